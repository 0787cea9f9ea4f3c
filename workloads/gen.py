"""Workload table and seeded input generation (no attention arithmetic here).

The five shapes follow the workloads the FlashAttention pages discuss: a tiny
fp32 case, a GPT-2-small-shaped causal self-attention (the GPT-2 1K-length run
in "Wyniki empiryczne" of the systems-analysis page), a BERT-large-shaped one
(length 512, same section), a long-context causal case whose score matrix
would be 32 x 8192 x 8192 x 2 bytes (the chipfoundryservices glossary,
"Standard attention" paragraph) and a head-dim-256 case (FlashAttention-2
section of the systems-analysis page), the last one also in FP8 (the
FlashAttention-3 paragraphs of the pages).
"""

from dataclasses import dataclass, field, replace
import math

import numpy as np

from .encode import bf16_bits_from_f32, bf16_bits_to_f64, e4m3fn_bits_from_f32, e4m3fn_bits_to_f64, E4M3FN_MAX


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32" | "bf16" | "fp8"
    causal: bool
    seed: int
    scale: float = None  # default 1/sqrt(d)
    H_kv: int = None     # K/V heads (grouped-query attention); default H
    N_q: int = None      # query rows (decode shape: the last N_q of N keys); default N

    @property
    def softmax_scale(self):
        return 1.0 / math.sqrt(self.d) if self.scale is None else self.scale

    @property
    def kv_heads(self):
        return self.H if self.H_kv is None else self.H_kv

    @property
    def q_rows(self):
        return self.N if self.N_q is None else self.N_q

    @property
    def group(self):
        """Query heads per K/V head; query head h reads K/V head h // group."""
        return self.H // self.kv_heads

    @property
    def flops(self):
        """Matmul FLOPs by the usual convention 4*B*H*N^2*d, halved for causal
        (decode shape: 4*B*H*N_q*N*d, the mask removing almost nothing)."""
        if self.N_q is not None:
            return 4.0 * self.B * self.H * self.N_q * self.N * self.d
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    @property
    def elem_bytes(self):
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]

    @property
    def out_elem_bytes(self):
        return {"f32": 4, "bf16": 2, "fp8": 2}[self.dtype]

    @property
    def compulsory_bytes(self):
        """Q, K, V read once; O and the fp32 logsumexp written once."""
        n = self.B * self.H * self.q_rows
        nkv = self.B * self.kv_heads * self.N
        return (n + 2 * nkv) * self.d * self.elem_bytes + n * self.d * self.out_elem_bytes + 4 * n

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = [
    Workload("tiny_f32_b1h2n256d64", 1, 2, 256, 64, "f32", False, seed=1),
    Workload("gpt2s_causal_bf16_b8h12n1024d64", 8, 12, 1024, 64, "bf16", True, seed=2),
    Workload("bertl_bf16_b16h16n512d64", 16, 16, 512, 64, "bf16", False, seed=3),
    Workload("long_causal_bf16_b1h32n8192d128", 1, 32, 8192, 128, "bf16", True, seed=4),
    Workload("wide_bf16_b2h8n16384d256", 2, 8, 16384, 256, "bf16", False, seed=5),
    Workload("wide_fp8_b2h8n16384d256", 2, 8, 16384, 256, "fp8", False, seed=5),
    # grouped-query attention: 32 query heads over 8 K/V heads, long causal context
    Workload("gqa_causal_bf16_b1h32kv8n8192d128", 1, 32, 8192, 128, "bf16", True, seed=6, H_kv=8),
]


# decode shapes (split-KV): one new token per sequence against a long cache
DECODE_WORKLOADS = [
    Workload("decode_gqa_bf16_b8h32kv8q1n32768d128", 8, 32, 32768, 128, "bf16", True, seed=7, H_kv=8, N_q=1),
    Workload("decode_mha_bf16_b4h32q1n16384d128", 4, 32, 16384, 128, "bf16", True, seed=8, N_q=1),
    # the first one with an fp8 K/V cache (e4m3 Q, K, V with per-tensor descales)
    Workload("decode_gqa_fp8_b8h32kv8q1n32768d128", 8, 32, 32768, 128, "fp8", True, seed=7, H_kv=8, N_q=1),
]


def by_name(name):
    for w in WORKLOADS + DECODE_WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


@dataclass
class AttnInputs:
    """Storage-format tensors plus their exact float64 meaning: q [B,H,N,d],
    k and v [B,H_kv,N,d] (H_kv = H unless the workload groups query heads).

    q/k/v hold float32 values (f32), uint16 bf16 bits (bf16) or uint8 e4m3fn
    bits (fp8).  ``descale`` is (s_q, s_k, s_v): the value of an fp8 element is
    its e4m3 value times s (1.0 for the other dtypes).
    """
    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    descale: tuple = (1.0, 1.0, 1.0)

    def f64(self, which, b=None, h=None):
        """float64 values of q, k or v (optionally one (b, h) slice; h indexes that tensor's own
        heads) exactly as the kernel sees them."""
        x = getattr(self, which)
        if b is not None:
            x = x[b, h]
        dt = self.workload.dtype
        if dt == "f32":
            return x.astype(np.float64)
        if dt == "bf16":
            return bf16_bits_to_f64(x)
        s = {"q": 0, "k": 1, "v": 2}[which]
        return e4m3fn_bits_to_f64(x) * float(self.descale[s])


def _draw(B, H, N, d, seed, H_kv=None, N_q=None):
    rng = np.random.default_rng(seed)
    kv_shape = (B, H if H_kv is None else H_kv, N, d)
    q = rng.standard_normal((B, H, N if N_q is None else N_q, d), dtype=np.float32)
    k = rng.standard_normal(kv_shape, dtype=np.float32)
    v = rng.standard_normal(kv_shape, dtype=np.float32)
    return q, k, v


def quantize_e4m3_per_tensor(x32):
    """float32 tensor -> (e4m3fn bits, float32 descale s) with s = amax|x| / 448."""
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    s = np.float32(amax / np.float32(E4M3FN_MAX)) if amax > 0 else np.float32(1.0)
    bits = e4m3fn_bits_from_f32((x32 / s).astype(np.float32))
    return bits, float(s)


def make_inputs(w, seed=None):
    """Draw the inputs of workload ``w`` (optionally with another seed)."""
    seed = w.seed if seed is None else seed
    q, k, v = _draw(w.B, w.H, w.N, w.d, seed, w.kv_heads, w.N_q)
    if w.dtype == "f32":
        return AttnInputs(w, q, k, v)
    qb, kb, vb = bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v)
    del q, k, v
    if w.dtype == "bf16":
        return AttnInputs(w, qb, kb, vb)
    outs, scales = [], []
    for t in (qb, kb, vb):
        x32 = (t.astype(np.uint32) << 16).view(np.float32)
        bits, s = quantize_e4m3_per_tensor(x32)
        outs.append(bits)
        scales.append(s)
    return AttnInputs(w, outs[0], outs[1], outs[2], tuple(scales))


def from_f32(w, q, k, v):
    """Encode caller-built float32 tensors (structured test inputs) in the workload's dtype."""
    q, k, v = (np.ascontiguousarray(t, dtype=np.float32) for t in (q, k, v))
    if w.dtype == "f32":
        return AttnInputs(w, q, k, v)
    qb, kb, vb = bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v)
    if w.dtype == "bf16":
        return AttnInputs(w, qb, kb, vb)
    outs, scales = [], []
    for t in (qb, kb, vb):
        bits, s = quantize_e4m3_per_tensor((t.astype(np.uint32) << 16).view(np.float32))
        outs.append(bits)
        scales.append(s)
    return AttnInputs(w, outs[0], outs[1], outs[2], tuple(scales))


def make_grad_output(w, seed=None):
    """Upstream gradient dO [B, H, N, d] for the backward pass, as bf16 bits:
    ``standard_normal`` float32 from ``default_rng(seed + 7919)`` (a stream
    apart from the workload's Q, K, V), rounded to bfloat16."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed + 7919)
    return bf16_bits_from_f32(rng.standard_normal((w.B, w.H, w.q_rows, w.d), dtype=np.float32))
