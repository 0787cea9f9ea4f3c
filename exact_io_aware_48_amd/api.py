"""Python binding of the C ABI (include/fa_fwd.h, fa_bwd.h, fa_split.h), same names,
argument marshalling only.

torch supplies device memory and streams; every step of the attention forward
and backward runs in the HIP kernels of libfa_fwd.so.  There is no fallback: if the library
is missing or a call fails, these functions raise.
"""

import ctypes
import math

import torch

from . import _lib

_DTYPE_CODE = {torch.float32: _lib.FA_F32, torch.bfloat16: _lib.FA_BF16}
_FP8_DTYPES = (torch.float8_e4m3fn, torch.uint8)


class FaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)}")


def fa_status_string(status):
    return _lib.load().fa_status_string(int(status)).decode()


def fa_version():
    return int(_lib.load().fa_version())


def fa_plan(B, H, N, d, causal=False, dtype=_lib.FA_BF16):
    """The launch fa_fwd would make (no GPU needed)."""
    lib = _lib.load()
    br, bc, thr, lds = (ctypes.c_int() for _ in range(4))
    wg, tiles = ctypes.c_int64(), ctypes.c_int64()
    st = lib.fa_plan(B, H, N, d, int(bool(causal)), int(dtype), ctypes.byref(br), ctypes.byref(bc),
                     ctypes.byref(wg), ctypes.byref(thr), ctypes.byref(lds), ctypes.byref(tiles))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_plan")
    return {"block_rows": br.value, "block_cols": bc.value, "workgroups": wg.value, "threads": thr.value,
            "lds_bytes": lds.value, "kv_tiles": tiles.value}


def _check(t, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 4 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")


def _check_out(t, name, shape, dtype, device):
    """A caller-supplied output buffer: the kernels write shape-many dtype
    elements through its pointer, so anything else is refused before a launch."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.device != torch.device(device):
        raise ValueError(f"{name} must be on {device}, not {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _outputs(o, lse, o_shape, o_dtype, lse_shape, device):
    """Allocate o and lse when not given, else check them."""
    o = torch.empty(o_shape, dtype=o_dtype, device=device) if o is None else _check_out(o, "o", o_shape, o_dtype, device)
    lse = (torch.empty(lse_shape, dtype=torch.float32, device=device) if lse is None
           else _check_out(lse, "lse", lse_shape, torch.float32, device))
    return o, lse


def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def fa_fwd(q, k, v, o=None, lse=None, scale=None, causal=False, stream=None):
    """O and per-row logsumexp of softmax(scale * Q K^T) V.

    q, k, v: contiguous [B, H, N, d] device tensors, float32 or bfloat16
    (float8_e4m3fn/uint8 bytes are taken with unit descales).  o, lse:
    optional preallocated outputs ([B,H,N,d] of the input dtype -- bfloat16
    for fp8 -- and float32 [B,H,N]).  Returns (o, lse).
    """
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, nm)
    if q.dtype in _FP8_DTYPES:
        return fa_fwd_fp8(q, k, v, 1.0, 1.0, 1.0, o=o, lse=lse, scale=scale, causal=causal, stream=stream)
    if q.dtype not in _DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError(f"unsupported dtypes {q.dtype}/{k.dtype}/{v.dtype}")
    B, H, N, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _outputs(o, lse, q.shape, q.dtype, (B, H, N), q.device)
    st = _lib.load().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            B, H, N, d, float(scale), int(bool(causal)), _DTYPE_CODE[q.dtype],
                            _stream_ptr(stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd")
    return o, lse


def fa_fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, o=None, lse=None, scale=None, causal=False,
               stream=None):
    """FP8 (OCP e4m3fn) inputs with per-tensor descales; bfloat16 O, float32 lse."""
    for t, nm in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        _check(t, nm)
        if t.dtype not in _FP8_DTYPES:
            raise ValueError(f"{nm} must be float8_e4m3fn or uint8 bytes")
    B, H, N, d = q8.shape
    if k8.shape != q8.shape or v8.shape != q8.shape:
        raise ValueError("q8, k8 and v8 must have the same shape")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _outputs(o, lse, (B, H, N, d), torch.bfloat16, (B, H, N), q8.device)
    st = _lib.load().fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                B, H, N, d, float(scale), float(q_descale), float(k_descale),
                                float(v_descale), int(bool(causal)), _stream_ptr(stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_fp8")
    return o, lse


def _gqa_shapes(q, k, v, names):
    B, H, N, d = q.shape
    if k.shape != v.shape or k.dim() != 4 or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"{names[1]} and {names[2]} must both be [B, H_kv, N, d] with q's B, N and d")
    H_kv = k.shape[1]
    if H_kv < 1 or H % H_kv:
        raise ValueError(f"{H} query heads do not split into groups over {H_kv} K/V heads")
    return B, H, H_kv, N, d


def fa_fwd_gqa(q, k, v, o=None, lse=None, scale=None, causal=False, stream=None):
    """Grouped-query attention: q [B, H, N, d], k and v [B, H_kv, N, d]; query head h
    attends over K/V head h // (H / H_kv).  Same dtypes, outputs and options as fa_fwd."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, nm)
    if q.dtype in _FP8_DTYPES:
        return fa_fwd_gqa_fp8(q, k, v, 1.0, 1.0, 1.0, o=o, lse=lse, scale=scale, causal=causal, stream=stream)
    if q.dtype not in _DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError(f"unsupported dtypes {q.dtype}/{k.dtype}/{v.dtype}")
    B, H, H_kv, N, d = _gqa_shapes(q, k, v, ("q", "k", "v"))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _outputs(o, lse, q.shape, q.dtype, (B, H, N), q.device)
    st = _lib.load().fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                B, H, H_kv, N, d, float(scale), int(bool(causal)), _DTYPE_CODE[q.dtype],
                                _stream_ptr(stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_gqa")
    return o, lse


def fa_fwd_gqa_fp8(q8, k8, v8, q_descale, k_descale, v_descale, o=None, lse=None, scale=None, causal=False,
                   stream=None):
    """fa_fwd_gqa on FP8 (OCP e4m3fn) inputs with per-tensor descales; bfloat16 O, float32 lse."""
    for t, nm in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        _check(t, nm)
        if t.dtype not in _FP8_DTYPES:
            raise ValueError(f"{nm} must be float8_e4m3fn or uint8 bytes")
    B, H, H_kv, N, d = _gqa_shapes(q8, k8, v8, ("q8", "k8", "v8"))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _outputs(o, lse, (B, H, N, d), torch.bfloat16, (B, H, N), q8.device)
    st = _lib.load().fa_fwd_gqa_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    B, H, H_kv, N, d, float(scale), float(q_descale), float(k_descale),
                                    float(v_descale), int(bool(causal)), _stream_ptr(stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_gqa_fp8")
    return o, lse


def _square(q, k, v, names=("q", "k", "v"), fp8=False):
    """q, k, v of one shape and one dtype (the FP8 dtypes when fp8, else float32 or bfloat16)."""
    for t, nm in zip((q, k, v), names):
        _check(t, nm)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"{', '.join(names)} must have the same shape")
    if fp8:
        if any(t.dtype not in _FP8_DTYPES for t in (q, k, v)):
            raise ValueError(f"{', '.join(names)} must be float8_e4m3fn or uint8 bytes")
    elif q.dtype not in _DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError(f"unsupported dtypes {q.dtype}/{k.dtype}/{v.dtype}")
    return q.shape


def _slopes(slopes, H):
    if (not isinstance(slopes, torch.Tensor) or slopes.dtype != torch.float32 or tuple(slopes.shape) != (H,)
            or slopes.device.type != "cuda"):
        raise ValueError("slopes must be a float32 device tensor [H]")
    return slopes.contiguous()


def _block_mask(block_mask, B, H, N):
    """(mask, stride_b, stride_h) for a [B, H, nb, nb], [H, nb, nb] or [nb, nb] block mask."""
    nb = (N + 127) // 128
    m = block_mask
    if not isinstance(m, torch.Tensor):
        raise ValueError("block_mask must be a tensor")
    if m.dtype == torch.bool:
        m = m.to(torch.uint8)
    if m.dtype != torch.uint8 or m.device.type != "cuda" or m.dim() < 2 or m.dim() > 4 or \
            tuple(m.shape[-2:]) != (nb, nb):
        raise ValueError(f"block_mask must be a uint8 device tensor [..., {nb}, {nb}]")
    if m.dim() >= 3 and m.shape[-3] != H or m.dim() == 4 and m.shape[0] != B:
        raise ValueError("block_mask leading dimensions must be [B, H] or [H]")
    m = m.contiguous()
    sb = nb * nb * m.shape[-3] if m.dim() == 4 else 0
    sh = nb * nb if m.dim() >= 3 else 0
    return m, sb, sh


def fa_fwd_alibi(q, k, v, slopes, o=None, lse=None, scale=None, causal=False, stream=None):
    """fa_fwd with ALiBi biases -slopes[h] * |i - j| on the scaled scores.
    q, k, v: [B, H, N, d] of any fa_fwd dtype (FP8 with unit descales); slopes:
    float32 device tensor [H].  Returns (o, lse)."""
    if q.dtype in _FP8_DTYPES:
        return fa_fwd_alibi_fp8(q, k, v, slopes, 1.0, 1.0, 1.0, o=o, lse=lse, scale=scale, causal=causal,
                                stream=stream)
    B, H, N, d = _square(q, k, v)
    slopes = _slopes(slopes, H)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _outputs(o, lse, q.shape, q.dtype, (B, H, N), q.device)
    st = _lib.load().fa_fwd_alibi(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  slopes.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                                  _DTYPE_CODE[q.dtype], _stream_ptr(stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_alibi")
    return o, lse


def fa_fwd_alibi_fp8(q8, k8, v8, slopes, q_descale, k_descale, v_descale, o=None, lse=None, scale=None,
                     causal=False, stream=None):
    """fa_fwd_alibi on FP8 (OCP e4m3fn) inputs with per-tensor descales; bfloat16 O, float32 lse."""
    B, H, N, d = _square(q8, k8, v8, ("q8", "k8", "v8"), fp8=True)
    slopes = _slopes(slopes, H)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _outputs(o, lse, (B, H, N, d), torch.bfloat16, (B, H, N), q8.device)
    st = _lib.load().fa_fwd_alibi_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      slopes.data_ptr(), B, H, N, d, float(scale), float(q_descale),
                                      float(k_descale), float(v_descale), int(bool(causal)), _stream_ptr(stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_alibi_fp8")
    return o, lse


def fa_fwd_blocksparse(q, k, v, block_mask, o=None, lse=None, scale=None, causal=False, stream=None):
    """fa_fwd restricted to the allowed 128 x 128 blocks of block_mask, a uint8 (or
    bool) device tensor [B, H, nb, nb], [H, nb, nb] or [nb, nb] with nb = ceil(N / 128);
    missing leading dimensions are shared.  Any fa_fwd dtype (FP8 with unit
    descales).  Returns (o, lse)."""
    if q.dtype in _FP8_DTYPES:
        return fa_fwd_blocksparse_fp8(q, k, v, block_mask, 1.0, 1.0, 1.0, o=o, lse=lse, scale=scale,
                                      causal=causal, stream=stream)
    B, H, N, d = _square(q, k, v)
    m, sb, sh = _block_mask(block_mask, B, H, N)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _outputs(o, lse, q.shape, q.dtype, (B, H, N), q.device)
    st = _lib.load().fa_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                        m.data_ptr(), sb, sh, B, H, N, d, float(scale), int(bool(causal)),
                                        _DTYPE_CODE[q.dtype], _stream_ptr(stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_blocksparse")
    return o, lse


def fa_fwd_blocksparse_fp8(q8, k8, v8, block_mask, q_descale, k_descale, v_descale, o=None, lse=None, scale=None,
                           causal=False, stream=None):
    """fa_fwd_blocksparse on FP8 (OCP e4m3fn) inputs with per-tensor descales; bfloat16 O, float32 lse."""
    B, H, N, d = _square(q8, k8, v8, ("q8", "k8", "v8"), fp8=True)
    m, sb, sh = _block_mask(block_mask, B, H, N)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _outputs(o, lse, (B, H, N, d), torch.bfloat16, (B, H, N), q8.device)
    st = _lib.load().fa_fwd_blocksparse_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(),
                                            lse.data_ptr(), m.data_ptr(), sb, sh, B, H, N, d, float(scale),
                                            float(q_descale), float(k_descale), float(v_descale),
                                            int(bool(causal)), _stream_ptr(stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_blocksparse_fp8")
    return o, lse


def _workspace(ws, need, device):
    """A scratch buffer of at least need bytes on device (allocated when not given)."""
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or ws.device != torch.device(device) or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds fewer than {need} bytes")
    return ws


def fa_bwd_workspace_size(B, H, H_kv, N, d):
    """Bytes of workspace fa_bwd needs (no GPU needed)."""
    n = ctypes.c_int64()
    st = _lib.load().fa_bwd_workspace_size(B, H, H_kv, N, d, ctypes.byref(n))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_bwd_workspace_size")
    return n.value


def fa_bwd(q, k, v, o, do, lse, scale=None, causal=False, dq=None, dk=None, dv=None, workspace=None,
           stream=None):
    """dQ, dK, dV of attention, recomputing P from q, k and the forward's lse.

    q, o, do: contiguous bfloat16 [B, H, N, d]; k, v: bfloat16 [B, H_kv, N, d]
    (H_kv dividing H); lse: float32 [B, H, N] from the forward.  dq, dk, dv:
    optional float32 outputs shaped like q, k, v; workspace: optional device
    buffer of at least fa_bwd_workspace_size(B, H, H_kv, N, d) bytes.  Returns (dq, dk, dv).
    """
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, nm)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{nm} must be bfloat16")
    B, H, H_kv, N, d = _gqa_shapes(q, k, v, ("q", "k", "v"))
    if o.shape != q.shape or do.shape != q.shape:
        raise ValueError("o and do must have q's shape")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if lse.device != q.device:
        raise ValueError(f"lse must be on {q.device}")
    grads = []
    for g, nm, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        grads.append(torch.empty(ref.shape, dtype=torch.float32, device=q.device) if g is None
                     else _check_out(g, nm, ref.shape, torch.float32, q.device))
    dq, dk, dv = grads
    need = fa_bwd_workspace_size(B, H, H_kv, N, d)
    workspace = _workspace(workspace, need, q.device)
    st = _lib.load().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                            workspace.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, H_kv, N, d,
                            float(scale), int(bool(causal)), _lib.FA_BF16, _stream_ptr(stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def fa_fwd_split_plan(B, H, H_kv, N_q, N_k, d, num_splits=0, fp8=False):
    """(splits, workspace bytes) fa_fwd_split (fa_fwd_split_fp8 when fp8) would use."""
    sp, nb = ctypes.c_int(), ctypes.c_int64()
    dtype = _lib.FA_FP8_E4M3 if fp8 else _lib.FA_BF16
    st = _lib.load().fa_fwd_split_plan(B, H, H_kv, N_q, N_k, d, int(num_splits), dtype, ctypes.byref(sp),
                                       ctypes.byref(nb))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_split_plan")
    return sp.value, nb.value


def fa_fwd_split(q, k, v, scale=None, causal=False, num_splits=0, o=None, lse=None, workspace=None, stream=None):
    """Split-KV attention for decode shapes: q [B, H, N_q, d] (the last N_q positions),
    k and v [B, H_kv, N_k, d] with N_q <= N_k, all bfloat16.  Returns (o, lse):
    bfloat16 [B, H, N_q, d] and float32 [B, H, N_q]."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, nm)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{nm} must be bfloat16")
    B, H, N_q, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must both be [B, H_kv, N_k, d] with q's B and d")
    H_kv, N_k = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _, need = fa_fwd_split_plan(B, H, H_kv, N_q, N_k, d, num_splits)
    workspace = _workspace(workspace, need, q.device)
    o, lse = _outputs(o, lse, q.shape, q.dtype, (B, H, N_q), q.device)
    st = _lib.load().fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  workspace.data_ptr(), B, H, H_kv, N_q, N_k, d, float(scale), int(bool(causal)),
                                  int(num_splits), _lib.FA_BF16, _stream_ptr(stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_split")
    return o, lse


def fa_fwd_split_fp8(q8, k8, v8, q_descale, k_descale, v_descale, scale=None, causal=False, num_splits=0, o=None,
                     lse=None, workspace=None, stream=None):
    """fa_fwd_split on FP8 (OCP e4m3fn) inputs with per-tensor descales: q8 [B, H, N_q, d],
    k8 and v8 [B, H_kv, N_k, d].  Returns (o, lse): bfloat16 [B, H, N_q, d] and float32 [B, H, N_q]."""
    for t, nm in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        _check(t, nm)
        if t.dtype not in _FP8_DTYPES:
            raise ValueError(f"{nm} must be float8_e4m3fn or uint8 bytes")
    B, H, N_q, d = q8.shape
    if k8.shape != v8.shape or k8.shape[0] != B or k8.shape[3] != d:
        raise ValueError("k8 and v8 must both be [B, H_kv, N_k, d] with q8's B and d")
    H_kv, N_k = k8.shape[1], k8.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _, need = fa_fwd_split_plan(B, H, H_kv, N_q, N_k, d, num_splits, fp8=True)
    workspace = _workspace(workspace, need, q8.device)
    o, lse = _outputs(o, lse, q8.shape, torch.bfloat16, (B, H, N_q), q8.device)
    st = _lib.load().fa_fwd_split_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      workspace.data_ptr(), B, H, H_kv, N_q, N_k, d, float(scale), float(q_descale),
                                      float(k_descale), float(v_descale), int(bool(causal)), int(num_splits),
                                      _stream_ptr(stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_split_fp8")
    return o, lse


def fa_split_scratch_bytes():
    """Size of the fixed device array fa_fwd_split_noalloc keeps its partials in."""
    return int(_lib.load().fa_split_scratch_bytes())


def fa_fwd_split_noalloc(q, k, v, o, lse, scale=None, causal=False, num_splits=0, stream=None):
    """fa_fwd_split for callers that cannot allocate: the partials go to the
    library's fixed per-GPU array instead of a workspace, and the outputs are
    the caller's (o bfloat16 [B, H, N_q, d], lse float32 [B, H, N_q]).  Calls
    that can overlap on one GPU race on that array.  Returns (o, lse)."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, nm)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{nm} must be bfloat16")
    B, H, N_q, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must both be [B, H_kv, N_k, d] with q's B and d")
    H_kv, N_k = k.shape[1], k.shape[2]
    if o is None or lse is None:
        raise ValueError("o and lse are the caller's buffers")
    _check_out(o, "o", q.shape, q.dtype, q.device)
    _check_out(lse, "lse", (B, H, N_q), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = _lib.load().fa_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                          B, H, H_kv, N_q, N_k, d, float(scale), int(bool(causal)), int(num_splits),
                                          _lib.FA_BF16, _stream_ptr(stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_fwd_split_noalloc")
    return o, lse


def fa_lse_merge(o_parts, lse_parts, out_dtype=torch.bfloat16, o=None, lse=None, stream=None):
    """Merge attention partials: o_parts float32 [S, rows, d], lse_parts float32 [S, rows].
    Returns (o [rows, d] of out_dtype (bfloat16 or float32), lse float32 [rows])."""
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("partials must be float32")
    if o_parts.dim() != 3 or lse_parts.shape != o_parts.shape[:2]:
        raise ValueError("o_parts must be [S, rows, d] and lse_parts [S, rows]")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()) or o_parts.device.type != "cuda":
        raise ValueError("partials must be contiguous device tensors")
    S, rows, d = o_parts.shape
    code = {torch.bfloat16: _lib.FA_BF16, torch.float32: _lib.FA_F32}.get(out_dtype)
    if code is None:
        raise ValueError("out_dtype must be bfloat16 or float32")
    o, lse = _outputs(o, lse, (rows, d), out_dtype, (rows,), o_parts.device)
    st = _lib.load().fa_lse_merge(o_parts.data_ptr(), lse_parts.data_ptr(), S, rows, d, o.data_ptr(), lse.data_ptr(),
                                  code, _stream_ptr(stream))
    if st != _lib.FA_OK:
        raise FaError(st, "fa_lse_merge")
    return o, lse
