"""Input generation: determinism, encoders against torch's CPU casts, workload sizes."""

import json
import os

import numpy as np
import pytest
import torch

from workloads import (WORKLOADS, bf16_bits_from_f32, bf16_bits_to_f64, by_name, e4m3fn_bits_from_f32,
                       e4m3fn_bits_to_f64, make_inputs)
from workloads.gen import from_f32, quantize_e4m3_per_tensor

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_encoder_matches_torch_random_and_edges():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(5_000_000).astype(np.float32),
        (rng.standard_normal(2_000_000) * 1e30).astype(np.float32),
        rng.integers(0, 2**32, 3_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45, 1.17549435e-38,
                  np.float32(1.00390625), np.float32(1.01171875), np.inf, -np.inf], dtype=np.float32),
    ])
    x = x[~np.isnan(x)]
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # ties go to even: 1 + 2**-8 lies halfway between bf16 1.0 and 1.0078125
    assert bf16_bits_from_f32(np.array([1.00390625], np.float32))[0] == 0x3F80
    assert bf16_bits_from_f32(np.array([1.01171875], np.float32))[0] == 0x3F82


def test_bf16_decode_roundtrip_all_finite_patterns():
    bits = np.arange(2**16, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f64(bits)
    fin = np.isfinite(vals)
    back = bf16_bits_from_f32(vals[fin].astype(np.float32))
    assert np.array_equal(back, bits[fin])


def test_e4m3fn_encoder_matches_torch_exhaustive_over_bf16():
    bits = np.arange(2**16, dtype=np.uint32).astype(np.uint16)
    x = bf16_bits_to_f64(bits).astype(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 464.0)]      # torch turns |x| >= 464 into NaN; we saturate
    ours = e4m3fn_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3fn_saturation_nan_and_decode():
    x = np.array([448.0, 464.0, 480.0, 1e6, np.inf, -1e6, -np.inf], np.float32)
    assert e4m3fn_bits_from_f32(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert e4m3fn_bits_from_f32(np.array([np.nan], np.float32))[0] & 0x7F == 0x7F
    allb = np.arange(256, dtype=np.uint8)
    vals = e4m3fn_bits_to_f64(allb)
    ref = torch.from_numpy(allb).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (vals == ref) | (np.isnan(vals) & np.isnan(ref))
    assert same.all()
    assert np.nanmax(vals) == 448.0 and np.nanmin(np.abs(vals[vals != 0])) == 2.0**-9


def test_per_tensor_quantisation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(10000).astype(np.float32) * 3
    bits, s = quantize_e4m3_per_tensor(x)
    deq = e4m3fn_bits_to_f64(bits) * s
    assert np.max(np.abs(deq)) <= 448 * s * (1 + 1e-7)
    assert np.abs(np.abs(deq).max() - np.abs(x).max()) <= 1e-6 * np.abs(x).max()  # amax maps onto 448
    rel = np.abs(deq - x) / np.maximum(np.abs(x), 2.0**-6 * s)
    assert rel.max() <= 2.0**-4 + 1e-9   # half an ulp of a 3-bit mantissa


@pytest.mark.parametrize("name", ["tiny_f32_b1h2n256d64", "bertl_bf16_b16h16n512d64"])
def test_generation_is_deterministic(name):
    w = by_name(name)
    a, b = make_inputs(w), make_inputs(w)
    for t in "qkv":
        assert np.array_equal(getattr(a, t), getattr(b, t))
    c = make_inputs(w, seed=w.seed + 100)
    assert not np.array_equal(a.q, c.q)


def test_dtypes_and_shapes():
    w = by_name("tiny_f32_b1h2n256d64")
    x = make_inputs(w)
    assert x.q.dtype == np.float32 and x.q.shape == (1, 2, 256, 64)
    w2 = w.with_(dtype="bf16")
    y = make_inputs(w2)
    assert y.q.dtype == np.uint16
    assert np.array_equal(y.f64("k"), bf16_bits_to_f64(bf16_bits_from_f32(x.k)))
    w3 = w.with_(dtype="fp8")
    z = make_inputs(w3)
    assert z.q.dtype == np.uint8 and all(s > 0 for s in z.descale)
    assert np.max(np.abs(z.f64("v") - y.f64("v"))) <= 2.0**-4 * np.max(np.abs(y.f64("v")))
    f = from_f32(w2, np.ones((1, 2, 256, 64)), x.k, x.v)
    assert np.all(f.f64("q") == 1.0)


def test_workload_table_closed_forms():
    with open(os.path.join(GOLDEN, "score_matrix_bytes.json")) as fh:
        g = json.load(fh)
    w = by_name("long_causal_bf16_b1h32n8192d128")
    assert w.B * w.H == g["batch_x_heads"] and w.N == g["seq_len"]
    nbytes = w.B * w.H * w.N * w.N * g["bytes_per_element"]
    assert nbytes == 2**32                      # 32 * 8192^2 * 2 = 4 GiB
    assert abs(nbytes / 1e9 - g["approx_gigabytes"]) / g["approx_gigabytes"] < 0.1
    # FLOP convention: 4*B*H*N^2*d, halved under the causal mask
    assert by_name("bertl_bf16_b16h16n512d64").flops == 4 * 16 * 16 * 512**2 * 64
    assert by_name("gpt2s_causal_bf16_b8h12n1024d64").flops == 2 * 8 * 12 * 1024**2 * 64
    assert len({w.name for w in WORKLOADS}) == len(WORKLOADS)
