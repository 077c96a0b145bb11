"""Seeded input generation: bf16 encoding, determinism, workload structure."""
import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_rne_matches_torch_bitwise():
    rng = np.random.default_rng(123)
    x = np.concatenate([
        rng.standard_normal(200_000, dtype=np.float32) * np.float32(3.0),
        (rng.standard_normal(50_000, dtype=np.float32) * np.float32(1e30)),
        (rng.standard_normal(50_000, dtype=np.float32) * np.float32(1e-38)),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38,
                  1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9], dtype=np.float32),
    ])
    # random bit patterns too (excluding NaNs, compared separately)
    raw = rng.integers(0, 2 ** 32, size=100_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, raw[~np.isnan(raw)]])
    ours = W.bf16_rne_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_nan_and_roundtrip():
    bits = W.bf16_rne_bits(np.array([np.nan], dtype=np.float32))
    assert bits[0] == 0x7FC0
    allbits = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    f = W.bf16_bits_to_f32(allbits)
    ok = ~np.isnan(f)
    assert np.array_equal(W.bf16_rne_bits(f[ok]), allbits[ok])


def test_generation_is_deterministic_and_shaped():
    w = W.small_case("t", "bf16", 2, 4, 2, 100, 64, True, 7, backward=True)
    a = W.gen_inputs(w)
    b = W.gen_inputs(w)
    for name in ("q", "k", "v", "do"):
        assert np.array_equal(getattr(a, name + "_bits"), getattr(b, name + "_bits"))
    assert a.q.shape == (2, 4, 100, 64) and a.k.shape == (2, 2, 100, 64)
    assert a.do.shape == a.q.shape
    # the float view is exactly the decoded bits
    assert np.array_equal(W.bf16_rne_bits(a.q), a.q_bits)


def test_fp32_workload_has_no_rounding():
    a = W.gen_inputs(W.C1)
    assert a.q.dtype == np.float32 and a.q_bits is None
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 256, 64), dtype=np.float32)
    assert np.array_equal(a.q, q)


def test_c3_outliers():
    w = W.C3.with_(N=1024)   # same recipe, smaller N
    a = W.gen_inputs(w)
    n_out = int(round(0.01 * 1024))
    assert a.outlier_rows.shape == (1, 8, n_out)
    rng = np.random.default_rng(w.seed)
    q = rng.standard_normal((1, 32, 1024, 128), dtype=np.float32)
    k = rng.standard_normal((1, 8, 1024, 128), dtype=np.float32)
    kb = W.bf16_round(k)
    for g in range(8):
        idx = a.outlier_rows[0, g]
        assert len(np.unique(idx)) == n_out
        assert np.array_equal(a.k[0, g, idx], kb[0, g, idx] * 8)   # x8 exact in bf16
        rest = np.setdiff1d(np.arange(1024), idx)
        assert np.array_equal(a.k[0, g, rest], kb[0, g, rest])


def test_c4_sampled_rows_include_fixed_rows():
    rng = np.random.default_rng(4)
    rows = W.sample_rows(rng, 32, 32768, 512)
    assert rows.shape == (512, 2)
    assert len({(int(h), int(i)) for h, i in rows}) == 512
    idx = set(int(i) for i in rows[:, 1])
    assert {0, 127, 128, 32767} <= idx


def test_workload_counts():
    assert W.C3.causal_adjusted_flops() == pytest.approx(549.755813888e9)
    assert W.C3.compulsory_bytes() == (64 + 32 + 64 + 1) * 2 ** 20
