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


# ---- FP8 (OCP E4M3) storage format -----------------------------------------

def test_e4m3_table_matches_the_format_definition():
    # values fixed by the OCP 8-bit floating point format, E4M3 variant
    t = W.E4M3_VALUES
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9            # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert t[0x08] == 2.0 ** -6            # smallest normal
    assert t[0x38] == 1.0
    assert t[0x3C] == 1.5
    assert t[0x7E] == 448.0                # largest finite
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0xFE] == -448.0 and t[0xB8] == -1.0
    finite = t[~np.isnan(t)]
    assert len(finite) == 254
    pos = t[1:0x7F]
    assert np.all(np.diff(pos) > 0)        # codes 0x01..0x7E increase


def test_e4m3_rounding_ties_to_even_and_saturates():
    enc = W.e4m3_rne_codes
    cases = {1.0625: 0x38, 1.1875: 0x3A, 3.0: 0x44, 2.0 ** -10: 0x00, 1.5 * 2.0 ** -10: 0x01,
             2.5 * 2.0 ** -9: 0x02, 3.5 * 2.0 ** -9: 0x04, 7.5 * 2.0 ** -9: 0x08, 464.0: 0x7E,
             1e6: 0x7E, -2.5: 0xC2, 232.0: 0x76, 0.3: 0x2A}
    for x, c in cases.items():
        assert enc(np.array([x]))[0] == c, (x, hex(c))
    assert enc(np.array([np.nan]))[0] == 0x7F


def test_e4m3_round_trip_and_nearest():
    codes = np.arange(256, dtype=np.uint8)
    vals = W.e4m3_decode(codes)
    ok = ~np.isnan(vals)
    assert np.array_equal(W.e4m3_rne_codes(vals[ok]), codes[ok])
    # nearest: no finite code is closer than the chosen one
    rng = np.random.default_rng(0)
    x = rng.standard_normal(2000) * np.exp2(rng.integers(-12, 9, 2000))
    x = np.clip(x, -448, 448)
    got = W.e4m3_decode(W.e4m3_rne_codes(x))
    grid = W.E4M3_VALUES[~np.isnan(W.E4M3_VALUES)]
    best = np.min(np.abs(x[:, None] - grid[None, :]), axis=1)
    assert np.all(np.abs(got - x) <= best + 0.0)


def test_fp8_workload_is_c3_quantized():
    w = W.F3.with_(N=256)
    inp = W.gen_inputs(w)
    ref = W.gen_inputs(W.C3.with_(N=256, dtype="f32"))
    for name in ("q", "k", "v"):
        codes = getattr(inp, name + "_codes")
        ds = inp.descale[name]
        assert codes.dtype == np.uint8 and codes.shape == getattr(ref, name).shape
        # the largest magnitude lands on +-448, and every value is the nearest
        # e4m3 point of the scaled draw
        assert np.max(np.abs(W.e4m3_decode(codes))) == 448.0
        np.testing.assert_array_equal(getattr(inp, name), W.e4m3_decode(codes) * ds)
        np.testing.assert_array_equal(codes, W.e4m3_rne_codes(getattr(ref, name).astype(np.float64) / ds))
