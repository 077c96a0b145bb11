"""GPU parity of the forward pass (fa_fwd, fa_fwd_f32) against the float64
oracle on the same seeded inputs.  Tolerances: see tests/gpu_util.py."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import (check_bf16, check_f32, check_lse, dev_bf16_bits, dev_bf16_to_f64,
                      dev_inputs, dev_to_f64, require_gpu)

pytestmark = pytest.mark.gpu


def run_fwd(inp, fa, torch, causal=None, scale=None):
    w = inp.w
    q, k, v, _ = dev_inputs(inp, torch)
    causal = w.causal if causal is None else causal
    scale = w.scale if scale is None else scale
    f = fa.fa_fwd if w.dtype == "bf16" else fa.fa_fwd_f32
    o, lse = f(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def compare_full(inp, o, lse, causal, scale, what):
    O, L = oracle.attention_fwd(inp.q, inp.k, inp.v, causal, scale)
    if inp.w.dtype == "bf16":
        info = check_bf16(dev_bf16_to_f64(o), O, what)
    else:
        info = {"max_abs": check_f32(dev_to_f64(o), O, what)}
    info["lse_max_abs"] = check_lse(dev_to_f64(lse), L, what)
    print(what, info, flush=True)
    return info


SMALL = [
    # name, dtype, B, H, Hkv, N, d, causal, seed
    ("bf16_d128_causal_ragged", "bf16", 2, 4, 2, 300, 128, True, 101),
    ("bf16_d128_noncausal_ragged", "bf16", 2, 4, 2, 300, 128, False, 102),
    ("bf16_d64_causal_ragged", "bf16", 1, 4, 1, 520, 64, True, 103),
    ("bf16_d64_noncausal_ragged", "bf16", 1, 2, 2, 257, 64, False, 104),
    ("bf16_d128_N1_causal", "bf16", 1, 2, 1, 1, 128, True, 105),
    ("bf16_d128_N1_noncausal", "bf16", 1, 2, 1, 1, 128, False, 106),
    ("bf16_d128_N17", "bf16", 1, 2, 2, 17, 128, True, 107),
    ("bf16_d128_N64", "bf16", 1, 2, 2, 64, 128, True, 108),
    ("bf16_d128_N128", "bf16", 1, 2, 2, 128, 128, True, 109),
    ("bf16_d128_N129", "bf16", 1, 2, 2, 129, 128, False, 110),
    ("bf16_d128_N1000_gqa8", "bf16", 1, 8, 1, 1000, 128, True, 111),
    # causal rows of 512+ keys on small grids take the key-split path; these
    # two put one and two query heads in a workgroup
    ("bf16_d128_N600_gqa2_split", "bf16", 2, 4, 2, 600, 128, True, 112),
    ("bf16_d64_N700_mha_split", "bf16", 1, 2, 2, 700, 64, True, 113),
    ("f32_d64_causal_ragged", "f32", 2, 4, 2, 300, 64, True, 121),
    ("f32_d128_noncausal_ragged", "f32", 1, 4, 4, 200, 128, False, 122),
    ("f32_d128_causal", "f32", 1, 2, 1, 256, 128, True, 123),
    ("f32_d64_N1", "f32", 1, 1, 1, 1, 64, True, 124),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases(case):
    torch, fa = require_gpu()
    name, dtype, B, H, Hkv, N, d, causal, seed = case
    inp = W.gen_inputs(W.small_case(name, dtype, B, H, Hkv, N, d, causal, seed))
    o, lse = run_fwd(inp, fa, torch)
    compare_full(inp, o, lse, causal, inp.w.scale, name)


def test_c3_recipe_reduced_with_outliers():
    # C3's structure (32 query heads on 8 kv heads, 1% of key rows x8) at N=1000.
    torch, fa = require_gpu()
    w = W.C3.with_(N=1000)
    inp = W.gen_inputs(w)
    o, lse = run_fwd(inp, fa, torch)
    compare_full(inp, o, lse, True, w.scale, "C3-reduced N=1000")


def test_c1_fp32_full():
    torch, fa = require_gpu()
    inp = W.gen_inputs(W.C1)
    o, lse = run_fwd(inp, fa, torch)
    compare_full(inp, o, lse, False, W.C1.scale, "C1")


def test_c2_full():
    torch, fa = require_gpu()
    inp = W.gen_inputs(W.C2)
    o, lse = run_fwd(inp, fa, torch)
    compare_full(inp, o, lse, True, W.C2.scale, "C2")


def _lse_bounds(inp, lse_dev, what):
    """Checks on every row that cost O(N d): LSE finite; LSE_i >= s_ii (key i
    is always visible); LSE_i <= scale |q_i| max_{j<=i} |k_j| + ln(i+1)
    (Cauchy-Schwarz on every visible score)."""
    w = inp.w
    L = dev_to_f64(lse_dev)
    assert np.isfinite(L).all(), what
    N = w.N
    for b in range(w.B):
        for h in range(w.H):
            g = oracle.kv_head_of(h, w.H, w.Hkv)
            q = inp.q[b, h].astype(np.float64)
            k = inp.k[b, g].astype(np.float64)
            sii = w.scale * np.einsum("ij,ij->i", q, k)
            assert (L[b, h] >= sii - 1e-3).all(), (what, b, h)
            kmax = np.maximum.accumulate(np.linalg.norm(k, axis=1))
            ub = w.scale * np.linalg.norm(q, axis=1) * kmax + np.log(np.arange(1, N + 1))
            assert (L[b, h] <= ub + 1e-3).all(), (what, b, h)


def _compare_rows(inp, o, lse, rows, what):
    Or, Lr = oracle.attention_rows(inp.q, inp.k, inp.v, inp.w.causal, inp.w.scale, rows)
    ob = dev_bf16_bits(o)
    L = dev_to_f64(lse)
    got = np.stack([W.bf16_bits_to_f32(ob[b, h, i]) for b, h, i in rows]).astype(np.float64)
    info = check_bf16(got, Or, what)
    info["lse_max_abs"] = check_lse(np.array([L[b, h, i] for b, h, i in rows]), Lr, what)
    print(what, info, flush=True)


def test_c3_full_size():
    torch, fa = require_gpu()
    w = W.C3
    inp = W.gen_inputs(w)
    o, lse = run_fwd(inp, fa, torch)
    # every head, element by element (rows dominated by one outlier key are
    # rare; sampling rows alone can miss them)
    for h in range(w.H):
        g = oracle.kv_head_of(h, w.H, w.Hkv)
        O, L = oracle.attention_fwd(inp.q[:, h:h + 1], inp.k[:, g:g + 1], inp.v[:, g:g + 1],
                                    True, w.scale)
        check_bf16(dev_bf16_to_f64(o[:, h:h + 1]), O, f"C3 head {h}")
        check_lse(dev_to_f64(lse[:, h:h + 1]), L, f"C3 head {h}")
    # 1024 sampled rows over all heads
    rng = np.random.default_rng(33)
    hi = W.sample_rows(rng, w.H, w.N, 1024)
    rows = np.concatenate([np.zeros((len(hi), 1), np.int64), hi], axis=1)
    _compare_rows(inp, o, lse, rows, "C3 sampled rows")
    _lse_bounds(inp, lse, "C3")


def test_c4_full_size_sampled_rows_prefix_and_workspace():
    torch, fa = require_gpu()
    w = W.C4
    inp = W.gen_inputs(w)
    q, k, v, _ = dev_inputs(inp, torch)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    # warm-up launch on a slice, so lazy code-object loading is not measured
    fa.fa_fwd(q[:, :, :256].contiguous(), k[:, :, :256].contiguous(), v[:, :, :256].contiguous(),
              causal=True, scale=w.scale)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    fa.fa_fwd(q, k, v, o=o, lse=lse, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    delta_long = (torch.cuda.max_memory_allocated() - alloc0, free0 - free1)

    rows = np.concatenate([np.zeros((len(inp.sampled_rows), 1), np.int64), inp.sampled_rows], axis=1)
    _compare_rows(inp, o, lse, rows, "C4 sampled rows")
    _lse_bounds(inp, lse, "C4")
    # one whole head per kv head, every row and column (a few seconds of host
    # time per head for the float64 oracle at this length on a 16-core host)
    for h in range(w.H // w.Hkv - 1, w.H, w.H // w.Hkv):
        g = oracle.kv_head_of(h, w.H, w.Hkv)
        O, L = oracle.attention_fwd(inp.q[:, h:h + 1], inp.k[:, g:g + 1], inp.v[:, g:g + 1],
                                    True, w.scale)
        info = check_bf16(dev_bf16_to_f64(o[:, h:h + 1]), O, f"C4 head {h}")
        info["lse_max_abs"] = check_lse(dev_to_f64(lse[:, h:h + 1]), L, f"C4 head {h}")
        print(f"C4 head {h}", info, flush=True)

    # Prefix consistency: causal rows i < 8192 see only keys < 8192, so a run
    # on the truncated inputs must give the same rows (same tile order: bitwise).
    n8 = 8192
    q8, k8, v8 = (t[:, :, :n8].contiguous() for t in (q, k, v))
    o8 = torch.empty_like(q8)
    l8 = torch.empty((w.B, w.H, n8), dtype=torch.float32, device=q.device)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    fa.fa_fwd(q8, k8, v8, o=o8, lse=l8, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    delta_short = (torch.cuda.max_memory_allocated() - alloc0, free0 - free1)
    assert np.array_equal(dev_bf16_bits(o8), dev_bf16_bits(o[:, :, :n8]))
    assert torch.equal(l8, lse[:, :, :n8])
    # the forward allocates nothing: workspace is zero at every N
    print("workspace deltas (torch peak, device free)", delta_long, delta_short, flush=True)
    assert delta_long == (0, 0) and delta_short == (0, 0)


def test_causal_row0_is_v0_bitwise():
    torch, fa = require_gpu()
    w = W.small_case("row0", "bf16", 2, 8, 2, 700, 128, True, 131)
    inp = W.gen_inputs(w)
    o, lse = run_fwd(inp, fa, torch)
    ob = dev_bf16_bits(o)
    L = dev_to_f64(lse)
    for b in range(w.B):
        for h in range(w.H):
            g = h // 4
            assert np.array_equal(ob[b, h, 0], inp.v_bits[b, g, 0])
            s00 = w.scale * float(inp.q[b, h, 0].astype(np.float64) @ inp.k[b, g, 0])
            assert abs(L[b, h, 0] - s00) <= 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_values(causal):
    torch, fa = require_gpu()
    w = W.small_case("samekeys", "bf16", 1, 2, 1, 333, 128, causal, 141)
    inp = W.gen_inputs(w)
    inp.k_bits[:] = inp.k_bits[:, :, :1]
    inp.k = W.bf16_bits_to_f32(inp.k_bits)
    o, lse = run_fwd(inp, fa, torch)
    v = inp.v[0, 0].astype(np.float64)
    cnt = np.arange(1, w.N + 1)[:, None] if causal else w.N
    mean = (np.cumsum(v, axis=0) / cnt) if causal else np.broadcast_to(v.mean(0), v.shape)
    for h in range(2):
        check_bf16(dev_bf16_to_f64(o[0, h]), mean, f"identical keys h={h}")


def test_deterministic_bitwise():
    torch, fa = require_gpu()
    inp = W.gen_inputs(W.C3.with_(N=2048))
    o1, l1 = run_fwd(inp, fa, torch)
    o2, l2 = run_fwd(inp, fa, torch)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.5])
def test_other_scales(scale):
    torch, fa = require_gpu()
    for dtype in ("bf16", "f32"):
        inp = W.gen_inputs(W.small_case("scale", dtype, 1, 2, 1, 200, 64, True, 151))
        o, lse = run_fwd(inp, fa, torch, scale=scale)
        compare_full(inp, o, lse, True, scale, f"{dtype} scale={scale}")


def test_empty_problem_is_a_noop():
    torch, fa = require_gpu()
    q = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = fa.fa_fwd(q, q[:, :1], q[:, :1], causal=True)
    assert o.shape == (1, 2, 0, 128) and lse.shape == (1, 2, 0)


@pytest.mark.parametrize("causal", [False, True])
def test_growing_keys_force_many_rebases(causal):
    # Key rows scaled by 1 + j/16 make the scores of later keys grow far past
    # the reference taken on the first tile (hundreds of log2 units by the end
    # of the sequence), so the reference is raised and O, l rebased on many
    # tiles; d=128 and d=64, bf16 (exact scaling up to rounding of the products,
    # applied to the float draws before the bf16 rounding).
    torch, fa = require_gpu()
    for d, seed in ((128, 161), (64, 162)):
        w = W.small_case(f"growing_keys_d{d}", "bf16", 1, 4, 2, 1000, d, causal, seed)
        inp = W.gen_inputs(w)
        grow = (1.0 + np.arange(w.N, dtype=np.float32) / 16.0)[None, None, :, None]
        inp.k_bits = W.bf16_rne_bits(W.bf16_bits_to_f32(inp.k_bits) * grow)
        inp.k = W.bf16_bits_to_f32(inp.k_bits)
        o, lse = run_fwd(inp, fa, torch)
        compare_full(inp, o, lse, causal, w.scale, f"growing keys d={d} causal={causal}")
