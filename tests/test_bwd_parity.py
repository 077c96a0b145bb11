"""GPU parity of the backward pass (fa_bwd) against the float64 oracle.

fa_bwd receives the O and LSE that fa_fwd produced on the GPU (its intended
use); the oracle computes the exact gradient of the definition from the same
bf16 inputs.  Tolerance: the bf16 rule of tests/gpu_util.py, applied to
dQ, dK and dV."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import check_bf16, dev_bf16_bits, dev_bf16_to_f64, dev_inputs, require_gpu

pytestmark = pytest.mark.gpu


def run_fwd_bwd(inp, fa, torch):
    w = inp.w
    q, k, v, do = dev_inputs(inp, torch)
    o, lse = fa.fa_fwd(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def compare(inp, dq, dk, dv, what, heads=None):
    w = inp.w
    dQ, dK, dV = oracle.attention_bwd(inp.q, inp.k, inp.v, inp.do, w.causal, w.scale, heads=heads)
    if heads is None:
        parts = [("dq", dq, dQ), ("dk", dk, dK), ("dv", dv, dV)]
        res = {n: check_bf16(dev_bf16_to_f64(a), b, f"{what} {n}") for n, a, b in parts}
    else:
        res = {}
        for b, h in heads:
            g = oracle.kv_head_of(h, w.H, w.Hkv)
            res[(b, h, "dq")] = check_bf16(dev_bf16_to_f64(dq[b, h]), dQ[b, h], f"{what} dq[{b},{h}]")
        kv = sorted({(b, oracle.kv_head_of(h, w.H, w.Hkv)) for b, h in heads})
        for b, g in kv:
            res[(b, g, "dk")] = check_bf16(dev_bf16_to_f64(dk[b, g]), dK[b, g], f"{what} dk[{b},{g}]")
            res[(b, g, "dv")] = check_bf16(dev_bf16_to_f64(dv[b, g]), dV[b, g], f"{what} dv[{b},{g}]")
    print(what, res, flush=True)
    return res


SMALL = [
    # name, B, H, Hkv, N, d, causal, seed
    ("d128_causal_ragged", 2, 4, 2, 300, 128, True, 201),
    ("d128_noncausal_ragged", 1, 4, 4, 300, 128, False, 202),
    ("d64_causal_ragged", 1, 4, 1, 260, 64, True, 203),
    ("d64_noncausal", 1, 2, 2, 256, 64, False, 204),
    ("d128_N1", 1, 2, 1, 1, 128, True, 205),
    ("d128_N17", 1, 2, 2, 17, 128, True, 206),
    ("d128_N129", 1, 2, 2, 129, 128, False, 207),
    ("d128_gqa8_N700", 1, 8, 1, 700, 128, True, 208),
    # every (d, causal, group size) combination of the dK/dV instances: P and dS
    # enter as one bf16 value for one head per kv head, P as a hi + lo pair
    # from two heads on, dS as well from four on
    ("d128_noncausal_gqa2", 1, 4, 2, 200, 128, False, 209),
    ("d128_noncausal_gqa4", 1, 4, 1, 200, 128, False, 210),
    ("d128_causal_gqa3", 1, 6, 2, 400, 128, True, 214),
    ("d64_causal_mha", 1, 2, 2, 330, 64, True, 211),
    ("d64_causal_gqa3", 1, 6, 2, 260, 64, True, 212),
    ("d64_noncausal_gqa2", 1, 4, 2, 200, 64, False, 215),
    ("d64_noncausal_gqa8", 1, 8, 1, 200, 64, False, 213),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases(case):
    torch, fa = require_gpu()
    name, B, H, Hkv, N, d, causal, seed = case
    inp = W.gen_inputs(W.small_case(name, "bf16", B, H, Hkv, N, d, causal, seed, backward=True))
    dq, dk, dv = run_fwd_bwd(inp, fa, torch)
    compare(inp, dq, dk, dv, name)


# dK/dV fetches its 64-query tiles three ahead into two register sets and runs
# two iterations per loop trip: a key block's tile count (query heads of its
# group x visible query tiles) sets which paths run.  Causal, one head per kv
# head: the first key block sees N/64 tiles, 1 .. 5 here; two heads per kv
# head non-causal: 2 * N/64 = 2 .. 10; three heads, ragged N: odd counts.
TILE_COUNTS = [
    ("mha_causal_N64", 1, 2, 2, 64, 128, True, 231),
    ("mha_causal_N128", 1, 2, 2, 128, 128, True, 232),
    ("mha_causal_N192", 1, 2, 2, 192, 128, True, 233),
    ("mha_causal_N256", 1, 2, 2, 256, 128, True, 234),
    ("mha_causal_N320", 1, 2, 2, 320, 128, True, 235),
    ("gqa2_noncausal_N64", 1, 4, 2, 64, 128, False, 236),
    ("gqa2_noncausal_N320", 1, 4, 2, 320, 128, False, 237),
    ("gqa3_causal_N100_d64", 1, 6, 2, 100, 64, True, 238),
    ("gqa3_noncausal_N190_d64", 1, 6, 2, 190, 64, False, 239),
]


@pytest.mark.parametrize("case", TILE_COUNTS, ids=[c[0] for c in TILE_COUNTS])
def test_dkdv_tile_counts(case):
    torch, fa = require_gpu()
    name, B, H, Hkv, N, d, causal, seed = case
    inp = W.gen_inputs(W.small_case(name, "bf16", B, H, Hkv, N, d, causal, seed, backward=True))
    dq, dk, dv = run_fwd_bwd(inp, fa, torch)
    compare(inp, dq, dk, dv, name)


def test_c5_reduced_full():
    # C5's recipe (B=2, H=16, causal, dO iid N(0,1)) at N=512, every element.
    torch, fa = require_gpu()
    inp = W.gen_inputs(W.C5.with_(N=512))
    dq, dk, dv = run_fwd_bwd(inp, fa, torch)
    compare(inp, dq, dk, dv, "C5 N=512")


def test_c5_full_size_all_heads():
    # Full size (B=2, H=16, N=4096, d=128, causal), in the launch configuration
    # the bench times: every element of dQ, dK and dV of all 32 heads against
    # the float64 oracle (about 0.7 s of host time per head).
    torch, fa = require_gpu()
    w = W.C5
    inp = W.gen_inputs(w)
    dq, dk, dv = run_fwd_bwd(inp, fa, torch)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    compare(inp, dq, dk, dv, "C5")


# Full-size shapes that take the other dK/dV instances and the non-causal
# kernels: every element of every head against the float64 oracle.
FULL = [
    # name, B, H, Hkv, N, d, causal, seed
    ("gqa4_causal_N4096", 1, 32, 8, 4096, 128, True, 241),    # hi + lo P and dS in dK/dV
    ("gqa2_causal_N4096", 1, 16, 8, 4096, 128, True, 242),    # hi + lo P in dK/dV
    ("mha_noncausal_N4096", 1, 8, 8, 4096, 128, False, 243),
]


@pytest.mark.parametrize("case", FULL, ids=[c[0] for c in FULL])
def test_full_size_shapes(case):
    name, B, H, Hkv, N, d, causal, seed = case
    torch, fa = require_gpu()
    w = W.C5.with_(name=name, B=B, H=H, Hkv=Hkv, N=N, d=d, causal=causal, seed=seed)
    inp = W.gen_inputs(w)
    dq, dk, dv = run_fwd_bwd(inp, fa, torch)
    compare(inp, dq, dk, dv, name)


def test_bwd_deterministic_bitwise():
    torch, fa = require_gpu()
    inp = W.gen_inputs(W.C5.with_(N=1024, B=1, H=4, Hkv=2))
    a = run_fwd_bwd(inp, fa, torch)
    b = run_fwd_bwd(inp, fa, torch)
    for x, y in zip(a, b):
        assert np.array_equal(dev_bf16_bits(x), dev_bf16_bits(y))


def test_bwd_rejects_short_workspace():
    torch, fa = require_gpu()
    q = torch.zeros((1, 2, 128, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 2, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        fa.fa_bwd(q, q, q, q, lse, q, workspace=ws, causal=True)


def test_bwd_does_not_read_o():
    # fa_bwd recomputes D_i = sum_j P_ij dP_ij from P and dP instead of
    # dO_i . O_i, so the `o` argument is validated but never read: an o full
    # of NaN must leave the gradients bitwise unchanged.
    torch, fa = require_gpu()
    inp = W.gen_inputs(W.C5.with_(N=640, B=1, H=4, Hkv=2))
    w = inp.w
    q, k, v, do = dev_inputs(inp, torch)
    o, lse = fa.fa_fwd(q, k, v, causal=True, scale=w.scale)
    ref = fa.fa_bwd(q, k, v, o, lse, do, causal=True, scale=w.scale)
    o_nan = torch.full_like(o, float("nan"))
    got = fa.fa_bwd(q, k, v, o_nan, lse, do, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for x, y in zip(ref, got):
        assert np.array_equal(dev_bf16_bits(x), dev_bf16_bits(y))
