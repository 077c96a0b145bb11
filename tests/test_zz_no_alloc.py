"""GPU: the allocation-free backward (fa_bwd_noalloc, the library's fixed
device scratch in place of a workspace) against fa_bwd on the same inputs:
two calls in a row, the second smaller, each bitwise equal to fa_bwd (the
same kernels run) and within the bf16 bound of the float64 oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import check_bf16, dev_bf16_bits, dev_bf16_to_f64, dev_inputs, require_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, Hkv, N, d, causal, seed -- the second call is the smaller one
    ("first_larger", 2, 8, 4, 1024, 128, True, 501),
    ("second_smaller", 1, 4, 2, 300, 64, False, 502),
]


def test_noalloc_matches_fa_bwd_two_calls_in_a_row():
    torch, fa = require_gpu()
    for name, B, H, Hkv, N, d, causal, seed in CASES:
        w = W.small_case(name, "bf16", B, H, Hkv, N, d, causal, seed, backward=True)
        inp = W.gen_inputs(w)
        q, k, v, do = dev_inputs(inp, torch)
        o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=w.scale)
        ref = fa.fa_bwd(q, k, v, o, lse, do, causal=causal, scale=w.scale)
        got = tuple(torch.full_like(t, float("nan")) for t in ref)
        fa.fa_bwd_noalloc(q, k, v, o, lse, do, *got, causal=causal, scale=w.scale)
        torch.cuda.synchronize()
        for n, x, y in zip(("dq", "dk", "dv"), ref, got):
            assert np.array_equal(dev_bf16_bits(x), dev_bf16_bits(y)), (name, n)
        dQ, dK, dV = oracle.attention_bwd(inp.q, inp.k, inp.v, inp.do, causal, w.scale)
        for n, t, r in (("dq", got[0], dQ), ("dk", got[1], dK), ("dv", got[2], dV)):
            info = check_bf16(dev_bf16_to_f64(t), r, f"{name} {n}")
            print(name, n, info, flush=True)


def test_noalloc_refuses_more_rows_than_its_scratch():
    torch, fa = require_gpu()
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    big = torch.zeros((1, 1, (1 << 22) + 64, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, big.shape[2]), dtype=torch.float32, device="cuda")
    outs = [torch.empty_like(big) for _ in range(3)]
    with pytest.raises(fa.FattnError) as e:
        fa.fa_bwd_noalloc(big, big, big, big, lse, big, *outs, causal=True)
    assert e.value.status == fa.FA_ERR_TOO_LARGE
    del q
