"""GPU parity of the bf16 forward at sizes that launch the 8-wave workgroup
shape for every variant: non-causal, d=64, two query heads per workgroup,
a ragged sequence and a local window above 2048 keys.  Smaller parity cases
stay under the 512-workgroup switch and run the 4-wave shape only, so these
cases are the evidence for the instances realistic calls take ("LLM
Architecture Refresh [3]: Flash Attention Is Exact", section 4 -- short tiles
at the end of the sequence -- and section 5, exactness with the causal mask
off and on).  Each case asserts the shape its sizes select, compares every
head element by element with the float64 oracle, and checks the LSE of every
row."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import (check_bf16, check_lse, dev_bf16_bits, dev_bf16_to_f64, dev_inputs,
                      dev_to_f64, fwd_launch_shape, require_gpu)

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, Hkv, N, d, causal, window, seed, expected (waves, hp)
    ("d128_noncausal_hp4", 1, 32, 8, 4096, 128, False, 0, 301, (8, 4)),
    ("d64_causal_hp4", 1, 32, 8, 4096, 64, True, 0, 302, (8, 4)),
    ("d64_noncausal_hp4_ragged", 1, 32, 8, 4100, 64, False, 0, 303, (8, 4)),
    ("d128_causal_hp2", 2, 16, 8, 4096, 128, True, 0, 304, (8, 2)),
    ("d64_noncausal_hp2", 2, 16, 8, 4096, 64, False, 0, 305, (8, 2)),
    ("d128_causal_hp1_ragged", 1, 32, 32, 4100, 128, True, 0, 306, (8, 1)),
    ("d64_local3000_hp4", 1, 32, 8, 4096, 64, True, 3000, 307, (8, 4)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_eight_wave_shape_whole_heads(case):
    name, B, H, Hkv, N, d, causal, window, seed, expect = case
    waves, hp, items = fwd_launch_shape(B, H, Hkv, N, causal, window)
    assert (waves, hp) == expect and items >= 512, (name, waves, hp, items)
    torch, fa = require_gpu()
    w = W.small_case(name, "bf16", B, H, Hkv, N, d, causal, seed)
    inp = W.gen_inputs(w)
    q, k, v, _ = dev_inputs(inp, torch)
    if window:
        o, lse = fa.fa_fwd_local(q, k, v, window, scale=w.scale)
    else:
        o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    got_o = dev_bf16_to_f64(o)
    got_l = dev_to_f64(lse)
    worst = {"max_abs": 0.0, "lse_max_abs": 0.0, "n_over_1e2": 0}
    for b in range(B):
        for h in range(H):
            g = oracle.kv_head_of(h, H, Hkv)
            O, L = oracle.attention_fwd(inp.q[b:b + 1, h:h + 1], inp.k[b:b + 1, g:g + 1],
                                        inp.v[b:b + 1, g:g + 1], causal, w.scale,
                                        window=window or None)
            info = check_bf16(got_o[b:b + 1, h:h + 1], O, f"{name} b={b} h={h}")
            e = check_lse(got_l[b:b + 1, h:h + 1], L, f"{name} b={b} h={h}")
            worst["max_abs"] = max(worst["max_abs"], info["max_abs"])
            worst["n_over_1e2"] += info["n_over_1e2"]
            worst["lse_max_abs"] = max(worst["lse_max_abs"], e)
    print(name, (waves, hp, items), worst, flush=True)


def test_c3_shape_noncausal_sampled_rows():
    # The headline head layout (32 query heads on 8 kv heads, N=8192, d=128,
    # 1% of key rows x8) with the causal mask off: 8-wave, 4 heads per
    # workgroup.  Two whole heads element by element, then 1024 sampled rows.
    w = W.C3.with_(causal=False)
    waves, hp, items = fwd_launch_shape(w.B, w.H, w.Hkv, w.N, False)
    assert (waves, hp) == (8, 4) and items >= 512
    torch, fa = require_gpu()
    inp = W.gen_inputs(w)
    q, k, v, _ = dev_inputs(inp, torch)
    o, lse = fa.fa_fwd(q, k, v, causal=False, scale=w.scale)
    torch.cuda.synchronize()
    for h in (0, w.H - 1):
        g = oracle.kv_head_of(h, w.H, w.Hkv)
        O, L = oracle.attention_fwd(inp.q[:, h:h + 1], inp.k[:, g:g + 1], inp.v[:, g:g + 1],
                                    False, w.scale)
        info = check_bf16(dev_bf16_to_f64(o[:, h:h + 1]), O, f"C3 non-causal head {h}")
        info["lse_max_abs"] = check_lse(dev_to_f64(lse[:, h:h + 1]), L, f"C3 non-causal head {h}")
        print("C3 non-causal head", h, info, flush=True)
    rng = np.random.default_rng(333)
    hi = W.sample_rows(rng, w.H, w.N, 1024)
    rows = np.concatenate([np.zeros((len(hi), 1), np.int64), hi], axis=1)
    Or, Lr = oracle.attention_rows(inp.q, inp.k, inp.v, False, w.scale, rows)
    ob = dev_bf16_bits(o)
    L = dev_to_f64(lse)
    got = np.stack([W.bf16_bits_to_f32(ob[b, h, i]) for b, h, i in rows]).astype(np.float64)
    info = check_bf16(got, Or, "C3 non-causal sampled rows")
    info["lse_max_abs"] = check_lse(np.array([L[b, h, i] for b, h, i in rows]), Lr,
                                    "C3 non-causal sampled rows")
    print("C3 non-causal sampled rows", info, flush=True)
