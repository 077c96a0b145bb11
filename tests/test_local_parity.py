"""GPU parity of the local (sliding-window) causal forward, fa_fwd_local,
against the float64 oracle's window variant on the same seeded inputs.
Tolerances: see tests/gpu_util.py."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import (check_bf16, check_lse, dev_bf16_bits, dev_bf16_to_f64, dev_inputs,
                      dev_to_f64, require_gpu)

pytestmark = pytest.mark.gpu


def run_local(inp, fa, torch, window):
    q, k, v, _ = dev_inputs(inp, torch)
    o, lse = fa.fa_fwd_local(q, k, v, window, scale=inp.w.scale)
    torch.cuda.synchronize()
    return o, lse


SMALL = [
    # name, B, H, Hkv, N, d, window, seed
    ("w1", 1, 2, 1, 200, 128, 1, 201),
    ("w17_ragged_gqa", 2, 4, 2, 300, 128, 17, 202),
    ("w64_d64", 1, 4, 1, 520, 64, 64, 203),
    ("w100_N257", 1, 2, 2, 257, 128, 100, 204),
    ("w255_N700", 1, 4, 2, 700, 128, 255, 205),
    ("w256_N1000_gqa8", 1, 8, 1, 1000, 128, 256, 206),
    ("w257_d64", 2, 2, 1, 600, 64, 257, 207),
    ("wNm1", 1, 2, 1, 333, 64, 332, 208),
    ("w5_N3", 1, 2, 2, 3, 128, 5, 209),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases(case):
    torch, fa = require_gpu()
    name, B, H, Hkv, N, d, window, seed = case
    inp = W.gen_inputs(W.small_case(name, "bf16", B, H, Hkv, N, d, True, seed))
    o, lse = run_local(inp, fa, torch, window)
    O, L = oracle.attention_fwd(inp.q, inp.k, inp.v, True, inp.w.scale, window=window)
    info = check_bf16(dev_bf16_to_f64(o), O, name)
    info["lse_max_abs"] = check_lse(dev_to_f64(lse), L, name)
    print(name, info, flush=True)


def test_window_one_returns_own_value_row_bitwise():
    torch, fa = require_gpu()
    w = W.small_case("w1_bitwise", "bf16", 1, 4, 2, 390, 128, True, 211)
    inp = W.gen_inputs(w)
    o, lse = run_local(inp, fa, torch, 1)
    ob = dev_bf16_bits(o)
    for h in range(w.H):
        assert np.array_equal(ob[0, h], inp.v_bits[0, h // 2]), h


def test_window_covering_sequence_equals_causal_forward_bitwise():
    torch, fa = require_gpu()
    w = W.small_case("wbig", "bf16", 1, 4, 2, 515, 128, True, 212)
    inp = W.gen_inputs(w)
    q, k, v, _ = dev_inputs(inp, torch)
    oc, lc = fa.fa_fwd(q, k, v, causal=True, scale=w.scale)
    for window in (515, 516, 1 << 30):
        o, lse = fa.fa_fwd_local(q, k, v, window, scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o, oc) and torch.equal(lse, lc), window


def test_c3_shape_window_256_with_outliers():
    # The headline shape (32 query heads on 8 kv heads, N=8192, d=128, 1% of
    # key rows x8) with the pages' window of 256, in the launch configuration
    # the bench times: every element of all 32 heads against the float64
    # oracle's window variant (about 0.2 s of host time per head).
    torch, fa = require_gpu()
    w = W.C3
    window = 256
    inp = W.gen_inputs(w)
    o, lse = run_local(inp, fa, torch, window)
    og, lg = dev_bf16_to_f64(o), dev_to_f64(lse)
    worst_o, worst_l = 0.0, 0.0
    for h in range(w.H):
        g = oracle.kv_head_of(h, w.H, w.Hkv)
        O, L = oracle.attention_fwd(inp.q[:, h:h + 1], inp.k[:, g:g + 1], inp.v[:, g:g + 1],
                                    True, w.scale, window=window)
        info = check_bf16(og[:, h:h + 1], O, f"C3 local head {h}")
        worst_o = max(worst_o, info["max_abs"])
        worst_l = max(worst_l, check_lse(lg[:, h:h + 1], L, f"C3 local head {h}"))
    print(f"C3 local w=256, all heads: O max abs {worst_o:.4g}, LSE max abs {worst_l:.3g}",
          flush=True)


def test_deterministic():
    torch, fa = require_gpu()
    w = W.small_case("wdet", "bf16", 1, 8, 2, 2000, 128, True, 213)
    inp = W.gen_inputs(w)
    q, k, v, _ = dev_inputs(inp, torch)
    o1, l1 = fa.fa_fwd_local(q, k, v, 300, scale=w.scale)
    o2, l2 = fa.fa_fwd_local(q, k, v, 300, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_growing_keys_force_many_rebases():
    # as in the full-attention test: later keys' scores grow far past the
    # reference taken on a row's first visible tile
    torch, fa = require_gpu()
    w = W.small_case("local_growing", "bf16", 1, 4, 2, 1000, 128, True, 214)
    inp = W.gen_inputs(w)
    grow = (1.0 + np.arange(w.N, dtype=np.float32) / 16.0)[None, None, :, None]
    inp.k_bits = W.bf16_rne_bits(W.bf16_bits_to_f32(inp.k_bits) * grow)
    inp.k = W.bf16_bits_to_f32(inp.k_bits)
    for window in (70, 300):
        o, lse = run_local(inp, fa, torch, window)
        O, L = oracle.attention_fwd(inp.q, inp.k, inp.v, True, w.scale, window=window)
        check_bf16(dev_bf16_to_f64(o), O, f"local growing w={window}")
        check_lse(dev_to_f64(lse), L, f"local growing w={window}")


def test_window_shape_switch():
    # Windows on both sides of the launch's switch from 4-wave workgroups
    # (windows up to 2048 keys) to 8-wave workgroups, at a size whose 8-wave
    # grid fills the chip (32 query heads on 8 kv heads, N=4096): two whole
    # heads element by element for each window.
    torch, fa = require_gpu()
    w = W.small_case("wswitch", "bf16", 1, 32, 8, 4096, 128, True, 215)
    inp = W.gen_inputs(w)
    for window in (2048, 2049, 3000):
        o, lse = run_local(inp, fa, torch, window)
        for h in (0, w.H - 1):
            g = oracle.kv_head_of(h, w.H, w.Hkv)
            O, L = oracle.attention_fwd(inp.q[:, h:h + 1], inp.k[:, g:g + 1], inp.v[:, g:g + 1],
                                        True, w.scale, window=window)
            info = check_bf16(dev_bf16_to_f64(o[:, h:h + 1]), O, f"window {window} head {h}")
            info["lse_max_abs"] = check_lse(dev_to_f64(lse[:, h:h + 1]), L,
                                            f"window {window} head {h}")
            print(f"window {window} head {h}", info, flush=True)
