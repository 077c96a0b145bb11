"""GPU: the debug build's device counters (libfattn_counters.so,
fa_debug_counters) on the headline workload (B=1, 32 query heads on 8 kv
heads, N=8192, d=128, causal, 1% of key rows x8).

  * tiles computed / skipped / masked against the oracle's walk of the tile
    grid (32-row x 64-key tiles; "LLM Architecture Refresh [3]: Flash
    Attention Is Exact", section 7, and the counters of section 8), also on
    the key-split path of short causal sequences;
  * reference raises against a host replay of the kernel's documented rule:
    a row block takes its reference from the row max of key tile 0; on each
    later tile, if any lane's sum of exp2(s*c - m) over its 32 keys exceeds
    2^48, every row of the block raises m to max(m, c * row max of the tile).
    A lane holds one row and the keys whose index mod 8 is below 4 (first
    half of the wave) or not (second half).  The replay runs in float32 like
    the kernel; scores come from a float32 matmul, whose summation order
    differs from the matrix cores', so an exact match is expected except for
    sums within rounding of the threshold (none on this input).
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import dev_inputs, require_gpu

pytestmark = pytest.mark.gpu

ROWS, KEYS = 32, 64


def replay_raises(q, k, scale, causal=True):
    """Number of reference raises after the first tile, summed over 32-row
    blocks, for one (query head, kv head) pair; q, k float32 [N, d]."""
    n = q.shape[0]
    c = np.float32(scale * np.log2(np.e))
    s = (q @ k.T).astype(np.float32)
    rows = np.arange(n)
    if causal:
        s = np.where(np.arange(n)[None, :] > rows[:, None], np.float32(-np.inf), s)
    half = (np.arange(KEYS) % 8) >= 4                       # keys of the second lane half
    n_kt = (n + KEYS - 1) // KEYS
    last_tile = (np.minimum((rows // ROWS) * ROWS + ROWS, n) - 1) // KEYS if causal \
        else np.full(n, n_kt - 1)
    m = c * s[:, :KEYS].max(axis=1)                         # reference from key tile 0
    raises = 0
    for kt in range(1, n_kt):
        live = last_tile >= kt                              # rows whose block computes tile kt
        if not live.any():
            break
        t = s[:, kt * KEYS:(kt + 1) * KEYS]
        x = np.exp2((t * c - m[:, None]).astype(np.float32)).astype(np.float32)
        lane_sums = np.stack([x[:, ~half].sum(axis=1), x[:, half].sum(axis=1)], axis=1)
        over_row = (lane_sums > np.float32(2.0 ** 48)).any(axis=1) & live
        blocks = np.unique(rows[over_row] // ROWS)
        raises += len(blocks)
        for bidx in blocks:
            r = slice(bidx * ROWS, min(bidx * ROWS + ROWS, n))
            m[r] = np.maximum(m[r], c * t[r].max(axis=1))
    return raises


def test_counters_match_tile_grid_and_replay_on_headline_workload():
    torch, fa = require_gpu()
    dbg = fa.counters_lib()
    w = W.C3
    inp = W.gen_inputs(w)
    q, k, v, _ = dev_inputs(inp, torch)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    fa.read_counters(dbg, reset=True)
    st = dbg.fa_fwd(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                    ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
                    ctypes.c_void_p(lse.data_ptr()), w.B, w.H, w.Hkv, w.N, w.d, 1, w.scale, None)
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    got = fa.read_counters(dbg, reset=True)
    computed, skipped, masked = oracle.tile_counts(w.N, ROWS, KEYS, True)
    heads = w.B * w.H
    assert got["tiles_computed"] == heads * computed
    assert got["tiles_skipped"] == heads * skipped
    assert got["tiles_masked"] == heads * masked
    expect = 0
    for h in range(w.H):
        g = oracle.kv_head_of(h, w.H, w.Hkv)
        expect += replay_raises(inp.q[0, h].astype(np.float32), inp.k[0, g].astype(np.float32),
                                w.scale)
    print("counters", got, "replayed raises", expect, flush=True)
    assert got["reference_raises"] == expect
    # the debug build computes the same result as the normal library
    o2, l2 = fa.fa_fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)


def test_counters_noncausal_ragged_and_reset():
    torch, fa = require_gpu()
    dbg = fa.counters_lib()
    w = W.small_case("ctr", "bf16", 2, 4, 2, 200, 64, False, 601)
    inp = W.gen_inputs(w)
    q, k, v, _ = dev_inputs(inp, torch)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    fa.read_counters(dbg, reset=True)
    for _ in range(2):   # counters accumulate over launches until reset
        assert dbg.fa_fwd(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                          ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
                          ctypes.c_void_p(lse.data_ptr()), w.B, w.H, w.Hkv, w.N, w.d, 0,
                          w.scale, None) == fa.FA_OK
    torch.cuda.synchronize()
    got = fa.read_counters(dbg, reset=True)
    computed, skipped, masked = oracle.tile_counts(w.N, ROWS, KEYS, False)
    heads = w.B * w.H
    assert got["tiles_computed"] == 2 * heads * computed
    assert got["tiles_skipped"] == 0 and skipped == 0
    assert got["tiles_masked"] == 2 * heads * masked
    assert fa.read_counters(dbg)["tiles_computed"] == 0


def test_counters_on_the_key_split_path():
    # causal rows of 600 keys on a small grid: two wave groups take alternate
    # key tiles of each row block; every (row block, tile) pair is still
    # computed once, and group 0 accounts for the block's skipped tiles
    torch, fa = require_gpu()
    dbg = fa.counters_lib()
    w = W.small_case("ctr_split", "bf16", 2, 4, 2, 600, 128, True, 602)
    inp = W.gen_inputs(w)
    q, k, v, _ = dev_inputs(inp, torch)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    fa.read_counters(dbg, reset=True)
    assert dbg.fa_fwd(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                      ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
                      ctypes.c_void_p(lse.data_ptr()), w.B, w.H, w.Hkv, w.N, w.d, 1,
                      w.scale, None) == fa.FA_OK
    torch.cuda.synchronize()
    got = fa.read_counters(dbg, reset=True)
    computed, skipped, masked = oracle.tile_counts(w.N, ROWS, KEYS, True)
    heads = w.B * w.H
    assert got["tiles_computed"] == heads * computed
    assert got["tiles_skipped"] == heads * skipped
    assert got["tiles_masked"] == heads * masked
    o2, l2 = fa.fa_fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)
