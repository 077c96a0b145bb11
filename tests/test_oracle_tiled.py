"""Pins for the online normaliser and the tiled loop (CPU only).

Values printed by the pages live in tests/golden/*.json with their citations.
"""
import math

import numpy as np
import pytest
import scipy.special

from conftest import load_golden
from oracle import (attention_fwd, causal_tile_counts, naive_counts, online_normaliser,
                    online_softmax, sliding_window_attention, softmax_direct,
                    tiled_attention)
import workloads as W

MiB = 2 ** 20


# ---------------------------------------------------------------- online softmax

def test_rebase_walkthrough_matches_printed_values():
    g = load_golden("rebase_walkthrough.json")
    x = np.array(sum(g["blocks"], []))
    trace = []
    m, l = online_normaliser(x, 2, trace)
    r = lambda a: round(float(a), g["decimals"])
    for bi, t in enumerate(trace):
        assert r(t["m_new"]) == g["m_after_block"][bi]
        assert r(t["l_new"]) == g["l_after_block"][bi]
        assert [r(a) for a in t["terms"]] == g["block_terms"][bi]
        if bi > 0:
            assert r(t["correction"]) == g["correction"][bi]
            assert r(t["rebased"]) == g["rebased_history"][bi]
    # one multiply == recomputing the held terms against the new reference
    recomputed = np.exp(np.array(g["blocks"][0]) - trace[1]["m_new"]).sum()
    assert r(recomputed) == g["recomputed_block1_history"]
    assert abs(recomputed - trace[1]["rebased"]) < 1e-15
    # streamed == one-shot
    one_shot = np.exp(x - x.max()).sum()
    assert r(one_shot) == g["one_shot_sum"]
    assert abs(one_shot - l) < 1e-15 and m == x.max()


@pytest.mark.parametrize("block", [64, 128, 512, 2048])
def test_online_softmax_hostile_rows(block):
    # Four rows of 2048 logits stretched x8 so each row spans ~60 (a hostile
    # dynamic range): every block size must give the one-shot softmax, and
    # every row must sum to 1.
    rng = np.random.default_rng(2048)
    x = rng.standard_normal((4, 2048)) * 8
    assert (x.max(1) - x.min(1)).min() > 40
    p = online_softmax(x, block)
    ref = scipy.special.softmax(x, axis=-1)
    np.testing.assert_allclose(p, ref, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    np.testing.assert_allclose(softmax_direct(x), ref, rtol=1e-13, atol=1e-300)


def test_correction_is_one_when_max_does_not_move():
    trace = []
    online_normaliser(np.array([5.0, 1.0, 2.0, 3.0, 4.0, 0.0]), 2, trace)
    assert trace[1]["correction"] == 1.0 and trace[2]["correction"] == 1.0


def test_all_masked_prefix_blocks_are_guarded():
    x = np.array([-np.inf, -np.inf, 1.0, 2.0])
    m, l = online_normaliser(x, 2)
    assert m == 2.0 and l == pytest.approx(1 + math.exp(-1.0), abs=1e-15)


# ---------------------------------------------------------------- tiled loop

TILES = [(64, 64), (128, 128), (256, 512), (64, 48), (100, 30), (300, 300)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bq,bk", TILES)
def test_tiled_equals_definition(bq, bk, causal):
    rng = np.random.default_rng(bq * 1000 + bk)
    N = 300   # ragged against every tile shape above but 300x300
    q = rng.standard_normal((1, 4, N, 16)) * 2
    k = rng.standard_normal((1, 2, N, 16)) * 2
    v = rng.standard_normal((1, 2, N, 16))
    O, L = attention_fwd(q, k, v, causal, 0.25)
    Ot, Lt = tiled_attention(q, k, v, causal, bq, bk, scale=0.25)
    np.testing.assert_allclose(Ot, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lt, L, rtol=0, atol=1e-12)


def test_tile_shape_does_not_change_the_result_with_outliers():
    w = W.C3.with_(N=1024, H=4, Hkv=1)
    inp = W.gen_inputs(w)
    outs = [tiled_attention(inp.q, inp.k, inp.v, True, bq, bk, scale=w.scale)[0]
            for bq, bk in ((64, 64), (128, 128), (256, 512))]
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=0, atol=1e-12)


def test_causal_skipping_table():
    g = load_golden("causal_skipping.json")
    n = g["n"]
    for row in g["rows"]:
        c, s = causal_tile_counts(n, row["block"])
        assert (c, s) == (row["computed"], row["skipped"])
        Bn = n // row["block"]
        assert s / (c + s) == (Bn - 1) / (2 * Bn)               # closed form
        assert c == Bn * (Bn + 1) // 2
        assert f"{100 * s / (c + s):.0f}%" == row["fraction_pct"]
    for ex in g["closed_form_examples"]:
        Bn = n // ex["block"]
        num, den = map(int, ex["fraction"].split("/"))
        assert (Bn - 1) * den == num * 2 * Bn


@pytest.mark.parametrize("Bn", [1, 2, 3, 16, 64, 256])
def test_skip_fraction_closed_form(Bn):
    c, s = causal_tile_counts(Bn * 128, 128)
    assert s * 2 * Bn == (Bn - 1) * (c + s)


def test_emulator_counts_skipped_tiles():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 2048, 4))
    for block in (128, 256, 512):
        cnt = {}
        tiled_attention(q, q, q, True, block, block, counters=cnt)
        assert (cnt["tiles_computed"], cnt["blocks_skipped"]) == causal_tile_counts(2048, block)


def _gflop_str(x):
    return f"{x / 1e9:.1f}"


def test_flops_and_traffic_tables():
    g = load_golden("flops_vs_bytes.json")
    sh = g["shape"]
    H, d, e, blk = sh["heads"], sh["dim"], sh["elem_bytes"], sh["block"]
    for row_nc, row_c, row_t in zip(g["noncausal"], g["causal"], g["all_tensor_traffic_noncausal"]):
        n = row_nc["n"]
        rng = np.random.default_rng(n)
        q = rng.standard_normal((1, H, n, d))
        k = rng.standard_normal((1, H, n, d))
        v = rng.standard_normal((1, H, n, d))
        nv = naive_counts(1, H, n, d, e)
        c_nc, c_c = {}, {}
        tiled_attention(q, k, v, False, blk, blk, counters=c_nc, elem=e)
        tiled_attention(q, k, v, True, blk, blk, counters=c_c, elem=e)
        # non-causal: tiled flops equal the naive flops to the digit
        assert c_nc["matmul_flops"] == nv["matmul_flops"] == 4 * H * n * n * d
        assert _gflop_str(nv["matmul_flops"]) == row_nc["naive_gflop"]
        assert _gflop_str(c_nc["matmul_flops"]) == row_nc["tiled_gflop"]
        assert nv["score_traffic"] == row_nc["naive_score_mib"] * MiB
        # causal: the ratio is (B+1)/(2B)
        Bn = n // blk
        assert c_c["matmul_flops"] * 2 * Bn == nv["matmul_flops"] * (Bn + 1)
        assert _gflop_str(c_c["matmul_flops"]) == row_c["tiled_gflop"]
        assert f"{c_c['matmul_flops'] / nv['matmul_flops']:.2f}x" == row_c["ratio"]
        # all-tensor traffic: K/V re-read once per query block, plus Q in and O out
        qo = 2 * H * n * d * e
        tiled_all = c_nc["hbm_bytes"] + qo
        assert tiled_all == row_t["tiled_mib"] * MiB
        assert nv["all_tensor_traffic"] == row_t["naive_mib"] * MiB
        assert f"{nv['all_tensor_traffic'] / tiled_all:.1f}x" == row_t["reduction"]
        assert f"{c_nc['hbm_bytes'] // (2 * H * n * d * e)}x" == row_t["kv_rereads"]


def test_memory_columns():
    g = load_golden("memory_scaling.json")
    H, e, t = g["heads"], g["elem_bytes"], g["tile"]
    for row in g["rows"]:
        assert f"{H * row['n'] ** 2 * e / MiB:.1f}" == row["score_mib"]
        assert f"{H * t * t * e / MiB:.1f}" == row["tile_mib"]
    for row in g["extrapolation"]:
        n = row["n"]
        assert f"{8 * n * n * 4 / 2 ** 30:.1f}" == row["h8_fp32_gib"]
        assert f"{32 * n * n * 2 / 2 ** 30:.1f}" == row["h32_bf16_gib"]


# ---------------------------------------------------------------- negative controls

def test_missing_accumulator_rescale_is_caught():
    # Planted mistake: the accumulator is not rebased when the max moves.
    w = W.C3.with_(N=1024, H=4, Hkv=1)
    inp = W.gen_inputs(w)
    O, _ = attention_fwd(inp.q, inp.k, inp.v, True, w.scale)
    Obad, _ = tiled_attention(inp.q, inp.k, inp.v, True, 128, 128, scale=w.scale,
                              rescale_accumulator=False)
    err = np.abs(Obad - O)
    assert err.max() > 0.1                       # fails the bf16 bound (1e-2) by far
    assert not np.all(err <= 1e-2 + 2 ** -8 * np.abs(O))


def test_sliding_window_is_a_different_function():
    rng = np.random.default_rng(256)
    q, k, v = (rng.standard_normal((1, 2, 1024, 64)) for _ in range(3))
    O, _ = attention_fwd(q, k, v, True, 1 / 8)
    for w, floor in ((256, 0.1), (64, 0.3)):
        err = np.abs(sliding_window_attention(q, k, v, w) - O).max()
        assert err > floor
    # a window covering the whole sequence is exact causal attention
    np.testing.assert_allclose(sliding_window_attention(q, k, v, 1024), O, atol=1e-12)


def test_counters_with_ragged_tiles():
    # Unequal blocks and a ragged tail: K/V are read once per query block, and
    # the flop total still equals the naive count.
    rng = np.random.default_rng(300)
    H, n, d, e = 2, 300, 8, 4
    q, k, v = (rng.standard_normal((1, H, n, d)) for _ in range(3))
    for bq, bk in ((64, 128), (128, 64), (100, 30)):
        cnt = {}
        tiled_attention(q, k, v, False, bq, bk, counters=cnt, elem=e)
        nqb = -(-n // bq)
        assert cnt["hbm_bytes"] == nqb * 2 * H * n * d * e
        assert cnt["matmul_flops"] == 4 * H * n * n * d
        assert cnt["tiles_computed"] == nqb * -(-n // bk)


@pytest.mark.parametrize("order", ["reverse", "tree"])
def test_partial_results_merge_in_any_order(order):
    # Partial results over disjoint key tiles combine by rescaling to a common
    # reference ("How FlashAttention Uses Tiling", "Why the Correction Factor
    # Works"); the merge is associative and commutative, so folding the tiles
    # right to left, or as a balanced tree, must give the definition too.  A
    # merge that scaled the wrong operand or dropped a factor fails here even
    # when a left fold happens to look right.
    from oracle.tiled import _combine, _tile_statistics
    rng = np.random.default_rng(77)
    q = rng.standard_normal((1, 2, 97, 16))
    k = rng.standard_normal((1, 2, 97, 16)) * np.linspace(0.5, 4.0, 97)[None, None, :, None]
    v = rng.standard_normal((1, 2, 97, 16))
    scale = 0.3
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    tiles = [_tile_statistics(s[..., j:j + 13], v[:, :, j:j + 13]) for j in range(0, 97, 13)]
    if order == "reverse":
        state = tiles[-1]
        for t in reversed(tiles[:-1]):
            state = _combine(t, state)
    else:
        level = tiles
        while len(level) > 1:
            level = [(_combine(level[i], level[i + 1]) if i + 1 < len(level) else level[i])
                     for i in range(0, len(level), 2)]
        state = level[0]
    m, l, u = state
    O, L = attention_fwd(q, k, v, False, scale)
    assert np.abs(u / l - O).max() < 1e-12
    assert np.abs((m + np.log(l))[..., 0] - L).max() < 1e-12


def test_rectangular_tile_counts():
    # Square blocks reduce to the pages' causal table; rectangular blocks agree
    # with the emulator's own counters (skip rule of section 7) and with the
    # closed form of a 32-row x 64-key grid (query block t computes
    # floor(t/2) + 1 key tiles); masked tiles are the computed tiles that hold
    # a key after the block's first row: one per query block when block_k is
    # a multiple of block_q.
    from oracle import tile_counts
    for n, b in ((2048, 128), (2048, 256), (2048, 512), (300, 64)):
        c, s, _ = tile_counts(n, b, b, True)
        assert (c, s) == causal_tile_counts(n, b)
    n = 8192
    c, s, m = tile_counts(n, 32, 64, True)
    assert c == sum(t // 2 + 1 for t in range(n // 32)) == 16512
    assert c + s == (n // 32) * (n // 64)
    assert m == n // 32
    for n, bq, bk, causal in ((300, 32, 64, True), (257, 64, 32, True), (200, 32, 64, False)):
        ctr = {}
        q = np.zeros((1, 1, n, 2))
        tiled_attention(q, q, q, causal, bq, bk, scale=1.0, counters=ctr)
        c, s, m = tile_counts(n, bq, bk, causal)
        assert (c, s) == (ctr["tiles_computed"], ctr["blocks_skipped"]), (n, bq, bk)
    # non-causal: every tile computed; only the ragged last key tile is masked
    assert tile_counts(200, 32, 64, False) == (7 * 4, 0, 7)
    assert tile_counts(256, 32, 64, False) == (8 * 4, 0, 0)
