"""Tiled attention in float64, with the pages' counters (oracle; test
infrastructure only).

The computation follows "LLM Architecture Refresh [3]: Flash Attention Is
Exact" and "How FlashAttention Uses Tiling":
  * per query block, each key tile yields its own (max, sum, unnormalised
    output); partial results over disjoint key sets merge exactly once both
    are rescaled to a common reference (the update equations of "The Running
    Statistics", section 2 and 3 of the other page), so folding the tiles in
    key order is the streaming loop of section 4, with one division at the
    end;
  * section 7 "Causal masking gets a bonus": a tile whose first key lies
    after the block's last query is skipped and counted, never computed;
  * section 8 "Where the speed actually comes from": per computed tile the
    matmul flop counter grows by 2 * (2 * batch * heads * rows * cols * dim),
    and the K/V traffic counter by 2 * batch * heads * cols * dim * elem.
The "FlashAttention" explainer (attention-lab), "Tiling and online softmax",
describes the same running max / sum / output per query row.

Rows and cols may be smaller than the block at the end of the sequence
(appendix notation of the same page).  Within a computed tile, scores of
keys after the query are set to -inf (section 5).  A reference of 0 replaces
an all -inf running max (never reached in ascending key order for square
causal attention, kept as a guard).

This is not the reference for GPU outputs (``attention.attention_fwd`` is);
it pins the tiling properties: tile shape does not change the result, and the
counters reproduce the pages' tables.
"""
from __future__ import annotations

import numpy as np

from .attention import kv_head_of


def _expand_kv(k, H):
    """[B, Hkv, N, d] -> [B, H, N, d], query head h reading kv head h // (H/Hkv)."""
    Hkv = k.shape[1]
    idx = [kv_head_of(h, H, Hkv) for h in range(H)]
    return k[:, idx]


def _tile_statistics(s, v_tile):
    """Statistics of one tile on its own, relative to the tile's own row max
    ("How FlashAttention Uses Tiling", "Building Intuition: Two Blocks"):
    (m_t, l_t, u_t) with m_t = max_j s_j, l_t = sum_j exp(s_j - m_t) and the
    unnormalised output u_t = sum_j exp(s_j - m_t) v_j.  A row whose scores are
    all -inf (every key masked) gives (-inf, 0, 0)."""
    m_t = s.max(axis=-1, keepdims=True)
    shift = np.where(np.isfinite(m_t), m_t, 0.0)
    w = np.exp(s - shift)
    return m_t, w.sum(axis=-1, keepdims=True), w @ v_tile


def _combine(a, b, rescale_first: bool = True):
    """Merge two partial results over disjoint key sets ("How FlashAttention
    Uses Tiling", "The Running Statistics" and "Why the Correction Factor
    Works"; "LLM Architecture Refresh [3]", section 3): both are brought to the
    common reference max(m_a, m_b) by the factors exp(m_a - m) and exp(m_b - m)
    and added.  The merge is associative, so folding tiles in key order gives
    the streaming result.  ``rescale_first=False`` leaves the first output
    unscaled (the pages' "quietly wrong" variant; negative control only)."""
    m_a, l_a, u_a = a
    m_b, l_b, u_b = b
    m = np.maximum(m_a, m_b)
    ref = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(invalid="ignore"):
        f_a = np.where(np.isfinite(m_a), np.exp(m_a - ref), 0.0)
        f_b = np.where(np.isfinite(m_b), np.exp(m_b - ref), 0.0)
    u = (u_a * f_a if rescale_first else u_a) + u_b * f_b
    return m, l_a * f_a + l_b * f_b, u


def tiled_attention(q, k, v, causal: bool, block_q: int, block_k: int,
                    scale: float | None = None, counters: dict | None = None,
                    elem: int = 4, rescale_accumulator: bool = True):
    """O [B,H,N,d] and LSE [B,H,N] by tiles, float64.

    For each query block, every key tile that is not skipped contributes its
    own statistics (``_tile_statistics``); they are folded left to right with
    ``_combine`` and the output is divided by the running sum once, at the end
    ("LLM Architecture Refresh [3]", section 4; the skip rule of section 7;
    the counters of section 8).

    ``counters`` (if given) accumulates ``blocks_skipped``, ``tiles_computed``,
    ``matmul_flops`` and ``hbm_bytes`` (K/V tile reads, ``elem`` bytes per
    element).  ``rescale_accumulator=False`` plants the pages' "quietly wrong"
    mistake (the output accumulated so far is not rebased when the max moves);
    it exists only for the oracle's own sensitivity test.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, N, d = q.shape
    k = _expand_kv(np.asarray(k, dtype=np.float64), H)
    v = _expand_kv(np.asarray(v, dtype=np.float64), H)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if counters is not None:
        for key in ("blocks_skipped", "tiles_computed", "matmul_flops", "hbm_bytes"):
            counters.setdefault(key, 0)
    out = np.empty_like(q)
    lse = np.empty((B, H, N))
    for q_start in range(0, N, block_q):
        q_blk = q[:, :, q_start:q_start + block_q]
        n_rows = q_blk.shape[2]
        q_last = q_start + n_rows - 1
        # the empty partial result: no key seen yet
        state = (np.full((B, H, n_rows, 1), -np.inf), np.zeros((B, H, n_rows, 1)),
                 np.zeros((B, H, n_rows, d)))
        for k_start in range(0, N, block_k):
            if causal and k_start > q_last:          # wholly in the future
                if counters is not None:
                    counters["blocks_skipped"] += 1
                continue
            k_blk = k[:, :, k_start:k_start + block_k]
            n_cols = k_blk.shape[2]
            s = scale * np.einsum("bhid,bhjd->bhij", q_blk, k_blk)
            if causal:
                later = (np.arange(k_start, k_start + n_cols)[None, :]
                         > np.arange(q_start, q_start + n_rows)[:, None])
                s = np.where(later, -np.inf, s)
            tile = _tile_statistics(s, v[:, :, k_start:k_start + n_cols])
            state = _combine(state, tile, rescale_first=rescale_accumulator)
            if counters is not None:
                counters["tiles_computed"] += 1
                counters["matmul_flops"] += 2 * (2 * B * H * n_rows * n_cols * d)
                counters["hbm_bytes"] += 2 * B * H * n_cols * d * elem
        m, l, u = state
        with np.errstate(divide="ignore", invalid="ignore"):
            out[:, :, q_start:q_start + n_rows] = u / l
            lse[:, :, q_start:q_start + n_rows] = (m + np.log(l))[..., 0]
    return out, lse


def causal_tile_counts(n: int, block: int):
    """(computed, skipped) tiles of the square causal loop with equal blocks,
    counted by walking the tile grid with the skip rule."""
    computed = skipped = 0
    for i in range(0, n, block):
        rows = min(block, n - i)
        for j in range(0, n, block):
            if j > i + rows - 1:
                skipped += 1
            else:
                computed += 1
    return computed, skipped


def tile_counts(n: int, block_q: int, block_k: int, causal: bool = True):
    """(computed, skipped, masked) tiles of the loop over query blocks of
    ``block_q`` rows and key blocks of ``block_k`` keys on a square n x n
    problem.  A tile is skipped when its first key lies after the query
    block's last row ("LLM Architecture Refresh [3]", section 7); a computed
    tile is masked when it holds a key after the block's first row (section 5)
    or the sequence ends inside it.  Counted by walking the grid."""
    computed = skipped = masked = 0
    for i in range(0, n, block_q):
        last = min(i + block_q, n) - 1
        for j in range(0, n, block_k):
            if causal and j > last:
                skipped += 1
                continue
            computed += 1
            if (causal and j + block_k - 1 > i) or j + block_k > n:
                masked += 1
    return computed, skipped, masked


def naive_counts(batch: int, heads: int, n: int, d: int, elem: int = 4):
    """Counts for standard attention (section 1 and section 8 of the same page):
    two full n x n matmuls; the score matrix crosses HBM four times (write S,
    read S, write P, read P); Q, K, V are read and O written once."""
    flops = 2 * (2 * batch * heads * n * n * d)
    score_traffic = 4 * batch * heads * n * n * elem
    qkvo = 4 * batch * heads * n * d * elem
    return dict(matmul_flops=flops, score_traffic=score_traffic,
                all_tensor_traffic=score_traffic + qkvo)


def sliding_window_attention(q, k, v, window: int, scale: float | None = None):
    """Local causal attention: query i sees keys i-window+1 .. i only.

    A different function from exact attention ("LLM Architecture Refresh [3]",
    section 5); used only as a negative control, which must fail the parity
    tolerances.  Single kv head per query head (H == Hkv)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape[-2], q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    s = (q @ np.swapaxes(k, -1, -2)) * scale
    lag = np.arange(N)[:, None] - np.arange(N)[None, :]      # query index - key index
    s = np.where((lag >= 0) & (lag < window), s, -np.inf)      # the visible band
    w = np.exp(s - s.max(axis=-1, keepdims=True))
    return (w / w.sum(axis=-1, keepdims=True)) @ v
