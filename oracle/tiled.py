"""Tiled attention loop in float64, with the pages' counters (oracle; test
infrastructure only).

The algorithm follows "LLM Architecture Refresh [3]: Flash Attention Is
Exact":
  * section 4 "Tiled attention in 40 lines": an outer loop over query blocks
    and an inner loop over key/value blocks; per tile, scores = scale * q k^T,
    the running max and normaliser are updated as in section 2, the
    accumulator is multiplied by the same correction before the tile's
    p @ v is added, and the division by the normaliser happens once, after
    the inner loop;
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


def tiled_attention(q, k, v, causal: bool, block_q: int, block_k: int,
                    scale: float | None = None, counters: dict | None = None,
                    elem: int = 4, rescale_accumulator: bool = True):
    """O [B,H,N,d] and LSE [B,H,N] by the tiled loop, float64.

    ``counters`` (if given) accumulates ``blocks_skipped``, ``tiles_computed``,
    ``matmul_flops`` and ``hbm_bytes`` (K/V tile reads, ``elem`` bytes per
    element).  ``rescale_accumulator=False`` plants the pages' "quietly wrong"
    mistake (the accumulator is not rebased when the max moves); it exists only
    for the oracle's own sensitivity test.
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
    for i in range(0, N, block_q):
        qi = q[:, :, i:i + block_q]
        rows = qi.shape[2]
        m = np.full((B, H, rows, 1), -np.inf)
        l = np.zeros((B, H, rows, 1))
        acc = np.zeros((B, H, rows, d))
        qpos = np.arange(i, i + rows)
        for j in range(0, N, block_k):
            if causal and j > i + rows - 1:
                if counters is not None:
                    counters["blocks_skipped"] += 1
                continue
            kj = k[:, :, j:j + block_k]
            vj = v[:, :, j:j + block_k]
            cols = kj.shape[2]
            s = (qi @ np.swapaxes(kj, -1, -2)) * scale
            if causal:
                kpos = np.arange(j, j + cols)
                s = np.where(kpos[None, :] > qpos[:, None], -np.inf, s)
            m_new = np.maximum(m, s.max(axis=-1, keepdims=True))
            ref = np.where(np.isfinite(m_new), m_new, 0.0)
            with np.errstate(invalid="ignore"):
                corr = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
            p = np.exp(s - ref)
            l = l * corr + p.sum(axis=-1, keepdims=True)
            if rescale_accumulator:
                acc = acc * corr + p @ vj
            else:
                acc = acc + p @ vj
            m = m_new
            if counters is not None:
                counters["tiles_computed"] += 1
                counters["matmul_flops"] += 2 * (2 * B * H * rows * cols * d)
                counters["hbm_bytes"] += 2 * B * H * cols * d * elem
        with np.errstate(divide="ignore", invalid="ignore"):
            out[:, :, i:i + rows] = acc / l
            lse[:, :, i:i + rows] = (m + np.log(l))[..., 0]
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
    pos = np.arange(N)
    hidden = (pos[None, :] < pos[:, None] - window + 1) | (pos[None, :] > pos[:, None])
    s = np.where(hidden, -np.inf, s)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return (e / e.sum(axis=-1, keepdims=True)) @ v
