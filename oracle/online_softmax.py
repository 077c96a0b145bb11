"""Online softmax normaliser (oracle; test infrastructure only).

The streaming form of the numerically stable softmax, as the pages state it
("How FlashAttention Uses Tiling", section "The Running Statistics", update
equations for m and l; "LLM Architecture Refresh [3]: Flash Attention Is
Exact", section 2 "Online softmax: the one idea", the update equation and its
derivation, after Milakov & Gimelshein 2018):

    m_new = max(m_old, max(block))
    l_new = l_old * exp(m_old - m_new) + sum(exp(block - m_new))

starting from m = -inf, l = 0.  The factor exp(m_old - m_new) is the
correction that rebases every term already held onto the new reference in a
single multiply.  After the last block, the probabilities are
exp(x - m) / l.
"""
from __future__ import annotations

import numpy as np


def online_normaliser(x, block: int, trace: list | None = None):
    """Stream the last axis of ``x`` in blocks; return the final (m, l).

    If ``trace`` is a list, one dict per block is appended with the block's
    m_old, m_new, correction, rebased history l_old*correction, the block's
    own terms exp(block - m_new) and l_new (float64 values).
    """
    x = np.asarray(x, dtype=np.float64)
    lead = x.shape[:-1]
    n = x.shape[-1]
    m = np.full(lead, -np.inf)
    l = np.zeros(lead)
    for start in range(0, n, block):
        blk = x[..., start:start + block]
        m_new = np.maximum(m, blk.max(axis=-1))
        # -inf guard: while nothing finite has been seen, the reference is 0
        ref = np.where(np.isfinite(m_new), m_new, 0.0)
        with np.errstate(invalid="ignore"):
            corr = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
        terms = np.exp(blk - ref[..., None])
        rebased = l * corr
        l_new = rebased + terms.sum(axis=-1)
        if trace is not None:
            trace.append(dict(m_old=m.copy(), m_new=m_new.copy(), correction=corr.copy(),
                              rebased=rebased.copy(), terms=terms.copy(),
                              l_new=l_new.copy()))
        m, l = m_new, l_new
    return m, l


def online_softmax(x, block: int):
    """Softmax over the last axis computed with the streaming normaliser."""
    x = np.asarray(x, dtype=np.float64)
    m, l = online_normaliser(x, block)
    return np.exp(x - m[..., None]) / l[..., None]


def softmax_direct(x):
    """The one-shot stable softmax exp(x - max) / sum exp(x - max)."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)
