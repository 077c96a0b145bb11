"""The attention definition in float64 (oracle; test infrastructure only).

Definition followed ("LLM Architecture Refresh [3]: Flash Attention Is
Exact", section 1 "The problem is memory traffic" -- S = Q K^T, P =
softmax(S), O = P V -- and section 2's numerically stable softmax, which
subtracts the row max; section 5 for the causal mask, which sends scores of
keys after the query to minus infinity; "How FlashAttention Uses Tiling",
softmax equation):

    s_ij   = scale * sum_c q[b,h,i,c] * k[b,g,j,c]         g = h // (H / Hkv)
    valid  = ((not causal) or j <= i) and (window is None or i - j < window)
    m_i    = max over valid j of s_ij
    l_i    = sum over valid j of exp(s_ij - m_i)
    O_i    = sum over valid j of exp(s_ij - m_i) * v[b,g,j,:] / l_i
    LSE_i  = m_i + ln(l_i)

Readings where the pages are silent (stated once here, listed in the design doc):
  * LSE is the natural log of the row normaliser in scaled-score units.
  * Grouped heads: query head h reads key/value head h // (H / Hkv).
  * Causal masking is square and includes the diagonal (key j <= query i).
  * The scale multiplies Q K^T before the max is taken.
  * A row with no visible key (impossible for square causal or non-causal
    attention with N >= 1) is defined as O = 0, LSE = -inf.

The local (sliding-window) variant is the approximation the same page sets
against exact attention in section 5: query i sees only the keys
i - window + 1 .. i (window >= 1; causal is implied).  With window >= N it is
causal attention; with window = 1 every row returns its own value row.

The backward is the calculus of the same definition (the pages say only that
it recomputes the probabilities from Q, K, V and the saved statistics,
section 8 of the same page):

    P_ij  = exp(s_ij - LSE_i) on valid pairs (0 elsewhere)
    dV_j  = sum_i P_ij dO_i
    dP_ij = dO_i . v_j
    D_i   = dO_i . O_i
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = scale * sum_j dS_ij k_j
    dK_j  = scale * sum_i dS_ij q_i
and dK, dV of a key/value head sum over the query heads that read it.

Inputs are float64 arrays upcast exactly from the stored bf16/fp32 values.
Matrix products use numpy's float64 matmul as a library primitive; rows are
processed in blocks only to bound host memory (no reordering of the
definition's sums beyond what matmul does).
"""
from __future__ import annotations

import numpy as np


def kv_head_of(h: int, H: int, Hkv: int) -> int:
    """Key/value head read by query head h (consecutive query heads share)."""
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError(f"H={H} must be a positive multiple of Hkv={Hkv}")
    return h // (H // Hkv)


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    B, H, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    Hkv = k.shape[1]
    kv_head_of(0, H, Hkv)
    return B, H, Hkv, N, d


def _check_window(causal: bool, window):
    if window is None:
        return
    if not causal:
        raise ValueError("a window implies causal attention")
    if int(window) < 1:
        raise ValueError("window must be >= 1")


def _scores(qb: np.ndarray, kk: np.ndarray, rows: np.ndarray, causal: bool,
            scale: float, window=None, k0: int = 0) -> np.ndarray:
    """scale * q_rows . k^T with invisible pairs set to -inf.
    ``rows`` holds the absolute query index of each row of ``qb``; ``kk``
    holds keys k0, k0 + 1, ... ."""
    s = scale * (qb @ kk.T)
    cols = k0 + np.arange(kk.shape[0])
    if causal:
        s[cols[None, :] > rows[:, None]] = -np.inf
    if window is not None:
        s[cols[None, :] <= rows[:, None] - window] = -np.inf
    return s


def _normalise(s: np.ndarray):
    """Row max, exp(s - max), row sum, guarded for rows with no visible key."""
    m = s.max(axis=1)
    dead = ~np.isfinite(m)
    m_safe = np.where(dead, 0.0, m)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for masked pairs
    l = e.sum(axis=1)
    return m, e, l, dead


def attention_fwd(q, k, v, causal: bool, scale: float, row_block: int = 1024, window=None):
    """O [B,H,N,d] and LSE [B,H,N] of the definition, float64 (``window``
    selects the local variant)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Hkv, N, d = _check(q, k, v)
    _check_window(causal, window)
    O = np.zeros((B, H, N, d), dtype=np.float64)
    LSE = np.full((B, H, N), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            for r0 in range(0, N, row_block):
                r1 = min(N, r0 + row_block)
                kmax = r1 if causal else N   # later keys are invisible to every row
                kmin = 0 if window is None else max(0, r0 - window + 1)   # and older ones
                rows = np.arange(r0, r1)
                s = _scores(q[b, h, r0:r1], k[b, g, kmin:kmax], rows, causal, scale, window,
                            kmin)
                m, e, l, dead = _normalise(s)
                with np.errstate(divide="ignore", invalid="ignore"):
                    o = (e @ v[b, g, kmin:kmax]) / l[:, None]
                    lse = m + np.log(l)
                o[dead] = 0.0
                lse[dead] = -np.inf
                O[b, h, r0:r1] = o
                LSE[b, h, r0:r1] = lse
    return O, LSE


def attention_rows(q, k, v, causal: bool, scale: float, rows, window=None):
    """O and LSE for selected (b, h, i) query rows only (for full-size checks).

    ``rows`` is an int array [n, 3] of (b, h, i).  Returns O [n, d], LSE [n].
    Each row is the definition evaluated on its own.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, Hkv, N, d = _check(q, k, v)
    _check_window(causal, window)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    O = np.zeros((rows.shape[0], d), dtype=np.float64)
    LSE = np.full(rows.shape[0], -np.inf, dtype=np.float64)
    for n, (b, h, i) in enumerate(rows):
        g = kv_head_of(int(h), H, Hkv)
        kmax = int(i) + 1 if causal else N
        kmin = 0 if window is None else max(0, int(i) - window + 1)
        kk = k[b, g, kmin:kmax].astype(np.float64)
        vv = v[b, g, kmin:kmax].astype(np.float64)
        qi = q[b, h, i].astype(np.float64)[None, :]
        s = _scores(qi, kk, np.array([i]), causal, scale, window, kmin)
        m, e, l, dead = _normalise(s)
        if dead[0]:
            continue
        O[n] = (e @ vv)[0] / l[0]
        LSE[n] = m[0] + np.log(l[0])
    return O, LSE


def attention_probs(q, k, causal: bool, scale: float):
    """The full probability matrix P [B, H, N, N] (small inputs only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    P = np.zeros((B, H, N, N), dtype=np.float64)
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            s = _scores(q[b, h], k[b, g], rows, causal, scale)
            m, e, l, dead = _normalise(s)
            with np.errstate(divide="ignore", invalid="ignore"):
                p = e / l[:, None]
            p[dead] = 0.0
            P[b, h] = p
    return P


def attention_bwd(q, k, v, do, causal: bool, scale: float, row_block: int = 512,
                  heads=None):
    """dQ [B,H,N,d], dK [B,Hkv,N,d], dV [B,Hkv,N,d] of the definition, float64.

    ``heads`` optionally restricts the work to a list of (b, h) query heads;
    then dQ is filled for those heads only, and dK/dV hold the contributions
    of those heads only (complete for a kv head when every query head that
    reads it is listed).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, Hkv, N, d = _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must have the shape of Q")
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        g = kv_head_of(h, H, Hkv)
        for r0 in range(0, N, row_block):
            r1 = min(N, r0 + row_block)
            kmax = r1 if causal else N
            rows = np.arange(r0, r1)
            qb = q[b, h, r0:r1]
            dob = do[b, h, r0:r1]
            kk = k[b, g, :kmax]
            vv = v[b, g, :kmax]
            s = _scores(qb, kk, rows, causal, scale)
            m, e, l, dead = _normalise(s)
            with np.errstate(divide="ignore", invalid="ignore"):
                P = e / l[:, None]
            P[dead] = 0.0
            O = P @ vv
            D = (dob * O).sum(axis=1)
            dV[b, g, :kmax] += P.T @ dob
            dP = dob @ vv.T
            dS = P * (dP - D[:, None])
            dQ[b, h, r0:r1] = scale * (dS @ kk)
            dK[b, g, :kmax] += scale * (dS.T @ qb)
    return dQ, dK, dV
