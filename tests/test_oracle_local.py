"""Pins for the oracle's local (sliding-window) forward (CPU only).

The local variant is the approximation set against exact attention in
"LLM Architecture Refresh [3]: Flash Attention Is Exact", section 5: query i
sees keys i - window + 1 .. i.  The oracle's window path is checked against
pure-Python loops, against the exact causal definition on a sliced sequence
(the last row of causal attention over keys i - window + 1 .. i), against the
separately written negative-control function of the tiled module, and against
the special cases window = 1 and window >= N.
"""
import math

import numpy as np
import pytest

from oracle import attention_fwd, attention_rows
from oracle.tiled import sliding_window_attention


def brute_force_local(q, k, v, window, scale):
    """Pure-Python loops over the visible keys only, math.exp, no max."""
    B, H, N, d = q.shape
    rep = H // k.shape[1]
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            g = h // rep
            for i in range(N):
                keys = [j for j in range(N) if j <= i and i - j < window]
                ws = []
                for j in keys:
                    s = sum(float(q[b, h, i, c]) * float(k[b, g, j, c]) for c in range(d))
                    ws.append(math.exp(scale * s))
                z = sum(ws)
                L[b, h, i] = math.log(z)
                for c in range(d):
                    O[b, h, i, c] = sum(w * float(v[b, g, j, c]) for w, j in zip(ws, keys)) / z
    return O, L


def _inputs(shape, seed):
    B, H, Hkv, N, d = shape
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, N, d)), rng.standard_normal((B, Hkv, N, d)),
            rng.standard_normal((B, Hkv, N, d)))


@pytest.mark.parametrize("window", [1, 2, 3, 5, 9])
@pytest.mark.parametrize("shape", [(1, 2, 1, 9, 3), (2, 4, 2, 7, 2)])
def test_brute_force(shape, window):
    q, k, v = _inputs(shape, 1000 + window)
    scale = 1.0 / math.sqrt(shape[-1])
    O, L = attention_fwd(q, k, v, True, scale, window=window)
    Ob, Lb = brute_force_local(q, k, v, window, scale)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [1, 4, 13, 64])
def test_row_is_causal_attention_over_the_window(window):
    # O_local[i] = last row of causal attention over keys i-w+1 .. i, with q_i
    # as the query at that last position.
    q, k, v = _inputs((1, 2, 2, 80, 8), 7 + window)
    scale = 0.4
    O, L = attention_fwd(q, k, v, True, scale, row_block=16, window=window)
    for (h, i) in [(0, 0), (1, 3), (0, 40), (1, 79), (0, window - 1 if window <= 80 else 0)]:
        lo = max(0, i - window + 1)
        n = i - lo + 1
        qs = np.zeros((1, 2, n, 8))
        qs[0, h, n - 1] = q[0, h, i]
        ks = k[:, :, lo:i + 1]
        vs = v[:, :, lo:i + 1]
        Or, Lr = attention_rows(qs, ks, vs, True, scale, np.array([[0, h, n - 1]]))
        np.testing.assert_allclose(O[0, h, i], Or[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[0, h, i], Lr[0], rtol=0, atol=1e-13)


def test_window_one_returns_own_value_row():
    q, k, v = _inputs((2, 4, 2, 33, 5), 11)
    scale = 0.3
    O, L = attention_fwd(q, k, v, True, scale, window=1)
    for h in range(4):
        g = h // 2
        np.testing.assert_array_equal(O[:, h], v[:, g])
        np.testing.assert_allclose(L[:, h], scale * np.einsum("bnd,bnd->bn", q[:, h], k[:, g]),
                                   rtol=0, atol=1e-13)


@pytest.mark.parametrize("window", [50, 51, 1000])
def test_window_covering_the_sequence_is_causal(window):
    q, k, v = _inputs((1, 2, 1, 50, 4), 3)
    O, L = attention_fwd(q, k, v, True, 0.5, window=window)
    Oc, Lc = attention_fwd(q, k, v, True, 0.5)
    np.testing.assert_allclose(O, Oc, rtol=0, atol=1e-14)
    np.testing.assert_allclose(L, Lc, rtol=0, atol=1e-14)


@pytest.mark.parametrize("window", [1, 7, 64])
def test_matches_the_negative_control_function(window):
    q, k, v = _inputs((1, 3, 3, 100, 16), 5)
    O, _ = attention_fwd(q, k, v, True, 0.25, row_block=32, window=window)
    for h in range(3):
        ref = sliding_window_attention(q[0, h], k[0, h], v[0, h], window, 0.25)
        np.testing.assert_allclose(O[0, h], ref, rtol=0, atol=1e-12)


def test_rows_helper_and_blocking():
    q, k, v = _inputs((1, 2, 1, 70, 4), 21)
    O1, L1 = attention_fwd(q, k, v, True, 0.5, row_block=1024, window=9)
    O2, L2 = attention_fwd(q, k, v, True, 0.5, row_block=8, window=9)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-14)
    rows = np.array([[0, 0, 0], [0, 1, 8], [0, 1, 9], [0, 0, 69]])
    Or, Lr = attention_rows(q, k, v, True, 0.5, rows, window=9)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(Or[n], O1[b, h, i], rtol=0, atol=1e-14)
        np.testing.assert_allclose(Lr[n], L1[b, h, i], rtol=0, atol=1e-14)


def test_invalid_windows():
    q, k, v = _inputs((1, 1, 1, 4, 2), 0)
    with pytest.raises(ValueError):
        attention_fwd(q, k, v, True, 1.0, window=0)
    with pytest.raises(ValueError):
        attention_fwd(q, k, v, False, 1.0, window=3)
