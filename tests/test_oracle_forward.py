"""Pins for the oracle's forward definition (CPU only).

Each test checks the float64 oracle against something other than itself:
brute force, closed forms, invariants of softmax attention, or special cases.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import attention_fwd, attention_rows, attention_probs


def brute_force(q, k, v, causal, scale):
    """Pure-Python loops, math.exp, no max subtraction (inputs kept small)."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    rep = H // Hkv
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            g = h // rep
            for i in range(N):
                ws = []
                for j in range(N):
                    if causal and j > i:
                        ws.append(0.0)
                        continue
                    s = 0.0
                    for c in range(d):
                        s += float(q[b, h, i, c]) * float(k[b, g, j, c])
                    ws.append(math.exp(scale * s))
                z = sum(ws)
                L[b, h, i] = math.log(z)
                for c in range(d):
                    O[b, h, i, c] = sum(ws[j] * float(v[b, g, j, c]) for j in range(N)) / z
    return O, L


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 3), (1, 2, 1, 5, 4), (2, 4, 2, 8, 3), (1, 3, 3, 7, 2)])
def test_brute_force(shape, causal):
    B, H, Hkv, N, d = shape
    rng = np.random.default_rng(hash((shape, causal)) % 2 ** 32)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    for scale in (1.0 / math.sqrt(d), 0.7):
        O, L = attention_fwd(q, k, v, causal, scale)
        Ob, Lb = brute_force(q, k, v, causal, scale)
        np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one_via_one_hot_values(causal):
    # With v[j] = e_j, the output row equals the probability row.
    N = 24
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, N, 16)) * 3
    k = rng.standard_normal((1, 1, N, 16)) * 3
    v = np.eye(N)[None, None]
    q = np.concatenate([q, np.zeros((1, 1, N, N - 16))], axis=-1)
    k = np.concatenate([k, np.zeros((1, 1, N, N - 16))], axis=-1)
    O, _ = attention_fwd(q, k, v, causal, 0.25)
    np.testing.assert_allclose(O.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert (O >= 0).all()
    if causal:
        assert np.all(np.triu(O[0, 0], k=1) == 0.0)
    P = attention_probs(q, k, causal, 0.25)
    np.testing.assert_allclose(P, O, rtol=0, atol=1e-15)


def test_probs_rows_sum_to_one_and_match_library_softmax():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 2, 50, 8))
    k = rng.standard_normal((2, 2, 50, 8))
    P = attention_probs(q, k, False, 0.5)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-12)
    S = 0.5 * q @ np.swapaxes(k, -1, -2)
    np.testing.assert_allclose(P, scipy.special.softmax(S, axis=-1), rtol=1e-13, atol=1e-15)


def test_causal_row_zero_is_v0():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 4, 33, 8))
    k = rng.standard_normal((2, 2, 33, 8))
    v = rng.standard_normal((2, 2, 33, 8))
    scale = 0.3
    O, L = attention_fwd(q, k, v, True, scale)
    for b in range(2):
        for h in range(4):
            g = h // 2
            assert np.array_equal(O[b, h, 0], v[b, g, 0])
            assert L[b, h, 0] == pytest.approx(scale * q[b, h, 0] @ k[b, g, 0], abs=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_values(causal):
    rng = np.random.default_rng(8)
    N, d = 40, 8
    q = rng.standard_normal((1, 1, N, d))
    k = np.repeat(rng.standard_normal((1, 1, 1, d)), N, axis=2)
    v = rng.standard_normal((1, 1, N, d))
    O, L = attention_fwd(q, k, v, causal, 0.5)
    s = 0.5 * (q[0, 0] @ k[0, 0, 0])
    for i in range(N):
        cnt = i + 1 if causal else N
        np.testing.assert_allclose(O[0, 0, i], v[0, 0, :cnt].mean(0), atol=1e-13)
        assert L[0, 0, i] == pytest.approx(s[i] + math.log(cnt), abs=1e-12)


def test_noncausal_permutation_invariance():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 2, 30, 8))
    k = rng.standard_normal((1, 2, 30, 8))
    v = rng.standard_normal((1, 2, 30, 8))
    perm = rng.permutation(30)
    O1, L1 = attention_fwd(q, k, v, False, 0.4)
    O2, L2 = attention_fwd(q, k[:, :, perm], v[:, :, perm], False, 0.4)
    np.testing.assert_allclose(O1, O2, atol=1e-13)
    np.testing.assert_allclose(L1, L2, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_moves_lse_only(causal):
    # Adding u to every key adds scale*q_i.u to a whole score row: softmax is
    # shift invariant, so O is unchanged and LSE moves by exactly that amount.
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 1, 20, 4))
    k = rng.standard_normal((1, 1, 20, 4))
    v = rng.standard_normal((1, 1, 20, 4))
    u = np.array([300.0, -200.0, 150.0, 400.0])   # shifts of hundreds: exp would overflow
    O1, L1 = attention_fwd(q, k, v, causal, 1.0)
    O2, L2 = attention_fwd(q, k + u, v, causal, 1.0)
    assert np.isfinite(O2).all() and np.isfinite(L2).all()
    np.testing.assert_allclose(O1, O2, atol=1e-9)
    np.testing.assert_allclose(L2 - L1, (q[0, 0] @ u)[None, None], atol=1e-9)


def test_single_token():
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((1, 1, 1, 5)) for _ in range(3))
    for causal in (False, True):
        O, L = attention_fwd(q, k, v, causal, 0.2)
        assert np.array_equal(O[0, 0, 0], v[0, 0, 0])
        assert L[0, 0, 0] == pytest.approx(0.2 * q[0, 0, 0] @ k[0, 0, 0], abs=1e-15)


def test_two_keys_closed_form():
    # Two visible keys: the weight of key 0 is the logistic function of the
    # score difference ("How FlashAttention Uses Tiling", two-block intuition).
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 1, 2, 3))
    k = rng.standard_normal((1, 1, 2, 3))
    v = rng.standard_normal((1, 1, 2, 3))
    O, L = attention_fwd(q, k, v, False, 1.0)
    for i in range(2):
        s0 = float(q[0, 0, i] @ k[0, 0, 0])
        s1 = float(q[0, 0, i] @ k[0, 0, 1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        np.testing.assert_allclose(O[0, 0, i], w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, 1], atol=1e-14)
        assert L[0, 0, i] == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))), abs=1e-14)


def test_grouped_heads_read_their_kv_head():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((1, 8, 16, 4))
    k = rng.standard_normal((1, 2, 16, 4))
    v = rng.standard_normal((1, 2, 16, 4))
    O, L = attention_fwd(q, k, v, True, 0.5)
    for h in range(8):
        g = h // 4
        Oh, Lh = attention_fwd(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], True, 0.5)
        assert np.array_equal(O[:, h], Oh[:, 0])
        assert np.array_equal(L[:, h], Lh[:, 0])
    with pytest.raises(ValueError):
        attention_fwd(q, k[:, :1].repeat(3, axis=1), v[:, :1].repeat(3, axis=1), True, 0.5)


def test_scale_multiplies_scores_before_max():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((1, 1, 12, 4))
    k = rng.standard_normal((1, 1, 12, 4))
    v = rng.standard_normal((1, 1, 12, 4))
    O1, L1 = attention_fwd(q, k, v, True, 2.0)
    O2, L2 = attention_fwd(2.0 * q, k, v, True, 1.0)
    np.testing.assert_allclose(O1, O2, atol=1e-14)
    np.testing.assert_allclose(L1, L2, atol=1e-14)


def test_rows_helper_matches_full():
    rng = np.random.default_rng(15)
    q = rng.standard_normal((2, 4, 70, 8)).astype(np.float32)
    k = rng.standard_normal((2, 2, 70, 8)).astype(np.float32)
    v = rng.standard_normal((2, 2, 70, 8)).astype(np.float32)
    for causal in (False, True):
        O, L = attention_fwd(q, k, v, causal, 0.35, row_block=16)
        rows = np.array([(0, 0, 0), (1, 3, 69), (0, 2, 33), (1, 1, 15), (1, 0, 16)])
        Or, Lr = attention_rows(q, k, v, causal, 0.35, rows)
        for n, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(Or[n], O[b, h, i], atol=1e-13)
            assert Lr[n] == pytest.approx(L[b, h, i], abs=1e-13)


def test_row_blocking_does_not_change_result():
    rng = np.random.default_rng(16)
    q = rng.standard_normal((1, 2, 130, 8))
    k = rng.standard_normal((1, 2, 130, 8))
    v = rng.standard_normal((1, 2, 130, 8))
    O1, L1 = attention_fwd(q, k, v, True, 0.4, row_block=1024)
    O2, L2 = attention_fwd(q, k, v, True, 0.4, row_block=7)
    np.testing.assert_allclose(O1, O2, atol=1e-14)
    np.testing.assert_allclose(L1, L2, atol=1e-14)
