"""Pins for the oracle's backward (CPU only): central finite differences of
the forward definition, and exact invariants of the gradient."""
import numpy as np
import pytest

from oracle import attention_bwd, attention_fwd


def _loss(q, k, v, do, causal, scale):
    O, _ = attention_fwd(q, k, v, causal, scale)
    return float((O * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    rng = np.random.default_rng(31 + causal)
    B, H, Hkv, N, d = 1, 2, 1, 5, 3
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    do = rng.standard_normal((B, H, N, d))
    scale = 0.6
    dq, dk, dv = attention_bwd(q, k, v, do, causal, scale)
    eps = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], do, causal, scale)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], do, causal, scale)
            num[idx] = (fp - fm) / (2 * eps)
        err = np.abs(num - g).max() / max(1.0, np.abs(g).max())
        assert err < 1e-7, (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    rng = np.random.default_rng(41 + causal)
    B, H, Hkv, N, d = 2, 4, 2, 37, 8
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    do = rng.standard_normal((B, H, N, d))
    dq, dk, dv = attention_bwd(q, k, v, do, causal, 0.3, row_block=8)
    # each row of dS sums to zero, hence sum_j dK_j = 0 for every kv head
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # each row of P sums to one, hence sum_j dV_j = sum of dO over the query heads
    for g in range(Hkv):
        want = do[:, 2 * g:2 * g + 2].sum(axis=(1, 2))
        np.testing.assert_allclose(dv[:, g].sum(axis=1), want, atol=1e-11)
    if causal:
        # the last key is seen only by the last query
        O, L = attention_fwd(q, k, v, True, 0.3)
        for b in range(B):
            for g in range(Hkv):
                want = 0
                for h in (2 * g, 2 * g + 1):
                    p = np.exp(0.3 * q[b, h, -1] @ k[b, g, -1] - L[b, h, -1])
                    want = want + p * do[b, h, -1]
                np.testing.assert_allclose(dv[b, g, -1], want, atol=1e-12)


def test_head_subset_matches_full():
    rng = np.random.default_rng(51)
    q = rng.standard_normal((2, 4, 20, 4))
    k = rng.standard_normal((2, 2, 20, 4))
    v = rng.standard_normal((2, 2, 20, 4))
    do = rng.standard_normal((2, 4, 20, 4))
    dq, dk, dv = attention_bwd(q, k, v, do, True, 0.5)
    dq1, dk1, dv1 = attention_bwd(q, k, v, do, True, 0.5, heads=[(1, 2), (1, 3)])
    np.testing.assert_allclose(dq1[1, 2:4], dq[1, 2:4], atol=1e-14)
    np.testing.assert_allclose(dk1[1, 1], dk[1, 1], atol=1e-14)
    np.testing.assert_allclose(dv1[1, 1], dv[1, 1], atol=1e-14)
    assert not dq1[0].any()
