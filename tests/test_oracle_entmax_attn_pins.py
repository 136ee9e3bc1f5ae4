"""Pins of the oracle's token-level alpha-entmax attention ("AdaSplash-2",
sections 1 and 2): textbook sort-based sparsemax and 1.5-entmax, a library
root finder for other alpha, the uniform case, causality.  CPU only."""
import math

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import _entmax15_sort, _sparsemax_sort, _tau_brentq


def _rng(seed):
    return np.random.default_rng(seed)


def _case(seed, n=37, d=16, hq=4, hkv=2, scale=3.0):
    rng = _rng(seed)
    Q = (scale * rng.standard_normal((1, hq, n, d))).astype(np.float32)
    K = rng.standard_normal((1, hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((1, hkv, n, d)).astype(np.float32)
    return Q, K, V


def _scores(Q, K, h, t, G):
    d = Q.shape[-1]
    return (K[0, h // G, :t + 1].astype(np.float64) @ Q[0, h, t].astype(np.float64)) / math.sqrt(d)


@pytest.mark.parametrize("alpha", [2.0, 1.5])
def test_entmax_attention_matches_sort_based_closed_forms(alpha):
    Q, K, V = _case(4000)
    O, tau, sup = oracle.entmax_attend(Q, K, V, alpha)
    hq, n = Q.shape[1], Q.shape[2]
    G = hq // K.shape[1]
    O = O.reshape(hq, n, -1)
    tau = tau.reshape(hq, n)
    for h in range(hq):
        for t in range(n):
            z = _scores(Q, K, h, t, G)
            if alpha == 2.0:
                p, tz = _sparsemax_sort(z)  # x = z for alpha = 2
            else:
                p, tz = _entmax15_sort(z)  # x = z / 2
            np.testing.assert_allclose(p.sum(), 1.0, atol=1e-12)
            np.testing.assert_allclose(tau[h, t], tz, rtol=0, atol=1e-12)
            np.testing.assert_allclose(O[h, t], p @ V[0, h // G, :t + 1].astype(np.float64),
                                       rtol=0, atol=1e-12)
    assert sup.min() >= 1 and sup.max() < n  # sparse somewhere


@pytest.mark.parametrize("alpha", [1.25, 1.75, 2.5, 3.0])
def test_entmax_attention_threshold_vs_library_root_finder(alpha):
    Q, K, V = _case(4100, n=29)
    req = np.array([[0, h, t] for h in range(4) for t in (0, 5, 17, 28)], np.int64)
    O, tau, sup = oracle.entmax_attend(Q, K, V, alpha, req=req)
    for r, (_, h, t) in enumerate(req):
        x = (alpha - 1) * _scores(Q, K, h, t, 2)
        if t == 0:
            assert sup[r] == 1
            np.testing.assert_allclose(O[r], V[0, h // 2, 0], rtol=0, atol=1e-12)
            continue
        tb = _tau_brentq(x, alpha)
        np.testing.assert_allclose(tau[r], tb, rtol=0, atol=1e-12)
        p = np.maximum(x - tb, 0) ** (1 / (alpha - 1))
        p /= p.sum()
        np.testing.assert_allclose(O[r], p @ V[0, h // 2, :t + 1].astype(np.float64), rtol=0,
                                   atol=1e-10)
        assert sup[r] == np.count_nonzero(p)


def test_entmax_attention_zero_query_is_the_causal_mean():
    _, K, V = _case(4200)
    Q = np.zeros((1, 4, 37, 16), np.float32)
    for alpha in (1.5, 2.0, 1.25):
        O, _, sup = oracle.entmax_attend(Q, K, V, alpha)
        O = O.reshape(4, 37, 16)
        for t in range(37):
            mean = V[0, :, :t + 1].astype(np.float64).mean(1)
            np.testing.assert_allclose(O[:, t], np.repeat(mean, 2, axis=0), rtol=0, atol=1e-12)
        assert np.array_equal(sup.reshape(4, 37), np.tile(np.arange(1, 38), (4, 1)))


def test_entmax_attention_weights_are_a_sparse_distribution_and_causal():
    """One-hot values expose the weights: nonnegative, summing to one, zero on
    future keys; changing future keys changes nothing."""
    Q, K, _ = _case(4300, n=30, d=32, hq=2, hkv=1, scale=6.0)
    V = np.eye(30, 32, dtype=np.float32)[None, None]
    O, _, sup = oracle.entmax_attend(Q, K, V, 1.5)
    O = O.reshape(2, 30, 32)
    assert np.all(O >= 0)
    np.testing.assert_allclose(O.sum(-1), 1.0, atol=1e-12)
    for t in range(30):
        assert np.all(O[:, t, t + 1:30] == 0)
    assert np.array_equal((O[:, :, :30] > 0).sum(-1).ravel(), sup)
    K2 = K.copy()
    K2[:, :, 20:] = 100.0
    O2, _, _ = oracle.entmax_attend(Q, K2, V, 1.5)
    np.testing.assert_array_equal(O2.reshape(2, 30, 32)[:, :20], O[:, :20])


# ---------------------------------------------------------------------------
# Backward of the entmax attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25])
def test_entmax_attention_backward_matches_central_differences(alpha):
    """dQ, dK, dV against central differences of the forward oracle's
    loss sum(dO * O) (exact thresholds, so the map is smooth away from
    support changes)."""
    Q, K, V = _case(4400, n=19, d=8, hq=2, hkv=1, scale=2.0)
    dO = _rng(4401).standard_normal(Q.shape).astype(np.float32)
    dQ, dK, dV = oracle.entmax_attend_backward(Q, K, V, dO, alpha)

    def loss(Qx, Kx, Vx):
        O, _, _ = oracle.entmax_attend(Qx, Kx, Vx, alpha)
        return float((O.reshape(dO.shape) * dO.astype(np.float64)).sum())

    rng = _rng(4402)
    h = np.float32(2.0 ** -12)
    for which, g in (("Q", dQ), ("K", dK), ("V", dV)):
        X = {"Q": Q, "K": K, "V": V}[which]
        for _ in range(10):
            pos = tuple(int(rng.integers(0, s)) for s in X.shape)
            xp, xm = X.copy(), X.copy()
            xp[pos] += h
            xm[pos] -= h
            step = float(xp[pos]) - float(xm[pos])
            args_p = {"Q": Q, "K": K, "V": V, which: xp}
            args_m = {"Q": Q, "K": K, "V": V, which: xm}
            fd = (loss(args_p["Q"], args_p["K"], args_p["V"]) -
                  loss(args_m["Q"], args_m["K"], args_m["V"])) / step
            np.testing.assert_allclose(g[pos], fd, rtol=2e-3, atol=2e-6)


def test_entmax_attention_backward_invariants():
    """Shifting every key leaves each query's entmax unchanged (its VJP sums
    to zero), so the key gradients sum to zero; the weights sum to one, so
    the value gradients sum to the upstream gradients; with alpha = 2 and a
    query whose support is one key, that query's dQ is zero."""
    Q, K, V = _case(4500, n=33, d=16, hq=4, hkv=2, scale=3.0)
    dO = _rng(4501).standard_normal(Q.shape).astype(np.float32)
    dQ, dK, dV = oracle.entmax_attend_backward(Q, K, V, dO, 1.5)
    np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-11)
    want = dO.astype(np.float64).reshape(1, 2, 2, 33, 16).sum(axis=(2, 3))
    np.testing.assert_allclose(dV.sum(axis=2), want, atol=1e-11)
    np.testing.assert_array_equal(dQ[:, :, 0], 0.0)  # token 0 attends only itself
