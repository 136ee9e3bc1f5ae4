"""Pins of the oracle's gradients through the prior-induced softmax and the
entmax routing ("DashAttention", Estágio 1: the routing is differentiable;
Estágio 2: the routing weights enter the logits as sigma ln w): the entmax
vector-Jacobian product against central differences of the oracle's own
entmax, dL/dw against central differences of the prior attention, and the
whole chain (summaries -> routing query -> entmax -> group mean -> biased
attention) against central differences of the full forward pipeline with
the selection held.  CPU only."""
import math

import numpy as np
import pytest

import oracle

B = 8


def _rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25])
def test_entmax_vjp_matches_central_differences(alpha):
    rng = _rng(6000)
    z = 0.3 / (alpha - 1) * rng.standard_normal(23)  # x = (alpha - 1) z spread 0.3
    dp = rng.standard_normal(23)

    def loss(zz):
        p, _, res, _, _, _ = oracle.entmax_row((alpha - 1) * zz, alpha, max_iter=60)
        assert res
        return float(p @ dp)

    p, _, res, _, _, _ = oracle.entmax_row((alpha - 1) * z, alpha, max_iter=60)
    assert res and 2 < np.count_nonzero(p) < 23  # a proper sparse support
    dz = oracle.entmax_vjp(p, dp, alpha)
    h = 1e-6
    for j in range(23):
        e = np.zeros(23)
        e[j] = h
        fd = (loss(z + e) - loss(z - e)) / (2 * h)
        np.testing.assert_allclose(dz[j], fd, rtol=0, atol=1e-7)
    # a direction along the support's constraint changes nothing: adding a
    # constant to every logit leaves p unchanged, so the VJP sums to zero
    assert abs(dz.sum()) < 1e-12


def _case(seed, n=51, hq=4, hkv=2, d=8, scale=1.0):
    rng = _rng(seed)
    Q = (scale * rng.standard_normal((1, hq, n, d))).astype(np.float32)
    K = rng.standard_normal((1, hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((1, hkv, n, d)).astype(np.float32)
    dO = rng.standard_normal((1, hq, n, d)).astype(np.float32)
    return Q, K, V, dO


def _route(Q, K, alpha, gamma, cap):
    S = oracle.summarize(K, B)
    qhat = oracle.qpool(Q, B)
    r = oracle.route_entmax(qhat, S, B, alpha, gamma, cap, force=oracle.FORCE_DIAG, max_iter=60)
    assert r["resolved"].all()
    return qhat, S, r


def test_prior_weight_gradient_matches_central_differences():
    Q, K, V, dO = _case(6100)
    _, _, r = _route(Q, K, 1.5, 6.0, 64)
    idx, cnt, wsel = r["idx"], r["cnt"], r["wsel"]
    sigma = 0.8
    *_, dw = oracle.attend_backward(Q, K, V, dO, B, idx, cnt, wsel=wsel, sigma=sigma)

    def loss(ww):
        O, _ = oracle.attend(Q, K, V, B, idx, cnt, wsel=ww, sigma=sigma)
        return float((O.reshape(dO.shape) * dO.astype(np.float64)).sum())

    checked = 0
    for pos in zip(*np.nonzero(wsel > 0)):
        h = 1e-6 * wsel[pos]
        wp, wm = wsel.copy(), wsel.copy()
        wp[pos] += h
        wm[pos] -= h
        fd = (loss(wp) - loss(wm)) / (2 * h)
        np.testing.assert_allclose(dw[pos], fd, rtol=1e-5, atol=1e-8)
        checked += 1
    assert checked > 10
    np.testing.assert_array_equal(dw[wsel <= 0], 0.0)


@pytest.mark.parametrize("cap,gamma", [(64, 6.0), (2, 6.0)])
def test_routing_chain_matches_central_differences_of_the_pipeline(cap, gamma):
    """Total dL/dQ and dL/dK = attention part (weights held) + routing part,
    against central differences of summarize -> q-pool -> entmax routing ->
    prior attention; cap = 2 cuts supported blocks (their weights then carry
    no gradient)."""
    alpha, sigma = 1.5, 1.0
    Q, K, V, dO = _case(6200 + cap)
    qhat, S, r = _route(Q, K, alpha, gamma, cap)
    idx, cnt, wsel = r["idx"], r["cnt"], r["wsel"]
    if cap == 2:
        assert np.isfinite(r["capgap"]).any()  # some rows had more blocks than the cap
    dQa, dKa, _, dw = oracle.attend_backward(Q, K, V, dO, B, idx, cnt, wsel=wsel, sigma=sigma)
    dQr, dKr = oracle.route_entmax_backward(qhat, S, r["probs"], idx, cnt, dw, Q.shape[2], B,
                                            alpha, gamma)
    assert np.abs(dQr).max() > 1e-3 and np.abs(dKr).max() > 1e-3  # the routing part is not void

    def loss(Qx, Kx):
        _, _, rr = _route(Qx, Kx, alpha, gamma, cap)
        assert np.array_equal(rr["idx"], idx) and np.array_equal(rr["cnt"], cnt)
        O, _ = oracle.attend(Qx, Kx, V, B, idx, cnt, wsel=rr["wsel"], sigma=sigma)
        return float((O.reshape(dO.shape) * dO.astype(np.float64)).sum())

    rng = _rng(6300 + cap)
    h = np.float32(2.0 ** -10)
    for which, total in (("Q", dQa + dQr), ("K", dKa + dKr)):
        X = Q if which == "Q" else K
        # random entries, plus two in the ragged last block (3 tokens: its
        # mean pool divides by 3, not B)
        picks = [tuple(int(rng.integers(0, s)) for s in X.shape) for _ in range(12)]
        picks += [(0, 1, X.shape[2] - 1, 3), (0, 0, X.shape[2] - 3, 5)]
        for pos in picks:
            xp, xm = X.copy(), X.copy()
            xp[pos] += h
            xm[pos] -= h
            step = float(xp[pos]) - float(xm[pos])  # exact fp32 perturbation
            lp = loss(xp, K) if which == "Q" else loss(Q, xp)
            lm = loss(xm, K) if which == "Q" else loss(Q, xm)
            np.testing.assert_allclose(total[pos], (lp - lm) / step, rtol=2e-3, atol=2e-5)


def test_routing_gradient_vanishes_without_a_prior_and_for_forced_blocks():
    """sigma = 0: the weights do not enter the output, so no gradient flows
    through the routing; forced (diagonal) entries carry w = 1 and no dw."""
    alpha, gamma = 1.5, 6.0
    Q, K, V, dO = _case(6400)
    qhat, S, r = _route(Q, K, alpha, gamma, 64)
    idx, cnt, wsel = r["idx"], r["cnt"], r["wsel"]
    *_, dw = oracle.attend_backward(Q, K, V, dO, B, idx, cnt, wsel=wsel, sigma=0.0)
    np.testing.assert_array_equal(dw, 0.0)
    dQr, dKr = oracle.route_entmax_backward(qhat, S, r["probs"], idx, cnt, dw, Q.shape[2], B,
                                            alpha, gamma)
    np.testing.assert_array_equal(dQr, 0.0)
    np.testing.assert_array_equal(dKr, 0.0)
    # the own block is listed with w = 1 (forced); its dw is sigma * sum dS
    *_, dw1 = oracle.attend_backward(Q, K, V, dO, B, idx, cnt, wsel=wsel, sigma=1.0)
    for rr in range(cnt.shape[2]):
        own = list(idx[0, 0, rr, :cnt[0, 0, rr]]).index(rr)
        assert wsel[0, 0, rr, own] == 1.0
    # a dw on a forced entry alone moves nothing through the routing
    only_forced = np.zeros_like(dw1)
    for rr in range(cnt.shape[2]):
        own = list(idx[0, 0, rr, :cnt[0, 0, rr]]).index(rr)
        only_forced[0, :, rr, own] = dw1[0, :, rr, own]
    dQf, dKf = oracle.route_entmax_backward(qhat, S, r["probs"], idx, cnt, only_forced,
                                            Q.shape[2], B, alpha, gamma)
    np.testing.assert_array_equal(dQf, 0.0)
    np.testing.assert_array_equal(dKf, 0.0)
