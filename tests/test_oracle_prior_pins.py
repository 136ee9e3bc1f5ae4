"""Pins of the oracle's prior-induced softmax ("DashAttention", Estágio 2):
the attention weights maximise z.p - KL(p || g) for a reference g that gives
every token of a listed block the weight w^sigma, and of the routing weights
the entmax router reports for each listed block.  CPU only."""
import math

import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _setup(seed, n=40, B=8, d=64, hq=2, hkv=1, k=3):
    rng = _rng(seed)
    nrow = -(-n // B)
    idx = np.full((1, hkv, nrow, k), -1, np.int32)
    cnt = np.zeros((1, hkv, nrow), np.int32)
    w = np.zeros((1, hkv, nrow, k))
    for g in range(hkv):
        for i in range(nrow):
            sel = sorted(set(rng.choice(i + 1, size=min(k - 1, i + 1), replace=False).tolist()) | {i})
            idx[0, g, i, :len(sel)] = sel
            cnt[0, g, i] = len(sel)
            w[0, g, i, :len(sel)] = rng.uniform(0.05, 1.0, len(sel))
    return rng, idx, cnt, w


def test_sigma_zero_is_plain_softmax():
    rng, idx, cnt, w = _setup(3000)
    Q = rng.standard_normal((1, 2, 40, 64)).astype(np.float32)
    K = rng.standard_normal((1, 1, 40, 64)).astype(np.float32)
    V = rng.standard_normal((1, 1, 40, 64)).astype(np.float32)
    O0, p0 = oracle.attend(Q, K, V, 8, idx, cnt)
    O1, p1 = oracle.attend(Q, K, V, 8, idx, cnt, wsel=w, sigma=0.0)
    np.testing.assert_array_equal(O0, O1)
    np.testing.assert_array_equal(p0, p1)


@pytest.mark.parametrize("sigma", [0.5, 1.0, 2.0])
def test_zero_query_gives_the_reference_distribution(sigma):
    """q = 0: every logit is 0, so p = g restricted to the attended tokens; with
    one-hot values o is that distribution: w_j^sigma per token of block j."""
    rng, idx, cnt, w = _setup(3100)
    n, B, d = 40, 8, 64
    Q = np.zeros((1, 2, n, d), np.float32)
    K = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    V = np.eye(n, d, dtype=np.float32)[None, None]
    w[0, 0, 2, 0] = 0.0  # a listed block with zero weight drops out
    O, pairs = oracle.attend(Q, K, V, B, idx, cnt, wsel=w, sigma=sigma)
    O = O.reshape(2, n, d)
    for t in range(n):
        i = t // B
        want = np.zeros(d)
        for s in range(cnt[0, 0, i]):
            j = idx[0, 0, i, s]
            if w[0, 0, i, s] <= 0:
                continue
            for tp in range(j * B, min((j + 1) * B, t + 1)):
                want[tp] = w[0, 0, i, s] ** sigma
        assert pairs[t] == np.count_nonzero(want)
        want /= want.sum()
        np.testing.assert_allclose(O[0, t], want, rtol=0, atol=1e-14)
        np.testing.assert_allclose(O[1, t], want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("sigma", [0.7, 1.0])
def test_weights_maximise_the_kl_regularised_objective(sigma):
    """With one-hot values o is the weight vector p itself; p must beat every
    other distribution on the attended set under z.p - KL(p || g), g the
    normalised reference (the variational form of the prior-induced softmax)."""
    rng, idx, cnt, w = _setup(3200, n=24, B=8, d=32, hq=1)
    n, B, d = 24, 8, 32
    Q = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    K = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    V = np.eye(n, d, dtype=np.float32)[None, None]
    O, _ = oracle.attend(Q, K, V, B, idx, cnt, wsel=w, sigma=sigma)
    scale = 1.0 / math.sqrt(d)
    for t in [5, 13, 23]:
        i = t // B
        toks, gw = [], []
        for s in range(cnt[0, 0, i]):
            j = idx[0, 0, i, s]
            for tp in range(j * B, min((j + 1) * B, t + 1)):
                toks.append(tp)
                gw.append(w[0, 0, i, s] ** sigma)
        toks = np.array(toks)
        g = np.array(gw) / np.sum(gw)
        z = (K[0, 0, toks].astype(np.float64) @ Q[0, 0, t].astype(np.float64)) * scale
        p = O[t, toks]
        assert abs(p.sum() - 1) < 1e-12 and np.all(p > 0)

        def F(q):
            return float(z @ q - np.sum(q * np.log(q / g)))
        best = F(p)
        for _ in range(200):
            q = p * np.exp(0.3 * rng.standard_normal(p.size))
            q /= q.sum()
            assert F(q) <= best + 1e-12


def test_entmax_routing_weights_of_the_listed_blocks():
    rng = _rng(3300)
    B, d, nblk, hq = 4, 8, 14, 4
    S = rng.standard_normal((1, 1, nblk, d))
    q = 3.0 * rng.standard_normal((1, hq, nblk, d))
    for force, cap in [(oracle.FORCE_DIAG, 64), (oracle.FORCE_DIAG | oracle.FORCE_FIRST, 3)]:
        r = oracle.route_entmax(q, S, B, 1.5, 4.0, cap=cap, force=force)
        wbar = r["probs"][0].mean(0)  # [nrow, nblk] group mean
        for i in range(nblk):
            c = r["cnt"][0, 0, i]
            sel = r["idx"][0, 0, i, :c]
            ws = r["wsel"][0, 0, i]
            assert np.all(ws[c:] == 0)
            for s, j in enumerate(sel):
                forced = (j == i and force & oracle.FORCE_DIAG) or (j == 0 and force & oracle.FORCE_FIRST)
                if forced:
                    assert ws[s] == 1.0
                else:
                    assert ws[s] > 0 and abs(ws[s] - wbar[i, j]) < 1e-15
