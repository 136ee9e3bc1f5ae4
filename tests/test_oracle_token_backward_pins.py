"""Pins of the oracle's gradients with per-token selections (the training
path of "DashAttention": every query token routed on its own by entmax,
Estágio 1, and its keys weighted by the prior-induced softmax, Estágio 2):
the attention part against a library autograd of the dense attention under
the per-token mask and additive prior, dL/dw against central differences of
the oracle's token-mode forward, the reduction to block rows when every token
of a block shares its block's selection, and the whole chain (summaries and
queries -> per-token entmax -> group mean -> biased attention) against
central differences of the token pipeline with the selection held.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle

TOK = oracle.MODE_TOKEN


def _rng(seed):
    return np.random.default_rng(seed)


def _tensors(rng, nb, hq, hkv, n, d, qscale=1.0):
    Q = (qscale * rng.standard_normal((nb, hq, n, d))).astype(np.float32)
    K = rng.standard_normal((nb, hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((nb, hkv, n, d)).astype(np.float32)
    dO = rng.standard_normal((nb, hq, n, d)).astype(np.float32)
    return Q, K, V, dO


def _token_selection(rng, nb, hkv, n, B, kmax, with_w):
    """Per-token lists: the own block plus a random subset of earlier ones in
    any order (and a future block now and then, which attends nothing), with
    random weights, some of them <= 0 (dropped by the prior)."""
    idx = np.full((nb, hkv, n, kmax), -1, np.int32)
    cnt = np.zeros((nb, hkv, n), np.int32)
    w = np.zeros((nb, hkv, n, kmax))
    nblk = -(-n // B)
    for b in range(nb):
        for g in range(hkv):
            for t in range(n):
                own = t // B
                prev = list(rng.permutation(own)[: rng.integers(0, kmax)])
                if own + 1 < nblk and len(prev) + 1 < kmax and rng.random() < 0.15:
                    prev.append(own + 1)
                sel = np.array([own] + prev, np.int32)
                rng.shuffle(sel)
                idx[b, g, t, :len(sel)] = sel
                cnt[b, g, t] = len(sel)
                if with_w:
                    w[b, g, t, :len(sel)] = rng.uniform(0.05, 1.0, len(sel))
                    if rng.random() < 0.1:
                        w[b, g, t, rng.integers(0, len(sel))] = 0.0
    return idx, cnt, w


def _torch_grads(Q, K, V, dO, B, idx, cnt, sm_scale, w=None, sigma=0.0):
    """Autograd of the dense attention with the per-token selection as a mask
    and sigma ln w added to the logits of the listed blocks' keys."""
    nb, hq, n, d = Q.shape
    G = hq // K.shape[1]
    q = torch.tensor(Q, dtype=torch.float64, requires_grad=True)
    k = torch.tensor(K, dtype=torch.float64, requires_grad=True)
    v = torch.tensor(V, dtype=torch.float64, requires_grad=True)
    outs = []
    for b in range(nb):
        for h in range(hq):
            g = h // G
            bias = np.full((n, n), -np.inf)
            for t in range(n):
                for e in range(cnt[b, g, t]):
                    j = idx[b, g, t, e]
                    lo, hi = j * B, min((j + 1) * B, t + 1)
                    if hi <= lo:
                        continue
                    if w is None:
                        bias[t, lo:hi] = 0.0
                    elif w[b, g, t, e] > 0:
                        bias[t, lo:hi] = sigma * math.log(w[b, g, t, e])
            # a row attending nothing gets p = 0 (no NaN enters the backward)
            live = np.isfinite(bias).any(1)
            bias[~live] = 0.0
            s = (q[b, h] @ k[b, g].T) * sm_scale + torch.tensor(bias)
            p = torch.softmax(s, -1) * torch.tensor(live, dtype=torch.float64)[:, None]
            outs.append(p @ v[b, g])
    O = torch.stack(outs).reshape(nb, hq, n, d)
    (O * torch.tensor(dO, dtype=torch.float64)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("seed,nb,hq,hkv,n,B,kmax", [(7000, 1, 4, 2, 37, 8, 3),
                                                    (7001, 2, 3, 1, 20, 4, 4)])
def test_token_backward_matches_library_autograd_of_masked_dense_attention(seed, nb, hq, hkv,
                                                                            n, B, kmax):
    rng = _rng(seed)
    Q, K, V, dO = _tensors(rng, nb, hq, hkv, n, 8)
    idx, cnt, _ = _token_selection(rng, nb, hkv, n, B, kmax, False)
    dQ, dK, dV = oracle.attend_backward(Q, K, V, dO, B, idx, cnt, mode=TOK)
    tq, tk, tv = _torch_grads(Q, K, V, dO, B, idx, cnt, 1.0 / math.sqrt(8))
    np.testing.assert_allclose(dQ, tq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, tk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, tv, rtol=0, atol=1e-12)


def test_token_backward_with_prior_matches_library_autograd():
    rng = _rng(7100)
    nb, hq, hkv, n, B, kmax, sigma = 1, 4, 2, 29, 4, 4, 0.7
    Q, K, V, dO = _tensors(rng, nb, hq, hkv, n, 8)
    idx, cnt, w = _token_selection(rng, nb, hkv, n, B, kmax, True)
    assert (w[..., :1] > 0).any() and ((w == 0) & (idx >= 0)).any()
    dQ, dK, dV, _ = oracle.attend_backward(Q, K, V, dO, B, idx, cnt, wsel=w, sigma=sigma,
                                           mode=TOK)
    tq, tk, tv = _torch_grads(Q, K, V, dO, B, idx, cnt, 1.0 / math.sqrt(8), w, sigma)
    np.testing.assert_allclose(dQ, tq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, tk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, tv, rtol=0, atol=1e-12)


def test_token_weight_gradient_matches_central_differences_of_the_forward():
    rng = _rng(7200)
    nb, hq, hkv, n, B, kmax, sigma = 1, 4, 2, 23, 4, 3, 0.9
    Q, K, V, dO = _tensors(rng, nb, hq, hkv, n, 8)
    idx, cnt, w = _token_selection(rng, nb, hkv, n, B, kmax, True)
    *_, dw = oracle.attend_backward(Q, K, V, dO, B, idx, cnt, wsel=w, sigma=sigma, mode=TOK)

    def loss(ww):
        O, _ = oracle.attend(Q, K, V, B, idx, cnt, mode=TOK, wsel=ww, sigma=sigma)
        return float((O.reshape(dO.shape) * dO.astype(np.float64)).sum())

    checked = 0
    for pos in zip(*np.nonzero(w > 0)):
        h = 1e-6 * w[pos]
        wp, wm = w.copy(), w.copy()
        wp[pos] += h
        wm[pos] -= h
        np.testing.assert_allclose(dw[pos], (loss(wp) - loss(wm)) / (2 * h), rtol=1e-5,
                                   atol=1e-8)
        checked += 1
    assert checked > 40
    np.testing.assert_array_equal(dw[w <= 0], 0.0)
    # a listed future block attends no key: its weight moves nothing
    fut = (idx * B > np.arange(n)[None, None, :, None]) & (w > 0)
    assert fut.any()
    np.testing.assert_array_equal(dw[fut], 0.0)


def test_token_rows_sharing_their_block_selection_are_block_rows():
    """Every token listing its block's selection (same order and weights):
    dQ, dK, dV equal the block-row gradients and each block row's dL/dw is
    the sum of its tokens'."""
    rng = _rng(7300)
    nb, hq, hkv, n, B, kmax, sigma = 1, 4, 2, 30, 8, 3, 0.6
    Q, K, V, dO = _tensors(rng, nb, hq, hkv, n, 8)
    nrow = -(-n // B)
    bidx = np.full((nb, hkv, nrow, kmax), -1, np.int32)
    bcnt = np.zeros((nb, hkv, nrow), np.int32)
    bw = np.zeros((nb, hkv, nrow, kmax))
    for g in range(hkv):
        for r in range(nrow):
            sel = np.concatenate([[r], rng.permutation(r)[: rng.integers(0, kmax)]])
            bidx[0, g, r, :len(sel)] = sel
            bcnt[0, g, r] = len(sel)
            bw[0, g, r, :len(sel)] = rng.uniform(0.1, 1.0, len(sel))
    rows = np.arange(n) // B
    tidx, tcnt, tw = bidx[:, :, rows], bcnt[:, :, rows], bw[:, :, rows]
    blk = oracle.attend_backward(Q, K, V, dO, B, bidx, bcnt, wsel=bw, sigma=sigma)
    tok = oracle.attend_backward(Q, K, V, dO, B, tidx, tcnt, wsel=tw, sigma=sigma, mode=TOK)
    for a, b in zip(blk[:3], tok[:3]):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-13)
    summed = np.zeros_like(bw)
    np.add.at(summed, (slice(None), slice(None), rows), tok[3])
    np.testing.assert_allclose(summed, blk[3], rtol=0, atol=1e-13)


@pytest.mark.parametrize("cap", [64, 2])
def test_token_routing_chain_matches_central_differences_of_the_pipeline(cap):
    """Total dL/dQ and dL/dK of the per-token pipeline (summaries; each
    token's own query routed by entmax over the earlier blocks; group mean;
    prior attention) = attention part (weights held) + routing part, against
    central differences with the selection held."""
    alpha, gamma, sigma, B = 1.5, 5.0, 1.0, 4
    rng = _rng(7400 + cap)
    Q, K, V, dO = _tensors(rng, 1, 4, 2, 27, 8)

    def route(Qx, Kx):
        S = oracle.summarize(Kx, B)
        r = oracle.route_entmax(Qx, S, B, alpha, gamma, cap, force=oracle.FORCE_DIAG,
                                max_iter=60, mode=TOK)
        assert r["resolved"].all()
        return S, r

    S, r = route(Q, K)
    idx, cnt, wsel = r["idx"], r["cnt"], r["wsel"]
    if cap == 2:
        assert np.isfinite(r["capgap"]).any()
    dQa, dKa, _, dw = oracle.attend_backward(Q, K, V, dO, B, idx, cnt, wsel=wsel, sigma=sigma,
                                             mode=TOK)
    dQr, dKr = oracle.route_entmax_backward(Q, S, r["probs"], idx, cnt, dw, Q.shape[2], B,
                                            alpha, gamma, mode=TOK)
    assert np.abs(dQr).max() > 1e-3 and np.abs(dKr).max() > 1e-3

    def loss(Qx, Kx):
        _, rr = route(Qx, Kx)
        assert np.array_equal(rr["idx"], idx) and np.array_equal(rr["cnt"], cnt)
        O, _ = oracle.attend(Qx, Kx, V, B, idx, cnt, mode=TOK, wsel=rr["wsel"], sigma=sigma)
        return float((O.reshape(dO.shape) * dO.astype(np.float64)).sum())

    h = np.float32(2.0 ** -10)
    for which, total in (("Q", dQa + dQr), ("K", dKa + dKr)):
        X = Q if which == "Q" else K
        picks = [tuple(int(rng.integers(0, s)) for s in X.shape) for _ in range(12)]
        picks += [(0, 1, X.shape[2] - 1, 3), (0, 0, X.shape[2] - 2, 5)]  # ragged last block
        for pos in picks:
            xp, xm = X.copy(), X.copy()
            xp[pos] += h
            xm[pos] -= h
            step = float(xp[pos]) - float(xm[pos])
            lp = loss(xp, K) if which == "Q" else loss(Q, xp)
            lm = loss(xm, K) if which == "Q" else loss(Q, xm)
            np.testing.assert_allclose(total[pos], (lp - lm) / step, rtol=2e-3, atol=2e-5)


def test_token_routing_gradient_of_forced_entries_and_first_block_is_zero():
    """Tokens of block 0 have no candidates (only the forced own block), and
    a dw on forced entries alone moves nothing through the routing."""
    alpha, gamma, B = 1.5, 5.0, 4
    rng = _rng(7500)
    Q, K, V, dO = _tensors(rng, 1, 2, 1, 18, 8)
    S = oracle.summarize(K, B)
    r = oracle.route_entmax(Q, S, B, alpha, gamma, 64, force=oracle.FORCE_DIAG, mode=TOK)
    idx, cnt = r["idx"], r["cnt"]
    dw = np.zeros(idx.shape)
    for t in range(18):
        own = list(idx[0, 0, t, :cnt[0, 0, t]]).index(t // B)
        dw[0, 0, t, own] = rng.standard_normal()
    dQ, dK = oracle.route_entmax_backward(Q, S, r["probs"], idx, cnt, dw, 18, B, alpha, gamma,
                                          mode=TOK)
    np.testing.assert_array_equal(dQ, 0.0)
    np.testing.assert_array_equal(dK, 0.0)
