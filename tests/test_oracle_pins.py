"""Pins of the fp64 oracle to things other than itself: closed forms, textbook
and library routines, brute force on tiny inputs, hand-worked fixtures and the
invariants the pages state.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.optimize
import scipy.special
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# Block summaries (DashAttention, Estágio 0)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,B", [(64, 16), (70, 16), (5, 8), (128, 128)])
def test_summary_is_block_mean(n, B):
    K = _rng(1).standard_normal((2, 3, n, 8)).astype(np.float32)
    S = oracle.summarize(K, B)
    for j in range(S.shape[2]):
        ref = K[:, :, j * B:(j + 1) * B, :].astype(np.float64).mean(axis=2)
        np.testing.assert_allclose(S[:, :, j], ref, rtol=0, atol=1e-15)


def test_summary_zero_learned_query_is_mean():
    K = _rng(2).standard_normal((1, 2, 40, 16)).astype(np.float32)
    np.testing.assert_allclose(oracle.summarize(K, 8, qbar=np.zeros((2, 16), np.float32)),
                               oracle.summarize(K, 8), rtol=0, atol=1e-14)


def test_summary_learned_query_matches_library_softmax():
    K = _rng(3).standard_normal((1, 2, 24, 8)).astype(np.float32)
    qbar = _rng(4).standard_normal((2, 8)).astype(np.float32)
    S = oracle.summarize(K, 8, qbar=qbar)
    for h in range(2):
        for j in range(3):
            kb = K[0, h, j * 8:(j + 1) * 8].astype(np.float64)
            w = scipy.special.softmax(kb @ qbar[h].astype(np.float64) / math.sqrt(8))
            np.testing.assert_allclose(S[0, h, j], w @ kb, rtol=1e-12, atol=1e-13)


def test_summary_huge_aligned_query_returns_that_key():
    K = _rng(5).standard_normal((1, 1, 16, 8)).astype(np.float32)
    K[0, 0, 3] = 4.0 * K[0, 0, 3] / np.linalg.norm(K[0, 0, 3])  # the longest key of block 0
    qbar = (1e3 * K[0, 0, 3]).reshape(1, 8).astype(np.float32)
    S = oracle.summarize(K, 8, qbar=qbar)
    np.testing.assert_allclose(S[0, 0, 0], K[0, 0, 3], rtol=0, atol=1e-6)


def test_qpool_is_block_mean_and_decode_is_identity():
    Q = _rng(6).standard_normal((2, 4, 50, 8)).astype(np.float32)
    qh = oracle.qpool(Q, 16)
    for i in range(4):
        np.testing.assert_allclose(qh[:, :, i], Q[:, :, i * 16:(i + 1) * 16].astype(np.float64).mean(2),
                                   rtol=0, atol=1e-15)
    q1 = Q[:, :, :1]
    np.testing.assert_array_equal(oracle.qpool(q1, 64)[:, :, 0], q1[:, :, 0].astype(np.float64))


# --------------------------------------------------------------------------
# Top-k routing
# --------------------------------------------------------------------------

def _numpy_scores(Q, K, B, hkv):
    """Independent scoring with numpy: mean-pooled queries summed over each
    GQA group, dotted with mean-pooled keys, divided by sqrt(d)."""
    nb, hq, n, d = Q.shape
    G = hq // hkv
    nblk = -(-n // B)
    qh = np.stack([Q[:, :, i * B:(i + 1) * B].astype(np.float64).mean(2) for i in range(nblk)], 2)
    s = np.stack([K[:, :, j * B:(j + 1) * B].astype(np.float64).mean(2) for j in range(nblk)], 2)
    qg = qh.reshape(nb, hkv, G, nblk, d).sum(2)
    return np.einsum("bgid,bgjd->bgij", qg, s) / math.sqrt(d)


def _brute_topk(scores, cands, m):
    """All subsets of size min(m, |cands|); the max-sum one, ties to the
    lexicographically smallest index tuple."""
    m = min(m, len(cands))
    best = None
    for sub in itertools.combinations(sorted(cands), m):
        tot = math.fsum(scores[j] for j in sub)
        # sums equal up to rounding are ties (exactly tied scores, summed in another order)
        if best is None or tot > best[0] + 1e-12 or (abs(tot - best[0]) <= 1e-12 and sub < best[1]):
            best = (tot, sub)
    return set(best[1]) if best else set()


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("force", [0, oracle.FORCE_DIAG, oracle.FORCE_DIAG | oracle.FORCE_FIRST])
def test_topk_matches_bruteforce_prefill(seed, force):
    rng = _rng(100 + seed)
    B, n, d, hq, hkv = 4, 36, 8, 4, 2
    if seed % 2:  # integer-valued data: exact ties between scores
        Q = rng.integers(-1, 2, (1, hq, n, d)).astype(np.float32)
        K = rng.integers(-1, 2, (1, hkv, n, d)).astype(np.float32)
    else:
        Q = rng.standard_normal((1, hq, n, d)).astype(np.float32)
        K = rng.standard_normal((1, hkv, n, d)).astype(np.float32)
    k_total = 4
    r = oracle.route_topk(oracle.qpool(Q, B), oracle.summarize(K, B), B, k_total, force)
    sc = _numpy_scores(Q, K, B, hkv)
    nblk = sc.shape[-1]
    for g in range(hkv):
        for i in range(nblk):
            np.testing.assert_allclose(r["scores"][0, g, i, :i + 1], sc[0, g, i, :i + 1], rtol=0, atol=1e-12)
            assert np.all(np.isneginf(r["scores"][0, g, i, i + 1:]))
            F = set()
            if force & oracle.FORCE_DIAG:
                F.add(i)
            if force & oracle.FORCE_FIRST:
                F.add(0)
            C = [j for j in range(i + 1) if j not in F]
            want = sorted(F | _brute_topk(sc[0, g, i], C, k_total - len(F)))
            got = r["idx"][0, g, i]
            assert r["cnt"][0, g, i] == len(want)
            assert list(got[:len(want)]) == want
            assert np.all(got[len(want):] == -1)


def test_topk_worked_example():
    fx = json.load(open(os.path.join(GOLDEN, "topk_worked.json")))
    K = np.array(fx["K"], np.float32)[None, None]
    Q = np.array(fx["Q"], np.float32)[None, None]
    B = fx["B"]
    S = oracle.summarize(K, B)
    np.testing.assert_array_equal(S[0, 0], np.array(fx["summaries"], np.float64))
    qh = oracle.qpool(Q, B)
    np.testing.assert_array_equal(qh[0, 0], np.array(fx["qhat"], np.float64))
    for key, k in (("k2_diag", 2), ("k3_diag", 3)):
        r = oracle.route_topk(qh, S, B, k, oracle.FORCE_DIAG)
        np.testing.assert_array_equal(r["idx"][0, 0], np.array(fx[key]["idx"]))
        np.testing.assert_array_equal(r["cnt"][0, 0], np.array(fx[key]["cnt"]))
        want = np.array([[np.nan if v is None else v / math.sqrt(2) for v in row]
                         for row in fx["scores_times_sqrt2"]])
        got = r["scores"][0, 0]
        mask = ~np.isnan(want)
        np.testing.assert_allclose(got[mask], want[mask], rtol=0, atol=1e-15)
    az = fx["attend_zero_q"]
    r = oracle.route_topk(qh, S, B, 3, oracle.FORCE_DIAG)
    O, _ = oracle.attend(np.zeros_like(Q), K, np.array(az["V"], np.float32)[None, None], B,
                         r["idx"], r["cnt"])
    np.testing.assert_allclose(O, np.array(az["O"]), rtol=0, atol=1e-15)


def test_topk_decode_permutation_equivariance():
    rng = _rng(7)
    B, L, d, hq, hkv = 8, 8 * 12 + 1, 16, 2, 1
    S = rng.standard_normal((1, hkv, 13, d))
    q = rng.standard_normal((1, hq, 1, d))
    perm = np.concatenate([rng.permutation(12), [12]])  # tail block 12 stays last
    r0 = oracle.route_topk(q, S, B, 5, oracle.FORCE_TAIL, mode=oracle.MODE_DECODE, kv_lens=[L])
    r1 = oracle.route_topk(q, S[:, :, perm], B, 5, oracle.FORCE_TAIL, mode=oracle.MODE_DECODE,
                           kv_lens=[L])
    sel0 = set(r0["idx"][0, 0, 0][:r0["cnt"][0, 0, 0]])
    sel1 = set(perm[r1["idx"][0, 0, 0][:r1["cnt"][0, 0, 0]]])
    assert sel0 == sel1 and 12 in sel0 and len(sel0) == 5


def test_topk_decode_candidates_and_tail():
    rng = _rng(8)
    B, d = 4, 8
    S = rng.standard_normal((3, 1, 6, d))
    q = rng.standard_normal((3, 1, 1, d))
    lens = [21, 8, 1]  # tails 5 (1 token), 1 (full block), 0 (first token)
    r = oracle.route_topk(q, S, B, 3, oracle.FORCE_TAIL, mode=oracle.MODE_DECODE, kv_lens=lens)
    for b, L in enumerate(lens):
        tail = (L - 1) // B
        sel = list(r["idx"][b, 0, 0][:r["cnt"][b, 0, 0]])
        assert tail in sel
        assert all(j <= tail for j in sel)
        assert np.all(np.isneginf(r["scores"][b, 0, 0, tail:]))
        assert r["cnt"][b, 0, 0] == min(3, tail + 1)


def test_topk_k_covers_everything():
    rng = _rng(9)
    S = rng.standard_normal((1, 1, 5, 4))
    q = rng.standard_normal((1, 1, 5, 4))
    r = oracle.route_topk(q, S, 4, 5, 0)
    for i in range(5):
        assert list(r["idx"][0, 0, i][:r["cnt"][0, 0, i]]) == list(range(i + 1))
        assert r["gap"][0, 0, i] == np.inf


# --------------------------------------------------------------------------
# Fine attention
# --------------------------------------------------------------------------

def _sdpa_causal(Q, K, V, scale=None):
    """torch's scaled_dot_product_attention (causal) in fp64 on CPU, GQA expanded."""
    hq, hkv = Q.shape[1], K.shape[1]
    Kx = np.repeat(K, hq // hkv, axis=1)
    Vx = np.repeat(V, hq // hkv, axis=1)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        t(Q), t(Kx), t(Vx), is_causal=True, scale=scale).numpy()


@pytest.mark.parametrize("n,B,hq,hkv", [(64, 16, 2, 2), (70, 16, 4, 2), (37, 8, 4, 1)])
def test_all_blocks_is_dense_causal_sdpa(n, B, hq, hkv):
    rng = _rng(10)
    d = 16
    Q = rng.standard_normal((2, hq, n, d)).astype(np.float32)
    K = rng.standard_normal((2, hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((2, hkv, n, d)).astype(np.float32)
    nblk = -(-n // B)
    r = oracle.route_topk(oracle.qpool(Q, B), oracle.summarize(K, B), B, nblk, oracle.FORCE_DIAG)
    O, pairs = oracle.attend(Q, K, V, B, r["idx"], r["cnt"])
    ref = _sdpa_causal(Q, K, V)
    np.testing.assert_allclose(O.reshape(ref.shape), ref, rtol=0, atol=1e-12)
    assert pairs.sum() == 2 * hq * n * (n + 1) // 2


def test_decode_all_blocks_is_dense_attention_over_cache():
    rng = _rng(11)
    B, d, hq, hkv, Lmax = 8, 16, 4, 2, 45
    lens = [45, 33, 8]
    K = rng.standard_normal((3, hkv, Lmax, d)).astype(np.float32)
    V = rng.standard_normal((3, hkv, Lmax, d)).astype(np.float32)
    q = rng.standard_normal((3, hq, 1, d)).astype(np.float32)
    nblk = -(-Lmax // B)
    S = oracle.summarize(K, B)
    r = oracle.route_topk(oracle.qpool(q, B), S, B, nblk, oracle.FORCE_TAIL, mode=oracle.MODE_DECODE,
                          kv_lens=lens)
    O, _ = oracle.attend(q, K, V, B, r["idx"], r["cnt"], mode=oracle.MODE_DECODE, kv_lens=lens)
    O = O.reshape(3, hq, d)
    for b, L in enumerate(lens):
        Kx = np.repeat(K[b:b + 1, :, :L], hq // hkv, 1)
        Vx = np.repeat(V[b:b + 1, :, :L], hq // hkv, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b:b + 1].astype(np.float64)), torch.from_numpy(Kx.astype(np.float64)),
            torch.from_numpy(Vx.astype(np.float64))).numpy()
        np.testing.assert_allclose(O[b], ref[0, :, 0], rtol=0, atol=1e-12)


def test_decode_equals_prefill_last_row_on_same_selection():
    rng = _rng(12)
    B, d, h, L = 8, 16, 2, 40
    Q = rng.standard_normal((1, h, L, d)).astype(np.float32)
    K = rng.standard_normal((1, h, L, d)).astype(np.float32)
    V = rng.standard_normal((1, h, L, d)).astype(np.float32)
    sel = np.array([[[[0, 2, 4, -1]] * 5]], np.int32).reshape(1, h // h, 5, 4)
    sel = np.repeat(sel, h, axis=1)
    cnt = np.full((1, h, 5), 3, np.int32)
    Op, _ = oracle.attend(Q, K, V, B, sel, cnt, req=[[0, hh, L - 1] for hh in range(h)])
    Od, _ = oracle.attend(Q[:, :, L - 1:], K, V, B, sel[:, :, 4:5], cnt[:, :, 4:5],
                          req=[[0, hh, 0] for hh in range(h)], mode=oracle.MODE_DECODE, kv_lens=[L])
    np.testing.assert_array_equal(Op, Od)


def test_zero_query_reveals_attended_token_set():
    """q = 0 gives uniform weights, and one-hot values make o the indicator of
    the attended set divided by its size."""
    rng = _rng(13)
    n, B, d = 48, 8, 64
    Q = np.zeros((1, 2, n, d), np.float32)
    K = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    V = np.eye(n, d, dtype=np.float32)[None, None]
    nblk = n // B
    idx = np.full((1, 1, nblk, 3), -1, np.int32)
    cnt = np.zeros((1, 1, nblk), np.int32)
    for i in range(nblk):
        sel = sorted(set(rng.choice(i + 1, size=min(2, i + 1), replace=False)) | {i})
        idx[0, 0, i, :len(sel)] = sel
        cnt[0, 0, i] = len(sel)
    O, pairs = oracle.attend(Q, K, V, B, idx, cnt)
    O = O.reshape(2, n, d)
    for t in range(n):
        i = t // B
        T = {tp for j in idx[0, 0, i, :cnt[0, 0, i]] for tp in range(j * B, (j + 1) * B) if tp <= t}
        want = np.zeros(d)
        want[sorted(T)] = 1.0 / len(T)
        np.testing.assert_allclose(O[0, t], want, rtol=0, atol=1e-15)
        np.testing.assert_allclose(O[1, t], want, rtol=0, atol=1e-15)
        assert pairs[t] == len(T)


def test_constant_values_and_first_token():
    rng = _rng(14)
    n, B, d = 40, 8, 16
    Q = rng.standard_normal((1, 2, n, d)).astype(np.float32)
    K = rng.standard_normal((1, 2, n, d)).astype(np.float32)
    V = np.full((1, 2, n, d), 0.375, np.float32)
    r = oracle.route_topk(oracle.qpool(Q, B), oracle.summarize(K, B), B, 2, oracle.FORCE_DIAG)
    O, _ = oracle.attend(Q, K, V, B, r["idx"], r["cnt"])
    np.testing.assert_allclose(O, 0.375, rtol=0, atol=1e-15)
    V = rng.standard_normal((1, 2, n, d)).astype(np.float32)
    O, _ = oracle.attend(Q, K, V, B, r["idx"], r["cnt"], req=[[0, 0, 0], [0, 1, 0]])
    np.testing.assert_array_equal(O[0], V[0, 0, 0].astype(np.float64))
    np.testing.assert_array_equal(O[1], V[0, 1, 0].astype(np.float64))


def test_empty_selection_gives_zero():
    Q = np.ones((1, 1, 8, 4), np.float32)
    idx = np.full((1, 1, 2, 2), -1, np.int32)
    cnt = np.zeros((1, 1, 2), np.int32)
    O, pairs = oracle.attend(Q, Q, Q, 4, idx, cnt)
    assert np.all(O == 0) and np.all(pairs == 0)


@pytest.mark.parametrize("seed", range(4))
def test_dropped_mass_bound(seed):
    """SSA page, sections 1 and 3: the sparse-vs-full error is linear in the
    dropped attention mass.  With delta = dense mass outside the attended set T,
    o_dense - o_sparse = sum_{not T} p v - delta/(1-delta) sum_{T} p v, hence
    |o_sparse - o_dense|_c <= 2 delta max_t |v_{t,c}|.  delta is computed here
    with numpy's softmax, independently of the oracle."""
    rng = _rng(200 + seed)
    n, B, d = 64, 8, 16
    Q = (2.0 * rng.standard_normal((1, 1, n, d))).astype(np.float32)
    K = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    V = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    nblk = n // B
    rs = oracle.route_topk(oracle.qpool(Q, B), oracle.summarize(K, B), B, 3, oracle.FORCE_DIAG)
    rd = oracle.route_topk(oracle.qpool(Q, B), oracle.summarize(K, B), B, nblk, oracle.FORCE_DIAG)
    Os, _ = oracle.attend(Q, K, V, B, rs["idx"], rs["cnt"])
    Od, _ = oracle.attend(Q, K, V, B, rd["idx"], rd["cnt"])
    for t in range(n):
        i = t // B
        T = {tp for j in rs["idx"][0, 0, i, :rs["cnt"][0, 0, i]] for tp in range(j * B, (j + 1) * B)
             if tp <= t}
        a = (K[0, 0, :t + 1].astype(np.float64) @ Q[0, 0, t].astype(np.float64)) / math.sqrt(d)
        p = scipy.special.softmax(a)
        delta = sum(p[u] for u in range(t + 1) if u not in T)
        bound = 2 * delta * np.abs(V[0, 0, :t + 1]).max(axis=0) + 1e-12
        assert np.all(np.abs(Os[t] - Od[t]) <= bound)
        if delta == 0:
            np.testing.assert_allclose(Os[t], Od[t], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# alpha-entmax and its histogram-started threshold (AdaSplash-2, 2.A)
# --------------------------------------------------------------------------

def _sparsemax_sort(z):
    """Sort-based sparsemax (Martins & Astudillo, 2016)."""
    zs = np.sort(z)[::-1]
    cs = np.cumsum(zs)
    k = np.arange(1, len(z) + 1)
    kk = k[1 + k * zs > cs][-1]
    tau = (cs[kk - 1] - 1) / kk
    return np.maximum(z - tau, 0), tau


def _entmax15_sort(z):
    """Exact sort-based 1.5-entmax (Peters, Niculae & Martins, 2019), with
    x = z/2 and p = [x - tau]_+^2."""
    x = np.sort(z / 2)[::-1]
    n = len(x)
    best = None
    for k in range(1, n + 1):
        m = x[:k].mean()
        ss = ((x[:k] - m) ** 2).sum()
        if ss > 1:
            break
        tau = m - math.sqrt((1 - ss) / k)
        if tau < x[k - 1]:
            best = tau
    return np.maximum(z / 2 - best, 0) ** 2, best


def _tau_brentq(x, alpha):
    f = lambda t: np.sum(np.maximum(x - t, 0) ** (1 / (alpha - 1))) - 1
    return scipy.optimize.brentq(f, x.max() - 1, x.max(), xtol=1e-15, rtol=1e-15, maxiter=500)


def test_entmax_worked_examples():
    fx = json.load(open(os.path.join(GOLDEN, "entmax_worked.json")))
    for c in fx["cases"]:
        alpha = c["alpha"]
        x = (alpha - 1) * np.array(c["z"])
        p, tau, res, _, _, _ = oracle.entmax_row(x, alpha)
        assert res
        np.testing.assert_allclose(p, c["p"], rtol=0, atol=1e-14)
        assert abs(tau - c["tau"]) < 1e-14


@pytest.mark.parametrize("seed", range(20))
@pytest.mark.parametrize("scale", [0.05, 1.0, 8.0])
def test_sparsemax_alpha2_matches_sort_based(seed, scale):
    z = scale * _rng(300 + seed).standard_normal(37)
    p, tau, res, _, _, _ = oracle.entmax_row(z, 2.0, max_iter=32)
    ps, ts = _sparsemax_sort(z)
    assert res
    np.testing.assert_allclose(p, ps, rtol=0, atol=1e-12)
    assert abs(tau - ts) < 1e-12


@pytest.mark.parametrize("seed", range(20))
@pytest.mark.parametrize("scale", [0.05, 1.0, 8.0])
def test_entmax15_matches_sort_based(seed, scale):
    z = scale * _rng(400 + seed).standard_normal(41)
    p, tau, res, _, _, _ = oracle.entmax_row(z / 2, 1.5, max_iter=32)
    ps, ts = _entmax15_sort(z)
    assert res
    np.testing.assert_allclose(p, ps, rtol=0, atol=1e-12)
    assert abs(tau - ts) < 1e-12


@pytest.mark.parametrize("alpha", [1.25, 1.5, 1.75, 2.0, 3.0])
@pytest.mark.parametrize("seed", range(6))
def test_entmax_threshold_vs_library_root_finder(alpha, seed):
    x = (alpha - 1) * 3.0 * _rng(500 + seed).standard_normal(50)
    p, tau, res, its, tlo, thi = oracle.entmax_row(x, alpha, max_iter=32)
    t_ref = _tau_brentq(x, alpha)
    # the histogram bracket holds the root (the lower edge is a proven lower bound)
    assert tlo <= t_ref + 1e-12 and t_ref <= thi + 1e-12
    assert thi - tlo <= 1.0 / 16 + 1e-12
    if res:
        assert abs(tau - t_ref) < 1e-9
        np.testing.assert_allclose(p, np.maximum(x - t_ref, 0) ** (1 / (alpha - 1)), rtol=0, atol=1e-8)


@pytest.mark.parametrize("seed", range(10))
def test_entmax_invariants(seed):
    rng = _rng(600 + seed)
    x = 0.5 * 4.0 * rng.standard_normal(64)
    p, tau, res, its, tlo, thi = oracle.entmax_row(x, 1.5)
    assert abs(p.sum() - 1) < 1e-12 and np.all(p >= 0)
    assert set(np.nonzero(p)[0]) == set(np.nonzero(x > tau)[0])
    # shift invariance
    p2, tau2, *_ = oracle.entmax_row(x + 0.3125, 1.5)
    np.testing.assert_allclose(p2, p, rtol=0, atol=1e-12)
    assert abs(tau2 - tau - 0.3125) < 1e-12
    # uniform input -> uniform output
    pu, *_ = oracle.entmax_row(np.full(17, 0.7), 1.5)
    np.testing.assert_allclose(pu, 1 / 17, rtol=0, atol=1e-14)
    # single candidate -> probability one
    p1, t1, r1, *_ = oracle.entmax_row(np.array([0.4]), 1.5)
    assert r1 and p1[0] == 1.0 and abs(t1 - (0.4 - 1)) < 1e-15


def test_entmax_unresolved_keeps_a_superset():
    """With no refinement steps, an unresolved bracket falls back to tau = lo,
    which is below the exact threshold, so the support can only grow."""
    seen_unresolved = False
    for seed in range(40):
        x = 0.5 * _rng(700 + seed).standard_normal(200)
        p, tau, res, its, tlo, thi = oracle.entmax_row(x, 1.5, max_iter=0)
        t_ref = _tau_brentq(x, 1.5)
        assert tau <= t_ref + 1e-12
        assert set(np.nonzero(x > t_ref)[0]) <= set(np.nonzero(p)[0])
        assert abs(p.sum() - 1) < 1e-12
        seen_unresolved |= not res
    assert seen_unresolved


def test_entmax_routing_gqa_identical_heads_and_cap():
    rng = _rng(800)
    B, d, nblk = 4, 8, 12
    S = rng.standard_normal((1, 1, nblk, d))
    q1 = 3.0 * rng.standard_normal((1, 1, nblk, d))
    q4 = np.repeat(q1, 4, axis=1)
    r1 = oracle.route_entmax(q1, S, B, 1.5, 4.0, cap=64)
    r4 = oracle.route_entmax(q4, S, B, 1.5, 4.0, cap=64)
    np.testing.assert_array_equal(r1["idx"], r4["idx"])
    np.testing.assert_allclose(r4["probs"][0, 3], r1["probs"][0, 0], rtol=0, atol=1e-15)
    for i in range(nblk):
        sel = list(r1["idx"][0, 0, i][:r1["cnt"][0, 0, i]])
        support = list(np.nonzero(r1["probs"][0, 0, i])[0])
        assert sel == sorted(set(support) | {i})
        # entmax over the blocks before the diagonal matches the sort-based closed form
        if i > 0:
            z = 4.0 * (S[0, 0, :i] @ q1[0, 0, i]) / math.sqrt(d)
            ps, _ = _entmax15_sort(z)
            np.testing.assert_allclose(r1["probs"][0, 0, i, :i], ps, rtol=0, atol=1e-10)
    # the cap keeps the blocks with the largest mean probability, lower index first on ties
    rc = oracle.route_entmax(q4, S, B, 1.5, 0.01, cap=3)
    wide = oracle.route_entmax(q4, S, B, 1.5, 0.01, cap=64)
    for i in range(nblk):
        w = wide["probs"][0, :, i].mean(0)
        nz = [j for j in range(i) if w[j] > 0]
        keep = sorted(sorted(nz, key=lambda j: (-w[j], j))[:3])
        want = sorted(set(keep) | {i})
        assert list(rc["idx"][0, 0, i][:rc["cnt"][0, 0, i]]) == want


def test_synthetic_generator_is_deterministic_and_sliceable():
    w = synth.WORKLOADS["bf16_gqa_prefill_n32k"].scaled(n=9000, hq=4, hkv=1)
    full = synth.gen(w, "k")
    part = synth.gen(w, "k", t0=4000, t1=8500)
    np.testing.assert_array_equal(full[:, :, 4000:8500], part)
    bits, f = synth.gen_stored(w, "k")
    assert bits.dtype == np.uint16
    ref = torch.from_numpy(full).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(f, ref)
