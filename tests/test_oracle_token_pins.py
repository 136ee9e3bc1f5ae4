"""Pins of the oracle's per-token routing mode (every query token routed on its
own, "DashAttention", Estágio 1) and of the per-tile active-block mask built
from per-token selections (Estágio 2, Implementação).  CPU only."""
import itertools
import math

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import _brute_topk, _entmax15_sort, _sdpa_causal


def _rng(seed):
    return np.random.default_rng(seed)


def _token_scores(Q, K, B, hkv):
    """numpy: every token's query summed over its GQA group, dotted with the
    mean-pooled keys of each block, over sqrt(d)."""
    nb, hq, n, d = Q.shape
    G = hq // hkv
    nblk = -(-n // B)
    s = np.stack([K[:, :, j * B:(j + 1) * B].astype(np.float64).mean(2) for j in range(nblk)], 2)
    qg = Q.astype(np.float64).reshape(nb, hkv, G, n, d).sum(2)
    return np.einsum("bgtd,bgjd->bgtj", qg, s) / math.sqrt(d)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("force", [0, oracle.FORCE_DIAG, oracle.FORCE_DIAG | oracle.FORCE_FIRST])
def test_token_topk_matches_bruteforce(seed, force):
    rng = _rng(2000 + seed)
    B, n, d, hq, hkv, k_total = 4, 22, 8, 4, 2, 3
    if seed % 2:  # exact ties between scores
        Q = rng.integers(-1, 2, (1, hq, n, d)).astype(np.float32)
        K = rng.integers(-1, 2, (1, hkv, n, d)).astype(np.float32)
    else:
        Q = rng.standard_normal((1, hq, n, d)).astype(np.float32)
        K = rng.standard_normal((1, hkv, n, d)).astype(np.float32)
    r = oracle.route_topk(Q, oracle.summarize(K, B), B, k_total, force, mode=oracle.MODE_TOKEN)
    sc = _token_scores(Q, K, B, hkv)
    assert r["idx"].shape == (1, hkv, n, k_total)
    for g in range(hkv):
        for t in range(n):
            own = t // B
            np.testing.assert_allclose(r["scores"][0, g, t, :own + 1], sc[0, g, t, :own + 1],
                                       rtol=0, atol=1e-12)
            assert np.all(np.isneginf(r["scores"][0, g, t, own + 1:]))
            F = set()
            if force & oracle.FORCE_DIAG:
                F.add(own)
            if force & oracle.FORCE_FIRST:
                F.add(0)
            C = [j for j in range(own + 1) if j not in F]
            want = sorted(F | _brute_topk(sc[0, g, t], C, k_total - len(F)))
            assert r["cnt"][0, g, t] == len(want)
            assert list(r["idx"][0, g, t, :len(want)]) == want
            assert np.all(r["idx"][0, g, t, len(want):] == -1)


@pytest.mark.parametrize("gamma", [1.0, 8.0])
def test_token_entmax_is_sort_based_entmax_over_earlier_blocks(gamma):
    rng = _rng(2100)
    B, n, d = 4, 30, 8
    Q = 2.0 * rng.standard_normal((1, 1, n, d)).astype(np.float32)
    K = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    S = oracle.summarize(K, B)
    r = oracle.route_entmax(Q, S, B, 1.5, gamma, cap=64, mode=oracle.MODE_TOKEN)
    for t in range(n):
        own = t // B
        sel = list(r["idx"][0, 0, t][:r["cnt"][0, 0, t]])
        if own == 0:
            assert sel == [0] and not np.any(r["probs"][0, 0, t])
            continue
        z = gamma * (S[0, 0, :own] @ Q[0, 0, t].astype(np.float64)) / math.sqrt(d)
        ps, _ = _entmax15_sort(z)
        np.testing.assert_allclose(r["probs"][0, 0, t, :own], ps, rtol=0, atol=1e-10)
        assert not np.any(r["probs"][0, 0, t, own:])
        assert sel == sorted(set(np.nonzero(ps)[0].tolist()) | {own})


@pytest.mark.parametrize("router", ["topk", "entmax"])
def test_token_mode_with_queries_constant_per_block_is_block_mode(router):
    """When every query of a block is the same vector, the block's mean query
    is that vector, so each token's selection is its block's selection and the
    attention outputs coincide."""
    rng = _rng(2200)
    B, n, d, hq, hkv = 8, 45, 16, 4, 2
    nblk = -(-n // B)
    base = rng.standard_normal((1, hq, nblk, d)).astype(np.float32)
    Q = np.repeat(base, B, axis=2)[:, :, :n].copy()
    K = rng.standard_normal((1, hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((1, hkv, n, d)).astype(np.float32)
    S = oracle.summarize(K, B)
    np.testing.assert_array_equal(oracle.qpool(Q, B), base.astype(np.float64))
    if router == "topk":
        blk = oracle.route_topk(oracle.qpool(Q, B), S, B, 3, oracle.FORCE_DIAG)
        tok = oracle.route_topk(Q, S, B, 3, oracle.FORCE_DIAG, mode=oracle.MODE_TOKEN)
    else:
        blk = oracle.route_entmax(oracle.qpool(Q, B), S, B, 1.5, 4.0, cap=2)
        tok = oracle.route_entmax(Q, S, B, 1.5, 4.0, cap=2, mode=oracle.MODE_TOKEN)
    rows = np.arange(n) // B
    np.testing.assert_array_equal(tok["idx"], blk["idx"][:, :, rows])
    np.testing.assert_array_equal(tok["cnt"], blk["cnt"][:, :, rows])
    Ob, pb = oracle.attend(Q, K, V, B, blk["idx"], blk["cnt"])
    Ot, pt = oracle.attend(Q, K, V, B, tok["idx"], tok["cnt"], mode=oracle.MODE_TOKEN)
    np.testing.assert_array_equal(Ot, Ob)
    np.testing.assert_array_equal(pt, pb)


@pytest.mark.parametrize("n,B,hq,hkv", [(40, 8, 2, 2), (37, 8, 4, 1)])
def test_token_all_blocks_is_dense_causal_sdpa(n, B, hq, hkv):
    rng = _rng(2300)
    d = 16
    Q = rng.standard_normal((2, hq, n, d)).astype(np.float32)
    K = rng.standard_normal((2, hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((2, hkv, n, d)).astype(np.float32)
    nblk = -(-n // B)
    r = oracle.route_topk(Q, oracle.summarize(K, B), B, nblk, 0, mode=oracle.MODE_TOKEN)
    O, pairs = oracle.attend(Q, K, V, B, r["idx"], r["cnt"], mode=oracle.MODE_TOKEN)
    ref = _sdpa_causal(Q, K, V)
    np.testing.assert_allclose(O.reshape(ref.shape), ref, rtol=0, atol=1e-12)
    assert pairs.sum() == 2 * hq * n * (n + 1) // 2


def test_token_zero_query_reveals_each_tokens_set():
    """q = 0 gives uniform weights; one-hot values make o the indicator of the
    token's own attended set divided by its size."""
    rng = _rng(2400)
    n, B, d = 44, 8, 64
    Q = np.zeros((1, 2, n, d), np.float32)
    K = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    V = np.eye(n, d, dtype=np.float32)[None, None]
    idx = np.full((1, 1, n, 3), -1, np.int32)
    cnt = np.zeros((1, 1, n), np.int32)
    for t in range(n):
        own = t // B
        sel = sorted(set(rng.choice(own + 1, size=min(2, own + 1), replace=False).tolist()) | {own})
        idx[0, 0, t, :len(sel)] = sel
        cnt[0, 0, t] = len(sel)
    O, pairs = oracle.attend(Q, K, V, B, idx, cnt, mode=oracle.MODE_TOKEN)
    O = O.reshape(2, n, d)
    for t in range(n):
        T = {tp for j in idx[0, 0, t, :cnt[0, 0, t]] for tp in range(j * B, (j + 1) * B) if tp <= t}
        want = np.zeros(d)
        want[sorted(T)] = 1.0 / len(T)
        np.testing.assert_allclose(O[0, t], want, rtol=0, atol=1e-15)
        np.testing.assert_allclose(O[1, t], want, rtol=0, atol=1e-15)
        assert pairs[t] == len(T)


def test_token_union_worked_example():
    # tile 0: token 0 selects {0, 2}, token 1 {2}, token 2 {1}, token 3 nothing
    idx = np.array([[[[0, 2], [2, -1], [1, -1], [-1, -1]]]], np.int32)
    cnt = np.array([[[2, 1, 1, 0]]], np.int32)
    uidx, ucnt, ubits = oracle.token_union(idx, cnt, 4)
    assert ucnt.tolist() == [[[3]]]
    assert uidx[0, 0, 0].tolist() == [0, 1, 2, -1]
    assert ubits[0, 0, 0].tolist() == [0b001, 0b100, 0b011, 0]


@pytest.mark.parametrize("n", [64, 150, 1])
def test_token_union_reconstructs_every_tokens_selection(n):
    rng = _rng(2500 + n)
    nb, hkv, width, nblk = 2, 3, 5, 12
    idx = np.full((nb, hkv, n, width), -1, np.int32)
    cnt = np.zeros((nb, hkv, n), np.int32)
    for b, g, t in itertools.product(range(nb), range(hkv), range(n)):
        c = int(rng.integers(0, width + 1))
        sel = np.sort(rng.choice(nblk, size=c, replace=False))
        idx[b, g, t, :c] = sel
        cnt[b, g, t] = c
    uidx, ucnt, ubits = oracle.token_union(idx, cnt, nblk)
    ntile = -(-n // 64)
    assert uidx.shape == (nb, hkv, ntile, nblk)
    for b, g, tile in itertools.product(range(nb), range(hkv), range(ntile)):
        c = ucnt[b, g, tile]
        u = uidx[b, g, tile, :c]
        bits = ubits[b, g, tile, :c]
        assert np.all(np.diff(u) > 0) and np.all(bits != 0)
        assert np.all(uidx[b, g, tile, c:] == -1) and np.all(ubits[b, g, tile, c:] == 0)
        for r in range(64):
            t = tile * 64 + r
            got = {int(j) for j, w in zip(u, bits) if (int(w) >> r) & 1}
            want = set(idx[b, g, t, :cnt[b, g, t]].tolist()) if t < n else set()
            assert got == want, (b, g, t)


@pytest.mark.parametrize("force", [oracle.FORCE_DIAG, oracle.FORCE_DIAG | oracle.FORCE_FIRST])
def test_token_entmax_row_equals_decode_row_at_its_position(force):
    """A token's entmax routing is the decode routing of a cache of length
    t + 1 with that token as the query (same candidates, blocks before t / B;
    same forced blocks), so single rows of a long sequence can be checked
    one by one."""
    rng = _rng(2600)
    B, n, d, hq, hkv = 8, 70, 16, 4, 2
    Q = rng.standard_normal((1, hq, n, d)).astype(np.float32)
    K = rng.standard_normal((1, hkv, n, d)).astype(np.float32)
    S = oracle.summarize(K, B)
    tok = oracle.route_entmax(Q, S, B, 1.5, 4.0, cap=3, force=force, mode=oracle.MODE_TOKEN)
    for t in [0, 7, 8, 33, 69]:
        one = oracle.route_entmax(Q[:, :, t:t + 1], S, B, 1.5, 4.0, cap=3, force=force,
                                  mode=oracle.MODE_DECODE, kv_lens=[t + 1])
        np.testing.assert_array_equal(one["idx"][:, :, 0], tok["idx"][:, :, t])
        np.testing.assert_array_equal(one["cnt"][:, :, 0], tok["cnt"][:, :, t])
        np.testing.assert_array_equal(one["probs"][:, :, 0], tok["probs"][:, :, t])
