"""Pins of the oracle's attention backward (the gradients of the fine
attention over the selected blocks for a fixed selection): a library autograd
of the dense masked softmax attention, central differences of the oracle's own
forward, and the invariants softmax fixes.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _case(seed, nb=1, hq=4, hkv=2, n=45, d=8, B=8, kmax=3):
    rng = _rng(seed)
    Q = rng.standard_normal((nb, hq, n, d)).astype(np.float32)
    K = rng.standard_normal((nb, hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((nb, hkv, n, d)).astype(np.float32)
    dO = rng.standard_normal((nb, hq, n, d)).astype(np.float32)
    nrow = -(-n // B)
    idx = np.full((nb, hkv, nrow, kmax), -1, np.int32)
    cnt = np.zeros((nb, hkv, nrow), np.int32)
    for b in range(nb):
        for g in range(hkv):
            for r in range(nrow):
                # the own block plus a random subset of earlier ones, in any order
                prev = rng.permutation(r)[: rng.integers(0, kmax)]
                sel = np.concatenate([[r], prev]).astype(np.int32)
                rng.shuffle(sel)
                idx[b, g, r, :len(sel)] = sel
                cnt[b, g, r] = len(sel)
    return Q, K, V, dO, idx, cnt


def _mask(n, B, idx, cnt, b, g):
    m = np.zeros((n, n), bool)
    for t in range(n):
        r = t // B
        for j in idx[b, g, r, :cnt[b, g, r]]:
            m[t, j * B:min((j + 1) * B, t + 1)] = True
    return m


def _torch_grads(Q, K, V, dO, B, idx, cnt, sm_scale):
    """Autograd of the dense attention with the selection as an additive mask."""
    nb, hq, n, d = Q.shape
    G = hq // K.shape[1]
    q = torch.tensor(Q, dtype=torch.float64, requires_grad=True)
    k = torch.tensor(K, dtype=torch.float64, requires_grad=True)
    v = torch.tensor(V, dtype=torch.float64, requires_grad=True)
    outs = []
    for b in range(nb):
        for h in range(hq):
            m = torch.tensor(_mask(n, B, idx, cnt, b, h // G))
            s = (q[b, h] @ k[b, h // G].T) * sm_scale
            p = torch.softmax(s.masked_fill(~m, -math.inf), -1)
            p = torch.nan_to_num(p, nan=0.0)  # rows with nothing attended
            outs.append(p @ v[b, h // G])
    O = torch.stack(outs).reshape(nb, hq, n, d)
    (O * torch.tensor(dO, dtype=torch.float64)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("seed,shape", [(5000, {}), (5001, dict(nb=2, hq=3, hkv=1, n=21, B=4)),
                                        (5002, dict(hq=2, hkv=2, n=16, B=16, kmax=1))])
def test_backward_matches_library_autograd_of_masked_dense_attention(seed, shape):
    Q, K, V, dO, idx, cnt = _case(seed, **shape)
    B = shape.get("B", 8)
    sc = 1.0 / math.sqrt(Q.shape[-1])
    dQ, dK, dV = oracle.attend_backward(Q, K, V, dO, B, idx, cnt)
    tq, tk, tv = _torch_grads(Q, K, V, dO, B, idx, cnt, sc)
    np.testing.assert_allclose(dQ, tq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, tk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, tv, rtol=0, atol=1e-12)


def test_backward_matches_central_differences_of_the_forward():
    """d/dx of sum(dO * O) by the forward oracle, x one entry of Q, K or V."""
    Q, K, V, dO, idx, cnt = _case(5100, hq=2, hkv=1, n=20, d=4, B=4)
    dQ, dK, dV = oracle.attend_backward(Q, K, V, dO, 4, idx, cnt)

    def loss(Qx, Kx, Vx):
        O, _ = oracle.attend(Qx, Kx, Vx, 4, idx, cnt)
        return float((O.reshape(dO.shape) * dO.astype(np.float64)).sum())

    rng = _rng(5101)
    h = 2.0 ** -8  # exactly representable steps in fp32
    for which, g in (("Q", dQ), ("K", dK), ("V", dV)):
        for _ in range(6):
            arrs = dict(Q=Q, K=K, V=V)
            pos = tuple(int(rng.integers(0, s)) for s in arrs[which].shape)
            plus = {k: a.copy() for k, a in arrs.items()}
            minus = {k: a.copy() for k, a in arrs.items()}
            plus[which][pos] += h
            minus[which][pos] -= h
            fd = (loss(plus["Q"], plus["K"], plus["V"]) -
                  loss(minus["Q"], minus["K"], minus["V"])) / (2 * h)
            # central differences err by O(h^2) times third derivatives
            np.testing.assert_allclose(g[pos], fd, rtol=0, atol=2e-4)


def test_backward_softmax_invariants():
    """Shifting every key of a KV head leaves each query's softmax unchanged,
    so the key gradients of that head sum to zero; the weights sum to one, so
    the value gradients sum to the upstream gradients of the rows that attend
    something; a query with a single attended token has zero gradient."""
    Q, K, V, dO, idx, cnt = _case(5200, n=40, B=8)
    dQ, dK, dV = oracle.attend_backward(Q, K, V, dO, 8, idx, cnt)
    np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-12)
    G = Q.shape[1] // K.shape[1]
    want = dO.astype(np.float64).reshape(1, K.shape[1], G, 40, 8).sum(axis=(2, 3))
    np.testing.assert_allclose(dV.sum(axis=2), want, atol=1e-12)
    # token 0 attends only itself (own block, causal)
    np.testing.assert_array_equal(dQ[:, :, 0], 0.0)


def test_backward_of_zero_upstream_is_zero_and_rows_without_blocks_contribute_nothing():
    Q, K, V, dO, idx, cnt = _case(5300, n=24, B=8)
    z = oracle.attend_backward(Q, K, V, np.zeros_like(dO), 8, idx, cnt)
    for g in z:
        np.testing.assert_array_equal(g, 0.0)
    cnt2 = cnt.copy()
    cnt2[:, :, 1] = 0  # query block 1 attends nothing
    dQ, dK, dV = oracle.attend_backward(Q, K, V, dO, 8, idx, cnt2)
    np.testing.assert_array_equal(dQ[:, :, 8:16], 0.0)
    dO2 = dO.copy()
    dO2[:, :, 8:16] = 123.0  # upstream gradient of those rows is ignored
    r = oracle.attend_backward(Q, K, V, dO2, 8, idx, cnt2)
    np.testing.assert_array_equal(r[1], dK)
    np.testing.assert_array_equal(r[2], dV)


def test_backward_row_sample_is_the_restriction_of_the_full_gradient():
    """Gradients are sums over queries: the sample of a set of query blocks
    plus the sample of the rest is the full gradient, a sampled query's dQ is
    its full dQ, and a key block whose selecting rows are all sampled gets its
    full dK, dV."""
    Q, K, V, dO, idx, cnt = _case(5400, n=48, B=8)
    full = oracle.attend_backward(Q, K, V, dO, 8, idx, cnt)
    mask = np.zeros(cnt.shape, bool)
    mask[0, 0, [1, 4]] = True
    mask[0, 1, 5] = True
    a = oracle.attend_backward(Q, K, V, dO, 8, idx, cnt, rowmask=mask)
    b = oracle.attend_backward(Q, K, V, dO, 8, idx, cnt, rowmask=~mask)
    for f, x, y in zip(full, a, b):
        np.testing.assert_allclose(x + y, f, rtol=0, atol=1e-12)
    G = Q.shape[1] // K.shape[1]
    for g, r in ((0, 1), (0, 4), (1, 5)):
        for h in range(g * G, (g + 1) * G):
            np.testing.assert_array_equal(a[0][0, h, 8 * r:8 * r + 8], full[0][0, h, 8 * r:8 * r + 8])
    # the last block of KV head 1 is selected only by its own row (5)
    sel = [r for r in range(6) if 5 in idx[0, 1, r, :cnt[0, 1, r]]]
    assert sel == [5]
    np.testing.assert_allclose(a[1][0, 1, 40:48], full[1][0, 1, 40:48], rtol=0, atol=1e-13)
    np.testing.assert_allclose(a[2][0, 1, 40:48], full[2][0, 1, 40:48], rtol=0, atol=1e-13)
