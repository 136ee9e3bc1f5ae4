"""GPU parity of the backward pass of the block-sparse fine attention: dQ,
dK, dV through the C ABI against the fp64 oracle's gradients on the same
seeded inputs, selection and upstream gradient.

Bar (bf16 inputs): every gradient element within
    |g - g_ref| <= TOL * scale + ulp_bf16(g_ref)/2 (bf16 gradients only),
with scale the largest |g_ref| of that tensor and TOL = 1e-2.  The kernels
round the weights P and dS = P (dP - Delta) to bf16 (relative error 2^-9)
before their MFMA products, and Delta is taken against the bf16 forward
output, so each gradient carries a relative error of a few 2^-9 of its
largest terms; 1e-2 of the tensor's scale bounds that with room for the
sums' lengths here (up to a few thousand terms).  A bf16 gradient adds its
own rounding."""
import numpy as np
import pytest

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)
import block_sparse_attention_summarize_amd as bsa  # noqa: E402

TOL = 1e-2
W = synth.WORKLOADS
BASE = W["bf16_gqa_prefill_n32k"]
CASES = {
    # GQA 4, several query blocks and a ragged tail
    "gqa_b64": BASE.scaled(hq=8, hkv=2, n=64 * 9 + 17, k_total=4, planted_blocks=2),
    # B = 128 (two 64-query tiles per block), d = 64, first block forced
    "b128_d64": BASE.scaled(hq=4, hkv=1, d=64, n=128 * 6 + 50, B=128, k_total=3,
                            force=synth.FORCE_DIAG | synth.FORCE_FIRST, planted_blocks=1),
    # block 0 selected by all 76 rows: split over three key-side work items
    "split_first": BASE.scaled(hq=2, hkv=2, n=64 * 75 + 3, k_total=3,
                               force=synth.FORCE_DIAG | synth.FORCE_FIRST, planted_blocks=2),
    # 8 query heads per KV head, B = 128
    "g8_b128": BASE.scaled(hq=8, hkv=1, n=128 * 5, B=128, k_total=2, planted_blocks=1),
    # two sequences
    "batch2": BASE.scaled(batch=2, hq=4, hkv=2, n=64 * 6 + 9, k_total=3, planted_blocks=1),
}


def _cpu(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _inputs(w):
    x = parity.make(w)
    do_st, do = synth.gen_stored(w, "do")
    x["dO"], x["do"] = parity.to_device(do_st, w.dtype), do
    return x


def _check(name, g, ref, bf16_out):
    g = _cpu(g).astype(np.float64).reshape(ref.shape)
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(g - ref)
    bound = TOL * scale + (parity.half_ulp_bf16(ref) if bf16_out else 0.0)
    worst = float((err / scale).max())
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{name}: {len(bad)} elements out of bounds, first {bad[0].tolist()}: "
                           f"{g[tuple(bad[0])]} vs {ref[tuple(bad[0])]} (scale {scale:.3g})")
    return worst


def _run(w, grad_dtype=None, o_f32=False):
    x = _inputs(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt = bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force)
    O, L = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt,
                              out_dtype=torch.float32 if o_f32 else None, want_lse=True)
    dQ, dK, dV = bsa.attend_backward(x["Q"], x["K"], x["V"], O, x["dO"], L, w.B, idx, cnt,
                                     grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return x, idx, cnt, O, L, (dQ, dK, dV)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("g_f32", [True, False])
def test_backward_matches_oracle(name, g_f32):
    w = CASES[name]
    print(f"[attend_backward] {name} g_f32={g_f32}", flush=True)
    x, idx, cnt, O, L, grads = _run(w, torch.float32 if g_f32 else None)
    ref = oracle.attend_backward(x["q"], x["k"], x["v"], x["do"], w.B, _cpu(idx), _cpu(cnt))
    errs = [_check(n, g, r, not g_f32) for n, g, r in zip(("dQ", "dK", "dV"), grads, ref)]
    print("max err / scale: dQ %.2e dK %.2e dV %.2e" % tuple(errs))


def test_backward_lse_is_the_log_normaliser():
    """The forward's lse equals the oracle's: ln sum exp over attended keys,
    checked through the weights it implies (O from P = exp(s - lse))."""
    w = CASES["gqa_b64"]
    x, idx, cnt, O, L, _ = _run(w)
    q, k = x["q"].astype(np.float64), x["k"].astype(np.float64)
    idx_c, cnt_c = _cpu(idx), _cpu(cnt)
    G = w.hq // w.hkv
    sc = 1.0 / np.sqrt(w.d)
    Lc = _cpu(L)
    for h in (0, 5):
        for t in (0, 63, 64, 300, w.n - 1):
            r = t // w.B
            toks = [u for j in idx_c[0, h // G, r, :cnt_c[0, h // G, r]]
                    for u in range(j * w.B, min((j + 1) * w.B, t + 1))]
            s = (k[0, h // G, toks] @ q[0, h, t]) * sc
            ref = s.max() + np.log(np.exp(s - s.max()).sum())
            assert abs(Lc[0, h, t] - ref) < 4e-3, (h, t, Lc[0, h, t], ref)


def test_backward_with_fp32_forward_output_and_determinism():
    w = CASES["gqa_b64"]
    x, idx, cnt, O, L, g1 = _run(w, torch.float32, o_f32=True)
    ref = oracle.attend_backward(x["q"], x["k"], x["v"], x["do"], w.B, _cpu(idx), _cpu(cnt))
    for n, g, r in zip(("dQ", "dK", "dV"), g1, ref):
        _check(n, g, r, False)
    g2 = bsa.attend_backward(x["Q"], x["K"], x["V"], O, x["dO"], L, w.B, idx, cnt,
                             grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b), "two calls differ"


def test_backward_autograd_wrapper():
    """sparse_attention(...).backward(dO) gives attend_backward's gradients."""
    w = CASES["b128_d64"]
    x = _inputs(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt = bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force)
    Q = x["Q"].clone().requires_grad_()
    K = x["K"].clone().requires_grad_()
    V = x["V"].clone().requires_grad_()
    O = bsa.sparse_attention(Q, K, V, w.B, idx, cnt)
    O.backward(x["dO"])
    O2, L = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, want_lse=True)
    ref = bsa.attend_backward(x["Q"], x["K"], x["V"], O2, x["dO"], L, w.B, idx, cnt)
    torch.cuda.synchronize()
    assert torch.equal(O.detach(), O2)
    for t, r in zip((Q, K, V), ref):
        assert torch.equal(t.grad, r)


def test_backward_keys_nobody_attends_get_zero():
    """A selection that leaves blocks unselected: their dK, dV are exactly 0,
    and rows with nothing to attend get dQ = 0."""
    w = CASES["gqa_b64"]
    x = _inputs(w)
    nrow = w.nblk
    idx = torch.full((1, w.hkv, nrow, 2), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((1, w.hkv, nrow), dtype=torch.int32, device="cuda")
    for r in range(nrow):
        if r % 3 == 2:
            continue  # this row attends nothing
        sel = [r] + ([r - 2] if r >= 2 else [])
        idx[0, :, r, :len(sel)] = torch.tensor(sel, dtype=torch.int32)
        cnt[0, :, r] = len(sel)
    O, L = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, want_lse=True)
    dQ, dK, dV = bsa.attend_backward(x["Q"], x["K"], x["V"], O, x["dO"], L, w.B, idx, cnt,
                                     grad_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.attend_backward(x["q"], x["k"], x["v"], x["do"], w.B, _cpu(idx), _cpu(cnt))
    for n, g, r in zip(("dQ", "dK", "dV"), (dQ, dK, dV), ref):
        _check(n, g, r, False)
    used = set()
    for r in range(nrow):
        used |= set(_cpu(idx)[0, 0, r, :_cpu(cnt)[0, 0, r]].tolist())
    for j in range(nrow):
        if j not in used:
            assert torch.all(dK[:, :, j * w.B:(j + 1) * w.B] == 0)
            assert torch.all(dV[:, :, j * w.B:(j + 1) * w.B] == 0)
    for r in range(2, nrow, 3):
        assert torch.all(dQ[:, :, r * w.B:min((r + 1) * w.B, w.n)] == 0)


def test_backward_full_size_headline_sampled():
    """bf16 GQA prefill at its full size (N = 32768, 32/8 heads, top-16): the
    oracle's gradients restricted to a sample of query blocks -- every row
    that selected three chosen key blocks (the most selected one, one in the
    middle, the last) -- against the GPU's dQ of those rows and dK, dV of those
    blocks; plus the softmax identities on the whole tensors."""
    w = BASE
    print("[attend_backward] full size", flush=True)
    x, idx, cnt, O, L, (dQ, dK, dV) = _run(w, torch.float32)
    idx_c, cnt_c = _cpu(idx), _cpu(cnt)
    nrow = w.nblk
    g = 3
    sel = np.zeros((nrow, nrow), bool)  # [row, block] for KV head g
    for r in range(nrow):
        sel[r, idx_c[0, g, r, :cnt_c[0, g, r]]] = True
    counts = sel.sum(0)
    blocks = [int(np.argmax(counts)), nrow // 2, nrow - 1]
    mask = np.zeros((1, w.hkv, nrow), bool)
    for j in blocks:
        mask[0, g, sel[:, j]] = True
    print(f"blocks {blocks} selected by {[int(counts[j]) for j in blocks]} rows; "
          f"{int(mask.sum())} rows sampled", flush=True)
    # only KV head g's query heads and the sampled rows enter the oracle
    G = w.hq // w.hkv
    heads = list(range(g * G, (g + 1) * G))
    q = x["q"][:, heads]
    do = x["do"][:, heads]
    k, v = x["k"][:, g:g + 1], x["v"][:, g:g + 1]
    rq, rk, rv = oracle.attend_backward(q, k, v, do, w.B, idx_c[:, g:g + 1], cnt_c[:, g:g + 1],
                                        rowmask=mask[:, g:g + 1])
    gq, gk, gv = _cpu(dQ)[:, heads], _cpu(dK)[:, g:g + 1], _cpu(dV)[:, g:g + 1]
    rows = np.nonzero(mask[0, g])[0]
    tq = np.concatenate([np.arange(r * w.B, min((r + 1) * w.B, w.n)) for r in rows])
    tk = np.concatenate([np.arange(j * w.B, (j + 1) * w.B) for j in blocks])
    e = [_check("dQ", torch.from_numpy(gq[:, :, tq]), rq[:, :, tq], False),
         _check("dK", torch.from_numpy(gk[:, :, tk]), rk[:, :, tk], False),
         _check("dV", torch.from_numpy(gv[:, :, tk]), rv[:, :, tk], False)]
    print("sampled max err / scale: dQ %.2e dK %.2e dV %.2e" % tuple(e))
    # softmax identities: the key gradients of a KV head sum to zero; the
    # value gradients sum to the upstream gradients of its query heads (every
    # query attends at least one key)
    sk = dK.double().sum(dim=2)
    assert float(sk.abs().max()) <= 1e-3 * float(dK.double().abs().sum(dim=2).max())
    sv = dV.double().sum(dim=2)
    ref_v = x["dO"].double().reshape(1, w.hkv, G, w.n, w.d).sum(dim=(2, 3))
    assert float((sv - ref_v).abs().max()) <= 1e-3 * float(ref_v.abs().max() + w.n)


ENT = W["entmax_prefill_n64k"]
PRIOR_CASES = {
    # entmax routing with a prior: the gradient reaches the routing weights,
    # then through the routing to Q and K
    "ent_b64": ENT.scaled(hq=8, hkv=2, n=64 * 12 + 17, gamma=16.0, cap=6, sigma=1.0,
                          planted_blocks=2),
    "ent_b128_d64": ENT.scaled(hq=8, hkv=2, d=64, n=128 * 7 + 40, B=128, gamma=24.0, cap=64,
                               sigma=0.7, planted_blocks=1),
}


@pytest.mark.parametrize("name", list(PRIOR_CASES))
@pytest.mark.parametrize("g_f32", [True, False])
def test_backward_through_prior_and_entmax_routing(name, g_f32):
    """The DashAttention chain: summaries -> entmax routing -> prior-induced
    attention; dL/dw of the listed blocks and the total dQ, dK, dV (attention
    part + routing part) against the oracle's chain on the oracle's own
    routing, which must select the same blocks."""
    w = PRIOR_CASES[name]
    print(f"[prior + routing backward] {name} g_f32={g_f32}", flush=True)
    x = _inputs(w)
    S = bsa.summarize(x["K"], w.B)
    width = w.idx_width
    wsel = torch.empty((w.batch, w.hkv, w.nblk, width), dtype=torch.float32, device="cuda")
    idx, cnt, probs, _ = bsa.route_entmax(x["Q"], S, w.B, w.alpha, w.gamma, w.cap, w.force,
                                          max_iter=w.max_iter, want_probs=True, wsel=wsel)
    O, L = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, wsel=wsel, sigma=w.sigma,
                              want_lse=True)
    dQ, dK, dV, dw = bsa.attend_backward(x["Q"], x["K"], x["V"], O, x["dO"], L, w.B, idx, cnt,
                                         grad_dtype=torch.float32 if g_f32 else None, wsel=wsel,
                                         sigma=w.sigma, want_dwsel=True)
    dQa, dKa = dQ.clone(), dK.clone()
    bsa.route_entmax_backward(x["Q"], S, probs, idx, cnt, dw, w.B, w.alpha, w.gamma, dQ, dK)
    torch.cuda.synchronize()

    So = oracle.summarize(x["k"], w.B)
    qh = oracle.qpool(x["q"], w.B)
    r = oracle.route_entmax(qh, So, w.B, w.alpha, w.gamma, w.cap, w.force, max_iter=w.max_iter,
                            idx_width=width)
    assert np.array_equal(r["idx"], _cpu(idx)) and np.array_equal(r["cnt"], _cpu(cnt))
    rq, rk, rv, rdw = oracle.attend_backward(x["q"], x["k"], x["v"], x["do"], w.B, r["idx"],
                                             r["cnt"], wsel=r["wsel"], sigma=w.sigma)
    gq, gk = oracle.route_entmax_backward(qh, So, r["probs"], r["idx"], r["cnt"], rdw, w.n, w.B,
                                          w.alpha, w.gamma)
    assert np.abs(gq).max() > 1e-2 * np.abs(rq).max()  # the routing part matters here
    if not g_f32:  # bf16 gradients: the totals, with their own rounding
        e = [_check(nm, g, ref, True) for nm, g, ref in
             (("dQ", dQ, rq + gq), ("dK", dK, rk + gk), ("dV", dV, rv))]
        print("max err / scale: dQ %.2e dK %.2e dV %.2e" % tuple(e))
        return
    e = [_check("dwsel", dw, rdw, False),
         _check("dQ attention part", dQa, rq, False),
         _check("dK attention part", dKa, rk, False),
         _check("dQ routing part", dQ - dQa, gq, False),
         _check("dK routing part", dK - dKa, gk, False),
         _check("dQ", dQ, rq + gq, False),
         _check("dK", dK, rk + gk, False),
         _check("dV", dV, rv, False)]
    print("max err / scale: dw %.2e dQa %.2e dKa %.2e dQr %.2e dKr %.2e dQ %.2e dK %.2e "
          "dV %.2e" % tuple(e))
