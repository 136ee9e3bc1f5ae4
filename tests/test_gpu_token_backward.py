"""GPU parity of the backward pass with per-token selections (the training
path of "DashAttention": Estágio 1 routes every query token, Estágio 2
weights its keys by the prior-induced softmax): dQ, dK, dV, dL/dw and the
routing gradient through the C ABI against the fp64 oracle's token mode on
seeded inputs, with the GPU's selections checked equal to the oracle's own
first.  Bar as in the block-row backward tests: every element within
TOL * scale (+ half a bf16 ulp for bf16 gradients), TOL = 1e-2, scale the
largest |reference| of the tensor."""
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
TOK = oracle.MODE_TOKEN
W = synth.WORKLOADS
TOPK = {
    # GQA 4, B = 64, a ragged last tile
    "tok_gqa_b64": W["bf16_gqa_prefill_n32k"].scaled(mode="token", hq=8, hkv=2, n=64 * 13 + 37,
                                                     k_total=5, force=synth.FORCE_DIAG,
                                                     planted_blocks=4, loc_amp=2.0),
    # B = 128 (two key sub-tiles a block), d = 64, nothing forced
    "tok_b128_d64": W["bf16_long_prefill_n256k"].scaled(mode="token", hq=4, hkv=1, d=64,
                                                        n=128 * 6 + 50, k_total=3, force=0,
                                                        planted_blocks=2, loc_amp=2.0),
    # 8 query heads a KV head: each query's heads span two query-side workgroups
    "tok_g8": W["bf16_gqa_prefill_n32k"].scaled(mode="token", hq=8, hkv=1, n=64 * 9 + 5,
                                                k_total=4,
                                                force=synth.FORCE_DIAG | synth.FORCE_FIRST,
                                                planted_blocks=3, loc_amp=2.0),
}
ENT = W["token_entmax_prefill_n32k"]
PRIOR = {
    "tokent_g4": ENT.scaled(hq=8, hkv=2, n=64 * 14 + 5, cap=8, gamma=4.0, sigma=1.0,
                            planted_blocks=4, loc_amp=2.0),
    # B = 128, d = 64, G = 8
    "tokent_g8_b128_d64": ENT.scaled(hq=8, hkv=1, d=64, n=128 * 6 + 33, B=128, cap=6, gamma=8.0,
                                     sigma=0.7, planted_blocks=2, loc_amp=2.0),
    # G = 3: a workgroup holds heads of two query sub-tiles
    "tokent_g3": ENT.scaled(hq=6, hkv=2, n=64 * 10 + 17, cap=5, gamma=6.0, sigma=1.2,
                            planted_blocks=3, loc_amp=2.0),
    # two sequences
    "tokent_batch2": ENT.scaled(batch=2, hq=4, hkv=1, n=64 * 5 + 3, cap=4, gamma=4.0, sigma=0.8,
                                planted_blocks=2, loc_amp=2.0),
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
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{name}: {len(bad)} elements out of bounds, first {bad[0].tolist()}: "
                           f"{g[tuple(bad[0])]} vs {ref[tuple(bad[0])]} (scale {scale:.3g})")
    return float((err / scale).max())


@pytest.mark.parametrize("name", list(TOPK))
@pytest.mark.parametrize("g_f32", [True, False])
def test_token_backward_matches_oracle(name, g_f32):
    w = TOPK[name]
    print(f"[token attend_backward] {name} g_f32={g_f32}", flush=True)
    x = _inputs(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt = bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force, token=True)
    O, L = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, token=True, want_lse=True)
    grads = bsa.attend_backward(x["Q"], x["K"], x["V"], O, x["dO"], L, w.B, idx, cnt,
                                grad_dtype=torch.float32 if g_f32 else None, token=True)
    torch.cuda.synchronize()
    r = oracle.route_topk(x["q"].astype(np.float64), oracle.summarize(x["k"], w.B), w.B,
                          w.k_total, w.force, mode=TOK)
    assert np.array_equal(r["idx"], _cpu(idx)) and np.array_equal(r["cnt"], _cpu(cnt))
    ref = oracle.attend_backward(x["q"], x["k"], x["v"], x["do"], w.B, r["idx"], r["cnt"],
                                 mode=TOK)
    errs = [_check(n, g, rf, not g_f32) for n, g, rf in zip(("dQ", "dK", "dV"), grads, ref)]
    print("max err / scale: dQ %.2e dK %.2e dV %.2e" % tuple(errs))


@pytest.mark.parametrize("name", list(PRIOR))
@pytest.mark.parametrize("g_f32", [True, False])
def test_token_backward_through_prior_and_entmax_routing(name, g_f32):
    """Per-token entmax routing -> prior-induced attention: dL/dw of every
    token's entries, the attention and routing parts of dQ and dK, and dV
    against the oracle's chain on its own routing, which must select the
    same blocks."""
    w = PRIOR[name]
    print(f"[token prior + routing backward] {name} g_f32={g_f32}", flush=True)
    x = _inputs(w)
    S = bsa.summarize(x["K"], w.B)
    width = w.idx_width
    wsel = torch.empty((w.batch, w.hkv, w.n, width), dtype=torch.float32, device="cuda")
    idx, cnt, probs, _ = bsa.route_entmax(x["Q"], S, w.B, w.alpha, w.gamma, w.cap, w.force,
                                          max_iter=w.max_iter, want_probs=True, wsel=wsel,
                                          token=True)
    O, L = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, token=True, wsel=wsel,
                              sigma=w.sigma, want_lse=True)
    dQ, dK, dV, dw = bsa.attend_backward(x["Q"], x["K"], x["V"], O, x["dO"], L, w.B, idx, cnt,
                                         grad_dtype=torch.float32 if g_f32 else None, wsel=wsel,
                                         sigma=w.sigma, want_dwsel=True, token=True)
    dQa, dKa = dQ.clone(), dK.clone()
    bsa.route_entmax_backward(x["Q"], S, probs, idx, cnt, dw, w.B, w.alpha, w.gamma, dQ, dK,
                              token=True)
    torch.cuda.synchronize()

    So = oracle.summarize(x["k"], w.B)
    r = oracle.route_entmax(x["q"], So, w.B, w.alpha, w.gamma, w.cap, w.force,
                            max_iter=w.max_iter, mode=TOK, idx_width=width)
    assert np.array_equal(r["idx"], _cpu(idx)) and np.array_equal(r["cnt"], _cpu(cnt))
    rq, rk, rv, rdw = oracle.attend_backward(x["q"], x["k"], x["v"], x["do"], w.B, r["idx"],
                                             r["cnt"], wsel=r["wsel"], sigma=w.sigma, mode=TOK)
    gq, gk = oracle.route_entmax_backward(x["q"], So, r["probs"], r["idx"], r["cnt"], rdw, w.n,
                                          w.B, w.alpha, w.gamma, mode=TOK)
    assert np.abs(gq).max() > 1e-2 * np.abs(rq).max()  # the routing part matters here
    if not g_f32:
        e = [_check(nm, g, ref, True) for nm, g, ref in
             (("dQ", dQ, rq + gq), ("dK", dK, rk + gk), ("dV", dV, rv))]
        print("max err / scale: dQ %.2e dK %.2e dV %.2e" % tuple(e))
        return
    e = [_check("dwsel", dw, rdw, False),
         _check("dQ attention part", dQa, rq, False),
         _check("dK attention part", dKa, rk, False),
         _check("dQ routing part", dQ - dQa, gq, False),
         _check("dK routing part", dK - dKa, gk, False),
         _check("dV", dV, rv, False)]
    print("max err / scale: dw %.2e dQa %.2e dKa %.2e dQr %.2e dKr %.2e dV %.2e" % tuple(e))
    # deterministic: a second call gives the same bits
    g2 = bsa.attend_backward(x["Q"], x["K"], x["V"], O, x["dO"], L, w.B, idx, cnt,
                             grad_dtype=torch.float32, wsel=wsel, sigma=w.sigma,
                             want_dwsel=True, token=True)
    torch.cuda.synchronize()
    for a, b in zip((dQa, dKa, dV, dw), g2):
        assert torch.equal(a, b), "two calls differ"


def test_token_backward_full_size_sampled():
    """The per-token entmax workload at its full size (N = 32768, 32/8 heads,
    cap 32, prior sigma = 1): with the GPU's per-token selection and weights
    as input, the oracle's gradients restricted to the tokens that chose two
    sampled key blocks (the last block and one selected by a few hundred
    tokens) against the GPU's dQ and dL/dw of those tokens and dK, dV of
    those blocks; plus the softmax identities on the whole tensors."""
    w = ENT
    print("[token attend_backward] full size", flush=True)
    x = _inputs(w)
    S = bsa.summarize(x["K"], w.B)
    width = w.idx_width
    wsel = torch.empty((w.batch, w.hkv, w.n, width), dtype=torch.float32, device="cuda")
    idx, cnt, _, _ = bsa.route_entmax(x["Q"], S, w.B, w.alpha, w.gamma, w.cap, w.force,
                                      max_iter=w.max_iter, wsel=wsel, token=True)
    O, L = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, token=True, wsel=wsel,
                              sigma=w.sigma, want_lse=True)
    dQ, dK, dV, dw = bsa.attend_backward(x["Q"], x["K"], x["V"], O, x["dO"], L, w.B, idx, cnt,
                                         grad_dtype=torch.float32, wsel=wsel, sigma=w.sigma,
                                         want_dwsel=True, token=True)
    torch.cuda.synchronize()
    idx_c, cnt_c, ws_c = _cpu(idx), _cpu(cnt), _cpu(wsel)
    g = 5
    chose = np.zeros((w.n, w.nblk), bool)
    for t in range(w.n):
        chose[t, idx_c[0, g, t, :cnt_c[0, g, t]]] = True
    counts = chose.sum(0)
    mid = [j for j in range(w.nblk // 4, w.nblk - 1) if 150 <= counts[j] <= 600]
    blocks = [w.nblk - 1] + mid[:1]
    mask = np.zeros((1, w.hkv, w.n), bool)
    for j in blocks:
        mask[0, g, chose[:, j]] = True
    print(f"blocks {blocks} chosen by {[int(counts[j]) for j in blocks]} tokens", flush=True)
    G = w.hq // w.hkv
    heads = list(range(g * G, (g + 1) * G))
    rq, rk, rv, rdw = oracle.attend_backward(
        x["q"][:, heads], x["k"][:, g:g + 1], x["v"][:, g:g + 1], x["do"][:, heads], w.B,
        idx_c[:, g:g + 1], cnt_c[:, g:g + 1], rowmask=mask[:, g:g + 1],
        wsel=ws_c[:, g:g + 1].astype(np.float64), sigma=w.sigma, mode=TOK)
    tq = np.nonzero(mask[0, g])[0]
    tk = np.concatenate([np.arange(j * w.B, (j + 1) * w.B) for j in blocks])
    e = [_check("dQ", torch.from_numpy(_cpu(dQ)[:, heads][:, :, tq]), rq[:, :, tq], False),
         _check("dK", torch.from_numpy(_cpu(dK)[:, g:g + 1][:, :, tk]), rk[:, :, tk], False),
         _check("dV", torch.from_numpy(_cpu(dV)[:, g:g + 1][:, :, tk]), rv[:, :, tk], False),
         _check("dwsel", torch.from_numpy(_cpu(dw)[:, g:g + 1][:, :, tq]), rdw[:, :, tq], False)]
    print("sampled max err / scale: dQ %.2e dK %.2e dV %.2e dw %.2e" % tuple(e))
    sk = dK.double().sum(dim=2)
    assert float(sk.abs().max()) <= 1e-3 * float(dK.double().abs().sum(dim=2).max())
    sv = dV.double().sum(dim=2)
    ref_v = x["dO"].double().reshape(1, w.hkv, G, w.n, w.d).sum(dim=(2, 3))
    assert float((sv - ref_v).abs().max()) <= 1e-3 * float(ref_v.abs().max() + w.n)


def test_token_autograd_wrapper_with_prior():
    """sparse_attention(..., wsel, token=True).backward(dO) gives
    attend_backward's dQ, dK, dV and dL/dw."""
    w = PRIOR["tokent_g4"]
    print("[token autograd wrapper]", flush=True)
    x = _inputs(w)
    S = bsa.summarize(x["K"], w.B)
    wsel = torch.empty((w.batch, w.hkv, w.n, w.idx_width), dtype=torch.float32, device="cuda")
    idx, cnt, _, _ = bsa.route_entmax(x["Q"], S, w.B, w.alpha, w.gamma, w.cap, w.force,
                                      max_iter=w.max_iter, wsel=wsel, token=True)
    Q = x["Q"].clone().requires_grad_()
    K = x["K"].clone().requires_grad_()
    V = x["V"].clone().requires_grad_()
    wp = wsel.clone().requires_grad_()
    O = bsa.sparse_attention(Q, K, V, w.B, idx, cnt, wsel=wp, sigma=w.sigma, token=True)
    O.backward(x["dO"])
    O2, L = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, token=True, wsel=wsel,
                               sigma=w.sigma, want_lse=True)
    ref = bsa.attend_backward(x["Q"], x["K"], x["V"], O2, x["dO"], L, w.B, idx, cnt, wsel=wsel,
                              sigma=w.sigma, want_dwsel=True, token=True)
    torch.cuda.synchronize()
    assert torch.equal(O.detach(), O2)
    for t, r in zip((Q, K, V, wp), ref):
        assert torch.equal(t.grad, r)
