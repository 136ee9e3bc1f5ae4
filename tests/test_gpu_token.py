"""GPU parity of per-token routing ("DashAttention", Estágio 1 routes every
query) and of the masked tile attention over per-token selections
(Estágio 2, Implementação), against the fp64 oracle's token mode on seeded
inputs small enough to check every row, spanning several tiles and a ragged
tail.  Calls go through the C ABI (ctypes binding)."""
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

W = synth.WORKLOADS
TOPK = {
    "tok_bf16_gqa": W["bf16_gqa_prefill_n32k"].scaled(mode="token", hq=8, hkv=2, n=64 * 21 + 37,
                                                      k_total=6, force=synth.FORCE_DIAG,
                                                      planted_blocks=5, loc_amp=2.0),
    "tok_f32_d64_first": W["fp32_prefill_n1k"].scaled(mode="token", n=64 * 9 + 17, hq=4, hkv=2,
                                                      k_total=3,
                                                      force=synth.FORCE_DIAG | synth.FORCE_FIRST),
    "tok_f32_d128": W["fp32_prefill_n1k"].scaled(mode="token", d=128, n=64 * 6 + 5, hq=2, hkv=1,
                                                 k_total=4, force=0, loc_amp=1.0),
    # B = 128: two 64-key sub-tiles per block; no forced diagonal
    "tok_b128_noforce": W["bf16_long_prefill_n256k"].scaled(mode="token", hq=4, hkv=1,
                                                            n=128 * 9 + 50, k_total=4, force=0,
                                                            planted_blocks=3, loc_amp=2.0),
    "tok_d64_mha": W["bf16_gqa_prefill_n32k"].scaled(mode="token", d=64, hq=3, hkv=3,
                                                     n=64 * 7 + 1, k_total=3,
                                                     force=synth.FORCE_DIAG, planted_blocks=2),
    # 4096 tiles of 64 token rows: the score tiles of a row tile are walked by
    # one workgroup, the next block tile's summaries loading during the
    # current tile's products (and the score matrix written in full)
    "tok_many_rows": W["bf16_gqa_prefill_n32k"].scaled(mode="token", batch=4, d=64, hq=8, hkv=8,
                                                       n=64 * 128, k_total=6,
                                                       force=synth.FORCE_DIAG, planted_blocks=4),
}
ENTMAX = {
    "tok_entmax_g4": W["entmax_prefill_n64k"].scaled(mode="token", hq=8, hkv=2, n=64 * 30 + 5,
                                                     cap=16, gamma=4.0, planted_blocks=5,
                                                     loc_amp=2.0),
    "tok_entmax_g1_cap64": W["entmax_prefill_n64k"].scaled(mode="token", hq=4, hkv=1, n=64 * 25,
                                                           cap=64, gamma=1.0, planted_blocks=4),
    "tok_entmax_a2": W["entmax_prefill_n64k"].scaled(mode="token", hq=4, hkv=2, n=64 * 12 + 33,
                                                     cap=6, gamma=16.0, alpha=2.0, loc_amp=1.0),
    # alpha outside {1.5, 2}: the histogram bracket by bisection
    "tok_entmax_a175": W["entmax_prefill_n64k"].scaled(mode="token", hq=4, hkv=2, n=64 * 20 + 7,
                                                       cap=8, gamma=8.0, alpha=1.75,
                                                       force=synth.FORCE_DIAG | synth.FORCE_FIRST),
    # 601 blocks: 16 logits per lane
    "tok_entmax_e16": W["entmax_prefill_n64k"].scaled(mode="token", hq=2, hkv=1, n=64 * 600 + 9,
                                                      cap=16, gamma=4.0, loc_amp=2.0,
                                                      planted_blocks=8),
}


def _cpu(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("name", list(TOPK))
def test_token_route_topk(name):
    w = TOPK[name]
    print(f"[token route_topk] {name}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt, sc = bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force, want_scores=True, token=True)
    assert idx.shape == (w.batch, w.hkv, w.n, w.k_total)
    ref = oracle.route_topk(x["q"].astype(np.float64), oracle.summarize(x["k"], w.B), w.B,
                            w.k_total, w.force, mode=oracle.MODE_TOKEN)
    gs = _cpu(sc)
    fin = np.isfinite(ref["scores"])
    assert np.array_equal(fin, np.isfinite(gs))
    np.testing.assert_allclose(gs[fin], ref["scores"][fin], rtol=0, atol=1e-5)
    rep = {}
    parity.check_topk_rows(w, _cpu(idx), _cpu(cnt), ref, rep)
    print(rep)


@pytest.mark.parametrize("name", list(ENTMAX))
def test_token_route_entmax(name):
    w = ENTMAX[name]
    print(f"[token route_entmax] {name}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    wsel = torch.empty((w.batch, w.hkv, w.n, w.idx_width), dtype=torch.float32, device="cuda")
    idx, cnt, probs, tau = bsa.route_entmax(x["Q"], S, w.B, w.alpha, w.gamma, w.cap, w.force,
                                            max_iter=w.max_iter, want_probs=True, want_tau=True,
                                            token=True, wsel=wsel)
    qt, Sref = x["q"].astype(np.float64), oracle.summarize(x["k"], w.B)
    ref = oracle.route_entmax(qt, Sref, w.B, w.alpha, w.gamma, w.cap, w.force,
                              max_iter=w.max_iter, mode=oracle.MODE_TOKEN)
    ref_x = oracle.route_entmax(qt, Sref, w.B, w.alpha, w.gamma, w.cap, w.force,
                                max_iter=parity.EXACT_ITERS, mode=oracle.MODE_TOKEN)
    own = np.arange(w.n) // w.B
    lg = parity.entmax_logits(w, qt, Sref, own)
    rep = {}
    parity.check_entmax_rows(w, _cpu(idx), _cpu(cnt), _cpu(probs), _cpu(tau), ref, ref_x, lg,
                             own, rep, gw=_cpu(wsel))
    print(rep)


def _random_token_selection(rng, w, width, p_invalid=0.0):
    """Per-token selections with varied sets (not from a router): each token
    picks a few causal blocks, sometimes none.  With p_invalid some listed ids
    are replaced by ids outside [0, nblk), which the library skips.  Returns
    (idx, cnt) with those ids and (idx, cnt) of the valid ids only, the form
    the oracle takes."""
    idx = np.full((w.batch, w.hkv, w.n, width), -1, np.int32)
    cnt = np.zeros((w.batch, w.hkv, w.n), np.int32)
    for b in range(w.batch):
        for g in range(w.hkv):
            for t in range(w.n):
                own = t // w.B
                c = int(rng.integers(0, min(width, own + 1) + 1))
                sel = np.sort(rng.choice(own + 1, size=c, replace=False))
                idx[b, g, t, :c] = sel
                cnt[b, g, t] = c
    clean_idx, clean_cnt = idx.copy(), cnt.copy()
    if p_invalid > 0:
        bad = rng.random(idx.shape) < p_invalid
        idx[bad] = rng.choice([-7, w.nblk, w.nblk + 100], size=int(bad.sum()))
        for r in zip(*np.nonzero(bad.any(-1))):
            keep = [j for j in idx[r][:cnt[r]] if 0 <= j < w.nblk]
            clean_idx[r] = -1
            clean_idx[r][:len(keep)] = keep
            clean_cnt[r] = len(keep)
    return idx, cnt, clean_idx, clean_cnt


@pytest.mark.parametrize("name", ["tok_bf16_gqa", "tok_b128_noforce"])
def test_token_mask_matches_oracle(name):
    w = TOPK[name]
    print(f"[token_mask] {name}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt = bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force, token=True)
    gi, gc = _cpu(idx), _cpu(cnt)
    cases = [(gi, gc)]
    rng = np.random.default_rng(w.seed + 77)
    ri, rc, _, _ = _random_token_selection(rng, w, 5, p_invalid=0.05)
    rc[0, 0, :3] = [-2, 9, 5]  # negative and over-width counts are clamped
    cases.append((ri, rc))
    for ci, cc in cases:
        uidx, ucnt, ubits = bsa.token_mask(torch.from_numpy(ci).cuda(), torch.from_numpy(cc).cuda(),
                                           w.B)
        ru, rn, rb = oracle.token_union(ci, cc, w.nblk)
        assert np.array_equal(_cpu(ucnt), rn)
        assert np.array_equal(_cpu(uidx), ru)
        assert np.array_equal(_cpu(ubits).view(np.uint64), rb)
    print(f"tiles {rn.size}, mean active blocks {rn.mean():.1f}")


@pytest.mark.parametrize("name", list(TOPK))
@pytest.mark.parametrize("out_f32", [False, True])
def test_token_attend(name, out_f32):
    w = TOPK[name]
    print(f"[token attend] {name} out_f32={out_f32}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt = bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force, token=True)
    O = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt,
                           out_dtype=torch.float32 if out_f32 else None, token=True)
    ref, pairs = oracle.attend(x["q"], x["k"], x["v"], w.B, _cpu(idx), _cpu(cnt),
                               mode=oracle.MODE_TOKEN)
    worst = parity.check_attention(w, _cpu(O).reshape(ref.shape), ref, out_f32 or w.dtype == "f32")
    print(f"max abs err {worst:.3e}, pairs {int(pairs.sum())}")


@pytest.mark.parametrize("name", ["tok_bf16_gqa", "tok_f32_d128", "tok_b128_noforce"])
def test_token_attend_varied_and_empty_selections(name):
    """Selections that differ token by token (including empty ones and
    invalid ids): every query attends exactly over its own token set."""
    w = TOPK[name]
    print(f"[token attend varied] {name}", flush=True)
    x = parity.make(w)
    rng = np.random.default_rng(w.seed + 99)
    ri, rc, ci, cc = _random_token_selection(rng, w, 4, p_invalid=0.03)
    O = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, torch.from_numpy(ri).cuda(),
                           torch.from_numpy(rc).cuda(), out_dtype=torch.float32, token=True)
    ref, pairs = oracle.attend(x["q"], x["k"], x["v"], w.B, ci, cc, mode=oracle.MODE_TOKEN)
    Oh = _cpu(O).reshape(ref.shape)
    worst = parity.check_attention(w, Oh, ref, True)
    assert np.all(Oh[pairs == 0] == 0)
    print(f"max abs err {worst:.3e}, empty rows {int((pairs == 0).sum())}")


@pytest.mark.parametrize("name", list(ENTMAX))
def test_token_entmax_pipeline_attention(name):
    w = ENTMAX[name]
    print(f"[token entmax pipeline] {name}", flush=True)
    x = parity.make(w)
    O, idx, cnt = bsa.prefill_token_entmax(x["Q"], x["K"], x["V"], w.B, w.alpha, w.gamma, w.cap,
                                           max_iter=w.max_iter)
    ref, _ = oracle.attend(x["q"], x["k"], x["v"], w.B, _cpu(idx), _cpu(cnt),
                           mode=oracle.MODE_TOKEN)
    worst = parity.check_attention(w, _cpu(O).reshape(ref.shape), ref, False)
    print(f"max abs err {worst:.3e}")


@pytest.mark.parametrize("name", ["tok_entmax_g4", "tok_entmax_a2"])
@pytest.mark.parametrize("sigma", [0.5, 1.0])
def test_token_prior_induced_attention(name, sigma):
    """Per-token entmax weights as each query's own prior: the tile kernel
    adds sigma * ln w of the query's token for every listed block."""
    w = ENTMAX[name]
    print(f"[token prior attention] {name} sigma={sigma}", flush=True)
    x = parity.make(w)
    O, idx, cnt = bsa.prefill_token_entmax(x["Q"], x["K"], x["V"], w.B, w.alpha, w.gamma, w.cap,
                                           max_iter=w.max_iter, out_dtype=torch.float32,
                                           sigma=sigma)
    S = bsa.summarize(x["K"], w.B)
    wsel = torch.empty(idx.shape, dtype=torch.float32, device="cuda")
    bsa.route_entmax(x["Q"], S, w.B, w.alpha, w.gamma, w.cap, w.force, max_iter=w.max_iter,
                     token=True, wsel=wsel)
    ref, _ = oracle.attend(x["q"], x["k"], x["v"], w.B, _cpu(idx), _cpu(cnt),
                           mode=oracle.MODE_TOKEN, wsel=_cpu(wsel), sigma=sigma)
    worst = parity.check_attention(w, _cpu(O).reshape(ref.shape), ref, True)
    print(f"max abs err {worst:.3e}")


@pytest.mark.parametrize("name", ["tok_bf16_gqa", "tok_f32_d128", "tok_b128_noforce"])
def test_token_prior_random_weights(name):
    """Varied per-token selections and hand-set weights (some zero: the
    block drops out for that token only)."""
    w = TOPK[name]
    x = parity.make(w)
    rng = np.random.default_rng(w.seed + 123)
    ri, rc, ci, cc = _random_token_selection(rng, w, 4, p_invalid=0.03)
    wh = rng.uniform(0.01, 1.0, ri.shape).astype(np.float32)
    wh[rng.random(ri.shape) < 0.15] = 0.0
    # the oracle's copy keeps the weights of the valid ids, in their order
    wc = np.zeros(ci.shape)
    for r in zip(*np.nonzero(rc)):
        keep = [wh[r][s] for s in range(rc[r]) if 0 <= ri[r][s] < w.nblk]
        wc[r][:len(keep)] = keep
    O = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, torch.from_numpy(ri).cuda(),
                           torch.from_numpy(rc).cuda(), out_dtype=torch.float32, token=True,
                           wsel=torch.from_numpy(wh).cuda(), sigma=0.7)
    ref, pairs = oracle.attend(x["q"], x["k"], x["v"], w.B, ci, cc, mode=oracle.MODE_TOKEN,
                               wsel=wc, sigma=0.7)
    Oh = _cpu(O).reshape(ref.shape)
    worst = parity.check_attention(w, Oh, ref, True)
    assert np.all(Oh[pairs == 0] == 0)
    print(f"max abs err {worst:.3e}, empty rows {int((pairs == 0).sum())}")


def test_token_all_blocks_equals_dense_attention():
    """k covering every causal block: per-token routing selects everything
    and the masked attention is dense causal attention."""
    w = TOPK["tok_bf16_gqa"]
    x = parity.make(w)
    O, idx, cnt = bsa.prefill_token_topk(x["Q"], x["K"], x["V"], w.B, w.nblk, force=0,
                                         out_dtype=torch.float32)
    t = np.arange(w.n)
    assert np.array_equal(_cpu(cnt), np.broadcast_to(t // w.B + 1, cnt.shape))
    G = w.hq // w.hkv
    q = torch.from_numpy(x["q"]).double()
    k = torch.from_numpy(np.repeat(x["k"], G, 1)).double()
    v = torch.from_numpy(np.repeat(x["v"], G, 1)).double()
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).numpy()
    parity.check_attention(w, _cpu(O), ref, True)


def test_token_mode_argument_errors():
    w = TOPK["tok_bf16_gqa"]
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt = bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force, token=True)
    with pytest.raises(bsa.BsaError, match="BSA_ERR_INVALID"):
        bsa.route_topk(x["Q"], S, w.B, w.k_total, synth.FORCE_TAIL, token=True)
    shape = bsa.make_shape(batch=w.batch, hq=w.hq, hkv=w.hkv, d=w.d, B=w.B, dtype=bsa.BF16,
                           mode=bsa.TOKEN, q_len=w.n, kv_len=w.n, q=x["Q"], k=x["K"], v=x["V"],
                           o=x["Q"])
    need = bsa.workspace_size(bsa.OP_ATTEND_PREFILL, shape, w.k_total)
    assert need > 0
    O = torch.empty_like(x["Q"])
    small = torch.empty(need // 2, dtype=torch.uint8, device="cuda")
    import ctypes
    rc = bsa.lib.bsa_attend_prefill(ctypes.byref(shape), bsa._ptr(x["Q"]), bsa._ptr(x["K"]),
                                    bsa._ptr(x["V"]), bsa._ptr(idx), bsa._ptr(cnt), w.k_total,
                                    0.0, None, 0.0, bsa._ptr(O), bsa.BF16, None,
                                    bsa._ptr(small), need // 2, None)
    assert rc == -4  # BSA_ERR_WORKSPACE, nothing enqueued
