"""Parity at the full sizes of the benchmark's workloads, in the launch
configuration the benchmark times.

Routing is checked on every row (bit-exact where the gap rule applies, valid
elsewhere; per-token routing on sampled tokens).  Attention is checked in full where the oracle finishes in
seconds (fp32 prefill N=1024, decode) and otherwise on every query token of a
few seeded query blocks for every head (the first, the last, and seeded
picks), against the fp64 oracle attending over the GPU's own selection.
Each test generates its inputs (up to ~26 GB of host memory for the decode
cache) and frees them before the next."""
import gc

import numpy as np
import pytest

import oracle
import synth
from tests import parity

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)
import block_sparse_attention_summarize_amd as bsa  # noqa: E402

W = synth.WORKLOADS


def _cpu(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _sample_blocks(w, extra, seed):
    rng = np.random.default_rng(seed)
    picks = {0, w.nblk - 1} | set(rng.choice(w.nblk, size=extra, replace=False).tolist())
    return sorted(picks)


def _requests(w, blocks):
    Bq = w.B
    return np.array([[0, h, t] for i in blocks for h in range(w.hq)
                     for t in range(i * Bq, min((i + 1) * Bq, w.n))], np.int64)


def _check_sampled(w, x, O, idx, cnt, blocks):
    req = _requests(w, blocks)
    ref, pairs = oracle.attend(x["q"], x["k"], x["v"], w.B, idx, cnt, req=req)
    Oh = _cpu(O)
    got = Oh[req[:, 0], req[:, 1], req[:, 2]]
    worst = parity.check_attention(w, got, ref, w.dtype == "f32")
    print(f"sampled query blocks {blocks}: {len(req)} rows, {int(pairs.sum())} pairs, "
          f"max abs err {worst:.3e}", flush=True)


def _free():
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["fp32_prefill_n1k", "bf16_gqa_prefill_n32k",
                                  "bf16_long_prefill_n256k"])
def test_full_topk_prefill(name):
    w = W[name]
    print(f"[full topk prefill] {w}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    shape_r = bsa._route_shape(x["Q"], S, w.B, False, None)
    ws = torch.empty(max(bsa.workspace_size(bsa.OP_ROUTE_TOPK, shape_r, w.k_total), 1),
                     dtype=torch.uint8, device="cuda")
    idx, cnt = bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force, ws=ws)
    O = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt)
    torch.cuda.synchronize()
    Sref = oracle.summarize(x["k"], w.B)
    assert np.abs(_cpu(S) - Sref).max() < 2e-6
    ref = oracle.route_topk(oracle.qpool(x["q"], w.B), Sref, w.B, w.k_total, w.force)
    gi, gc_ = _cpu(idx), _cpu(cnt)
    rep = {}
    parity.check_topk_rows(w, gi, gc_, ref, rep)
    print(f"routing: {rep}", flush=True)
    if w.n <= 4096:
        out, _ = oracle.attend(x["q"], x["k"], x["v"], w.B, gi, gc_)
        worst = parity.check_attention(w, _cpu(O).reshape(out.shape), out, w.dtype == "f32")
        print(f"attention: all rows, max abs err {worst:.3e}", flush=True)
    else:
        _check_sampled(w, x, O, gi, gc_, _sample_blocks(w, 3, w.seed + 100))
    del x, S, O, idx, cnt, ws
    _free()


def test_full_entmax_prefill():
    w = W["entmax_prefill_n64k"]
    print(f"[full entmax prefill] {w}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt, probs, tau = bsa.route_entmax(x["Q"], S, w.B, w.alpha, w.gamma, w.cap, w.force,
                                            max_iter=w.max_iter, want_probs=True, want_tau=True)
    O = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt)
    torch.cuda.synchronize()
    ref = oracle.route_entmax(oracle.qpool(x["q"], w.B), oracle.summarize(x["k"], w.B), w.B,
                              w.alpha, w.gamma, w.cap, w.force, max_iter=w.max_iter)
    gp, gt = _cpu(probs), _cpu(tau)
    rt = ref["tau"]
    fin = np.isfinite(rt)
    assert np.array_equal(fin, np.isfinite(gt))
    clear = parity.entmax_clear(w, ref)
    assert np.abs(gt[fin & clear] - rt[fin & clear]).max(initial=0) < 2e-5
    assert np.abs(gp - ref["probs"])[clear].max(initial=0) < 2e-5
    # the probabilities of every resolved head-row sum to one
    sums = gp.sum(-1)[fin]
    assert np.abs(sums - 1).max() < 1e-4
    gi, gc_ = _cpu(idx), _cpu(cnt)
    G = w.hq // w.hkv
    row_clear = clear.reshape(w.batch, w.hkv, G, -1).all(axis=2) & (ref["capgap"] > parity.GAP)
    same = (gi == ref["idx"]).all(-1) & (gc_ == ref["cnt"])
    assert same[row_clear].all(), f"{int((~same & row_clear).sum())} clear rows differ"
    for r in zip(*np.nonzero(~same)):
        sel = gi[r][:gc_[r]]
        assert r[2] in sel and np.all(np.diff(sel) > 0) and sel.max() <= r[2]
    print(f"routing: rows {same.size}, clear {int(row_clear.sum())}, match {same.mean():.4f}, "
          f"mean support {float((ref['probs'] > 0).sum(-1).mean()):.1f}, "
          f"mean count {float(gc_.mean()):.1f}", flush=True)
    del probs, tau, gp, ref
    _check_sampled(w, x, O, gi, gc_, _sample_blocks(w, 1, w.seed + 100))
    del x, S, O, idx, cnt
    _free()


def test_full_decode_step():
    w = W["bf16_decode_l128k"]
    print(f"[full decode step] {w}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    lens = torch.tensor(w.lens(), dtype=torch.int32, device="cuda")
    ws = bsa.decode_workspace(x["Q"], x["K"], w.B, w.k_total)
    O, idx, cnt = bsa.decode_step(x["Q"], x["K"], x["V"], S, w.B, w.k_total, w.force,
                                  kv_lens=lens, ws=ws)
    torch.cuda.synchronize()
    Sref = oracle.summarize(x["k"], w.B)
    assert np.abs(_cpu(S) - Sref).max() < 2e-6
    ref = oracle.route_topk(x["q"].astype(np.float64), Sref, w.B, w.k_total, w.force,
                            mode=oracle.MODE_DECODE, kv_lens=w.lens())
    gi, gc_ = _cpu(idx), _cpu(cnt)
    rep = {}
    parity.check_topk_rows(w, gi, gc_, ref, rep)
    print(f"routing: {rep}", flush=True)
    out, _ = oracle.attend(x["q"], x["k"], x["v"], w.B, gi, gc_, mode=oracle.MODE_DECODE,
                           kv_lens=w.lens())
    worst = parity.check_attention(w, _cpu(O).reshape(out.shape), out, False)
    print(f"attention: all {out.shape[0]} rows, max abs err {worst:.3e}", flush=True)
    del x, S, O, idx, cnt, ws, Sref
    _free()


def test_full_token_entmax_prefill():
    """Per-token entmax routing at full size: sampled tokens' rows are checked
    one by one (a token's row is the decode row of a cache of length t + 1),
    the tile masks of every tile, and attention on every query of a few
    sampled tiles for every head."""
    w = W["token_entmax_prefill_n32k"]
    print(f"[full token entmax prefill] {w}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    wsel = torch.empty((w.batch, w.hkv, w.n, w.idx_width), dtype=torch.float32, device="cuda")
    idx, cnt, probs, tau = bsa.route_entmax(x["Q"], S, w.B, w.alpha, w.gamma, w.cap, w.force,
                                            max_iter=w.max_iter, want_probs=True, want_tau=True,
                                            token=True, wsel=wsel)
    O = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, token=True, wsel=wsel,
                           sigma=w.sigma)
    uidx, ucnt, ubits = bsa.token_mask(idx, cnt, w.B)
    torch.cuda.synchronize()
    gi, gc, gw = _cpu(idx), _cpu(cnt), _cpu(wsel)
    Sref = oracle.summarize(x["k"], w.B)
    assert np.abs(_cpu(S) - Sref).max() < 2e-6
    rng = np.random.default_rng(w.seed + 200)
    tiles = sorted({0, (w.n - 1) // 64} | set(rng.choice(w.n // 64, size=2, replace=False).tolist()))
    toks = sorted(set(rng.choice(w.n, size=96, replace=False).tolist())
                  | {t for tl in tiles for t in (tl * 64, tl * 64 + 63)} | {w.n - 1})
    gp, gt = _cpu(probs), _cpu(tau)
    checked = same_n = clear_n = 0
    for t in toks:
        one = oracle.route_entmax(x["q"][:, :, t:t + 1].astype(np.float64), Sref, w.B, w.alpha,
                                  w.gamma, w.cap, w.force, max_iter=w.max_iter,
                                  mode=oracle.MODE_DECODE, kv_lens=[t + 1])
        clear = parity.entmax_clear(w, one)[:, :, 0]
        fin = np.isfinite(one["tau"][:, :, 0])
        assert np.array_equal(fin, np.isfinite(gt[:, :, t]))
        m = fin & clear
        assert np.abs(gt[:, :, t][m] - one["tau"][:, :, 0][m]).max(initial=0) < 2e-5
        assert np.abs(gp[:, :, t] - one["probs"][:, :, 0])[clear].max(initial=0) < 2e-5
        row_clear = clear.reshape(w.batch, w.hkv, -1).all(-1) & (one["capgap"][:, :, 0] > parity.GAP)
        same = (gi[:, :, t] == one["idx"][:, :, 0]).all(-1) & (gc[:, :, t] == one["cnt"][:, :, 0])
        assert same[row_clear].all(), f"token {t}: clear rows differ"
        assert np.abs(gw[:, :, t] - one["wsel"][:, :, 0])[row_clear].max(initial=0) < 2e-5
        for g in np.nonzero(~same[0])[0]:
            sel = gi[0, g, t, :gc[0, g, t]]
            assert t // w.B in sel and np.all(np.diff(sel) > 0) and sel.max() <= t // w.B
        checked += same.size
        same_n += int(same.sum())
        clear_n += int(row_clear.sum())
    print(f"routing: {checked} sampled rows, clear {clear_n}, match {same_n / checked:.4f}, "
          f"mean count {gc.mean():.1f}", flush=True)
    # the tile masks of every tile, bit-exact against the oracle's union of
    # the GPU's per-token selections
    ru, rn, rb = oracle.token_union(gi, gc, w.nblk)
    gu, gn, gb = _cpu(uidx), _cpu(ucnt), _cpu(ubits).view(np.uint64)
    assert np.array_equal(gn, rn) and np.array_equal(gu, ru) and np.array_equal(gb, rb)
    print(f"tile masks: {rn.size} tiles, mean active blocks {rn.mean():.1f}", flush=True)
    del probs, tau, gp, gu, gb, ru, rb, uidx, ubits
    req = np.array([[0, h, t] for tl in tiles for h in range(w.hq)
                    for t in range(tl * 64, min(tl * 64 + 64, w.n))], np.int64)
    ref, pairs = oracle.attend(x["q"], x["k"], x["v"], w.B, gi, gc, req=req,
                               mode=oracle.MODE_TOKEN, wsel=gw, sigma=w.sigma)
    got = _cpu(O)[req[:, 0], req[:, 1], req[:, 2]]
    worst = parity.check_attention(w, got, ref, False)
    print(f"attention: tiles {tiles}, {len(req)} rows, {int(pairs.sum())} pairs, "
          f"max abs err {worst:.3e}", flush=True)
    del x, S, O, idx, cnt
    _free()
