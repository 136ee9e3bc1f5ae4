"""Parity at the full sizes of the benchmark's workloads, in the launch
configuration the benchmark times.

Routing is checked on every row (bit-exact where the gap or margin rule
applies, valid elsewhere; per-token routing on sampled tokens).  Attention is
checked in full where the oracle finishes in seconds (fp32 prefill N=1024,
decode) and otherwise on every query token of sampled query blocks, for every
head of each KV head's group: per KV head 64 seeded blocks, the first and the
last, and the blocks holding planted queries (at most 64 of them), against the
fp64 oracle attending over the GPU's own selection (split over host threads,
each oracle call single-threaded).
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
# share of entmax rows whose selection equals the oracle's exactly (rows
# without a margin may differ near a threshold or at the cap and are then
# checked for validity)
ENTMAX_MATCH_FLOOR = 0.99


def _cpu(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _check_sampled(w, x, O, idx, cnt):
    """Attention on every token of the sampled query blocks (per KV head: 64
    seeded blocks, the first and last, and the planted-query blocks), every
    head of the group, against the oracle over the GPU's selection."""
    blocks = parity.sample_query_blocks(w)
    req = parity.block_requests(w, blocks)
    ref, pairs = parity.attend_threads(x["q"], x["k"], x["v"], w.B, idx, cnt, req)
    Oh = _cpu(O)
    got = Oh[req[:, 0], req[:, 1], req[:, 2]]
    worst = parity.check_attention(w, got, ref, w.dtype == "f32")
    nblk = sum(len(v) for v in blocks.values())
    print(f"sampled {nblk} query blocks over {len(blocks)} KV heads: {len(req)} rows, "
          f"{int(pairs.sum())} pairs, max abs err {worst:.3e}", flush=True)


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
        _check_sampled(w, x, O, gi, gc_)
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
    qh, Sref = oracle.qpool(x["q"], w.B), oracle.summarize(x["k"], w.B)
    ref = oracle.route_entmax(qh, Sref, w.B, w.alpha, w.gamma, w.cap, w.force,
                              max_iter=w.max_iter)
    ref_x = oracle.route_entmax(qh, Sref, w.B, w.alpha, w.gamma, w.cap, w.force,
                                max_iter=parity.EXACT_ITERS)
    own = np.arange(w.nblk)
    lg = parity.entmax_logits(w, qh, Sref, own)
    gp, gt = _cpu(probs), _cpu(tau)
    # the probabilities of every head-row with candidates sum to one
    fin = np.isfinite(ref["tau"])
    assert np.abs(gp.sum(-1)[fin] - 1).max() < 1e-4
    gi, gc_ = _cpu(idx), _cpu(cnt)
    rep = {}
    parity.check_entmax_rows(w, gi, gc_, gp, gt, ref, ref_x, lg, own, rep)
    rep["mean_support"] = float((ref["probs"] > 0).sum(-1).mean())
    print(f"routing: {rep}", flush=True)
    # rows without a margin may still differ near a threshold or at the cap;
    # on this workload they almost never do
    assert rep["match_rate"] >= ENTMAX_MATCH_FLOOR, rep
    del probs, tau, gp, gt, ref, ref_x, lg
    _check_sampled(w, x, O, gi, gc_)
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
    the tile masks of every tile, and attention on every query of 18
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
    tiles = sorted({0, (w.n - 1) // 64} | set(rng.choice(w.n // 64, size=16, replace=False).tolist()))
    toks = sorted(set(rng.choice(w.n, size=256, replace=False).tolist())
                  | {t for tl in tiles for t in (tl * 64, tl * 64 + 63)} | {w.n - 1})
    gp, gt = _cpu(probs), _cpu(tau)
    toks = np.array(toks)
    ones = [oracle.route_entmax(x["q"][:, :, t:t + 1].astype(np.float64), Sref, w.B, w.alpha,
                                w.gamma, w.cap, w.force, max_iter=it, mode=oracle.MODE_DECODE,
                                kv_lens=[t + 1])
            for it in (w.max_iter, parity.EXACT_ITERS) for t in toks]
    ref, ref_x = ({k: np.concatenate([o[k] for o in part], axis=2) for k in part[0]}
                  for part in (ones[:len(toks)], ones[len(toks):]))
    own = toks // w.B
    lg = parity.entmax_logits(w, x["q"][:, :, toks].astype(np.float64), Sref, own)
    rep = {}
    parity.check_entmax_rows(w, gi[:, :, toks], gc[:, :, toks], gp[:, :, toks], gt[:, :, toks],
                             ref, ref_x, lg, own, rep, gw=gw[:, :, toks])
    print(f"routing: {len(toks)} sampled tokens, {rep}", flush=True)
    assert rep["match_rate"] >= ENTMAX_MATCH_FLOOR, rep
    # the tile masks of every tile, bit-exact against the oracle's union of
    # the GPU's per-token selections
    ru, rn, rb = oracle.token_union(gi, gc, w.nblk)
    gu, gn, gb = _cpu(uidx), _cpu(ucnt), _cpu(ubits).view(np.uint64)
    assert np.array_equal(gn, rn) and np.array_equal(gu, ru) and np.array_equal(gb, rb)
    print(f"tile masks: {rn.size} tiles, mean active blocks {rn.mean():.1f}", flush=True)
    del probs, tau, gp, gu, gb, ru, rb, uidx, ubits
    req = np.array([[0, h, t] for tl in tiles for h in range(w.hq)
                    for t in range(tl * 64, min(tl * 64 + 64, w.n))], np.int64)
    ref, pairs = parity.attend_threads(x["q"], x["k"], x["v"], w.B, gi, gc, req,
                                       mode=oracle.MODE_TOKEN, wsel=gw, sigma=w.sigma)
    got = _cpu(O)[req[:, 0], req[:, 1], req[:, 2]]
    worst = parity.check_attention(w, got, ref, False)
    print(f"attention: tiles {tiles}, {len(req)} rows, {int(pairs.sum())} pairs, "
          f"max abs err {worst:.3e}", flush=True)
    del x, S, O, idx, cnt
    _free()
