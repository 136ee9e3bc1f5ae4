"""Parity helpers: run the HIP path and the oracle on the same seeded inputs
and compare them under the stated bars.

Bars (from the method's target):
  * selected block ids bit-exact wherever the k-th/(k+1)-th routed score gap
    exceeds 1e-4 (entmax: every head's min |x - tau| and the cap gap exceed
    1e-4); elsewhere the GPU selection must be a valid one (top-k: a top set
    within 1e-4; entmax: see check_entmax_rows);
  * attention output max abs error <= 1e-4 for fp32 inputs and <= 1e-2 for
    bf16 inputs, against the fp64 oracle attending over the GPU's own
    selection.  A bf16 *output* additionally carries its own rounding:
    |O - O_ref| <= 1e-2 + ulp_bf16(O_ref)/2.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import synth

GAP = 1e-4
TOL_F32 = 1e-4
TOL_BF16 = 1e-2


def to_device(stored: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(stored.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(stored).to("cuda")


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def make(w: synth.Workload):
    """Seeded inputs for workload w: dict with host exact fp32 and device tensors."""
    q_st, q = synth.gen_stored(w, "q")
    k_st, k = synth.gen_stored(w, "k")
    v_st, v = synth.gen_stored(w, "v")
    return dict(q=q, k=k, v=v, Q=to_device(q_st, w.dtype), K=to_device(k_st, w.dtype),
                V=to_device(v_st, w.dtype))


def topk_mode(w):
    return {"decode": oracle.MODE_DECODE, "token": oracle.MODE_TOKEN}.get(w.mode,
                                                                          oracle.MODE_PREFILL)


def own_block(w, row):
    """The routing row's own block in prefill (the row) or token mode (row // B)."""
    return row // w.B if w.mode == "token" else row


def forced_set(w, b, row, kv_lens=None):
    """Forced blocks of a routing row (prefill: DIAG -> row, token: DIAG ->
    row // B, FIRST -> 0; decode: TAIL/DIAG -> the block of the query,
    FIRST -> 0)."""
    F = set()
    if w.force & synth.FORCE_FIRST:
        F.add(0)
    if w.mode in ("prefill", "token"):
        if w.force & synth.FORCE_DIAG:
            F.add(own_block(w, row))
    else:
        L = int(w.lens()[b] if kv_lens is None else kv_lens[b])
        if w.force & (synth.FORCE_DIAG | synth.FORCE_TAIL):
            F.add((L - 1) // w.B)
    return F


def entmax_clear(w, ref):
    """Head-rows whose entmax threshold is decided robustly: every logit is
    more than GAP from tau, and the bisection resolved the support before its
    last allowed step.  A support resolved only at the last step can flip to
    unresolved (tau = the bracket's lower end) under a 1e-7 change of the
    logits, e.g. their fp32 rounding, so its tau is compared for validity
    only."""
    early = (ref["resolved"] != 0) & (ref["iters"] < w.max_iter)
    return (ref["margin"] > GAP) & (early | (w.max_iter == 0))


def check_topk_rows(w, gidx, gcnt, ref, report=None):
    """Selections: exact where the gap rule applies, valid elsewhere."""
    idx, cnt, scores, gap = ref["idx"], ref["cnt"], ref["scores"], ref["gap"]
    exact = gap > GAP
    same = (gidx == idx).all(axis=-1) & (gcnt == cnt)
    bad = exact & ~same
    assert not bad.any(), f"{int(bad.sum())} rows differ although their gap exceeds {GAP}"
    for r in zip(*np.nonzero(~exact & ~same)):
        b, g, row = (int(x) for x in r)
        F = forced_set(w, b, row)
        sel = set(gidx[r][:gcnt[r]].tolist())
        assert gcnt[r] == cnt[r], f"row {r}: count {gcnt[r]} != {cnt[r]}"
        assert np.all(gidx[r][gcnt[r]:] == -1)
        assert F <= sel, f"row {r}: forced blocks missing"
        sc = scores[r]
        routed = [j for j in sel - F]
        unsel = [j for j in np.nonzero(np.isfinite(sc))[0] if j not in sel and j not in F]
        assert all(np.isfinite(sc[j]) for j in routed), f"row {r}: non-candidate routed"
        if routed and unsel:
            assert min(sc[j] for j in routed) >= max(sc[j] for j in unsel) - GAP, f"row {r}"
    if report is not None:
        report["rows"] = int(gap.size)
        report["exact_rule_rows"] = int(exact.sum())
        report["match_rate"] = float(same.mean())


def check_attention(w, O_gpu, O_ref, out_f32):
    tol = TOL_F32 if w.dtype == "f32" else TOL_BF16
    err = np.abs(O_gpu.astype(np.float64) - O_ref)
    if w.dtype == "bf16" and not out_f32:
        lim = tol + half_ulp_bf16(O_ref)
    else:
        lim = tol
    worst = float(err.max()) if err.size else 0.0
    assert np.all(err <= lim), f"max abs error {worst:.3e} exceeds the bar ({tol})"
    return worst


EXACT_ITERS = 32  # bisections of the oracle run that stands in for the exact threshold


def entmax_logits(w, qhat, S, own):
    """Routing logits x = (alpha - 1) * gamma * qhat.s_j / sqrt(d) of the
    candidate blocks of each row r (-inf elsewhere), fp64: the blocks before
    own[r], less block 0 when it is forced.  qhat [nb, hq, R, d] (block means,
    or the tokens' own queries), S [nb, hkv, nblk, d] oracle summaries, own [R]
    each row's own (diagonal) block."""
    nb, hq, R, d = qhat.shape
    hkv, nblk = S.shape[1], S.shape[2]
    G = hq // hkv
    x = np.empty((nb, hq, R, nblk), np.float64)
    for b in range(nb):
        for h in range(hq):
            x[b, h] = qhat[b, h] @ S[b, h // G].T
    x *= (w.alpha - 1.0) * w.gamma / np.sqrt(d)
    x[:, :, np.arange(nblk)[None, :] >= np.asarray(own)[:, None]] = -np.inf
    if w.force & synth.FORCE_FIRST:
        x[..., 0] = -np.inf
    return x


def check_entmax_rows(w, gi, gc, gp, gt, ref, ref_x, x, own, report=None, gw=None):
    """Entmax selections of the GPU against the oracle, on every row.

    gi/gc [nb, hkv, R, width] / [nb, hkv, R] GPU lists and counts; gp/gt
    [nb, hq, R, nblk] / [nb, hq, R] GPU probabilities and thresholds; ref the
    oracle run with the workload's bisection budget (the GPU's algorithm);
    ref_x the oracle run with EXACT_ITERS bisections (tau within 2^-36 of the
    exact root); x the logits (entmax_logits); own [R] each row's diagonal.

    Rows whose decision has margin (entmax_clear on every head and a cap gap
    above GAP) must match the oracle bit for bit, with tau and p within 2e-5.
    Every row, clear or not, must satisfy:
      * tau lies in [tau* - 2^-(4 + max_iter) - 2e-5, tau* + 2e-5]: the 16-bin
        bracket is 1/16 wide and each bisection halves it, and an unresolved
        row keeps its lower end;
      * p equals the renormalised [x - tau]_+^(1/(alpha-1)) at the GPU's own
        tau (within 2e-5);
      * the support {p > 0} holds every block more than GAP above tau* and
        none more than GAP below the bracket's reach;
      * the list is the forced blocks plus min(|U|, cap) blocks of U (U: blocks with
        group-mean p > 0), ascending, and the kept blocks are a top-cap set of
        U within GAP by the oracle's group-mean weights and by those of the
        oracle's logits at the GPU's tau, and within 1e-6 by the GPU's own;
      * with gw (the GPU's routing weights in the layout of gi): each listed
        routed block's weight is the GPU's group-mean p (within 1e-6), a
        forced block's is 1."""
    G = w.hq // w.hkv
    nb, hq, R, nblk = gp.shape
    own = np.asarray(own)
    width = 2.0 ** -(4 + w.max_iter)
    tx = ref_x["tau"]
    fin = np.isfinite(tx)
    assert np.array_equal(fin, np.isfinite(gt)), "rows with and without candidates differ"
    assert np.array_equal(fin, np.isfinite(ref["tau"]))
    d_tau = gt[fin].astype(np.float64) - tx[fin]
    assert d_tau.max(initial=0) <= 2e-5, f"tau above the exact root by {d_tau.max():.3e}"
    assert d_tau.min(initial=0) >= -width - 2e-5, f"tau below the bracket by {-d_tau.min():.3e}"
    # p from the GPU's own tau, renormalised
    tg = np.where(fin, gt.astype(np.float64), np.inf)[..., None]
    pw = np.clip(x - tg, 0.0, None) ** (1.0 / (w.alpha - 1.0))
    z = pw.sum(-1, keepdims=True)
    pt = np.divide(pw, z, out=np.zeros_like(pw), where=z > 0)
    perr = np.abs(gp.astype(np.float64) - pt).max(initial=0)
    assert perr <= 2e-5, f"p differs from the renormalised weights at the GPU's tau by {perr:.3e}"
    wt = pt.reshape(nb, w.hkv, G, R, nblk).mean(2)
    del pw, pt, tg
    sup = gp > 0
    txe = np.where(fin, tx, np.inf)[..., None]
    must = x > txe + GAP
    may = x > txe - width - GAP
    assert not (must & ~sup).any(), f"{int((must & ~sup).sum())} supported blocks missing"
    assert not (sup & ~may).any(), f"{int((sup & ~may).sum())} blocks beyond the bracket kept"
    del must, may, txe
    # lists: diagonal, ascending, causal, padding
    width_l = gi.shape[-1]
    pos = np.arange(width_l)
    valid = pos[None, None, None, :] < gc[..., None]
    assert np.all(np.where(valid, gi >= 0, gi == -1)), "padding or negative ids"
    asc = (np.diff(gi, axis=-1) > 0) | ~valid[..., 1:]
    assert asc.all(), "ids not strictly ascending"
    rows_own = np.broadcast_to(own[None, None, :, None], gi.shape)
    assert np.all(np.where(valid, gi <= rows_own, True)), "a block after the row's own"
    has_own = (valid & (gi == rows_own)).any(-1)
    assert has_own.all(), f"{int((~has_own).sum())} rows without their diagonal"
    first = bool(w.force & synth.FORCE_FIRST)
    if first:
        has_first = (valid & (gi == 0)).any(-1)
        assert has_first.all(), f"{int((~has_first).sum())} rows without block 0"
    forced = (gi == rows_own) | ((gi == 0) & first)
    kept = np.zeros((nb, w.hkv, R, nblk + 1), bool)
    np.put_along_axis(kept, np.where(valid, gi, nblk), True, axis=-1)
    kept = kept[..., :nblk]
    kept[:, :, np.arange(R), own] = False
    if first:
        kept[..., 0] = False
    wg = gp.astype(np.float64).reshape(nb, w.hkv, G, R, nblk).mean(2)
    wr = ref["probs"].reshape(nb, w.hkv, G, R, nblk).mean(2)
    U = wg > 0
    assert not (kept & ~U).any(), "a kept block outside the group support"
    nk = kept.sum(-1)
    nforced = (valid & forced).sum(-1)
    assert np.array_equal(nk, gc - nforced), "duplicate ids"
    assert np.array_equal(nk, np.minimum(U.sum(-1), w.cap)), "count != min(|U|, cap)"
    drop = U & ~kept
    for wb, tol in ((wr, GAP), (wt, GAP), (wg, 1e-6)):
        lo_k = np.where(kept, wb, np.inf).min(-1)
        hi_d = np.where(drop, wb, -np.inf).max(-1)
        bad = lo_k < hi_d - tol
        assert not bad.any(), f"{int(bad.sum())} rows keep a block below a dropped one"
    if gw is not None:
        ent = np.take_along_axis(wg, np.where(valid, gi, 0), axis=-1)
        ent = np.where(forced, 1.0, ent)
        werr = np.abs(np.where(valid, gw - ent, 0.0)).max(initial=0)
        assert werr <= 1e-6, f"routing weights differ from the group-mean p by {werr:.3e}"
    # exact rows
    clear = entmax_clear(w, ref)
    rt = ref["tau"]
    assert np.abs(gt[fin & clear] - rt[fin & clear]).max(initial=0) < 2e-5
    assert np.abs(gp - ref["probs"])[clear].max(initial=0) < 2e-5
    row_clear = clear.reshape(nb, w.hkv, G, R).all(axis=2) & (ref["capgap"] > GAP)
    same = (gi == ref["idx"]).all(-1) & (gc == ref["cnt"])
    assert same[row_clear].all(), f"{int((~same & row_clear).sum())} clear rows differ"
    if gw is not None:
        assert np.abs(gw - ref["wsel"])[row_clear].max(initial=0) < 2e-5
    if report is not None:
        report["rows"] = int(same.size)
        report["clear_rows"] = int(row_clear.sum())
        report["match_rate"] = float(same.mean())
        report["tau_below_exact_max"] = float(-d_tau.min(initial=0))
        report["mean_count"] = float(gc.mean())
    return same, row_clear


def attend_threads(q, k, v, B, idx, cnt, req, **kw):
    """oracle.attend over the requested rows, split across host threads (each
    oracle call stays single-threaded; ctypes releases the GIL)."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.float32) for a in (q, k, v))
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    cnt = np.ascontiguousarray(cnt, dtype=np.int32)
    nt = max(1, min(16, os.cpu_count() or 1))
    parts = np.array_split(np.ascontiguousarray(req, dtype=np.int64), nt * 4)
    parts = [p for p in parts if len(p)]
    with ThreadPoolExecutor(nt) as ex:
        res = list(ex.map(lambda r: oracle.attend(q, k, v, B, idx, cnt, req=r, **kw), parts))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def sample_query_blocks(w, per_kv=64, planted_cap=64):
    """Query blocks whose attention is checked at full size, per KV head: a
    seeded sample of per_kv blocks, the first and the last block, and the
    blocks holding planted queries (a seeded subset of at most planted_cap of
    them).  Returns {kv_head: sorted block ids}."""
    nq = -(-w.q_len // w.B)
    pq = np.unique(synth.planted_query_positions(w) // w.B)
    out = {}
    for g in range(w.hkv):
        rng = np.random.default_rng(np.random.SeedSequence([w.seed, 900, g]))
        picks = set(rng.choice(nq, size=min(per_kv, nq), replace=False).tolist())
        picks |= {0, nq - 1}
        if len(pq) > planted_cap:
            picks |= set(rng.choice(pq, size=planted_cap, replace=False).tolist())
        else:
            picks |= set(pq.tolist())
        out[g] = sorted(int(i) for i in picks)
    return out


def block_requests(w, blocks):
    """(b, h, t) rows of every query token of the given blocks, for every
    head of each KV head's group and every batch entry."""
    G = w.hq // w.hkv
    rows = []
    for g, blks in blocks.items():
        for b in range(w.batch):
            for h in range(g * G, (g + 1) * G):
                for i in blks:
                    t = np.arange(i * w.B, min((i + 1) * w.B, w.q_len))
                    rows.append(np.stack([np.full_like(t, b), np.full_like(t, h), t], 1))
    return np.concatenate(rows).astype(np.int64)
