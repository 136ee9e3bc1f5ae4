"""Parity helpers: run the HIP path and the oracle on the same seeded inputs
and compare them under the stated bars.

Bars (from the method's target):
  * selected block ids bit-exact wherever the k-th/(k+1)-th routed score gap
    exceeds 1e-4 (entmax: every head's min |x - tau| and the cap gap exceed
    1e-4); elsewhere the GPU selection must be a valid one;
  * attention output max abs error <= 1e-4 for fp32 inputs and <= 1e-2 for
    bf16 inputs, against the fp64 oracle attending over the GPU's own
    selection.  A bf16 *output* additionally carries its own rounding:
    |O - O_ref| <= 1e-2 + ulp_bf16(O_ref)/2.
"""
from __future__ import annotations

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
