"""The entmax validity rule of tests/parity.py, on the CPU.

The rule must accept the oracle's own routing (with its outputs rounded to
fp32, as a GPU reports them) and reject each plausible mistake planted in a
copy of that output: a kept block swapped for a lower-weight one, a missing
diagonal, a block dropped from the count, a threshold above the exact root,
weights that do not follow from the threshold, a supported block cut from a
head's support."""
import copy

import numpy as np
import pytest

import oracle
import synth
from tests import parity

W = synth.WORKLOADS


@pytest.fixture(scope="module")
def case():
    # 300 query blocks at gamma 1: supports hold nearly every earlier block and
    # the cap of 64 binds with gaps below 1e-4, so most rows are not exact
    w = W["entmax_prefill_n64k"].scaled(hq=8, hkv=2, n=64 * 300)
    q = synth.gen(w, "q")
    k = synth.gen(w, "k")
    qh = oracle.qpool(q, w.B)
    S = oracle.summarize(k, w.B)
    ref = oracle.route_entmax(qh, S, w.B, w.alpha, w.gamma, w.cap, w.force, max_iter=w.max_iter)
    refx = oracle.route_entmax(qh, S, w.B, w.alpha, w.gamma, w.cap, w.force,
                               max_iter=parity.EXACT_ITERS)
    own = np.arange(w.nblk)
    x = parity.entmax_logits(w, qh, S, own)
    got = dict(idx=ref["idx"].copy(), cnt=ref["cnt"].copy(),
               probs=ref["probs"].astype(np.float32), tau=ref["tau"].astype(np.float32))
    return w, ref, refx, x, own, got


def _run(case, got):
    w, ref, refx, x, own, _ = case
    rep = {}
    parity.check_entmax_rows(w, got["idx"], got["cnt"], got["probs"], got["tau"], ref, refx, x,
                             own, rep)
    return rep


def test_accepts_oracle_output(case):
    rep = _run(case, case[5])
    assert rep["match_rate"] == 1.0
    # the case exercises the non-exact path
    assert rep["clear_rows"] < rep["rows"] // 2


def _capped_row(case):
    w, ref, _, _, _, got = case
    G = w.hq // w.hkv
    wbar = ref["probs"].reshape(1, w.hkv, G, -1, w.nblk).mean(2)
    U = (wbar > 0).sum(-1)
    r = tuple(int(v) for v in np.argwhere(U > w.cap + 8)[-1])
    return r, wbar[r]


def test_rejects_swapped_block(case):
    w = case[0]
    got = copy.deepcopy(case[5])
    r, wb = _capped_row(case)
    sel = got["idx"][r][:got["cnt"][r]].tolist()
    routed = [j for j in sel if j != r[2]]
    dropped = [j for j in np.nonzero(wb > 0)[0] if j not in sel]
    best = max(routed, key=lambda j: wb[j])
    worst = min(dropped, key=lambda j: wb[j])
    assert wb[best] - wb[worst] > parity.GAP
    sel = sorted(set(sel) - {best} | {int(worst)})
    got["idx"][r][:len(sel)] = sel
    with pytest.raises(AssertionError, match="keep a block below"):
        _run(case, got)
    assert w.cap < len(routed) + len(dropped)


def test_rejects_missing_diagonal(case):
    got = copy.deepcopy(case[5])
    r, _ = _capped_row(case)
    n = got["cnt"][r]
    sel = got["idx"][r][:n].tolist()
    sel.remove(r[2])
    got["idx"][r][:n] = sel + [-1]
    got["cnt"][r] = n - 1
    with pytest.raises(AssertionError):
        _run(case, got)


def test_rejects_short_count(case):
    got = copy.deepcopy(case[5])
    r, _ = _capped_row(case)
    n = got["cnt"][r]
    got["idx"][r][n - 2] = got["idx"][r][n - 1]   # drop one routed block, keep the diagonal last
    got["idx"][r][n - 1] = -1
    got["cnt"][r] = n - 1
    with pytest.raises(AssertionError, match="count"):
        _run(case, got)


def test_rejects_high_tau(case):
    got = copy.deepcopy(case[5])
    got["tau"][0, 3, 200] += 1e-3
    with pytest.raises(AssertionError, match="above the exact root"):
        _run(case, got)


def test_rejects_inconsistent_weights(case):
    got = copy.deepcopy(case[5])
    p = got["probs"][0, 5, 250]
    j = int(np.argmax(p))
    p[j] *= 1.01
    with pytest.raises(AssertionError, match="renormalised"):
        _run(case, got)


def test_rejects_cut_support(case):
    got = copy.deepcopy(case[5])
    p = got["probs"][0, 1, 120]
    j = int(np.argmax(p))
    p[j] = 0.0
    with pytest.raises(AssertionError):
        _run(case, got)


def test_accepts_token_rows_with_block0_forced():
    """Per-token rows with block 0 forced as well as the diagonal, and an
    alpha other than 1.5."""
    w = W["entmax_prefill_n64k"].scaled(mode="token", hq=4, hkv=2, n=64 * 20 + 7, cap=8,
                                        gamma=8.0, alpha=1.75,
                                        force=synth.FORCE_DIAG | synth.FORCE_FIRST)
    q = synth.gen(w, "q").astype(np.float64)
    S = oracle.summarize(synth.gen(w, "k"), w.B)
    ref = oracle.route_entmax(q, S, w.B, w.alpha, w.gamma, w.cap, w.force, max_iter=w.max_iter,
                              mode=oracle.MODE_TOKEN)
    refx = oracle.route_entmax(q, S, w.B, w.alpha, w.gamma, w.cap, w.force,
                               max_iter=parity.EXACT_ITERS, mode=oracle.MODE_TOKEN)
    own = np.arange(w.n) // w.B
    x = parity.entmax_logits(w, q, S, own)
    rep = {}
    parity.check_entmax_rows(w, ref["idx"], ref["cnt"], ref["probs"].astype(np.float32),
                             ref["tau"].astype(np.float32), ref, refx, x, own, rep,
                             gw=ref["wsel"].astype(np.float32))
    assert rep["match_rate"] == 1.0
