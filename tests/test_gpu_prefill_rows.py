"""Prefill attention at mid sizes (hundreds of query blocks, key lists of 16
to 40 tiles: the four-wavefront and the ping-pong kernels), its output
checked on sampled query blocks and its lse on sampled queries against the
oracle over the GPU's own selection, and on selections edited so that rows
are empty, hold one block or hold only invalid ids between rows that do not
("DashAttention", Estágio 2: attention over the selected blocks only; an
empty selection attends nothing)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_summarize_amd as bsa
import synth
from tests import parity

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
CASES = {
    # 8 KV heads x 256 query blocks, one head each, 16 tiles a row
    "b64_h8_k16": W["bf16_gqa_prefill_n32k"].scaled(hq=8, hkv=8, n=64 * 256, k_total=16,
                                                    planted_blocks=6),
    # B = 128, d = 64, 4 KV heads x 256 query blocks
    "b128_d64_k8": W["bf16_long_prefill_n256k"].scaled(hq=4, hkv=4, d=64, n=128 * 256, k_total=8,
                                                       planted_blocks=4),
    # two sequences with a ragged tail
    "batch2_ragged_k17": W["bf16_gqa_prefill_n32k"].scaled(batch=2, hq=4, hkv=2,
                                                           n=64 * 23 + 13, k_total=17,
                                                           planted_blocks=3),
    # B = 128 with four query heads per KV head (two workgroups per row)
    "b128_g4_k9": W["bf16_long_prefill_n256k"].scaled(hq=8, hkv=2, n=128 * 15 + 100, k_total=9,
                                                      planted_blocks=3),
    # 40 tiles a row (the ping-pong kernel), ragged tail
    "b64_g4_k40": W["bf16_gqa_prefill_n32k"].scaled(hq=8, hkv=2, n=64 * 200 + 33, k_total=40,
                                                    planted_blocks=5),
}


def _cpu(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def _lse_ref(w, x, idx_c, cnt_c, b, h, t):
    G = w.hq // w.hkv
    r = t // w.B
    g = h // G
    ids = [j for j in idx_c[b, g, r, :cnt_c[b, g, r]] if 0 <= j < w.nblk]
    toks = [u for j in ids for u in range(j * w.B, min((j + 1) * w.B, t + 1))]
    if not toks:
        return -np.inf
    s = (x["k"][b, g, toks].astype(np.float64) @ x["q"][b, h, t].astype(np.float64)) / np.sqrt(w.d)
    return s.max() + np.log(np.exp(s - s.max()).sum())


def _check(w, x, O, L, idx, cnt, per_kv):
    idx_c, cnt_c = _cpu(idx), _cpu(cnt)
    blocks = parity.sample_query_blocks(w, per_kv=per_kv, planted_cap=16)
    req = parity.block_requests(w, blocks)
    ref, pairs = parity.attend_threads(x["q"], x["k"], x["v"], w.B, idx_c, cnt_c, req)
    got = _cpu(O)[req[:, 0], req[:, 1], req[:, 2]]
    worst = parity.check_attention(w, got, ref, False)
    Lc = _cpu(L)
    rng = np.random.default_rng(5)
    for row in req[rng.choice(len(req), size=min(48, len(req)), replace=False)]:
        b, h, t = (int(v) for v in row)
        lr = _lse_ref(w, x, idx_c, cnt_c, b, h, t)
        if np.isinf(lr):
            assert Lc[b, h, t] == -np.inf
        else:
            assert abs(Lc[b, h, t] - lr) < 4e-3, (b, h, t, Lc[b, h, t], lr)
    return worst, len(req), int(pairs.sum())


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_rows_sampled(name):
    w = CASES[name]
    print(f"[prefill rows] {name}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt = bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force)
    O, L = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, want_lse=True)
    torch.cuda.synchronize()
    worst, nreq, pairs = _check(w, x, O, L, idx, cnt, per_kv=24)
    print(f"{nreq} rows, {pairs} pairs, max abs err {worst:.3e}")


@pytest.mark.parametrize("name", ["b64_h8_k16", "batch2_ragged_k17", "b64_g4_k40"])
def test_prefill_empty_short_and_invalid_rows(name):
    """Every fifth row empty, every seventh left with its first block only and
    every eleventh with its ids replaced by invalid ones (-1 and past the
    last block)."""
    w = CASES[name]
    print(f"[prefill edited rows] {name}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt = bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force)
    nrow = idx.shape[2]
    rows = torch.arange(nrow, device="cuda")
    cnt[:, :, rows % 5 == 2] = 0
    cnt[:, :, rows % 7 == 3] = torch.clamp(cnt[:, :, rows % 7 == 3], max=1)
    bad = rows % 11 == 4
    idx[:, :, bad, 0::2] = -1
    idx[:, :, bad, 1::2] = w.nblk + 3
    O, L = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, out_dtype=torch.float32,
                              want_lse=True)
    torch.cuda.synchronize()
    # empty and all-invalid rows: zero output and lse -inf on every head
    dead = ((rows % 5 == 2) | bad).cpu().numpy()
    Oc, Lc = _cpu(O), _cpu(L)
    for i in np.nonzero(dead)[0]:
        t0, t1 = i * w.B, min((i + 1) * w.B, w.n)
        assert np.all(Oc[:, :, t0:t1] == 0) and np.all(Lc[:, :, t0:t1] == -np.inf), i
    # sampled rows against the oracle on the edited selection, plus every
    # row next to an edited one
    # the library skips ids outside [0, n_blk); the oracle is given each row's
    # valid ids only
    idx_c, cnt_c = _cpu(idx).copy(), _cpu(cnt).copy()
    for b in range(idx_c.shape[0]):
        for g in range(idx_c.shape[1]):
            for i in range(nrow):
                ids = [j for j in idx_c[b, g, i, :cnt_c[b, g, i]] if 0 <= j < w.nblk]
                idx_c[b, g, i, :] = -1
                idx_c[b, g, i, :len(ids)] = ids
                cnt_c[b, g, i] = len(ids)
    blocks = parity.sample_query_blocks(w, per_kv=16, planted_cap=8)
    near = [i for i in range(nrow) if i % 5 in (1, 3) or i % 7 == 3 or i % 11 in (3, 5)][:40]
    blocks = {g: sorted(set(v) | set(near)) for g, v in blocks.items()}
    req = parity.block_requests(w, blocks)
    ref, _ = parity.attend_threads(x["q"], x["k"], x["v"], w.B, idx_c, cnt_c, req)
    got = Oc[req[:, 0], req[:, 1], req[:, 2]]
    worst = parity.check_attention(w, got, ref, True)
    print(f"{len(req)} rows, max abs err {worst:.3e}")
