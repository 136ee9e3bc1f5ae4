#!/usr/bin/env python3
"""Benchmark of block-sparse attention with summary-based block routing on one
MI355X.

A step is one pass of the whole hot path over one batch of seeded synthetic
input already resident in HBM: key summaries (Stage 0), top-k routing
(Stage 1) and fine attention over the selected blocks (Stage 2).  The headline
workload is the largest single-GPU prefill: causal bf16 GQA prefill, batch 1,
16 query / 2 KV heads, N = 262144, d = 128, B = 128, top-32 blocks per
128-query block (diagonal and block 0 always kept).

Printed: one JSON line.  `value` is prefill TFLOP/s counted on the selected
blocks only (4 d flops per causal query-key pair actually attended) over the
whole step.  `roofline` covers the dominant kernel (the MFMA attention) timed
with HIP events on its stream inside the timed region (mean, median and min
launch time); `cpu_baseline` is the fp64 oracle timed on one pinned host core
on a bounded sample of the same workload, with the host described.  `extra`
holds the other workloads: `bf16_gqa_prefill_n32k` (32/8 heads, N = 32768,
B = 64, top-16), `fp32_prefill_n1k` (fp32, 2 heads, N = 1024, d = 64, top-4),
`decode` (batch 16, 32/8 heads, L = 131072, top-32 + tail; GB/s with the
last-level cache flushed between steps; `paged`: the same step over the
cache stored as a shuffled pool of 64-token pages), `entmax_prefill_n64k`
(alpha = 1.5 entmax routing, N = 65536, cap 64) and
`token_entmax_prefill_n32k` (every query token routed by alpha-entmax, cap
32, attention over 64-query tile masks), each with its step time, per-stage
times and attention TFLOP/s, and `entmax_attn_prefill_n16k` (token-level
alpha-entmax attention, dense causal with zero key tiles skipped) timed
beside the dense causal softmax of the same inputs (every block selected),
`backward` (the gradients dQ, dK, dV of the N = 32768 attention for its
selection, beside the forward that feeds them), `train_entmax_prior` (a
training pass of entmax routing with the prior-induced softmax, sigma = 1, on
the N = 65536 entmax inputs: forward, then the attention gradients with
dL/dw and the routing gradient into dQ and dK) and `train_token_prior` (the
same pass with every query token routed, on the per-token inputs);
`cpu_baselines` times the oracle on the other workloads (in full where it
finishes in seconds, else on a sample).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# fp32 VALU without packed fp32 (disabled in every kernel here): 256 CUs x 4
# SIMDs x 16 lanes x 2 flops (fma) x 2.4 GHz
PEAK_F32_VALU_TFLOPS = 78.6
HEADLINE = "bf16_long_prefill_n256k"
GQA32K = "bf16_gqa_prefill_n32k"
FP32 = "fp32_prefill_n1k"
DECODE = "bf16_decode_l128k"
ENTMAX = "entmax_prefill_n64k"
LONG = "bf16_long_prefill_n256k"
TOKEN = "token_entmax_prefill_n32k"
ENTMAX_ATTN = "entmax_attn_prefill_n16k"
PROFILES = os.path.join(HERE, "profiles")
COUNTERS = {ENTMAX_ATTN: "entmax_attn_bf16_n16k_counters.txt",
            HEADLINE: "attend_prefill_bf16_long_n256k_counters.txt",
            GQA32K: "attend_prefill_bf16_gqa_n32k_counters.txt"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=HEADLINE,
                   help="prefill workload of the headline line (a profiling aid)")
    p.add_argument("--only", action="store_true",
                   help="the headline workload alone: no extras, no CPU baseline")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--no-decode", action="store_true", help="skip the decode extra")
    p.add_argument("--no-backward", action="store_true", help="skip the backward extra")
    p.add_argument("--no-train", action="store_true",
                   help="skip the training-pass extras (entmax routing with the prior)")
    p.add_argument("--no-entmax", action="store_true", help="skip the entmax prefill extra")
    p.add_argument("--no-gqa", action="store_true",
                   help="skip the N=32768 prefill extra (and the backward that uses it)")
    p.add_argument("--no-fp32", action="store_true", help="skip the fp32 N=1024 prefill extra")
    p.add_argument("--no-token", action="store_true", help="skip the per-token routing extra")
    p.add_argument("--no-entmax-attn", action="store_true",
                   help="skip the token-level entmax attention extra")
    p.add_argument("--cpu-sample-blocks", type=int, default=6,
                   help="query blocks (all heads) of the headline's CPU-baseline sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (counter calibration)")
    p.add_argument("--entmax-attn-only", action="store_true",
                   help="only run the token-level entmax attention forward (counter runs)")
    return p.parse_args()


def entmax_attn_only(steps, warmup, refine=2):
    """The token-level entmax attention forward alone, for counter runs."""
    import torch
    import block_sparse_attention_summarize_amd as bsa
    w = synth.WORKLOADS[ENTMAX_ATTN]
    x = device_inputs(w, torch)
    O = torch.empty_like(x["Q"])
    for _ in range(warmup + steps):
        bsa.attend_entmax(x["Q"], x["K"], x["V"], w.alpha, refine=refine, out=O)
    torch.cuda.synchronize()
    print(json.dumps({"entmax_attn_launches": warmup + steps, "refine": refine}))


def copy_calibration(mib, reps=3):
    """A plain device-to-device copy of known size: the reference reading for
    the FETCH_SIZE / WRITE_SIZE counters (each launch reads and writes MIB MiB)."""
    import torch
    x = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": mib * 1024 * 1024, "launches": reps}))


def device_inputs(w, torch):
    """Seeded q, k, v of workload w: exact fp32 host copies, device tensors and
    the SHA-256 (first 16 hex digits) of each stored tensor."""
    out = {"sha256": {}}
    for name in ("q", "k", "v"):
        stored, exact = synth.gen_stored(w, name)
        out["sha256"][name] = hashlib.sha256(np.ascontiguousarray(stored).data).hexdigest()[:16]
        if w.dtype == "bf16":
            dev = torch.from_numpy(stored.view(np.int16)).to("cuda").view(torch.bfloat16)
        else:
            dev = torch.from_numpy(stored).to("cuda")
        out[name] = exact
        out[name.upper()] = dev
    return out


def prefill_pairs(w, idx, cnt):
    """Causal query-key pairs attended per the runtime selection, all heads."""
    G = w.hq // w.hkv
    nb = w.nblk
    ntok = np.minimum(w.B, w.n - np.arange(nb) * w.B).astype(np.int64)
    total = 0
    for b in range(idx.shape[0]):
        for g in range(idx.shape[1]):
            for i in range(idx.shape[2]):
                sel = idx[b, g, i, :cnt[b, g, i]]
                sel = sel[(sel >= 0) & (sel <= i)]
                below = sel[sel < i]
                total += int(ntok[i] * ntok[below].sum())
                if (sel == i).any():
                    total += int(ntok[i] * (ntok[i] + 1) // 2)
    return total * G


def token_pairs(w, idx, cnt):
    """Causal query-key pairs attended with per-token selections, all heads:
    a selected block before the token's own is B keys, its own block
    t mod B + 1 keys."""
    t = np.arange(w.n)
    own = (t // w.B)[None, None, :, None]
    listed = np.arange(idx.shape[-1])[None, None, None, :] < cnt[..., None]
    below = listed & (idx >= 0) & (idx < own)
    diag = listed & (idx == own)
    pairs = int(below.sum()) * w.B + int((diag * ((t % w.B) + 1)[None, None, :, None]).sum())
    return pairs * (w.hq // w.hkv)


def source_digest(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def read_traffic(workload, kernel_src):
    """HBM bytes per launch from the committed counter summary of the
    workload's attention, if it was taken on the current kernel source."""
    name = COUNTERS.get(workload)
    path = os.path.join(PROFILES, name) if name else None
    if not path or not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != source_digest(kernel_src):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_info():
    """The host the CPU baseline runs on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": model}


class pinned_core:
    """Pins this process to one core of its affinity set for the duration
    (the oracle is single-threaded), then restores the set."""

    def __enter__(self):
        self.saved = os.sched_getaffinity(0)
        self.core = min(self.saved)
        os.sched_setaffinity(0, {self.core})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.saved)


def _sample_req(w, nsample, seed=12345):
    rng = np.random.default_rng(seed)
    blocks = np.sort(rng.choice(w.nblk, size=min(nsample, w.nblk), replace=False))
    req = np.array([[b, h, t] for b in range(w.batch) for i in blocks for h in range(w.hq)
                    for t in range(i * w.B, min((i + 1) * w.B, w.n))], np.int64)
    return blocks, req


def cpu_baseline(w, x, idx_h, cnt_h, total_flops, nsample):
    """The fp64 oracle on one pinned host core: summaries and routing of every
    row, attention on a seeded sample of query blocks (every head),
    extrapolated by attended pairs to the full step (top-k or entmax
    routing; a sample of every block is the full step)."""
    import oracle
    with pinned_core() as pin:
        t0 = time.perf_counter()
        S = oracle.summarize(x["k"], w.B)
        qh = oracle.qpool(x["q"], w.B)
        if w.router == "topk":
            oracle.route_topk(qh, S, w.B, w.k_total, w.force)
        else:
            oracle.route_entmax(qh, S, w.B, w.alpha, w.gamma, w.cap, w.force,
                                max_iter=w.max_iter)
        t_route = time.perf_counter() - t0
        blocks, req = _sample_req(w, nsample)
        t0 = time.perf_counter()
        _, pairs = oracle.attend(x["q"], x["k"], x["v"], w.B, idx_h, cnt_h, req=req)
        t_att = time.perf_counter() - t0
    total_pairs = total_flops / (4 * w.d)
    full = len(blocks) == w.nblk
    t_total = t_route + (t_att if full else t_att * total_pairs / max(int(pairs.sum()), 1))
    value = total_flops / t_total / 1e12
    host = host_info()
    return {"value": value, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": (f"routing of all {w.batch * w.hkv * w.nblk} rows ({t_route:.1f} s) + "
                       f"attention of {len(blocks)} seeded query blocks x {w.hq} heads "
                       f"({t_att:.1f} s, {int(pairs.sum())} pairs)"
                       + ("" if full else ", extrapolated by pair count to the full step")),
            "seconds_per_step": t_total, "measured": "full step" if full else "extrapolated",
            "pinned_core": pin.core, "host": host,
            "ideal_all_cores_not_measured": {"value": value * host["affinity_cpus"],
                                             "seconds_per_step": t_total / host["affinity_cpus"]}}


def cpu_baseline_decode(w, x, idx_h, cnt_h, total_bytes):
    """The oracle's decode step on one pinned core: routing of every (batch,
    KV head) row over the cached summaries and attention of every query head
    (the full step; the summaries are the cache, computed once and untimed)."""
    import oracle
    S = oracle.summarize(x["k"], w.B)
    with pinned_core() as pin:
        t0 = time.perf_counter()
        oracle.route_topk(x["q"].astype(np.float64), S, w.B, w.k_total, w.force,
                          mode=oracle.MODE_DECODE, kv_lens=w.lens())
        oracle.attend(x["q"], x["k"], x["v"], w.B, idx_h, cnt_h, mode=oracle.MODE_DECODE,
                      kv_lens=w.lens())
        t = time.perf_counter() - t0
    return {"value": total_bytes / t / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "the full step: routing of all rows and attention of every query head",
            "seconds_per_step": t, "pinned_core": pin.core}


def run_prefill(bsa, torch, w, steps, warmup, keep_inputs=True):
    """One prefill step = summaries + routing (top-k or entmax) + fine attention.
    Times `steps` steps back to back (host clock around the synchronised
    region) and each stage with HIP events on the current stream."""
    x = device_inputs(w, torch)
    Q, K, V = x["Q"], x["K"], x["V"]
    token = w.mode == "token"
    nrow = w.nrow
    S = torch.empty((w.batch, w.hkv, w.nblk, w.d), dtype=torch.float32, device="cuda")
    O = torch.empty_like(Q)
    shape_r = bsa._route_shape(Q, S, w.B, False, None, token)
    idx = torch.empty((w.batch, w.hkv, nrow, w.idx_width), dtype=torch.int32, device="cuda")
    cnt = torch.empty((w.batch, w.hkv, nrow), dtype=torch.int32, device="cuda")
    if w.router == "topk":
        ws = torch.empty(bsa.workspace_size(bsa.OP_ROUTE_TOPK, shape_r, w.k_total),
                         dtype=torch.uint8, device="cuda")
    else:
        ws = torch.empty(bsa.workspace_size(bsa.OP_ROUTE_ENTMAX, shape_r, w.cap),
                         dtype=torch.uint8, device="cuda")
    prior = w.router == "entmax" and w.sigma != 0.0
    wsel = torch.empty(idx.shape, dtype=torch.float32, device="cuda") if prior else None
    aws = None
    if token:  # the tile masks (and prior bias) of the per-token attention
        shape_a = bsa.make_shape(batch=w.batch, hq=w.hq, hkv=w.hkv, d=w.d, B=w.B,
                                 dtype=bsa.BF16, mode=bsa.TOKEN, q_len=w.n, kv_len=w.n)
        op = bsa.OP_ATTEND_PREFILL_PRIOR if prior else bsa.OP_ATTEND_PREFILL
        aws = torch.empty(bsa.workspace_size(op, shape_a, w.idx_width), dtype=torch.uint8,
                          device="cuda")
    sel = {"idx": idx, "cnt": cnt}
    ev = []

    def route():
        if w.router == "topk":
            bsa.route_topk(Q, S, w.B, w.k_total, w.force, ws=ws, out=(idx, cnt), token=token)
        else:
            bsa.route_entmax(Q, S, w.B, w.alpha, w.gamma, w.cap, w.force, n_bins=w.n_bins,
                             max_iter=w.max_iter, ws=ws, token=token, out=(idx, cnt), wsel=wsel)

    def step(record=False):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            e[0].record()
        bsa.summarize(K, w.B, out=S)
        if record:
            e[1].record()
        route()
        if record:
            e[2].record()
        bsa.attend_prefill(Q, K, V, w.B, idx, cnt, out=O, token=token, ws=aws, wsel=wsel,
                           sigma=w.sigma)
        if record:
            e[3].record()
            ev.append(e)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(record=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    flops = 4.0 * w.d * (token_pairs(w, idx_h, cnt_h) if token else prefill_pairs(w, idx_h, cnt_h))
    stage = lambda a_, b_: float(np.mean([e[a_].elapsed_time(e[b_]) for e in ev]))
    att_ms = [e[2].elapsed_time(e[3]) for e in ev]
    res = {"workload": w.name, "flops": flops, "elapsed_s": elapsed,
           "attend_s": stage(2, 3) * 1e-3,
           "attend_ms": {"mean": float(np.mean(att_ms)), "median": float(np.median(att_ms)),
                         "min": float(np.min(att_ms)), "max": float(np.max(att_ms))},
           "stages_ms": {"summarize": stage(0, 1), "route": stage(1, 2), "attend": stage(2, 3)},
           "sparsity_vs_causal": 1.0 - flops / (4.0 * w.d * w.hq * w.n * (w.n + 1) / 2),
           "idx_h": idx_h, "cnt_h": cnt_h, "steps": steps}
    if token:
        # the tile masks alone, and how much of the tiles' query x key area
        # the tokens' own selections cover
        uidx, ucnt, ubits = bsa.token_mask(idx, cnt, w.B)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            bsa.token_mask(idx, cnt, w.B, out=(uidx, ucnt, ubits))
        e1.record()
        torch.cuda.synchronize()
        area = float(ucnt.double().sum().item()) * 64 * w.B * (w.hq // w.hkv)
        res["token"] = {"mask_ms": e0.elapsed_time(e1) / 10,
                        "mean_active_blocks_per_tile": float(ucnt.float().mean().item()),
                        "selected_fraction_of_tile_area": flops / (4.0 * w.d) / area}
        del uidx, ucnt, ubits
    if keep_inputs:
        res["x"] = x
        res["sel"] = (idx, cnt)
    else:
        del x, Q, K, V, O, S, sel, idx, cnt, ws, aws, wsel
        torch.cuda.empty_cache()
    return res


def prefill_extra(r):
    """JSON summary of a non-headline prefill workload."""
    w = synth.WORKLOADS[r["workload"]]
    ms = r["elapsed_s"] / r["steps"] * 1e3
    att = r["flops"] / r["attend_s"] / 1e12
    f32 = w.dtype == "f32"
    peak = PEAK_F32_VALU_TFLOPS if f32 else PEAK_BF16_TFLOPS
    out = {"workload": w.name, "router": w.router, "dtype": w.dtype, "batch": w.batch,
           "q_heads": w.hq, "kv_heads": w.hkv, "seq_len": w.n, "head_dim": w.d, "block": w.B,
           "ms_per_step": ms, "flops_per_step": r["flops"],
           "TFLOP_per_s_step": r["flops"] / ms / 1e9,
           "attend_TFLOP_per_s": att, "attend_ms": r["attend_ms"],
           "attend_TFLOP_per_s_median": r["flops"] / r["attend_ms"]["median"] / 1e9,
           ("attend_frac_fp32_valu_peak" if f32 else "attend_frac_mfma_peak"): att / peak,
           "stages_ms": r["stages_ms"], "sparsity_vs_causal": r["sparsity_vs_causal"],
           "mean_selected_blocks": float(r["cnt_h"].mean())}
    if w.router == "topk":
        out["top_k"] = w.k_total
    else:
        out.update(alpha=w.alpha, gamma=w.gamma, cap=w.cap, max_iter=w.max_iter)
    if "token" in r:
        out["routing"] = "per token"
        out["query_locality_amp"] = w.loc_amp
        out.update(r["token"])
    if w.router == "entmax":
        out["prior_sigma"] = w.sigma
    if r.get("traffic") is not None:
        out["attend_hbm_bytes_per_launch"] = r["traffic"]
    return out


def run_entmax_attn(bsa, torch, steps, warmup, refine=2):
    """Token-level alpha-entmax attention (one call per step) and, on the same
    inputs, the dense causal softmax through the block-sparse kernel with
    every block selected.  TFLOP/s are dense-causal equivalents (4 d flops
    per causal pair), the unit in which both are compared."""
    w = synth.WORKLOADS[ENTMAX_ATTN]
    x = device_inputs(w, torch)
    Q, K, V = x["Q"], x["K"], x["V"]
    O = torch.empty_like(Q)
    nb = w.nblk
    idx = torch.arange(nb, dtype=torch.int32, device="cuda").repeat(w.batch * w.hkv * nb, 1) \
        .reshape(w.batch, w.hkv, nb, nb)
    cnt = (torch.arange(nb, dtype=torch.int32, device="cuda") + 1).repeat(w.batch * w.hkv, 1) \
        .reshape(w.batch, w.hkv, nb)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    t_ent = timed(lambda: bsa.attend_entmax(Q, K, V, w.alpha, refine=refine, out=O))
    # one refinement step ("AdaSplash-2", 2.A: 1-2 iterations from the
    # histogram start): its time, and its distance from a converged run
    # (refine 8) of the same kernel
    t_ent1 = timed(lambda: bsa.attend_entmax(Q, K, V, w.alpha, refine=1, out=O))
    O8, tau8 = bsa.attend_entmax(Q, K, V, w.alpha, refine=8, want_tau=True)

    def distance(r):
        Or, taur = bsa.attend_entmax(Q, K, V, w.alpha, refine=r, want_tau=True)
        dt, do_ = (taur - tau8).abs(), (Or.float() - O8.float()).abs()
        return {"tau_max_abs_diff_vs_refine8": float(dt.max()),
                "tau_p99_abs_diff_vs_refine8": float(torch.quantile(dt.flatten()[::64], 0.99)),
                "out_max_abs_diff_vs_refine8": float(do_.max())}
    one_step = {"ms_per_step": t_ent1, **distance(1)}
    default_steps = distance(refine)
    del O8, tau8
    t_soft = timed(lambda: bsa.attend_prefill(Q, K, V, w.B, idx, cnt, out=O))
    dense = 4.0 * w.d * w.hq * w.batch * w.n * (w.n + 1) / 2
    _, tau, live = bsa.attend_entmax(Q, K, V, w.alpha, refine=refine, want_tau=True,
                                     want_live=True)
    nt = (w.n + 63) // 64
    lv = live.cpu().numpy().view(np.uint32)
    live_frac = float(np.unpackbits(lv.view(np.uint8)).sum()) / (w.batch * w.hkv * nt * (nt + 1) / 2)
    # the backward from the forward's tau (walking its live tiles, and every
    # causal tile), for a seeded upstream gradient
    do_st, _ = synth.gen_stored(w, "do")
    dO = torch.from_numpy(do_st.view(np.int16)).to("cuda").view(torch.bfloat16)
    shape = bsa.make_shape(batch=w.batch, hq=w.hq, hkv=w.hkv, d=w.d, B=64, dtype=bsa.BF16,
                           mode=bsa.PREFILL, q_len=w.n, kv_len=w.n, q=Q, k=K, v=V, o=dO)
    ews = torch.empty(bsa.workspace_size(bsa.OP_ATTEND_ENTMAX_BACKWARD, shape, 0),
                      dtype=torch.uint8, device="cuda")
    t_bwd = timed(lambda: bsa.attend_entmax_backward(Q, K, V, dO, tau, w.alpha, ws=ews, live=live))
    t_bwd_all = timed(lambda: bsa.attend_entmax_backward(Q, K, V, dO, tau, w.alpha, ws=ews))
    del ews
    # the dense softmax's own backward on the same inputs (every block
    # selected), for the training-step comparison ("AdaSplash-2", 4)
    Os, Ls = bsa.attend_prefill(Q, K, V, w.B, idx, cnt, want_lse=True)
    dshape = bsa.make_shape(batch=w.batch, hq=w.hq, hkv=w.hkv, d=w.d, B=w.B, dtype=bsa.BF16,
                            mode=bsa.PREFILL, q_len=w.n, kv_len=w.n, q=Q, k=K, v=V, o=Os)
    dws = torch.empty(bsa.workspace_size(bsa.OP_ATTEND_BACKWARD, dshape, nb), dtype=torch.uint8,
                      device="cuda")
    t_soft_bwd = timed(lambda: bsa.attend_backward(Q, K, V, Os, dO, Ls, w.B, idx, cnt, ws=dws))
    torch.cuda.synchronize()
    del x, Q, K, V, O, idx, cnt, tau, live, dO, Os, Ls, dws
    torch.cuda.empty_cache()
    return {"workload": w.name, "batch": w.batch, "q_heads": w.hq, "kv_heads": w.hkv,
            "seq_len": w.n, "head_dim": w.d, "alpha": w.alpha, "refine": refine,
            "query_scale": w.q_scale, "ms_per_step": t_ent,
            "dense_equiv_TFLOP_per_s": dense / t_ent / 1e9,
            "dense_softmax_ms": t_soft, "dense_softmax_TFLOP_per_s": dense / t_soft / 1e9,
            "speedup_vs_dense_softmax": t_soft / t_ent, "live_tile_fraction": live_frac,
            "backward_ms": t_bwd, "backward_dense_equiv_TFLOP_per_s": 2.5 * dense / t_bwd / 1e9,
            "backward_all_tiles_ms": t_bwd_all, "dense_softmax_backward_ms": t_soft_bwd,
            "training_pass_ms": t_ent + t_bwd, "dense_softmax_training_pass_ms": t_soft + t_soft_bwd,
            "training_pass_speedup_vs_dense_softmax": (t_soft + t_soft_bwd) / (t_ent + t_bwd),
            "refine_1": one_step, "refine_default_vs_refine8": default_steps,
            "hbm_bytes_per_launch": read_traffic(
                ENTMAX_ATTN, os.path.join(HERE, "block_sparse_attention_summarize_amd", "csrc",
                                          "entmax_attn.hip")),
            "algorithmic_bytes_per_launch": (2 * w.hq + 2 * w.hkv) * w.batch * w.n * w.d * 2}


def run_decode(bsa, torch, steps, warmup, with_paged=True, with_cpu=False):
    w = synth.WORKLOADS[DECODE]
    x = device_inputs(w, torch)
    S = bsa.summarize(x["K"], w.B)  # cached summaries, computed once
    lens = torch.tensor(w.lens(), dtype=torch.int32, device="cuda")
    idx = torch.empty((w.batch, w.hkv, 1, w.k_total), dtype=torch.int32, device="cuda")
    cnt = torch.empty((w.batch, w.hkv, 1), dtype=torch.int32, device="cuda")
    O = torch.empty_like(x["Q"])
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    ws = bsa.decode_workspace(x["Q"], x["K"], w.B, w.k_total)

    def step():
        # routing over the cached summaries + attention
        bsa.decode_step(x["Q"], x["K"], x["V"], S, w.B, w.k_total, w.force, kv_lens=lens, out=O,
                        sel=(idx, cnt), ws=ws)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(steps, 5)):
            flush.sum()  # evict the last-level cache by reading 512 MiB (untimed, no dirty lines)
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return ts

    times = timed(step)
    O_ref = O.clone()
    c = cnt.cpu().numpy()
    kv_bytes = int(c.sum()) * w.B * w.d * 2 * 2  # selected K and V blocks (all full here)
    sum_bytes = w.batch * w.hkv * (w.nblk - 1) * w.d * 4  # fp32 summaries of the candidates
    qo_bytes = 2 * w.batch * w.hq * w.d * 2
    total = kv_bytes + sum_bytes + qo_bytes
    cpu = cpu_baseline_decode(w, x, idx.cpu().numpy(), c, total) if with_cpu else None
    paged = None
    if with_paged:
        # the same cache as a shuffled pool of pages of B tokens behind page tables
        nb = w.nblk
        perm = torch.randperm(w.batch * nb, generator=torch.Generator().manual_seed(7))
        pool_of = lambda T: T.reshape(w.batch, w.hkv, nb, w.B, w.d).permute(0, 2, 1, 3, 4) \
            .reshape(w.batch * nb, w.hkv, w.B, w.d)[perm.to("cuda")].contiguous()
        Kp, Vp = pool_of(x["K"]), pool_of(x["V"])
        table = torch.empty(w.batch * nb, dtype=torch.int32)
        table[perm] = torch.arange(w.batch * nb, dtype=torch.int32)
        table = table.reshape(w.batch, nb).to("cuda")
        del x["K"], x["V"]

        def pstep():
            bsa.decode_step_paged(x["Q"], Kp, Vp, table, S, w.B, w.k_total, w.force, kv_lens=lens,
                                  kv_len=w.n, out=O, want_selection=False, ws=ws)

        ptimes = timed(pstep)
        paged = {"us_per_step_median": float(np.median(ptimes)) * 1e6,
                 "same_output_as_contiguous": bool(torch.equal(O, O_ref)),
                 "pages": int(w.batch * nb), "page_tokens": w.B}
    t = float(np.median(times))
    return {"workload": w.name, "batch": w.batch, "hq": w.hq, "hkv": w.hkv, "kv_len": w.n,
            "head_dim": w.d, "block": w.B, "top_k": w.k_total - 1, "forced": "tail",
            "us_per_step_median": t * 1e6, "us_per_step_min": float(np.min(times)) * 1e6,
            "bytes_per_step": total, "kv_bytes": kv_bytes, "summary_bytes": sum_bytes,
            "GB_per_s": total / t / 1e9, "KV_GB_per_s": kv_bytes / t / 1e9,
            "frac_hbm_peak": total / t / 1e9 / PEAK_HBM_GBS,
            "cache_flush": "512 MiB read before every timed step"} | (
        {} if paged is None else {"paged": paged | {
            "GB_per_s": total / (paged["us_per_step_median"] * 1e-6) / 1e9}}) | (
        {} if cpu is None else {"cpu_baseline": cpu})


def run_backward(bsa, torch, w, r, steps, warmup):
    """Training pass of the fine attention on the headline inputs and
    selection: the forward with its log-normaliser, then the gradients dQ, dK,
    dV for a seeded upstream gradient (bf16, same shapes as the inputs).
    TFLOP/s use the usual accounting of 2.5x the forward's flops for the
    backward (five products of the pair's size against the forward's two,
    10 d flops per attended pair); the kernels execute seven (dQ recomputes
    the scores and dP instead of atomically accumulating)."""
    x = r["x"]
    Q, K, V = x["Q"], x["K"], x["V"]
    idx, cnt = r["sel"]
    do_st, _ = synth.gen_stored(w, "do")
    dO = torch.from_numpy(do_st.view(np.int16)).to("cuda").view(torch.bfloat16)
    del do_st
    O = torch.empty_like(Q)
    L = torch.empty((w.batch, w.hq, w.n), dtype=torch.float32, device="cuda")
    shape = bsa.make_shape(batch=w.batch, hq=w.hq, hkv=w.hkv, d=w.d, B=w.B, dtype=bsa.BF16,
                           mode=bsa.PREFILL, q_len=w.n, kv_len=w.n, q=Q, k=K, v=V, o=O)
    ws = torch.empty(bsa.workspace_size(bsa.OP_ATTEND_BACKWARD, shape, idx.shape[-1]),
                     dtype=torch.uint8, device="cuda")

    def fwd():
        O_, L_ = bsa.attend_prefill(Q, K, V, w.B, idx, cnt, out=O, want_lse=True)
        L.copy_(L_)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    t_plain = timed(lambda: bsa.attend_prefill(Q, K, V, w.B, idx, cnt, out=O))
    fwd()
    t_bwd = timed(lambda: bsa.attend_backward(Q, K, V, O, dO, L, w.B, idx, cnt, ws=ws))
    fwd_flops = r["flops"]
    bwd_flops = 2.5 * fwd_flops
    out = {"workload": w.name, "forward_ms": t_plain, "backward_ms": t_bwd,
           "train_step_ms": t_plain + t_bwd,
           "backward_TFLOP_per_s": bwd_flops / t_bwd / 1e9,
           "backward_frac_mfma_peak": bwd_flops / t_bwd / 1e9 / PEAK_BF16_TFLOPS,
           "backward_executed_TFLOP_per_s": 3.5 * fwd_flops / t_bwd / 1e9,
           "workspace_MiB": ws.numel() / 2**20,
           "accounting": "backward flops = 2.5 x forward (10 d per attended pair)"}
    del dO, O, L, ws
    torch.cuda.empty_cache()
    return out


def run_train_entmax(bsa, torch, steps, warmup, name=ENTMAX, sigma=1.0):
    """One training pass of entmax-routed prefill with the prior (the
    N = 65536 entmax workload, or the per-token one, with sigma = 1): forward
    = summaries, entmax routing (probabilities and weights kept), biased
    attention with its log-normaliser; backward = attention gradients with
    dL/dw, then the routing gradient added to dQ and dK.  Timed as two
    event-bracketed phases per step."""
    w = synth.WORKLOADS[name]
    token = w.mode == "token"
    nrow = w.n if token else w.nblk
    x = device_inputs(w, torch)
    Q, K, V = x["Q"], x["K"], x["V"]
    del x
    do_st, _ = synth.gen_stored(w, "do")
    dO = torch.from_numpy(do_st.view(np.int16)).to("cuda").view(torch.bfloat16)
    del do_st
    width = w.idx_width
    S = torch.empty((w.batch, w.hkv, w.nblk, w.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.batch, w.hkv, nrow, width), dtype=torch.int32, device="cuda")
    cnt = torch.empty((w.batch, w.hkv, nrow), dtype=torch.int32, device="cuda")
    wsel = torch.empty(idx.shape, dtype=torch.float32, device="cuda")
    O = torch.empty_like(Q)
    shape_r = bsa._route_shape(Q, S, w.B, False, None, token)
    rws = torch.empty(bsa.workspace_size(bsa.OP_ROUTE_ENTMAX, shape_r, w.cap), dtype=torch.uint8,
                      device="cuda")
    shape = bsa.make_shape(batch=w.batch, hq=w.hq, hkv=w.hkv, d=w.d, B=w.B, dtype=bsa.BF16,
                           mode=bsa.TOKEN if token else bsa.PREFILL, q_len=w.n, kv_len=w.n, q=Q,
                           k=K, v=V, o=O)
    aws = torch.empty(max(bsa.workspace_size(bsa.OP_ATTEND_PREFILL_PRIOR, shape, width), 1),
                      dtype=torch.uint8, device="cuda")
    bws = torch.empty(bsa.workspace_size(bsa.OP_ATTEND_BACKWARD_PRIOR, shape, width),
                      dtype=torch.uint8, device="cuda")
    gws = torch.empty(bsa.workspace_size(bsa.OP_ROUTE_ENTMAX_BACKWARD, shape, 0),
                      dtype=torch.uint8, device="cuda")
    st = {}

    def forward():
        bsa.summarize(K, w.B, out=S)
        _, _, st["probs"], _ = bsa.route_entmax(Q, S, w.B, w.alpha, w.gamma, w.cap, w.force,
                                                n_bins=w.n_bins, max_iter=w.max_iter, ws=rws,
                                                out=(idx, cnt), wsel=wsel, want_probs=True,
                                                token=token)
        _, st["L"] = bsa.attend_prefill(Q, K, V, w.B, idx, cnt, out=O, wsel=wsel, sigma=sigma,
                                        want_lse=True, token=token, ws=aws)

    def backward():
        dQ, dK, dV, dw = bsa.attend_backward(Q, K, V, O, dO, st["L"], w.B, idx, cnt, ws=bws,
                                             wsel=wsel, sigma=sigma, want_dwsel=True,
                                             grad_dtype=torch.float32, token=token)
        bsa.route_entmax_backward(Q, S, st["probs"], idx, cnt, dw, w.B, w.alpha, w.gamma, dQ, dK,
                                  ws=gws, token=token)

    for _ in range(warmup):
        forward()
        backward()
    torch.cuda.synchronize()
    ev = []
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        forward()
        e[1].record()
        backward()
        e[2].record()
        ev.append(e)
    torch.cuda.synchronize()
    fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    flops = 4.0 * w.d * (token_pairs(w, idx_h, cnt_h) if token else prefill_pairs(w, idx_h, cnt_h))
    del Q, K, V, dO, S, idx, cnt, wsel, O, rws, aws, bws, gws, st
    torch.cuda.empty_cache()
    return {"workload": w.name, "prior_sigma": sigma, "forward_ms": fwd, "backward_ms": bwd,
            "train_step_ms": fwd + bwd, "attention_flops": flops,
            "backward_attention_TFLOP_per_s": 2.5 * flops / bwd / 1e9,
            "note": "backward = attention gradients with dL/dw + routing gradient into dQ, dK; "
                    "fp32 gradients"}


def main():
    a = parse()
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
        return
    if a.entmax_attn_only:
        entmax_attn_only(a.steps, a.warmup)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the hot path runs on a single MI355X with no collectives)", file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_attention_summarize_amd as bsa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    w = synth.WORKLOADS[a.workload]
    assert w.mode == "prefill" and w.dtype == "bf16"
    if a.only:
        a.no_cpu = a.no_decode = a.no_backward = a.no_train = a.no_entmax = True
        a.no_gqa = a.no_fp32 = a.no_token = a.no_entmax_attn = True
    kernel_src = os.path.join(HERE, "block_sparse_attention_summarize_amd", "csrc", "attend.hip")

    def done(name):  # progress on stderr; the result line stays alone on stdout
        print(f"[bench] {name} done", file=sys.stderr, flush=True)

    r = run_prefill(bsa, torch, w, a.steps, a.warmup)
    done(w.name)
    flops, elapsed = r["flops"], r["elapsed_s"]
    ms = elapsed / a.steps * 1e3
    value = flops * a.steps / elapsed / 1e12
    att_s = r["attend_s"]
    achieved = flops / att_s / 1e12
    out = {
        "metric": "block-sparse attn prefill TFLOP/s (% MFMA peak); decode KV GB/s (% HBM)",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) with planted blocks)",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.hq, "kv_heads": w.hkv,
                   "seq_len": w.n, "head_dim": w.d, "block": w.B, "top_k": w.k_total,
                   "forced": {0: "none", 1: "diagonal", 3: "diagonal + block 0"}.get(w.force),
                   "flops_per_step": flops, "sparsity_vs_causal": r["sparsity_vs_causal"],
                   "inputs_sha256": r["x"]["sha256"]},
        "frac_mfma_peak_step": value / PEAK_BF16_TFLOPS,
        "stages_ms": r["stages_ms"],
        # the library serves plain block rows of 32 or more 64-key tiles with its
        # ping-pong kernel, shorter rows with the 4-wavefront one
        "roofline": {"kernel": "attend_prefill_pp" if w.idx_width * (w.B // 64) >= 32
                     else "attend_prefill_bf16", "bound": "mfma", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": read_traffic(w.name, kernel_src), "avg_launch_ms": att_s * 1e3,
                     "launch_ms": r["attend_ms"],
                     "frac_at_median_launch": flops / r["attend_ms"]["median"] / 1e9
                     / PEAK_BF16_TFLOPS,
                     "algorithmic_flops_per_launch": flops},
    }
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, r["x"], r["idx_h"], r["cnt_h"], flops,
                                           a.cpu_sample_blocks)
        done("cpu_baseline")
    del r
    torch.cuda.empty_cache()
    extra = {}
    cpu_extra = {}
    if not a.no_gqa:
        w2 = synth.WORKLOADS[GQA32K]
        r2 = run_prefill(bsa, torch, w2, a.steps, a.warmup)
        r2["traffic"] = read_traffic(GQA32K, kernel_src)
        extra[GQA32K] = prefill_extra(r2)
        done(GQA32K)
        if not a.no_cpu:
            cpu_extra[GQA32K] = cpu_baseline(w2, r2["x"], r2["idx_h"], r2["cnt_h"], r2["flops"], 8)
            done(f"{GQA32K} cpu")
        if not a.no_backward:
            extra["backward"] = run_backward(bsa, torch, w2, r2, a.steps, a.warmup)
            done("backward")
        del r2
        torch.cuda.empty_cache()
    if not a.no_fp32:
        w1 = synth.WORKLOADS[FP32]
        r1 = run_prefill(bsa, torch, w1, a.steps, a.warmup)
        extra[FP32] = prefill_extra(r1)
        done(FP32)
        if not a.no_cpu:
            cpu_extra[FP32] = cpu_baseline(w1, r1["x"], r1["idx_h"], r1["cnt_h"], r1["flops"],
                                           w1.nblk)
        del r1
    if not a.no_backward and not a.no_train:
        extra["train_entmax_prior"] = run_train_entmax(bsa, torch, a.steps, a.warmup)
        done("train_entmax_prior")
        if not a.no_token:
            extra["train_token_prior"] = run_train_entmax(bsa, torch, a.steps, a.warmup,
                                                          name=TOKEN)
            done("train_token_prior")
    if not a.no_decode:
        extra["decode"] = run_decode(bsa, torch, a.steps, a.warmup, with_cpu=not a.no_cpu)
        done("decode")
    if not a.no_entmax:
        w4 = synth.WORKLOADS[ENTMAX]
        r4 = run_prefill(bsa, torch, w4, a.steps, a.warmup, keep_inputs=not a.no_cpu)
        extra[ENTMAX] = prefill_extra(r4)
        done(ENTMAX)
        if not a.no_cpu:
            cpu_extra[ENTMAX] = cpu_baseline(w4, r4["x"], r4["idx_h"], r4["cnt_h"], r4["flops"], 4)
            done(f"{ENTMAX} cpu")
        del r4
        torch.cuda.empty_cache()
    if not a.no_token:
        extra[TOKEN] = prefill_extra(run_prefill(bsa, torch, synth.WORKLOADS[TOKEN], a.steps,
                                                 a.warmup, keep_inputs=False))
        done(TOKEN)
    if not a.no_entmax_attn:
        extra[ENTMAX_ATTN] = run_entmax_attn(bsa, torch, a.steps, a.warmup)
        done(ENTMAX_ATTN)
    if cpu_extra:
        extra["cpu_baselines"] = cpu_extra
    if extra:
        out["extra"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
