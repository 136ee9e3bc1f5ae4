"""GPU parity of every stage against the fp64 oracle on seeded inputs small
enough for the oracle to check every row, spanning several tiles and a ragged
tail, plus edge cases.  Calls go through the C ABI (ctypes binding)."""
import math

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
SMALL = {
    # the fp32 workload is small enough to check in full
    "fp32_n1k": W["fp32_prefill_n1k"],
    "fp32_d128_ragged": W["fp32_prefill_n1k"].scaled(d=128, n=64 * 9 + 17, hq=4, hkv=2, k_total=3,
                                                    force=synth.FORCE_DIAG | synth.FORCE_FIRST),
    "bf16_gqa": W["bf16_gqa_prefill_n32k"].scaled(hq=8, hkv=2, n=64 * 21 + 37, k_total=6,
                                                  planted_blocks=5),
    "bf16_gqa_d64_diag": W["bf16_gqa_prefill_n32k"].scaled(d=64, hq=4, hkv=1, n=64 * 17, k_total=4,
                                                           force=synth.FORCE_DIAG, planted_blocks=3),
    "bf16_mha": W["bf16_gqa_prefill_n32k"].scaled(hq=3, hkv=3, n=64 * 7 + 1, k_total=3,
                                                  planted_blocks=2),
    "long_b128": W["bf16_long_prefill_n256k"].scaled(hq=8, hkv=1, n=128 * 14 + 50, k_total=5,
                                                     planted_blocks=4),
    "long_b128_g2": W["bf16_long_prefill_n256k"].scaled(hq=4, hkv=2, n=128 * 9 + 127, k_total=4,
                                                        planted_blocks=3),
    # two sequences (bf16 and fp32)
    "bf16_batch2": W["bf16_gqa_prefill_n32k"].scaled(batch=2, hq=4, hkv=2, n=64 * 8 + 21,
                                                     k_total=3, planted_blocks=2),
    "fp32_batch2": W["fp32_prefill_n1k"].scaled(batch=2, n=64 * 5 + 7, hq=2, hkv=1, k_total=3),
    # lists of 32 or more key tiles: the ping-pong prefill kernel
    "wide_gqa": W["bf16_gqa_prefill_n32k"].scaled(hq=8, hkv=2, n=64 * 45 + 13, k_total=34,
                                                  planted_blocks=5),
    "wide_b128_g8": W["bf16_long_prefill_n256k"].scaled(hq=8, hkv=1, n=128 * 24 + 77, k_total=16,
                                                        planted_blocks=4),
    "wide_d64_batch2": W["bf16_gqa_prefill_n32k"].scaled(batch=2, d=64, hq=4, hkv=2,
                                                         n=64 * 40 + 5, k_total=33,
                                                         force=synth.FORCE_DIAG,
                                                         planted_blocks=3),
    "wide_g3_dense": W["bf16_gqa_prefill_n32k"].scaled(hq=3, hkv=1, n=64 * 36, k_total=36,
                                                       planted_blocks=2),
}
DECODE = {
    "decode": W["bf16_decode_l128k"].scaled(batch=4, hq=8, hkv=2, n=64 * 40, k_total=9,
                                            kv_lens=(2560, 1537, 64, 1)),
    "decode_b128_g8": W["bf16_decode_l128k"].scaled(batch=2, hq=8, hkv=1, n=128 * 30 + 3, B=128,
                                                    k_total=6, kv_lens=(3843, 700),
                                                    force=synth.FORCE_TAIL | synth.FORCE_FIRST),
    "decode_f32_d64": W["bf16_decode_l128k"].scaled(dtype="f32", d=64, batch=2, hq=4, hkv=4,
                                                    n=64 * 12, k_total=4, kv_lens=(768, 300)),
}
ENTMAX = {
    "entmax_g1": W["entmax_prefill_n64k"].scaled(hq=8, hkv=2, n=64 * 30 + 5, cap=64, gamma=1.0),
    "entmax_g8_cap8": W["entmax_prefill_n64k"].scaled(hq=8, hkv=2, n=64 * 30 + 5, cap=8, gamma=8.0),
    "entmax_g64": W["entmax_prefill_n64k"].scaled(hq=4, hkv=1, n=64 * 40, cap=16, gamma=64.0),
    "entmax_a2": W["entmax_prefill_n64k"].scaled(hq=4, hkv=2, n=64 * 25, cap=6, gamma=16.0,
                                                 alpha=2.0),
    "entmax_a175_iter0": W["entmax_prefill_n64k"].scaled(hq=4, hkv=2, n=64 * 25, cap=10, gamma=32.0,
                                                         alpha=1.75, max_iter=0),
    # 16 heads x 1030 blocks of logits exceed 64 KiB: the passes run on the
    # workspace rows instead of LDS
    "entmax_g16_global": W["entmax_prefill_n64k"].scaled(hq=16, hkv=1, n=64 * 1030, cap=16,
                                                         gamma=64.0, planted_blocks=8),
}


def _cpu(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _kv_lens_dev(w):
    return torch.tensor(w.lens(), dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("name", list(SMALL) + list(DECODE))
def test_summarize(name):
    w = {**SMALL, **DECODE}[name]
    print(f"[summarize] {name} {w}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    ref = oracle.summarize(x["k"], w.B)
    np.testing.assert_allclose(_cpu(S), ref, rtol=0, atol=2e-6)
    qbar = np.random.default_rng(5).standard_normal((w.hkv, w.d)).astype(np.float32)
    S2 = bsa.summarize(x["K"], w.B, qbar=torch.from_numpy(qbar).cuda())
    ref2 = oracle.summarize(x["k"], w.B, qbar=qbar)
    np.testing.assert_allclose(_cpu(S2), ref2, rtol=0, atol=2e-5)


def test_summarize_blocks_incremental():
    """Per-sequence block update of a decode cache: each named block equals the
    full summary bit for bit (same kernel arithmetic) and the oracle; entries
    outside [0, n_blk) leave their sequence untouched."""
    w = DECODE["decode"]  # lengths 2560, 1537, 64, 1
    x = parity.make(w)
    full = bsa.summarize(x["K"], w.B)
    qbar = torch.from_numpy(np.random.default_rng(6).standard_normal((w.hkv, w.d)).astype(np.float32)).cuda()
    full_q = bsa.summarize(x["K"], w.B, qbar=qbar)
    # the block each token append just completed (L % B == 0), and arbitrary ones
    for blk_list in ([int(L) // w.B - 1 if L % w.B == 0 else -1 for L in w.lens()], [39, 5, 0, 40]):
        blk = torch.tensor(blk_list, dtype=torch.int32, device="cuda")
        for ref_full, q in ((full, None), (full_q, qbar)):
            S = ref_full.clone()
            for b, j in enumerate(blk_list):
                if 0 <= j < w.nblk:
                    S[b, :, j, :] = float("nan")
            before = S.clone()
            bsa.summarize_blocks(x["K"], w.B, blk, S, qbar=q)
            torch.cuda.synchronize()
            assert torch.equal(S, ref_full), blk_list
            for b, j in enumerate(blk_list):
                if not (0 <= j < w.nblk):
                    assert torch.equal(S[b].isnan(), before[b].isnan())
    ref = oracle.summarize(x["k"], w.B)
    np.testing.assert_allclose(_cpu(full), ref, rtol=0, atol=2e-6)


def _route_ref(w, x):
    S = oracle.summarize(x["k"], w.B)
    if w.mode == "decode":
        qh = x["q"].astype(np.float64)
        return oracle.route_topk(qh, S, w.B, w.k_total, w.force, mode=oracle.MODE_DECODE,
                                 kv_lens=w.lens())
    return oracle.route_topk(oracle.qpool(x["q"], w.B), S, w.B, w.k_total, w.force)


def _route_gpu(w, x):
    S = bsa.summarize(x["K"], w.B)
    if w.mode == "decode":
        return bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force, decode=True, kv_len=w.n,
                              kv_lens=_kv_lens_dev(w), want_scores=True)
    return bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force, want_scores=True)


@pytest.mark.parametrize("name", list(SMALL) + list(DECODE))
def test_route_topk(name):
    w = {**SMALL, **DECODE}[name]
    print(f"[route_topk] {name}", flush=True)
    x = parity.make(w)
    idx, cnt, sc = _route_gpu(w, x)
    ref = _route_ref(w, x)
    gs = _cpu(sc)
    fin = np.isfinite(ref["scores"])
    assert np.array_equal(fin, np.isfinite(gs))
    np.testing.assert_allclose(gs[fin], ref["scores"][fin], rtol=0, atol=1e-5)
    rep = {}
    parity.check_topk_rows(w, _cpu(idx), _cpu(cnt), ref, rep)
    print(rep)


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("out_f32", [False, True])
def test_attend_prefill(name, out_f32):
    w = SMALL[name]
    print(f"[attend_prefill] {name} out_f32={out_f32}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt = bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force)
    O = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt,
                           out_dtype=torch.float32 if out_f32 else None)
    ref, pairs = oracle.attend(x["q"], x["k"], x["v"], w.B, _cpu(idx), _cpu(cnt))
    worst = parity.check_attention(w, _cpu(O).reshape(ref.shape), ref, out_f32 or w.dtype == "f32")
    print(f"max abs err {worst:.3e}, pairs {int(pairs.sum())}")


@pytest.mark.parametrize("name", list(DECODE))
@pytest.mark.parametrize("out_f32", [False, True])
def test_attend_decode(name, out_f32):
    w = DECODE[name]
    print(f"[attend_decode] {name} out_f32={out_f32}", flush=True)
    x = parity.make(w)
    idx, cnt, _ = _route_gpu(w, x)
    O = bsa.attend_decode(x["Q"], x["K"], x["V"], w.B, idx, cnt, kv_lens=_kv_lens_dev(w),
                          out_dtype=torch.float32 if out_f32 else None)
    ref, _ = oracle.attend(x["q"], x["k"], x["v"], w.B, _cpu(idx), _cpu(cnt),
                           mode=oracle.MODE_DECODE, kv_lens=w.lens())
    worst = parity.check_attention(w, _cpu(O).reshape(ref.shape), ref, out_f32 or w.dtype == "f32")
    print(f"max abs err {worst:.3e}")


@pytest.mark.parametrize("name", list(ENTMAX))
def test_route_entmax(name):
    w = ENTMAX[name]
    print(f"[route_entmax] {name}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    wsel = torch.empty((w.batch, w.hkv, w.nblk, w.idx_width), dtype=torch.float32, device="cuda")
    idx, cnt, probs, tau = bsa.route_entmax(x["Q"], S, w.B, w.alpha, w.gamma, w.cap, w.force,
                                            max_iter=w.max_iter, want_probs=True, want_tau=True,
                                            wsel=wsel)
    qh, Sref = oracle.qpool(x["q"], w.B), oracle.summarize(x["k"], w.B)
    ref = oracle.route_entmax(qh, Sref, w.B, w.alpha, w.gamma, w.cap, w.force,
                              max_iter=w.max_iter)
    ref_x = oracle.route_entmax(qh, Sref, w.B, w.alpha, w.gamma, w.cap, w.force,
                                max_iter=parity.EXACT_ITERS)
    own = np.arange(w.nblk)
    lg = parity.entmax_logits(w, qh, Sref, own)
    # exact on rows decided with margin; threshold, weights, support, count
    # and cap order valid on every row
    rep = {}
    parity.check_entmax_rows(w, _cpu(idx), _cpu(cnt), _cpu(probs), _cpu(tau), ref, ref_x, lg,
                             own, rep, gw=_cpu(wsel))
    print(rep)


@pytest.mark.parametrize("sigma", [0.5, 1.0])
@pytest.mark.parametrize("out_f32", [False, True])
def test_prior_induced_attention(sigma, out_f32):
    """Entmax routing weights as the prior of the fine softmax: the scores of
    each listed block's keys gain sigma * ln w."""
    w = ENTMAX["entmax_g8_cap8"]
    print(f"[prior attention] sigma={sigma} out_f32={out_f32}", flush=True)
    x = parity.make(w)
    O, idx, cnt = bsa.prefill_entmax(x["Q"], x["K"], x["V"], w.B, w.alpha, w.gamma, w.cap,
                                     out_dtype=torch.float32 if out_f32 else None, sigma=sigma)
    # the same selection's weights, as the pipeline computed them
    S = bsa.summarize(x["K"], w.B)
    wsel = torch.empty(idx.shape, dtype=torch.float32, device="cuda")
    bsa.route_entmax(x["Q"], S, w.B, w.alpha, w.gamma, w.cap, w.force, wsel=wsel)
    ref, _ = oracle.attend(x["q"], x["k"], x["v"], w.B, _cpu(idx), _cpu(cnt), wsel=_cpu(wsel),
                           sigma=sigma)
    plain, _ = oracle.attend(x["q"], x["k"], x["v"], w.B, _cpu(idx), _cpu(cnt))
    worst = parity.check_attention(w, _cpu(O).reshape(ref.shape), ref, out_f32)
    print(f"max abs err {worst:.3e}; the prior moves the output by {np.abs(ref - plain).max():.3e}")


def test_prior_weights_zero_and_forced():
    """Hand-set weights: zero drops a block, 1 leaves it unbiased."""
    w = SMALL["bf16_gqa"]
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt = bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force)
    rng = np.random.default_rng(5)
    wh = rng.uniform(0.01, 1.0, idx.shape).astype(np.float32)
    wh[rng.random(idx.shape) < 0.2] = 0.0
    wsel = torch.from_numpy(wh).cuda()
    O = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, out_dtype=torch.float32,
                           wsel=wsel, sigma=0.8)
    ref, pairs = oracle.attend(x["q"], x["k"], x["v"], w.B, _cpu(idx), _cpu(cnt), wsel=wh,
                               sigma=0.8)
    Oh = _cpu(O).reshape(ref.shape)
    parity.check_attention(w, Oh, ref, True)
    assert np.all(Oh[pairs == 0] == 0)
    # fp32 inputs: the VALU kernel
    wf = SMALL["fp32_d128_ragged"]
    xf = parity.make(wf)
    Sf = bsa.summarize(xf["K"], wf.B)
    idx, cnt = bsa.route_topk(xf["Q"], Sf, wf.B, wf.k_total, wf.force)
    wh = rng.uniform(0.01, 1.0, idx.shape).astype(np.float32)
    wh[rng.random(idx.shape) < 0.2] = 0.0
    O = bsa.attend_prefill(xf["Q"], xf["K"], xf["V"], wf.B, idx, cnt,
                           wsel=torch.from_numpy(wh).cuda(), sigma=1.3)
    ref, _ = oracle.attend(xf["q"], xf["k"], xf["v"], wf.B, _cpu(idx), _cpu(cnt), wsel=wh,
                           sigma=1.3)
    parity.check_attention(wf, _cpu(O).reshape(ref.shape), ref, True)


def test_prefill_entmax_pipeline_attention():
    w = ENTMAX["entmax_g8_cap8"]
    x = parity.make(w)
    O, idx, cnt = bsa.prefill_entmax(x["Q"], x["K"], x["V"], w.B, w.alpha, w.gamma, w.cap,
                                     out_dtype=torch.float32)
    ref, _ = oracle.attend(x["q"], x["k"], x["v"], w.B, _cpu(idx), _cpu(cnt))
    parity.check_attention(w, _cpu(O).reshape(ref.shape), ref, True)


def test_all_blocks_equals_dense_attention():
    w = SMALL["bf16_gqa"]
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt = bsa.route_topk(x["Q"], S, w.B, w.nblk, 0)
    O = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, out_dtype=torch.float32)
    G = w.hq // w.hkv
    q, k, v = (torch.from_numpy(a).double() for a in (x["q"], x["k"], x["v"]))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(G, 1), v.repeat_interleave(G, 1), is_causal=True).numpy()
    assert np.abs(_cpu(O) - ref).max() <= parity.TOL_BF16


def test_zero_query_reveals_token_set():
    """q = 0: every weight is exactly 1 before normalisation, so o is the mean
    of V over the attended tokens; one-hot values expose that set exactly."""
    w = SMALL["bf16_gqa"].scaled(d=128, n=64 * 3 + 20, hq=4, hkv=1)
    n = w.n
    Q = torch.zeros((1, 4, n, 128), dtype=torch.bfloat16, device="cuda")
    K = torch.randn((1, 1, n, 128), device="cuda").to(torch.bfloat16)
    Vh = np.zeros((1, 1, n, 128), np.float32)
    Vh[0, 0, np.arange(n), np.arange(n) % 128] = 1.0
    V = torch.from_numpy(Vh).to("cuda").to(torch.bfloat16)
    idx = torch.tensor([[[[0, -1], [0, 1], [0, 2], [1, 3]]]], dtype=torch.int32, device="cuda")
    cnt = torch.tensor([[[1, 2, 2, 2]]], dtype=torch.int32, device="cuda")
    O = bsa.attend_prefill(Q, K, V, 64, idx, cnt, out_dtype=torch.float32)
    ref, _ = oracle.attend(np.zeros((1, 4, n, 128), np.float32), _cpu(K), Vh, 64, _cpu(idx), _cpu(cnt))
    np.testing.assert_allclose(_cpu(O).reshape(ref.shape), ref, rtol=0, atol=1e-6)


def test_edge_cases_empty_and_invalid_ids():
    w = SMALL["bf16_gqa"]
    x = parity.make(w)
    nrow = w.nblk
    idx = torch.full((1, w.hkv, nrow, 3), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((1, w.hkv, nrow), dtype=torch.int32, device="cuda")
    O = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, out_dtype=torch.float32)
    assert torch.all(O == 0)
    # invalid ids in the list are skipped; counts above the width are clamped
    idx[:, :, :, 0] = 0
    idx[:, :, :, 1] = 10 ** 6
    cnt.fill_(7)
    O = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, idx, cnt, out_dtype=torch.float32)
    only0 = torch.full((1, w.hkv, nrow, 1), 0, dtype=torch.int32, device="cuda")
    O0 = bsa.attend_prefill(x["Q"], x["K"], x["V"], w.B, only0,
                            torch.ones((1, w.hkv, nrow), dtype=torch.int32, device="cuda"),
                            out_dtype=torch.float32)
    assert torch.equal(O, O0)


@pytest.mark.parametrize("n", [1, 5, 64, 65])
def test_tiny_sequences(n):
    w = SMALL["bf16_gqa"].scaled(n=n, hq=4, hkv=2, k_total=2, planted_blocks=0)
    x = parity.make(w)
    O, idx, cnt = bsa.prefill_topk(x["Q"], x["K"], x["V"], w.B, w.k_total, out_dtype=torch.float32)
    ref, _ = oracle.attend(x["q"], x["k"], x["v"], w.B, _cpu(idx), _cpu(cnt))
    parity.check_attention(w, _cpu(O).reshape(ref.shape), ref, True)
    r = _route_ref(w, x)
    assert np.array_equal(_cpu(idx), r["idx"]) and np.array_equal(_cpu(cnt), r["cnt"])


def test_determinism_and_strides():
    w = SMALL["bf16_gqa"]
    x = parity.make(w)
    O1, i1, c1 = bsa.prefill_topk(x["Q"], x["K"], x["V"], w.B, w.k_total)
    O2, i2, c2 = bsa.prefill_topk(x["Q"], x["K"], x["V"], w.B, w.k_total)
    assert torch.equal(i1, i2) and torch.equal(c1, c2) and torch.equal(O1, O2)
    # token-major storage [b, N, h, d] viewed as [b, h, N, d]
    Qt = x["Q"].transpose(1, 2).contiguous().transpose(1, 2)
    Kt = x["K"].transpose(1, 2).contiguous().transpose(1, 2)
    Vt = x["V"].transpose(1, 2).contiguous().transpose(1, 2)
    O3, i3, c3 = bsa.prefill_topk(Qt, Kt, Vt, w.B, w.k_total)
    assert torch.equal(i1, i3) and torch.equal(O1, O3)


DECODE_WIDE = {
    # 16 query heads per KV head: the single-kernel decode path (heads split)
    "decode_g16": W["bf16_decode_l128k"].scaled(batch=2, hq=16, hkv=1, n=64 * 33 + 5, k_total=7,
                                                kv_lens=(64 * 33 + 5, 999)),
    # more routed blocks than the partitioned path keeps
    "decode_k300": W["bf16_decode_l128k"].scaled(batch=1, hq=4, hkv=1, n=64 * 400, k_total=301,
                                                 kv_lens=(64 * 400,)),
    # more 256-candidate slices than wavefronts (12: four wavefronts take two
    # each, the ragged row 6), and a top-100 whose slice survivors need two
    # more tournament rounds (11 x 100 -> 5 x 100 -> 2 x 100 -> 100)
    "decode_slices": W["bf16_decode_l128k"].scaled(batch=2, hq=4, hkv=1, n=64 * 3000 + 17,
                                                   k_total=33, kv_lens=(64 * 3000 + 17, 64 * 1300 + 5)),
    "decode_slices_k101": W["bf16_decode_l128k"].scaled(batch=1, hq=8, hkv=2, n=64 * 2600,
                                                        k_total=101, kv_lens=(64 * 2600,)),
}


@pytest.mark.parametrize("name", list(DECODE) + list(DECODE_WIDE))
@pytest.mark.parametrize("partitioned", [True, False])
def test_route_topk_decode_kernels(name, partitioned):
    """Decode routing without scores_out: partitioned kernels (with workspace)
    or the single-workgroup-per-row kernel (without)."""
    w = {**DECODE, **DECODE_WIDE}[name]
    print(f"[route_topk decode] {name} partitioned={partitioned}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    idx, cnt = bsa.route_topk(x["Q"], S, w.B, w.k_total, w.force, decode=True, kv_len=w.n,
                              kv_lens=_kv_lens_dev(w), partitioned=partitioned)
    parity.check_topk_rows(w, _cpu(idx), _cpu(cnt), _route_ref(w, x))


@pytest.mark.parametrize("name", list(DECODE) + list(DECODE_WIDE))
@pytest.mark.parametrize("out_f32", [False, True])
def test_decode_step(name, out_f32):
    w = {**DECODE, **DECODE_WIDE}[name]
    print(f"[decode_step] {name} out_f32={out_f32}", flush=True)
    x = parity.make(w)
    S = bsa.summarize(x["K"], w.B)
    O, idx, cnt = bsa.decode_step(x["Q"], x["K"], x["V"], S, w.B, w.k_total, w.force,
                                  kv_lens=_kv_lens_dev(w),
                                  out_dtype=torch.float32 if out_f32 else None)
    parity.check_topk_rows(w, _cpu(idx), _cpu(cnt), _route_ref(w, x))
    ref, _ = oracle.attend(x["q"], x["k"], x["v"], w.B, _cpu(idx), _cpu(cnt),
                           mode=oracle.MODE_DECODE, kv_lens=w.lens())
    parity.check_attention(w, _cpu(O).reshape(ref.shape), ref, out_f32 or w.dtype == "f32")
    # without selection outputs, and on a reused (dirty) workspace, the result is identical
    ws = torch.full((1 << 22,), 255, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        O2, _, _ = bsa.decode_step(x["Q"], x["K"], x["V"], S, w.B, w.k_total, w.force,
                                   kv_lens=_kv_lens_dev(w), want_selection=False, ws=ws,
                                   out_dtype=torch.float32 if out_f32 else None)
        assert torch.equal(O, O2)
