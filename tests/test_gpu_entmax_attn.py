"""GPU parity of token-level alpha-entmax attention ("AdaSplash-2") against
the fp64 oracle on seeded inputs: every row of small shapes spanning several
64-query tiles and a ragged tail, sampled rows at a longer length.  Calls go
through the C ABI (ctypes binding)."""
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

BASE = synth.WORKLOADS["entmax_attn_prefill_n16k"]
CASES = {
    "a15_gqa": BASE.scaled(hq=8, hkv=2, n=64 * 5 + 17, planted_blocks=2),
    "a15_dense_scores": BASE.scaled(hq=4, hkv=1, n=64 * 4 + 3, q_scale=1.0, planted_blocks=2),
    "a2_sparsemax": BASE.scaled(hq=4, hkv=2, n=64 * 3 + 40, alpha=2.0, planted_blocks=2),
    "a125": BASE.scaled(hq=4, hkv=4, n=64 * 3 + 1, alpha=1.25, q_scale=2.0, planted_blocks=1),
    "a175_newton": BASE.scaled(hq=4, hkv=2, n=64 * 3 + 9, alpha=1.75, q_scale=3.0, planted_blocks=1),
    "a15_d64": BASE.scaled(hq=6, hkv=3, d=64, n=64 * 6, planted_blocks=2),
    "a15_batch2": BASE.scaled(batch=2, hq=4, hkv=2, n=64 * 3 + 21, planted_blocks=1),
    # a group of 8 heads: two workgroups per query tile share the live rows
    "a15_g8": BASE.scaled(hq=16, hkv=2, n=64 * 4 + 50, planted_blocks=2),
}


def _cpu(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("out_f32", [False, True])
def test_entmax_attention_matches_oracle(name, out_f32):
    w = CASES[name]
    print(f"[entmax attention] {name} out_f32={out_f32}", flush=True)
    x = parity.make(w)
    O, tau = bsa.attend_entmax(x["Q"], x["K"], x["V"], w.alpha, refine=2,
                               out_dtype=torch.float32 if out_f32 else None, want_tau=True)
    ref, rtau, sup = oracle.entmax_attend(x["q"], x["k"], x["v"], w.alpha)
    worst = parity.check_attention(w, _cpu(O).reshape(ref.shape), ref, out_f32)
    terr = np.abs(_cpu(tau).ravel() - rtau)
    # Halley / Newton from the histogram bracket: converged after two steps
    assert terr.max() < 1e-3, terr.max()
    print(f"max abs err {worst:.3e}, tau err max {terr.max():.2e} median {np.median(terr):.2e}, "
          f"mean support {sup.mean():.1f} of {(w.n + 1) / 2:.0f} keys")


SECANT = {
    "a25_secant": (BASE.scaled(hq=4, hkv=2, n=64 * 4 + 9, alpha=2.5, q_scale=2.0,
                               planted_blocks=2), 10),
    "a3_secant": (BASE.scaled(hq=4, hkv=2, n=64 * 4 + 33, alpha=3.0, q_scale=2.0,
                              planted_blocks=2), 14),
    "a3_sharp": (BASE.scaled(hq=4, hkv=1, n=64 * 3 + 5, alpha=3.0, q_scale=6.0,
                             planted_blocks=1), 14),
    "a25_d64_batch2": (BASE.scaled(batch=2, hq=4, hkv=2, d=64, n=64 * 3 + 1, alpha=2.5,
                                   planted_blocks=1), 10),
}


@pytest.mark.parametrize("name", list(SECANT))
@pytest.mark.parametrize("out_f32", [False, True])
def test_entmax_attention_secant_above_alpha_2(name, out_f32):
    """alpha > 2 ("AdaSplash-2", 2.B: secant with a bisection safeguard) against
    the oracle's exact threshold, with the refinement budget the header
    states for these alphas."""
    w, refine = SECANT[name]
    print(f"[entmax attention, secant] {name} refine={refine} out_f32={out_f32}", flush=True)
    x = parity.make(w)
    O, tau = bsa.attend_entmax(x["Q"], x["K"], x["V"], w.alpha, refine=refine,
                               out_dtype=torch.float32 if out_f32 else None, want_tau=True)
    ref, rtau, sup = oracle.entmax_attend(x["q"], x["k"], x["v"], w.alpha)
    worst = parity.check_attention(w, _cpu(O).reshape(ref.shape), ref, out_f32)
    terr = np.abs(_cpu(tau).ravel() - rtau)
    assert terr.max() < 1e-3, terr.max()
    print(f"max abs err {worst:.3e}, tau err max {terr.max():.2e} median {np.median(terr):.2e}, "
          f"mean support {sup.mean():.1f}")


def test_entmax_attention_zero_query_is_the_causal_mean():
    w = CASES["a15_gqa"]
    x = parity.make(w)
    Q = torch.zeros_like(x["Q"])
    O = bsa.attend_entmax(Q, x["K"], x["V"], 1.5, out_dtype=torch.float32)
    G = w.hq // w.hkv
    v = np.repeat(x["v"].astype(np.float64), G, axis=1)
    ref = np.cumsum(v, axis=2) / np.arange(1, w.n + 1)[None, None, :, None]
    np.testing.assert_allclose(_cpu(O), ref, rtol=0, atol=2e-3)


def test_entmax_attention_long_sampled():
    w = BASE.scaled(n=8192, hq=8, hkv=2)
    x = parity.make(w)
    O = bsa.attend_entmax(x["Q"], x["K"], x["V"], w.alpha, out_dtype=torch.float32)
    rng = np.random.default_rng(9)
    rows = sorted({0, 63, 64, w.n - 1} | set(rng.choice(w.n, 60, replace=False).tolist()))
    req = np.array([[0, h, t] for h in range(w.hq) for t in rows], np.int64)
    ref, _, sup = oracle.entmax_attend(x["q"], x["k"], x["v"], w.alpha, req=req)
    got = _cpu(O)[req[:, 0], req[:, 1], req[:, 2]]
    worst = parity.check_attention(w, got, ref, True)
    print(f"{len(req)} sampled rows, max abs err {worst:.3e}, mean support {sup.mean():.1f}")


def test_entmax_attention_full_size_two_passes_converge():
    """Every row of the token-level entmax workload at full size (N = 16384,
    32/8 heads) reaches its threshold in the two refinement passes: against
    sixteen passes on all 524 288 rows, and against the oracle's exact root on
    rows whose root lies within 2e-4 of the bracket's upper end with a key
    leaving the support in between (where an unguarded Halley step
    overshoots) plus seeded ones."""
    w = synth.WORKLOADS["entmax_attn_prefill_n16k"]
    print("[entmax attention] full size, two passes", flush=True)
    x = parity.make(w)
    _, tau2 = bsa.attend_entmax(x["Q"], x["K"], x["V"], w.alpha, refine=2, want_tau=True)
    _, tau16 = bsa.attend_entmax(x["Q"], x["K"], x["V"], w.alpha, refine=16, want_tau=True)
    t2, t16 = _cpu(tau2)[0], _cpu(tau16)[0]
    gap = np.abs(t2 - t16)
    assert gap.max() < 1e-4, (gap.max(), np.unravel_index(gap.argmax(), gap.shape))
    rng = np.random.default_rng(13)
    rows = [(10, 200), (17, 11158), (18, 4808), (26, 11205)]
    rows += [(int(h), int(t)) for h, t in zip(rng.integers(0, w.hq, 12), rng.integers(0, w.n, 12))]
    req = np.array([[0, h, t] for h, t in rows], np.int64)
    _, rtau, _ = oracle.entmax_attend(x["q"], x["k"], x["v"], w.alpha, req=req)
    got = np.array([t2[h, t] for h, t in rows])
    assert np.abs(got - rtau).max() < 1e-4, np.abs(got - rtau).max()
    print(f"max |tau(2) - tau(16)| {gap.max():.2e}, vs exact on {len(rows)} rows "
          f"{np.abs(got - rtau).max():.2e}")


def test_entmax_attention_longest_sequence_sampled():
    """The longest sequence the kernel takes (2048 key tiles, ragged: N =
    131072 - 5), one head: sampled rows, the last ones included, against the
    oracle."""
    w = BASE.scaled(hq=1, hkv=1, n=131072 - 5, planted_blocks=8)
    print("[entmax attention] N = 131067", flush=True)
    x = parity.make(w)
    O, tau = bsa.attend_entmax(x["Q"], x["K"], x["V"], w.alpha, out_dtype=torch.float32,
                               want_tau=True)
    rng = np.random.default_rng(21)
    rows = sorted({0, 64, 65535, w.n - 64, w.n - 2, w.n - 1}
                  | set(rng.choice(w.n, 18, replace=False).tolist()))
    req = np.array([[0, 0, t] for t in rows], np.int64)
    ref, rtau, sup = oracle.entmax_attend(x["q"], x["k"], x["v"], w.alpha, req=req)
    got = _cpu(O)[0, 0, rows]
    worst = parity.check_attention(w, got, ref, True)
    terr = np.abs(_cpu(tau)[0, 0, rows] - rtau)
    assert terr.max() < 1e-3, terr.max()
    print(f"{len(rows)} rows, max abs err {worst:.3e}, tau err max {terr.max():.2e}, "
          f"mean support {sup.mean():.1f}")


def test_entmax_attention_argument_errors():
    w = CASES["a15_gqa"]
    x = parity.make(w)
    with pytest.raises(bsa.BsaError, match="alpha"):
        bsa.attend_entmax(x["Q"], x["K"], x["V"], 1.0)
    with pytest.raises(bsa.BsaError, match="alpha <= 16"):
        bsa.attend_entmax(x["Q"], x["K"], x["V"], 17.0)
    with pytest.raises(bsa.BsaError, match="refine"):
        bsa.attend_entmax(x["Q"], x["K"], x["V"], 1.5, refine=25)
    with pytest.raises(bsa.BsaError, match="bf16"):
        bsa.attend_entmax(x["Q"].float(), x["K"].float(), x["V"].float(), 1.5)


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

BWD_TOL = 1e-2  # of each gradient tensor's largest magnitude (as the block-sparse backward)


def _check_grad(name, g, ref, bf16_out):
    g = _cpu(g).astype(np.float64).reshape(ref.shape)
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(g - ref)
    bound = BWD_TOL * scale + (parity.half_ulp_bf16(ref) if bf16_out else 0.0)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{name}: {len(bad)} out of bounds, first {bad[0].tolist()}: "
                           f"{g[tuple(bad[0])]} vs {ref[tuple(bad[0])]} (scale {scale:.3g})")
    return float((err / scale).max())


@pytest.mark.parametrize("name", ["a15_gqa", "a2_sparsemax", "a125", "a175_newton", "a15_d64",
                                  "a15_batch2"])
@pytest.mark.parametrize("g_f32", [True, False])
@pytest.mark.parametrize("use_live", [False, True])
def test_entmax_attention_backward_matches_oracle(name, g_f32, use_live):
    """dQ, dK, dV from the forward's tau (and, with use_live, walking only
    the forward's live key tiles) against the oracle's gradients with exact
    thresholds."""
    w = CASES[name]
    print(f"[entmax attention backward] {name} g_f32={g_f32} live={use_live}", flush=True)
    x = parity.make(w)
    do_st, do = synth.gen_stored(w, "do")
    dO = parity.to_device(do_st, w.dtype)
    O, tau, live = bsa.attend_entmax(x["Q"], x["K"], x["V"], w.alpha, refine=2, want_tau=True,
                                     want_live=True)
    grads = bsa.attend_entmax_backward(x["Q"], x["K"], x["V"], dO, tau, w.alpha,
                                       grad_dtype=torch.float32 if g_f32 else None,
                                       live=live if use_live else None)
    torch.cuda.synchronize()
    refs = oracle.entmax_attend_backward(x["q"], x["k"], x["v"], do, w.alpha)
    e = [_check_grad(nm, g, r, not g_f32) for nm, g, r in zip(("dQ", "dK", "dV"), grads, refs)]
    print("max err / scale: dQ %.2e dK %.2e dV %.2e" % tuple(e))


def test_entmax_attention_backward_sums_and_determinism():
    """The key gradients of a KV head sum to zero and the value gradients to
    the upstream gradients (entmax weights sum to one); two calls agree."""
    w = CASES["a15_gqa"]
    x = parity.make(w)
    dO = torch.randn(x["Q"].shape, generator=torch.Generator().manual_seed(9)).to(
        "cuda", torch.bfloat16)
    _, tau = bsa.attend_entmax(x["Q"], x["K"], x["V"], w.alpha, want_tau=True)
    g1 = bsa.attend_entmax_backward(x["Q"], x["K"], x["V"], dO, tau, w.alpha,
                                    grad_dtype=torch.float32)
    g2 = bsa.attend_entmax_backward(x["Q"], x["K"], x["V"], dO, tau, w.alpha,
                                    grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    dK, dV = g1[1].double(), g1[2].double()
    assert float(dK.sum(dim=2).abs().max()) <= 1e-3 * float(dK.abs().sum(dim=2).max())
    G = w.hq // w.hkv
    ref = dO.double().reshape(1, w.hkv, G, w.n, w.d).sum(dim=(2, 3))
    assert float((dV.sum(dim=2) - ref).abs().max()) <= 1e-2 * float(ref.abs().max())


@pytest.mark.parametrize("name", ["a15_gqa", "a2_sparsemax", "a175_newton", "a15_g8"])
@pytest.mark.parametrize("refine", [2, 0])
def test_entmax_live_tiles_cover_every_support(name, refine):
    """The forward's live key tiles hold every key with a nonzero oracle
    weight for every query of the tile and every head of the group (and,
    with refine = 0, are every causal tile); the same output either way."""
    w = CASES[name]
    print(f"[entmax live tiles] {name} refine={refine}", flush=True)
    x = parity.make(w)
    O1 = bsa.attend_entmax(x["Q"], x["K"], x["V"], w.alpha, refine=refine)
    O2, live = bsa.attend_entmax(x["Q"], x["K"], x["V"], w.alpha, refine=refine, want_live=True)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)
    nt = (w.n + 63) // 64
    lv = _cpu(live).astype(np.int64) & 0xFFFFFFFF
    bits = np.zeros((w.hkv, nt, nt), bool)
    for j in range(nt):
        bits[:, :, j] = (lv[0, :, :, j >> 5] >> (j & 31)) & 1
    causal = np.tril(np.ones((nt, nt), bool))
    assert not (bits & ~causal).any()
    if refine == 0:
        assert (bits == causal).all()
        return
    G = w.hq // w.hkv
    rng = np.random.default_rng(31)
    req = np.array([[0, h, t] for h in range(w.hq) for t in rng.choice(w.n, 24, replace=False)])
    _, tau, _ = oracle.entmax_attend(x["q"], x["k"], x["v"], w.alpha, req=req)
    q = x["q"].astype(np.float64)
    k = x["k"].astype(np.float64)
    sc = (w.alpha - 1) / np.sqrt(w.d)
    for (b, h, t), tt in zip(req, tau):
        xs = sc * (k[0, h // G, :t + 1] @ q[0, h, t])
        # (a margin far below the bracket's width keeps fp32 scores' rounding out)
        for j in np.unique(np.nonzero(xs > tt + 1e-4)[0] // 64):
            assert bits[h // G, t // 64, j], (h, t, j)
    frac = bits.sum() / (causal.sum() * w.hkv)
    print(f"live fraction {frac:.3f}")


def test_entmax_attention_backward_full_size_live_tiles_change_nothing():
    """The token-level entmax attention workload at its full size (N = 16384,
    32/8 heads): walking only the forward's live key tiles gives the same
    gradient bits as walking every causal tile (the skipped tiles hold no
    weight, and the kept ones are summed in the same order), and the
    gradients obey the identities of normalised weights."""
    w = synth.WORKLOADS["entmax_attn_prefill_n16k"]
    print("[entmax attention backward] full size", flush=True)
    x = parity.make(w)
    dO = torch.randn(x["Q"].shape, generator=torch.Generator().manual_seed(11)).to(
        "cuda", torch.bfloat16)
    _, tau, live = bsa.attend_entmax(x["Q"], x["K"], x["V"], w.alpha, want_tau=True,
                                     want_live=True)
    g_live = bsa.attend_entmax_backward(x["Q"], x["K"], x["V"], dO, tau, w.alpha,
                                        grad_dtype=torch.float32, live=live)
    g_all = bsa.attend_entmax_backward(x["Q"], x["K"], x["V"], dO, tau, w.alpha,
                                       grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for nm, a_, b_ in zip(("dQ", "dK", "dV"), g_live, g_all):
        assert torch.equal(a_, b_), nm
    dK, dV = g_live[1].double(), g_live[2].double()
    assert float(dK.sum(dim=2).abs().max()) <= 1e-3 * float(dK.abs().sum(dim=2).max())
    G = w.hq // w.hkv
    ref = dO.double().reshape(w.batch, w.hkv, G, w.n, w.d).sum(dim=(2, 3))
    assert float((dV.sum(dim=2) - ref).abs().max()) <= 1e-2 * float(ref.abs().max())
