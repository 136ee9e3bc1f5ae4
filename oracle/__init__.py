"""fp64 CPU oracle for block-sparse attention with summary-based block routing.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers; the product path never imports this
package.  It shares no code with the HIP library: the arithmetic lives in
``bsa_oracle.c`` (plain C, fp64, single-threaded) and this module only
marshals numpy arrays through ctypes.

Layouts are dense row-major ``[batch, heads, tokens, d]``.  bf16 data is passed
as its exact fp32 upcast.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FORCE_DIAG = 1
FORCE_FIRST = 2
FORCE_TAIL = 4
MODE_PREFILL = 0
MODE_DECODE = 1
MODE_TOKEN = 2  # causal prefill routed per query token


def build(force: bool = True) -> str:
    """Compile the oracle with gcc -O2 (no fast-math, no threads)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        D = ctypes.c_double
        lib.orc_summarize.argtypes = [P, I, I, I, I, I, P, P]
        lib.orc_qpool.argtypes = [P, I, I, I, I, I, P]
        lib.orc_route_topk.argtypes = [P, P, I, I, I, I, I, I, I, ctypes.c_int, P, I,
                                       ctypes.c_uint32, D, P, P, P, P]
        lib.orc_entmax_row.argtypes = [P, I, D, ctypes.c_int, ctypes.c_int, P, P, P, P, P]
        lib.orc_entmax_row.restype = D
        lib.orc_route_entmax.argtypes = [P, P, I, I, I, I, I, I, I, ctypes.c_int, P, D, D,
                                         ctypes.c_int, ctypes.c_int, I, ctypes.c_uint32, D, I,
                                         P, P, P, P, P, P, P, P, P]
        lib.orc_attend.argtypes = [P, P, P, I, I, I, I, I, I, I, ctypes.c_int, P, P, P, I, D,
                                   P, I, P, P, P, D]
        lib.orc_token_union.argtypes = [P, P, I, I, I, I, I, P, P, P]
        lib.orc_entmax_attend.argtypes = [P, P, P, I, I, I, I, I, D, D, P, I, P, P, P]
        lib.orc_attend_backward.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_int, P, P, I,
                                            D, P, P, D, P, P, P, P]
        lib.orc_entmax_vjp.argtypes = [P, P, I, D, P]
        lib.orc_entmax_attend_backward.argtypes = [P, P, P, P, I, I, I, I, I, D, D, P, P, P]
        lib.orc_route_entmax_backward.argtypes = [P, P, P, P, P, I, P, I, I, I, I, I, I,
                                                  ctypes.c_int, D, D, D, ctypes.c_uint32, P, P]
        lib.orc_version.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def summarize(K, B, qbar=None):
    """Block summaries of K [nb, nh, n, d] -> fp64 [nb, nh, ceil(n/B), d]."""
    K = _f32(K)
    nb, nh, n, d = K.shape
    nblk = (n + B - 1) // B
    S = np.empty((nb, nh, nblk, d), np.float64)
    qb = None if qbar is None else _f32(qbar)
    _load().orc_summarize(_ptr(K), nb, nh, n, d, B, _ptr(qb), _ptr(S))
    return S


def qpool(Q, B):
    """Per-head mean of each query block: Q [nb, nh, n, d] -> [nb, nh, ceil(n/B), d]."""
    Q = _f32(Q)
    nb, nh, n, d = Q.shape
    nblk = (n + B - 1) // B
    out = np.empty((nb, nh, nblk, d), np.float64)
    _load().orc_qpool(_ptr(Q), nb, nh, n, d, B, _ptr(out))
    return out


def route_topk(qhat, S, B, k_total, force=0, mode=MODE_PREFILL, kv_lens=None, score_scale=None):
    """Top-k routing.  qhat [nb, hq, nrow, d], S [nb, hkv, nblk, d] (fp64).

    Returns dict(idx, cnt, scores, gap)."""
    qhat = _f64(qhat)
    S = _f64(S)
    nb, hq, nrow, d = qhat.shape
    _, hkv, nblk, _ = S.shape
    if score_scale is None:
        score_scale = 1.0 / np.sqrt(d)
    kl = None if kv_lens is None else np.ascontiguousarray(kv_lens, dtype=np.int64)
    idx = np.empty((nb, hkv, nrow, k_total), np.int32)
    cnt = np.empty((nb, hkv, nrow), np.int32)
    scores = np.empty((nb, hkv, nrow, nblk), np.float64)
    gap = np.empty((nb, hkv, nrow), np.float64)
    _load().orc_route_topk(_ptr(qhat), _ptr(S), nb, hq, hkv, nrow, nblk, d, B, mode, _ptr(kl),
                           k_total, force, float(score_scale), _ptr(idx), _ptr(cnt),
                           _ptr(scores), _ptr(gap))
    return dict(idx=idx, cnt=cnt, scores=scores, gap=gap)


def entmax_row(x, alpha, n_bins=16, max_iter=8):
    """alpha-entmax of one row x (already scaled by alpha-1), histogram-started
    bisection.  Returns (p, tau, resolved, iters, tau_lo, tau_hi)."""
    x = _f64(x)
    n = x.shape[0]
    p = np.empty(n, np.float64)
    res = ctypes.c_int(0)
    its = ctypes.c_int(0)
    tlo = ctypes.c_double(0)
    thi = ctypes.c_double(0)
    tau = _load().orc_entmax_row(_ptr(x), n, float(alpha), n_bins, max_iter, _ptr(p),
                                 ctypes.byref(res), ctypes.byref(its), ctypes.byref(tlo),
                                 ctypes.byref(thi))
    return p, tau, bool(res.value), its.value, tlo.value, thi.value


def route_entmax(qhat, S, B, alpha, gamma, cap, force=FORCE_DIAG, n_bins=16, max_iter=8,
                 mode=MODE_PREFILL, kv_lens=None, score_scale=None, idx_width=None):
    """Entmax routing.  Returns dict(idx, cnt, probs, tau, margin, capgap,
    resolved, iters, wsel)."""
    qhat = _f64(qhat)
    S = _f64(S)
    nb, hq, nrow, d = qhat.shape
    _, hkv, nblk, _ = S.shape
    if score_scale is None:
        score_scale = 1.0 / np.sqrt(d)
    if idx_width is None:
        idx_width = cap + bin(force & 7).count("1")
    kl = None if kv_lens is None else np.ascontiguousarray(kv_lens, dtype=np.int64)
    idx = np.empty((nb, hkv, nrow, idx_width), np.int32)
    cnt = np.empty((nb, hkv, nrow), np.int32)
    probs = np.empty((nb, hq, nrow, nblk), np.float64)
    tau = np.empty((nb, hq, nrow), np.float64)
    margin = np.empty((nb, hq, nrow), np.float64)
    capgap = np.empty((nb, hkv, nrow), np.float64)
    resolved = np.empty((nb, hq, nrow), np.int32)
    iters = np.empty((nb, hq, nrow), np.int32)
    wsel = np.empty((nb, hkv, nrow, idx_width), np.float64)
    _load().orc_route_entmax(_ptr(qhat), _ptr(S), nb, hq, hkv, nrow, nblk, d, B, mode, _ptr(kl),
                             float(alpha), float(gamma), n_bins, max_iter, cap, force,
                             float(score_scale), idx_width, _ptr(idx), _ptr(cnt), _ptr(probs),
                             _ptr(tau), _ptr(margin), _ptr(capgap), _ptr(resolved), _ptr(iters),
                             _ptr(wsel))
    return dict(idx=idx, cnt=cnt, probs=probs, tau=tau, margin=margin, capgap=capgap,
                resolved=resolved, iters=iters, wsel=wsel)


def attend(Q, K, V, B, idx, cnt, req=None, mode=MODE_PREFILL, kv_lens=None, sm_scale=None,
           wsel=None, sigma=0.0):
    """Fine attention over the selected blocks for the requested (b, h, t) rows;
    with wsel (routing weights in the layout of idx) the prior-induced softmax
    of strength sigma.

    Returns (O [nreq, d] fp64, pairs [nreq] int64).  req=None means every row."""
    Q = _f32(Q)
    K = _f32(K)
    V = _f32(V)
    nb, hq, nq, d = Q.shape
    _, hkv, nk, _ = K.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    if req is None:
        bb, hh, tt = np.meshgrid(np.arange(nb), np.arange(hq), np.arange(nq), indexing="ij")
        req = np.stack([bb.ravel(), hh.ravel(), tt.ravel()], axis=1)
    req = np.ascontiguousarray(req, dtype=np.int64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    cnt = np.ascontiguousarray(cnt, dtype=np.int32)
    kmax = idx.shape[-1]
    kl = None if kv_lens is None else np.ascontiguousarray(kv_lens, dtype=np.int64)
    O = np.empty((req.shape[0], d), np.float64)
    pairs = np.empty(req.shape[0], np.int64)
    if wsel is not None:
        wsel = np.ascontiguousarray(wsel, dtype=np.float64)
        assert wsel.shape == idx.shape
    _load().orc_attend(_ptr(Q), _ptr(K), _ptr(V), nb, hq, hkv, nq, nk, d, B, mode, _ptr(kl),
                       _ptr(idx), _ptr(cnt), kmax, float(sm_scale), _ptr(req), req.shape[0],
                       _ptr(O), _ptr(pairs), _ptr(wsel), float(sigma))
    return O, pairs


def token_union(idx, cnt, nblk):
    """Active blocks of every 64-query tile from per-token selections.
    idx [nb, hkv, n, width], cnt [nb, hkv, n].  Returns (uidx, ucnt, ubits):
    uidx [nb, hkv, ntile, nblk] ascending, -1 padded; ucnt [nb, hkv, ntile];
    ubits [nb, hkv, ntile, nblk] uint64, bit r = token 64*tile + r selected it."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    cnt = np.ascontiguousarray(cnt, dtype=np.int32)
    nb, hkv, n, width = idx.shape
    ntile = (n + 63) // 64
    uidx = np.empty((nb, hkv, ntile, nblk), np.int32)
    ucnt = np.empty((nb, hkv, ntile), np.int32)
    ubits = np.empty((nb, hkv, ntile, nblk), np.uint64)
    _load().orc_token_union(_ptr(idx), _ptr(cnt), nb, hkv, n, width, nblk, _ptr(uidx),
                            _ptr(ucnt), _ptr(ubits))
    return uidx, ucnt, ubits


def entmax_attend(Q, K, V, alpha, req=None, sm_scale=None):
    """Causal token-level alpha-entmax attention for the requested (b, h, t)
    rows (all rows when req is None).  Returns (O [nreq, d] fp64,
    tau [nreq], support [nreq])."""
    Q = _f32(Q)
    K = _f32(K)
    V = _f32(V)
    nb, hq, n, d = Q.shape
    hkv = K.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    if req is None:
        bb, hh, tt = np.meshgrid(np.arange(nb), np.arange(hq), np.arange(n), indexing="ij")
        req = np.stack([bb.ravel(), hh.ravel(), tt.ravel()], axis=1)
    req = np.ascontiguousarray(req, dtype=np.int64)
    O = np.empty((req.shape[0], d), np.float64)
    tau = np.empty(req.shape[0], np.float64)
    sup = np.empty(req.shape[0], np.int64)
    _load().orc_entmax_attend(_ptr(Q), _ptr(K), _ptr(V), nb, hq, hkv, n, d, float(alpha),
                              float(sm_scale), _ptr(req), req.shape[0], _ptr(O), _ptr(tau),
                              _ptr(sup))
    return O, tau, sup


def attend_backward(Q, K, V, dO, B, idx, cnt, sm_scale=None, rowmask=None, wsel=None,
                    sigma=0.0, mode=MODE_PREFILL):
    """Gradients (dQ, dK, dV) in fp64 of the causal block-sparse attention
    (prefill rows, selection idx/cnt per query block; mode=MODE_TOKEN:
    per query token) for upstream dO.
    rowmask [nb, hkv, nrow] (bool): only those selection rows contribute.
    wsel, sigma: the prior-induced softmax; then (dQ, dK, dV, dwsel) with
    dwsel = dL/dw in the layout of idx."""
    Q, K, V, dO = _f32(Q), _f32(K), _f32(V), _f32(dO)
    nb, hq, n, d = Q.shape
    hkv = K.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    cnt = np.ascontiguousarray(cnt, dtype=np.int32)
    dQ = np.empty(Q.shape, np.float64)
    dK = np.empty(K.shape, np.float64)
    dV = np.empty(V.shape, np.float64)
    if rowmask is not None:
        rowmask = np.ascontiguousarray(rowmask, dtype=np.uint8)
        assert rowmask.shape == cnt.shape
    dwsel = None
    if wsel is not None:
        wsel = np.ascontiguousarray(wsel, dtype=np.float64)
        assert wsel.shape == idx.shape
        dwsel = np.empty(idx.shape, np.float64)
    _load().orc_attend_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), nb, hq, hkv, n, d, B,
                                int(mode), _ptr(idx), _ptr(cnt), idx.shape[-1], float(sm_scale),
                                _ptr(rowmask), _ptr(wsel), float(sigma), _ptr(dwsel), _ptr(dQ),
                                _ptr(dK), _ptr(dV))
    return (dQ, dK, dV) if wsel is None else (dQ, dK, dV, dwsel)


def entmax_attend_backward(Q, K, V, dO, alpha, sm_scale=None):
    """Gradients (dQ, dK, dV) in fp64 of the causal token-level alpha-entmax
    attention for upstream dO."""
    Q, K, V, dO = _f32(Q), _f32(K), _f32(V), _f32(dO)
    nb, hq, n, d = Q.shape
    hkv = K.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    dQ = np.empty(Q.shape, np.float64)
    dK = np.empty(K.shape, np.float64)
    dV = np.empty(V.shape, np.float64)
    _load().orc_entmax_attend_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), nb, hq, hkv, n, d,
                                       float(alpha), float(sm_scale), _ptr(dQ), _ptr(dK),
                                       _ptr(dV))
    return dQ, dK, dV


def entmax_vjp(p, dp, alpha):
    """dL/dz of alpha-entmax at probabilities p (logits z, x = (alpha-1) z)
    for dL/dp = dp."""
    p = _f64(p)
    dp = _f64(dp)
    dz = np.empty_like(p)
    _load().orc_entmax_vjp(_ptr(p), _ptr(dp), p.size, float(alpha), _ptr(dz))
    return dz


def route_entmax_backward(qhat, S, probs, idx, cnt, dwsel, n, B, alpha, gamma,
                          score_scale=None, force=FORCE_DIAG, mode=MODE_PREFILL):
    """Routing part of the gradient (prefill block rows; mode=MODE_TOKEN: a
    row per query token, qhat the queries themselves): dL/dQ and dL/dK in
    fp64 through qhat -> logits -> entmax -> group mean w, given dL/dw."""
    qhat, S, probs, dwsel = _f64(qhat), _f64(S), _f64(probs), _f64(dwsel)
    nb, hq, nrow, d = qhat.shape
    hkv = S.shape[1]
    if score_scale is None:
        score_scale = 1.0 / np.sqrt(d)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    cnt = np.ascontiguousarray(cnt, dtype=np.int32)
    dQ = np.empty((nb, hq, n, d), np.float64)
    dK = np.empty((nb, hkv, n, d), np.float64)
    _load().orc_route_entmax_backward(_ptr(qhat), _ptr(S), _ptr(probs), _ptr(idx), _ptr(cnt),
                                      idx.shape[-1], _ptr(dwsel), nb, hq, hkv, n, d, B,
                                      int(mode), float(alpha), float(gamma), float(score_scale),
                                      force,
                                      _ptr(dQ), _ptr(dK))
    return dQ, dK


def version() -> str:
    return _load().orc_version().decode()
