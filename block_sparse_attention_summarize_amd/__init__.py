"""Block-sparse attention with summary-based block routing on MI355X (gfx950).

Thin ctypes binding of ``libbsa.so`` (C ABI in ``include/bsa.h``).  PyTorch is
used only for device memory and streams: every step runs in the library's HIP
kernels.  The library is loaded at the first call into it, which raises
ImportError if it has not been built
(``python -m block_sparse_attention_summarize_amd.build``).

Stages (names as in the C ABI):
  summarize        keys -> per-block summaries (mean pool, or learned query)
  route_topk       top-k block selection with forced blocks
  route_entmax     alpha-entmax block support (histogram-started bisection)
  attend_prefill   causal attention over the selected blocks' tokens
  attend_decode    single-token decode over the selected blocks (split-KV)
  token_mask       per-token selections -> active-block masks of 64-query tiles
Per-token routing (every query token routed on its own) is the `token=True`
variant of route_topk / route_entmax / attend_prefill.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

F32, BF16 = 0, 1
PREFILL, DECODE, TOKEN = 0, 1, 2
FORCE_DIAG, FORCE_FIRST, FORCE_TAIL = 1, 2, 4
OP_SUMMARIZE, OP_ROUTE_TOPK, OP_ROUTE_ENTMAX, OP_ATTEND_PREFILL, OP_ATTEND_DECODE, \
    OP_DECODE_TOPK, OP_ATTEND_PREFILL_PRIOR, OP_ATTEND_BACKWARD, OP_ROUTE_ENTMAX_BACKWARD, \
    OP_ATTEND_ENTMAX_BACKWARD, OP_ATTEND_BACKWARD_PRIOR = range(11)
STATUS = {0: "BSA_OK", -1: "BSA_ERR_INVALID", -2: "BSA_ERR_UNSUPPORTED", -3: "BSA_ERR_DEVICE",
          -4: "BSA_ERR_WORKSPACE"}

EXPORTS = ("bsa_summarize", "bsa_summarize_blocks", "bsa_summarize_blocks_paged",
           "bsa_route_topk", "bsa_route_entmax", "bsa_attend_prefill", "bsa_token_mask",
           "bsa_attend_decode", "bsa_decode_topk", "bsa_decode_topk_noalloc",
           "bsa_decode_topk_paged", "bsa_attend_entmax",
           "bsa_attend_backward", "bsa_route_entmax_backward", "bsa_attend_entmax_backward",
           "bsa_workspace_size",
           "bsa_last_error", "bsa_version")


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("mode", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("q_len", ctypes.c_int64), ("kv_len", ctypes.c_int64),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
    ]


class Pages(ctypes.Structure):
    _fields_ = [("table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("k_page_stride", ctypes.c_int64),
                ("v_page_stride", ctypes.c_int64)]


_P = ctypes.c_void_p
_i32 = ctypes.c_int32
_u32 = ctypes.c_uint32
_f32 = ctypes.c_float
_sz = ctypes.c_size_t
_SP = ctypes.POINTER(Shape)
_PP = ctypes.POINTER(Pages)


def _declare(lib):
    """Sets the argument and result types of every exported entry point."""
    lib.bsa_summarize.argtypes = [_SP, _P, _P, _P, _P]
    lib.bsa_summarize_blocks.argtypes = [_SP, _P, _P, _P, _P, _P]
    lib.bsa_summarize_blocks_paged.argtypes = [_SP, _PP, _P, _P, _P, _P, _P]
    lib.bsa_decode_topk_paged.argtypes = [_SP, _PP, _P, _P, _P, _P, _P, _i32, _u32, _f32, _f32, _P, _P,
                                          _P, _i32, _P, _sz, _P]
    lib.bsa_route_topk.argtypes = [_SP, _P, _P, _P, _i32, _u32, _f32, _P, _P, _P, _P, _sz, _P]
    lib.bsa_route_entmax.argtypes = [_SP, _P, _P, _P, _f32, _f32, _i32, _i32, _i32, _u32, _f32, _P,
                                     _P, _P, _P, _P, _P, _sz, _P]
    lib.bsa_attend_prefill.argtypes = [_SP, _P, _P, _P, _P, _P, _i32, _f32, _P, _f32, _P, _i32, _P, _P,
                                       _sz, _P]
    lib.bsa_attend_backward.argtypes = [_SP, _P, _P, _P, _P, _i32, _P, _P, _P, _P, _i32, _f32, _P, _f32,
                                        _P, _P, _P, _P, _i32, _P, _sz, _P]
    lib.bsa_attend_entmax_backward.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _f32, _f32, _P, _P, _P, _i32,
                                               _P, _sz, _P]
    lib.bsa_route_entmax_backward.argtypes = [_SP, _P, _P, _P, _P, _P, _i32, _P, _f32, _f32, _f32, _P,
                                              _P, _i32, _P, _sz, _P]
    lib.bsa_token_mask.argtypes = [_SP, _P, _P, _i32, _P, _P, _P, _P]
    lib.bsa_attend_entmax.argtypes = [_SP, _P, _P, _P, _f32, _i32, _f32, _P, _i32, _P, _P, _P]
    lib.bsa_attend_decode.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _i32, _f32, _P, _i32, _P, _sz, _P]
    lib.bsa_decode_topk.argtypes = [_SP, _P, _P, _P, _P, _P, _i32, _u32, _f32, _f32, _P, _P, _P, _i32,
                                    _P, _sz, _P]
    lib.bsa_decode_topk_noalloc.argtypes = [_SP, _P, _P, _P, _P, _P, _i32, _u32, _f32, _f32, _P, _P,
                                            _P, _i32, _P]
    for f in (lib.bsa_summarize, lib.bsa_summarize_blocks, lib.bsa_summarize_blocks_paged,
               lib.bsa_route_topk, lib.bsa_route_entmax, lib.bsa_attend_prefill, lib.bsa_token_mask,
               lib.bsa_attend_decode, lib.bsa_decode_topk, lib.bsa_decode_topk_noalloc,
               lib.bsa_decode_topk_paged,
               lib.bsa_attend_entmax, lib.bsa_attend_backward, lib.bsa_route_entmax_backward,
               lib.bsa_attend_entmax_backward):
        f.restype = ctypes.c_int
    lib.bsa_workspace_size.argtypes = [_i32, _SP, _i32]
    lib.bsa_workspace_size.restype = _sz
    lib.bsa_last_error.restype = ctypes.c_char_p
    lib.bsa_version.restype = ctypes.c_char_p


class _Library:
    """libbsa.so, loaded at the first call into it.

    Loading on first use lets the package be imported to build the library
    from a clean checkout; any call made before the library exists raises
    ImportError (there is no fallback path)."""

    _cdll = None

    def __getattr__(self, name):
        if _Library._cdll is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"libbsa.so not found at {LIB_PATH}; build it with "
                    "`python -m block_sparse_attention_summarize_amd.build`")
            cdll = ctypes.CDLL(LIB_PATH)
            _declare(cdll)
            _Library._cdll = cdll
        return getattr(_Library._cdll, name)


lib = _Library()


class BsaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def version() -> str:
    return lib.bsa_version().decode()


def _check(rc):
    if rc != 0:
        raise BsaError(rc, lib.bsa_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _strides(t):
    if t is None:
        return (0, 0, 0)
    if t.stride(3) != 1:
        raise ValueError("head_dim must be contiguous")
    return tuple(int(s) for s in t.stride()[:3])


def make_shape(*, batch, hq, hkv, d, B, dtype, mode, q_len, kv_len, q=None, k=None, v=None,
               o=None) -> Shape:
    s = Shape()
    s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.block = batch, hq, hkv, d, B
    s.dtype, s.mode, s.reserved = dtype, mode, 0
    s.q_len, s.kv_len = q_len, kv_len
    s.q_stride[:] = _strides(q)
    s.k_stride[:] = _strides(k)
    s.v_stride[:] = _strides(v)
    s.o_stride[:] = _strides(o)
    return s


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def workspace_size(op: int, shape: Shape, k_or_cap: int) -> int:
    return int(lib.bsa_workspace_size(op, ctypes.byref(shape), k_or_cap))


def _workspace(op, shape, k, device, ws=None):
    n = workspace_size(op, shape, k)
    if ws is not None and ws.numel() * ws.element_size() >= n:
        return ws, n
    return (torch.empty(max(n, 1), dtype=torch.uint8, device=device), n)


def summarize(K: torch.Tensor, B: int, qbar: torch.Tensor | None = None,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """K [b, Hkv, L, d] -> fp32 summaries [b, Hkv, ceil(L/B), d]."""
    b, hkv, L, d = K.shape
    nblk = (L + B - 1) // B
    S = out if out is not None else torch.empty((b, hkv, nblk, d), dtype=torch.float32,
                                                device=K.device)
    shape = make_shape(batch=b, hq=hkv, hkv=hkv, d=d, B=B, dtype=_dtype_code(K), mode=PREFILL,
                       q_len=L, kv_len=L, k=K)
    if qbar is not None:
        qbar = qbar.contiguous().to(torch.float32)
    _check(lib.bsa_summarize(ctypes.byref(shape), _ptr(K), _ptr(qbar), _ptr(S), _stream(K)))
    return S


def _route_shape(Q, S, B, decode, kv_len, token=False):
    b, hq, n, d = Q.shape
    hkv, nblk = S.shape[1], S.shape[2]
    if decode:
        kv_len = kv_len if kv_len is not None else nblk * B
        return make_shape(batch=b, hq=hq, hkv=hkv, d=d, B=B, dtype=_dtype_code(Q), mode=DECODE,
                          q_len=1, kv_len=kv_len, q=Q)
    return make_shape(batch=b, hq=hq, hkv=hkv, d=d, B=B, dtype=_dtype_code(Q),
                      mode=TOKEN if token else PREFILL, q_len=n, kv_len=n, q=Q)


def _nrow(shape, B):
    if shape.mode == DECODE:
        return 1
    return shape.q_len if shape.mode == TOKEN else (shape.q_len + B - 1) // B


def summarize_blocks(K: torch.Tensor, B: int, blk: torch.Tensor, S: torch.Tensor,
                     qbar: torch.Tensor | None = None) -> torch.Tensor:
    """Recompute S[b, :, blk[b], :] of a cache K [b, Hkv, L, d] (blk int32 [b]
    on the device; out-of-range entries skip their sequence).  Returns S."""
    b, hkv, L, d = K.shape
    shape = make_shape(batch=b, hq=hkv, hkv=hkv, d=d, B=B, dtype=_dtype_code(K), mode=PREFILL,
                       q_len=L, kv_len=L, k=K)
    if qbar is not None:
        qbar = qbar.contiguous().to(torch.float32)
    _check(lib.bsa_summarize_blocks(ctypes.byref(shape), _ptr(K), _ptr(qbar), _ptr(blk), _ptr(S),
                                    _stream(K)))
    return S


def route_topk(Q, S, B, k_total, force=0, decode=False, kv_len=None, kv_lens=None,
               score_scale=0.0, want_scores=False, ws=None, out=None, partitioned=True,
               token=False):
    """Top-k routing.  Returns (idx, cnt) or (idx, cnt, scores).  In decode,
    partitioned=False passes no workspace (one workgroup per row routes).
    token=True routes every query token (rows = tokens)."""
    shape = _route_shape(Q, S, B, decode, kv_len, token)
    b, hkv, nblk = shape.batch, shape.n_kv_heads, S.shape[2]
    nrow = _nrow(shape, B)
    dev = Q.device
    if out is not None:
        idx, cnt = out
    else:
        idx = torch.empty((b, hkv, nrow, k_total), dtype=torch.int32, device=dev)
        cnt = torch.empty((b, hkv, nrow), dtype=torch.int32, device=dev)
    scores = torch.empty((b, hkv, nrow, nblk), dtype=torch.float32, device=dev) if want_scores else None
    if decode and not partitioned and not want_scores:
        wsb, n = None, 0
    else:
        wsb, n = _workspace(OP_ROUTE_TOPK, shape, k_total, dev, ws)
    _check(lib.bsa_route_topk(ctypes.byref(shape), _ptr(Q), _ptr(S), _ptr(kv_lens), k_total, force,
                              score_scale, _ptr(idx), _ptr(cnt), _ptr(scores), _ptr(wsb), n,
                              _stream(Q)))
    return (idx, cnt, scores) if want_scores else (idx, cnt)


def route_entmax(Q, S, B, alpha, gamma, cap, force=FORCE_DIAG, n_bins=16, max_iter=8,
                 decode=False, kv_len=None, kv_lens=None, score_scale=0.0, want_probs=False,
                 want_tau=False, ws=None, token=False, out=None, wsel=None):
    """alpha-entmax routing.  Returns (idx, cnt, probs or None, tau or None).
    token=True routes every query token (rows = tokens).  wsel: an fp32 tensor
    shaped like idx to receive the routing weight of every listed block."""
    shape = _route_shape(Q, S, B, decode, kv_len, token)
    b, hq, hkv, nblk = shape.batch, shape.n_q_heads, shape.n_kv_heads, S.shape[2]
    nrow = _nrow(shape, B)
    dev = Q.device
    width = cap + bin(force & 7).count("1")
    if out is not None:
        idx, cnt = out
    else:
        idx = torch.empty((b, hkv, nrow, width), dtype=torch.int32, device=dev)
        cnt = torch.empty((b, hkv, nrow), dtype=torch.int32, device=dev)
    probs = torch.empty((b, hq, nrow, nblk), dtype=torch.float32, device=dev) if want_probs else None
    tau = torch.empty((b, hq, nrow), dtype=torch.float32, device=dev) if want_tau else None
    wsb, n = _workspace(OP_ROUTE_ENTMAX, shape, cap, dev, ws)
    if wsel is not None:
        assert wsel.shape == idx.shape and wsel.dtype == torch.float32 and wsel.is_contiguous()
    _check(lib.bsa_route_entmax(ctypes.byref(shape), _ptr(Q), _ptr(S), _ptr(kv_lens), alpha, gamma,
                                n_bins, max_iter, cap, force, score_scale, _ptr(idx), _ptr(cnt),
                                _ptr(probs), _ptr(tau), _ptr(wsel), _ptr(wsb), n, _stream(Q)))
    return idx, cnt, probs, tau


def attend_prefill(Q, K, V, B, idx, cnt, sm_scale=0.0, out_dtype=None, out=None, token=False,
                   ws=None, wsel=None, sigma=0.0, want_lse=False):
    """Causal attention over the selected blocks.  Q [b, Hq, N, d], K/V [b, Hkv, N, d].
    token=True: idx/cnt are per-token selections [b, Hkv, N, width].
    wsel (routing weights shaped like idx) and sigma: prior-induced softmax.
    want_lse: also return the log-normaliser [b, Hq, N] fp32 the backward needs."""
    b, hq, n, d = Q.shape
    hkv = K.shape[1]
    odt = out_dtype or Q.dtype
    O = out if out is not None else torch.empty((b, hq, n, d), dtype=odt, device=Q.device)
    L = torch.empty((b, hq, n), dtype=torch.float32, device=Q.device) if want_lse else None
    shape = make_shape(batch=b, hq=hq, hkv=hkv, d=d, B=B, dtype=_dtype_code(Q),
                       mode=TOKEN if token else PREFILL, q_len=n, kv_len=K.shape[2], q=Q, k=K,
                       v=V, o=O)
    op = OP_ATTEND_PREFILL if wsel is None else OP_ATTEND_PREFILL_PRIOR
    wsb, nws = _workspace(op, shape, idx.shape[-1], Q.device, ws) if token else (None, 0)
    if wsel is not None:
        assert wsel.shape == idx.shape and wsel.dtype == torch.float32 and wsel.is_contiguous()
    _check(lib.bsa_attend_prefill(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx),
                                  _ptr(cnt), idx.shape[-1], sm_scale, _ptr(wsel), sigma, _ptr(O),
                                  _dtype_code(O), _ptr(L), _ptr(wsb), nws, _stream(Q)))
    return (O, L) if want_lse else O


def attend_backward(Q, K, V, O, dO, lse, B, idx, cnt, sm_scale=0.0, grad_dtype=None, ws=None,
                    wsel=None, sigma=0.0, want_dwsel=False, token=False):
    """Gradients (dQ, dK, dV) of attend_prefill's output (bf16; block rows,
    or token=True for per-token selections) for upstream gradient dO, given
    the forward's O and lse.  The gradients take the strides of Q, K, V; dO
    is brought to O's strides and Q's dtype.  wsel, sigma: the forward's
    prior; want_dwsel: also return dL/dw."""
    b, hq, n, d = Q.shape
    gdt = grad_dtype or Q.dtype
    dQ = torch.empty_strided(Q.size(), Q.stride(), dtype=gdt, device=Q.device)
    dK = torch.empty_strided(K.size(), K.stride(), dtype=gdt, device=K.device)
    dV = torch.empty_strided(V.size(), V.stride(), dtype=gdt, device=V.device)
    if dO.dtype != Q.dtype or dO.stride() != O.stride():
        t = torch.empty_strided(O.size(), O.stride(), dtype=Q.dtype, device=O.device)
        t.copy_(dO)
        dO = t
    shape = make_shape(batch=b, hq=hq, hkv=K.shape[1], d=d, B=B, dtype=_dtype_code(Q),
                       mode=TOKEN if token else PREFILL, q_len=n, kv_len=K.shape[2], q=Q, k=K,
                       v=V, o=O)
    op = OP_ATTEND_BACKWARD if wsel is None else OP_ATTEND_BACKWARD_PRIOR
    wsb, nws = _workspace(op, shape, idx.shape[-1], Q.device, ws)
    dw = torch.empty(idx.shape, dtype=torch.float32, device=Q.device) if want_dwsel else None
    if wsel is not None:
        assert wsel.shape == idx.shape and wsel.dtype == torch.float32 and wsel.is_contiguous()
    _check(lib.bsa_attend_backward(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                   _dtype_code(O), _ptr(dO), _ptr(lse), _ptr(idx), _ptr(cnt),
                                   idx.shape[-1], sm_scale, _ptr(wsel), sigma, _ptr(dw), _ptr(dQ),
                                   _ptr(dK), _ptr(dV), _dtype_code(dQ), _ptr(wsb), nws,
                                   _stream(Q)))
    return (dQ, dK, dV, dw) if want_dwsel else (dQ, dK, dV)


def route_entmax_backward(Q, S, probs, idx, cnt, dwsel, B, alpha, gamma, dQ, dK,
                          score_scale=0.0, ws=None, token=False):
    """Adds the gradient through the entmax routing weights (prefill block
    rows; token=True: a row per query token) to dQ and dK in place: dwsel
    from attend_backward, probs the routing's probs_out, S the summaries it
    scored.  Returns (dQ, dK)."""
    b, hq, n, d = Q.shape
    assert dQ.stride() == Q.stride() and dQ.dtype == dK.dtype
    shape = make_shape(batch=b, hq=hq, hkv=S.shape[1], d=d, B=B, dtype=_dtype_code(Q),
                       mode=TOKEN if token else PREFILL, q_len=n, kv_len=n, q=Q, k=dK, v=dK,
                       o=Q)
    wsb, nws = _workspace(OP_ROUTE_ENTMAX_BACKWARD, shape, 0, Q.device, ws)
    _check(lib.bsa_route_entmax_backward(ctypes.byref(shape), _ptr(Q), _ptr(S), _ptr(probs),
                                         _ptr(idx), _ptr(cnt), idx.shape[-1], _ptr(dwsel), alpha,
                                         gamma, score_scale, _ptr(dQ), _ptr(dK),
                                         _dtype_code(dQ), _ptr(wsb), nws, _stream(Q)))
    return dQ, dK


class _SparseAttention(torch.autograd.Function):
    """attend_prefill with attend_backward as its gradient; the selection is
    an input without gradient, the routing weights wsel (prior) get dL/dw."""

    @staticmethod
    def forward(ctx, Q, K, V, wsel, B, idx, cnt, sm_scale, sigma, token):
        O, L = attend_prefill(Q, K, V, B, idx, cnt, sm_scale, token=token, wsel=wsel,
                              sigma=sigma, want_lse=True)
        ctx.save_for_backward(Q, K, V, O, L, idx, cnt, wsel)
        ctx.B, ctx.sm_scale, ctx.sigma, ctx.token = B, sm_scale, sigma, token
        return O

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, O, L, idx, cnt, wsel = ctx.saved_tensors
        want_dw = wsel is not None and ctx.needs_input_grad[3]
        g = attend_backward(Q, K, V, O, dO, L, ctx.B, idx, cnt, ctx.sm_scale, wsel=wsel,
                            sigma=ctx.sigma, want_dwsel=want_dw, token=ctx.token)
        dw = g[3] if want_dw else None
        return g[0], g[1], g[2], dw, None, None, None, None, None, None


def sparse_attention(Q, K, V, B, idx, cnt, sm_scale=0.0, wsel=None, sigma=0.0, token=False):
    """Differentiable causal block-sparse attention over a fixed selection
    (block rows, or per-token selections with token=True); with routing
    weights wsel (shaped like idx) the prior-induced softmax, whose weights
    receive dL/dw when they require grad."""
    return _SparseAttention.apply(Q, K, V, wsel, B, idx, cnt, sm_scale, sigma, token)


def attend_entmax(Q, K, V, alpha, refine=2, sm_scale=0.0, out_dtype=None, out=None,
                  want_tau=False, want_live=False):
    """Causal token-level alpha-entmax attention (bf16 Q [b, Hq, N, d],
    K/V [b, Hkv, N, d]).  Returns O, (O, tau) with want_tau, and the live
    key tiles [b, Hkv, T, ceil(T/32)] uint32 (T = ceil(N/64)) appended with
    want_live."""
    b, hq, n, d = Q.shape
    hkv = K.shape[1]
    odt = out_dtype or Q.dtype
    O = out if out is not None else torch.empty((b, hq, n, d), dtype=odt, device=Q.device)
    tau = torch.empty((b, hq, n), dtype=torch.float32, device=Q.device) if want_tau else None
    nt = (n + 63) // 64
    live = (torch.empty((b, hkv, nt, (nt + 31) // 32), dtype=torch.int32, device=Q.device)
            if want_live else None)
    shape = make_shape(batch=b, hq=hq, hkv=hkv, d=d, B=64, dtype=_dtype_code(Q),
                       mode=PREFILL, q_len=n, kv_len=K.shape[2], q=Q, k=K, v=V, o=O)
    _check(lib.bsa_attend_entmax(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), alpha, refine,
                                 sm_scale, _ptr(O), _dtype_code(O), _ptr(tau), _ptr(live),
                                 _stream(Q)))
    res = (O,) + ((tau,) if want_tau else ()) + ((live,) if want_live else ())
    return res if len(res) > 1 else O


def attend_entmax_backward(Q, K, V, dO, tau, alpha, sm_scale=0.0, grad_dtype=None, ws=None,
                           live=None):
    """Gradients (dQ, dK, dV) of attend_entmax's output for upstream dO, given
    the forward's tau (want_tau=True) and, optionally, its live key tiles
    (want_live=True), which the backward then walks alone.  Gradients take
    the strides of Q, K, V."""
    b, hq, n, d = Q.shape
    gdt = grad_dtype or Q.dtype
    dQ = torch.empty_strided(Q.size(), Q.stride(), dtype=gdt, device=Q.device)
    dK = torch.empty_strided(K.size(), K.stride(), dtype=gdt, device=K.device)
    dV = torch.empty_strided(V.size(), V.stride(), dtype=gdt, device=V.device)
    if dO.dtype != Q.dtype:
        dO = dO.to(Q.dtype)
    shape = make_shape(batch=b, hq=hq, hkv=K.shape[1], d=d, B=64, dtype=_dtype_code(Q),
                       mode=PREFILL, q_len=n, kv_len=K.shape[2], q=Q, k=K, v=V, o=dO)
    wsb, nws = _workspace(OP_ATTEND_ENTMAX_BACKWARD, shape, 0, Q.device, ws)
    _check(lib.bsa_attend_entmax_backward(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V),
                                          _ptr(dO), _ptr(tau), _ptr(live), alpha, sm_scale,
                                          _ptr(dQ),
                                          _ptr(dK), _ptr(dV), _dtype_code(dQ), _ptr(wsb), nws,
                                          _stream(Q)))
    return dQ, dK, dV


def token_mask(idx, cnt, B, kv_len=None, out=None):
    """Per-token selections idx [b, Hkv, N, width] / cnt [b, Hkv, N] -> the
    active blocks of every 64-query tile: (uidx [b, Hkv, T, nblk] int32,
    ucnt [b, Hkv, T] int32, ubits [b, Hkv, T, nblk] int64 holding the 64-bit
    token words), T = ceil(N / 64), nblk = ceil(kv_len / B)."""
    b, hkv, n, width = idx.shape
    kv_len = n if kv_len is None else kv_len
    nblk = (kv_len + B - 1) // B
    ntile = (n + 63) // 64
    if out is not None:
        uidx, ucnt, ubits = out
    else:
        uidx = torch.empty((b, hkv, ntile, nblk), dtype=torch.int32, device=idx.device)
        ucnt = torch.empty((b, hkv, ntile), dtype=torch.int32, device=idx.device)
        ubits = torch.empty((b, hkv, ntile, nblk), dtype=torch.int64, device=idx.device)
    shape = make_shape(batch=b, hq=hkv, hkv=hkv, d=64, B=B, dtype=F32, mode=TOKEN, q_len=n,
                       kv_len=kv_len)
    _check(lib.bsa_token_mask(ctypes.byref(shape), _ptr(idx), _ptr(cnt), width, _ptr(uidx),
                              _ptr(ucnt), _ptr(ubits), _stream(idx)))
    return uidx, ucnt, ubits


def attend_decode(q, K, V, B, idx, cnt, kv_lens=None, sm_scale=0.0, out_dtype=None, out=None):
    """One query token per sequence.  q [b, Hq, 1, d], K/V caches [b, Hkv, L, d]."""
    b, hq, _, d = q.shape
    hkv, L = K.shape[1], K.shape[2]
    odt = out_dtype or q.dtype
    O = out if out is not None else torch.empty((b, hq, 1, d), dtype=odt, device=q.device)
    shape = make_shape(batch=b, hq=hq, hkv=hkv, d=d, B=B, dtype=_dtype_code(q), mode=DECODE,
                       q_len=1, kv_len=L, q=q, k=K, v=V, o=O)
    _check(lib.bsa_attend_decode(ctypes.byref(shape), _ptr(q), _ptr(K), _ptr(V), _ptr(kv_lens),
                                 _ptr(idx), _ptr(cnt), idx.shape[-1], sm_scale, _ptr(O),
                                 _dtype_code(O), None, 0, _stream(q)))
    return O


def decode_step(q, K, V, S, B, k_total, force=FORCE_TAIL, kv_lens=None, score_scale=0.0,
                sm_scale=0.0, out_dtype=None, out=None, want_selection=True, sel=None, ws=None):
    """Top-k routing over cached summaries and decode attention in one launch.
    Returns (O, idx, cnt) (idx, cnt are None when want_selection is False)."""
    b, hq, _, d = q.shape
    hkv, L = K.shape[1], K.shape[2]
    odt = out_dtype or q.dtype
    O = out if out is not None else torch.empty((b, hq, 1, d), dtype=odt, device=q.device)
    if sel is not None:
        idx, cnt = sel
    elif want_selection:
        idx = torch.empty((b, hkv, 1, k_total), dtype=torch.int32, device=q.device)
        cnt = torch.empty((b, hkv, 1), dtype=torch.int32, device=q.device)
    else:
        idx = cnt = None
    shape = make_shape(batch=b, hq=hq, hkv=hkv, d=d, B=B, dtype=_dtype_code(q), mode=DECODE,
                       q_len=1, kv_len=L, q=q, k=K, v=V, o=O)
    wsb, n = _workspace(OP_DECODE_TOPK, shape, k_total, q.device, ws)
    _check(lib.bsa_decode_topk(ctypes.byref(shape), _ptr(q), _ptr(K), _ptr(V), _ptr(S),
                               _ptr(kv_lens), k_total, force, score_scale, sm_scale, _ptr(idx),
                               _ptr(cnt), _ptr(O), _dtype_code(O), _ptr(wsb), n, _stream(q)))
    return O, idx, cnt


def decode_step_noalloc(q, K, V, S, B, k_total, force=FORCE_TAIL, kv_lens=None,
                        score_scale=0.0, sm_scale=0.0, out_dtype=None, out=None, sel=None):
    """decode_step through bsa_decode_topk_noalloc: no workspace; the
    library's static per-GPU scratch is used instead (calls overlapping on
    one GPU race).  Returns (O, idx, cnt)."""
    b, hq, _, d = q.shape
    hkv, L = K.shape[1], K.shape[2]
    odt = out_dtype or q.dtype
    O = out if out is not None else torch.empty((b, hq, 1, d), dtype=odt, device=q.device)
    if sel is not None:
        idx, cnt = sel
    else:
        idx = torch.empty((b, hkv, 1, k_total), dtype=torch.int32, device=q.device)
        cnt = torch.empty((b, hkv, 1), dtype=torch.int32, device=q.device)
    shape = make_shape(batch=b, hq=hq, hkv=hkv, d=d, B=B, dtype=_dtype_code(q), mode=DECODE,
                       q_len=1, kv_len=L, q=q, k=K, v=V, o=O)
    _check(lib.bsa_decode_topk_noalloc(ctypes.byref(shape), _ptr(q), _ptr(K), _ptr(V), _ptr(S),
                                       _ptr(kv_lens), k_total, force, score_scale, sm_scale,
                                       _ptr(idx), _ptr(cnt), _ptr(O), _dtype_code(O),
                                       _stream(q)))
    return O, idx, cnt


def make_pages(table, Kp, Vp):
    """Page description of a pool Kp / Vp [num_pages, Hkv, B, d] addressed by
    table int32 [batch, max_pages] (device)."""
    pg = Pages()
    pg.table = table.data_ptr()
    pg.max_pages = int(table.shape[1])
    pg.num_pages = int(min(Kp.shape[0], Vp.shape[0]))
    pg.k_page_stride = int(Kp.stride(0))
    pg.v_page_stride = int(Vp.stride(0))
    return pg


def _paged_shape(q, Kp, Vp, B, kv_len, O=None):
    b, hq, _, d = q.shape
    s = make_shape(batch=b, hq=hq, hkv=Kp.shape[1], d=d, B=B, dtype=_dtype_code(q), mode=DECODE,
                   q_len=1, kv_len=kv_len, q=q, o=O)
    s.k_stride[:] = (0, int(Kp.stride(1)), int(Kp.stride(2)))
    s.v_stride[:] = (0, int(Vp.stride(1)), int(Vp.stride(2)))
    return s


def decode_step_paged(q, Kp, Vp, table, S, B, k_total, force=FORCE_TAIL, kv_lens=None,
                      kv_len=None, score_scale=0.0, sm_scale=0.0, out_dtype=None, out=None,
                      want_selection=True, ws=None):
    """decode_step over a paged cache: Kp / Vp [num_pages, Hkv, B, d], logical
    block j of sequence b in page table[b, j].  kv_len: the logical capacity
    (default table.shape[1] * B).  Returns (O, idx, cnt)."""
    b, hq, _, d = q.shape
    hkv = Kp.shape[1]
    kv_len = table.shape[1] * B if kv_len is None else kv_len
    odt = out_dtype or q.dtype
    O = out if out is not None else torch.empty((b, hq, 1, d), dtype=odt, device=q.device)
    if want_selection:
        idx = torch.empty((b, hkv, 1, k_total), dtype=torch.int32, device=q.device)
        cnt = torch.empty((b, hkv, 1), dtype=torch.int32, device=q.device)
    else:
        idx = cnt = None
    shape = _paged_shape(q, Kp, Vp, B, kv_len, O)
    pg = make_pages(table, Kp, Vp)
    wsb, n = _workspace(OP_DECODE_TOPK, shape, k_total, q.device, ws)
    _check(lib.bsa_decode_topk_paged(ctypes.byref(shape), ctypes.byref(pg), _ptr(q), _ptr(Kp),
                                     _ptr(Vp), _ptr(S), _ptr(kv_lens), k_total, force, score_scale,
                                     sm_scale, _ptr(idx), _ptr(cnt), _ptr(O), _dtype_code(O),
                                     _ptr(wsb), n, _stream(q)))
    return O, idx, cnt


def summarize_blocks_paged(Kp, table, B, blk, S, kv_len=None, qbar=None):
    """summarize_blocks over a paged key pool Kp [num_pages, Hkv, B, d]."""
    hkv, d = Kp.shape[1], Kp.shape[3]
    b = table.shape[0]
    kv_len = table.shape[1] * B if kv_len is None else kv_len
    shape = make_shape(batch=b, hq=hkv, hkv=hkv, d=d, B=B, dtype=_dtype_code(Kp), mode=DECODE,
                       q_len=1, kv_len=kv_len)
    shape.k_stride[:] = (0, int(Kp.stride(1)), int(Kp.stride(2)))
    pg = make_pages(table, Kp, Kp)
    if qbar is not None:
        qbar = qbar.contiguous().to(torch.float32)
    _check(lib.bsa_summarize_blocks_paged(ctypes.byref(shape), ctypes.byref(pg), _ptr(Kp),
                                          _ptr(qbar), _ptr(blk), _ptr(S), _stream(Kp)))
    return S


def decode_workspace(q, K, B, k_total):
    """A workspace for decode_step on these shapes (reusable across steps)."""
    b, hq, _, d = q.shape
    shape = make_shape(batch=b, hq=hq, hkv=K.shape[1], d=d, B=B, dtype=_dtype_code(q),
                       mode=DECODE, q_len=1, kv_len=K.shape[2], q=q, k=K, v=K, o=q)
    return torch.empty(max(workspace_size(OP_DECODE_TOPK, shape, k_total), 1), dtype=torch.uint8,
                       device=q.device)


def prefill_topk(Q, K, V, B, k_total, force=0, S=None, out_dtype=None):
    """Stage 0 + top-k routing + fine attention for causal prefill."""
    S = summarize(K, B) if S is None else S
    idx, cnt = route_topk(Q, S, B, k_total, force)
    return attend_prefill(Q, K, V, B, idx, cnt, out_dtype=out_dtype), idx, cnt


def _wsel_like(Q, S, B, cap, force, token, sigma):
    if sigma is None:
        return None
    b, hkv, nblk = Q.shape[0], S.shape[1], S.shape[2]
    nrow = Q.shape[2] if token else (Q.shape[2] + B - 1) // B
    width = cap + bin(force & 7).count("1")
    return torch.empty((b, hkv, nrow, width), dtype=torch.float32, device=Q.device)


def prefill_entmax(Q, K, V, B, alpha, gamma, cap, force=FORCE_DIAG, max_iter=8, S=None,
                   out_dtype=None, sigma=None):
    """Stage 0 + alpha-entmax routing + fine attention for causal prefill;
    sigma (not None): prior-induced softmax with the routing weights."""
    S = summarize(K, B) if S is None else S
    wsel = _wsel_like(Q, S, B, cap, force, False, sigma)
    idx, cnt, _, _ = route_entmax(Q, S, B, alpha, gamma, cap, force, max_iter=max_iter, wsel=wsel)
    O = attend_prefill(Q, K, V, B, idx, cnt, out_dtype=out_dtype, wsel=wsel,
                       sigma=sigma or 0.0)
    return O, idx, cnt


def prefill_token_topk(Q, K, V, B, k_total, force=FORCE_DIAG, S=None, out_dtype=None):
    """Stage 0 + per-token top-k routing + masked fine attention."""
    S = summarize(K, B) if S is None else S
    idx, cnt = route_topk(Q, S, B, k_total, force, token=True)
    return attend_prefill(Q, K, V, B, idx, cnt, out_dtype=out_dtype, token=True), idx, cnt


def prefill_token_entmax(Q, K, V, B, alpha, gamma, cap, force=FORCE_DIAG, max_iter=8, S=None,
                         out_dtype=None, sigma=None):
    """Stage 0 + per-token alpha-entmax routing + masked fine attention;
    sigma (not None): prior-induced softmax with the routing weights."""
    S = summarize(K, B) if S is None else S
    wsel = _wsel_like(Q, S, B, cap, force, True, sigma)
    idx, cnt, _, _ = route_entmax(Q, S, B, alpha, gamma, cap, force, max_iter=max_iter, token=True,
                                  wsel=wsel)
    O = attend_prefill(Q, K, V, B, idx, cnt, out_dtype=out_dtype, token=True, wsel=wsel,
                       sigma=sigma or 0.0)
    return O, idx, cnt


def decode_topk(q, K, V, S, B, k_total, force=FORCE_TAIL, kv_lens=None, out_dtype=None):
    """Top-k routing over cached summaries + decode attention (two calls)."""
    idx, cnt = route_topk(q, S, B, k_total, force, decode=True, kv_len=K.shape[2], kv_lens=kv_lens)
    return attend_decode(q, K, V, B, idx, cnt, kv_lens=kv_lens, out_dtype=out_dtype), idx, cnt
