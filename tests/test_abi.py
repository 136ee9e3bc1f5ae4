"""The C-ABI library loads, exports every entry point declared in
include/bsa.h, and rejects malformed arguments on the host before any HIP
call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
bsa = pytest.importorskip("block_sparse_attention_summarize_amd")
lib = bsa.lib

FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(os.path.join(ROOT, "include", "bsa.h")).read()
    return sorted(set(re.findall(r"\b(bsa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(bsa.EXPORTS) == set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version():
    assert "gfx950" in bsa.version()


def shape(**kw):
    base = dict(batch=1, hq=4, hkv=2, d=128, B=64, dtype=bsa.BF16, mode=bsa.PREFILL, q_len=256,
                kv_len=256)
    base.update(kw)
    s = bsa.make_shape(**base)
    st = (base["hq"] * base["kv_len"] * base["d"], base["kv_len"] * base["d"], base["d"])
    for f in ("q_stride", "k_stride", "v_stride", "o_stride"):
        getattr(s, f)[:] = st
    return s


def err():
    return lib.bsa_last_error().decode()


def topk(s, k=4, force=0, ws_bytes=None, Q=FAKE, S=FAKE, idx=FAKE, cnt=FAKE, scale=0.0):
    n = lib.bsa_workspace_size(bsa.OP_ROUTE_TOPK, ctypes.byref(s), k) if ws_bytes is None else ws_bytes
    return lib.bsa_route_topk(ctypes.byref(s), Q, S, None, k, force, scale, idx, cnt, None,
                              ctypes.c_void_p(0x200000), n, None)


def entmax(s, alpha=1.5, n_bins=16, max_iter=8, cap=64, force=1):
    n = lib.bsa_workspace_size(bsa.OP_ROUTE_ENTMAX, ctypes.byref(s), cap)
    return lib.bsa_route_entmax(ctypes.byref(s), FAKE, FAKE, None, alpha, 1.0, n_bins, max_iter,
                                cap, force, 0.0, FAKE, FAKE, None, None, None,
                                ctypes.c_void_p(0x200000), n, None)


def prefill(s, k_max=4, o_dtype=None, Q=FAKE, O=FAKE, sm_scale=0.0, wsel=None, sigma=0.0):
    return lib.bsa_attend_prefill(ctypes.byref(s), Q, FAKE, FAKE, FAKE, FAKE, k_max, sm_scale,
                                  wsel, sigma, O, s.dtype if o_dtype is None else o_dtype, None,
                                  None, 0, None)


def test_shape_validation():
    assert lib.bsa_summarize(None, FAKE, None, FAKE, None) == -1
    assert "NULL" in err()
    assert lib.bsa_summarize_blocks(ctypes.byref(shape()), FAKE, None, None, FAKE, None) == -1
    assert "blk" in err()
    assert topk(shape(hq=3, hkv=2)) == -1 and "multiple" in err()
    assert topk(shape(batch=0)) == -1
    assert topk(shape(d=96)) == -2 and "head_dim" in err()
    assert topk(shape(B=32)) == -2 and "block" in err()
    assert topk(shape(dtype=7)) == -2
    assert topk(shape(mode=3)) == -1
    assert topk(shape(q_len=128)) == -1 and "q_len == kv_len" in err()
    assert topk(shape(mode=bsa.DECODE, q_len=2)) == -1 and "q_len == 1" in err()
    s = shape()
    s.reserved = 1
    assert topk(s) == -1
    s = shape()
    s.q_stride[2] = 100  # not a multiple of 8 bf16 elements
    assert topk(s) == -2 and "stride" in err()
    s = shape()
    s.q_stride[0] = -8
    assert topk(s) == -1


def test_pointer_validation():
    assert topk(shape(), Q=None) == -1 and "Q is NULL" in err()
    assert topk(shape(), Q=ctypes.c_void_p(0x100002)) == -2 and "aligned" in err()
    assert topk(shape(), idx=None) == -1
    assert prefill(shape(), O=None) == -1


def test_route_topk_validation():
    assert topk(shape(), k=0) == -1
    assert topk(shape(), k=1, force=bsa.FORCE_DIAG | bsa.FORCE_FIRST) == -1 and "forced" in err()
    assert topk(shape(), force=bsa.FORCE_TAIL) == -1 and "decode" in err()
    assert topk(shape(), force=8) == -1
    assert topk(shape(), scale=float("nan")) == -1
    assert topk(shape(), ws_bytes=16) == -4 and "workspace" in err()


def test_route_entmax_validation():
    assert entmax(shape(), alpha=1.0) == -1 and "alpha" in err()
    assert entmax(shape(), alpha=0.5) == -1
    assert entmax(shape(), n_bins=8) == -1 and "n_bins" in err()
    assert entmax(shape(), max_iter=-1) == -1
    assert entmax(shape(), max_iter=33) == -1
    assert entmax(shape(), cap=0) == -1


def test_attend_validation():
    assert prefill(shape(), k_max=0) == -1
    assert prefill(shape(), o_dtype=5) == -2
    assert prefill(shape(), sm_scale=-0.1) == -1 and "sm_scale" in err()
    assert prefill(shape(), wsel=FAKE, sigma=float("inf")) == -1 and "sigma" in err()
    assert prefill(shape(), wsel=ctypes.c_void_p(0x100004), sigma=1.0) == -2
    assert prefill(shape(mode=bsa.DECODE, q_len=1)) == -1 and "PREFILL" in err()
    s = shape(mode=bsa.DECODE, q_len=1, hq=9, hkv=1)  # 9 heads per KV head: no even split
    assert lib.bsa_attend_decode(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, FAKE, 4, 0.0, FAKE,
                                 bsa.BF16, None, 0, None) == -2 and "8 heads" in err()
    s = shape(mode=bsa.DECODE, q_len=1, kv_len=64 * 40000)  # scores of a row exceed the LDS
    assert lib.bsa_attend_decode(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, FAKE, 4, 0.0, FAKE,
                                 bsa.BF16, None, 0, None) == -2 and "LDS" in err()
    s = shape(mode=bsa.DECODE, q_len=1)
    assert lib.bsa_attend_decode(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, FAKE, 4, 0.0, FAKE,
                                 bsa.BF16, None, 0, None) == -1
    assert lib.bsa_decode_topk(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, 4, bsa.FORCE_TAIL,
                               0.0, 0.0, FAKE, None, FAKE, bsa.BF16, FAKE, 1 << 20,
                               None) == -1 and "both" in err()
    assert lib.bsa_decode_topk(ctypes.byref(shape()), FAKE, FAKE, FAKE, FAKE, None, 4, 0,
                               0.0, 0.0, None, None, FAKE, bsa.BF16, FAKE, 1 << 20,
                               None) == -1 and "DECODE" in err()
    assert lib.bsa_decode_topk(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, 4, bsa.FORCE_TAIL,
                               0.0, 0.0, None, None, FAKE, bsa.BF16, FAKE, 16,
                               None) == -4 and "workspace" in err()


def test_workspace_sizes():
    s = shape(batch=2, hq=8, hkv=2, d=128, B=64, q_len=1000, kv_len=1000)
    nrow = nblk = 16
    rows = 2 * 2 * nrow
    al = lambda x: (x + 255) // 256 * 256
    assert lib.bsa_workspace_size(bsa.OP_ROUTE_TOPK, ctypes.byref(s), 4) == al(rows * 128 * 4) + al(rows * nblk * 4)
    hrows = 2 * 8 * nrow
    assert lib.bsa_workspace_size(bsa.OP_ROUTE_ENTMAX, ctypes.byref(s), 8) == al(hrows * 128 * 4) + al(hrows * nblk * 4)
    assert lib.bsa_workspace_size(bsa.OP_ATTEND_PREFILL, ctypes.byref(s), 4) == 0
    assert lib.bsa_workspace_size(bsa.OP_SUMMARIZE, ctypes.byref(s), 4) == 0
    assert lib.bsa_workspace_size(bsa.OP_ROUTE_TOPK, None, 4) == 0
    d = shape(batch=16, hq=32, hkv=8, mode=bsa.DECODE, q_len=1, kv_len=131072)
    # decode attention runs in one launch without scratch
    assert lib.bsa_workspace_size(bsa.OP_ATTEND_DECODE, ctypes.byref(d), 33) == 0
    # 128 rows: one fused launch, no scratch
    assert lib.bsa_workspace_size(bsa.OP_DECODE_TOPK, ctypes.byref(d), 33) == 0
    # 4 x 8 rows: 8 workgroups per row; candidates (keys + ids) and partial
    # states for 4 heads
    d = shape(batch=4, hq=32, hkv=8, mode=bsa.DECODE, q_len=1, kv_len=131072)
    rows, parts, G = 4 * 8, 8, 4
    want = 2 * al(rows * parts * 33 * 4) + al(rows * parts * G * 130 * 4)
    assert lib.bsa_workspace_size(bsa.OP_DECODE_TOPK, ctypes.byref(d), 33) == want


def test_error_string_is_thread_local_and_cleared():
    import threading
    assert topk(shape(), k=0) == -1
    msgs = []
    t = threading.Thread(target=lambda: msgs.append(err()))
    t.start()
    t.join()
    assert msgs == [""]
    assert err() != ""


def test_token_mode_validation_and_workspace():
    al = lambda x: (x + 255) // 256 * 256
    s = shape(batch=2, hq=8, hkv=2, d=128, B=64, mode=bsa.TOKEN, q_len=1000, kv_len=1000)
    nblk, ntile = 16, 16
    rows = 2 * 2 * 1000  # one routing row per token
    assert lib.bsa_workspace_size(bsa.OP_ROUTE_TOPK, ctypes.byref(s), 4) == \
        al(rows * 128 * 4) + al(rows * nblk * 4)
    hrows = 2 * 8 * 1000
    assert lib.bsa_workspace_size(bsa.OP_ROUTE_ENTMAX, ctypes.byref(s), 8) == \
        al(hrows * 128 * 4) + al(hrows * nblk * 4)
    trows = 2 * 2 * ntile  # 64-query tiles: active ids, token words, counts
    need = al(trows * nblk * 4) + al(trows * nblk * 8) + al(trows * 4)
    assert lib.bsa_workspace_size(bsa.OP_ATTEND_PREFILL, ctypes.byref(s), 4) == need
    assert topk(s, force=bsa.FORCE_TAIL) == -1 and "decode" in err()
    assert topk(shape(mode=bsa.TOKEN, q_len=128)) == -1 and "q_len == kv_len" in err()
    # the tile masks need their workspace
    assert lib.bsa_attend_prefill(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.0, None,
                                  0.0, FAKE, bsa.BF16, None, ctypes.c_void_p(0x200000),
                                  need - 1, None) == -4
    # with routing weights the tiles' per-query bias is added
    prior = lib.bsa_workspace_size(bsa.OP_ATTEND_PREFILL_PRIOR, ctypes.byref(s), 4)
    assert prior == need + al(trows * nblk * 64 * 4)
    assert lib.bsa_attend_prefill(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.0, FAKE,
                                  1.0, FAKE, bsa.BF16, None, ctypes.c_void_p(0x200000),
                                  prior - 1, None) == -4
    mask = lambda sh, idx=FAKE, width=4: lib.bsa_token_mask(ctypes.byref(sh), idx, FAKE, width,
                                                             FAKE, FAKE, FAKE, None)
    assert mask(shape()) == -1 and "BSA_TOKEN" in err()
    assert mask(s, idx=None) == -1
    assert mask(s, width=0) == -1
    big = shape(hq=2, hkv=2, mode=bsa.TOKEN, q_len=64 * 4097, kv_len=64 * 4097)
    assert mask(big) == -2 and "4096" in err()


def test_paged_validation():
    s = shape(batch=2, hq=8, hkv=2, mode=bsa.DECODE, q_len=1, kv_len=64 * 10)
    s.k_stride[:] = (0, 64 * 128, 128)
    s.v_stride[:] = (0, 64 * 128, 128)
    pg = bsa.Pages()
    pg.table, pg.max_pages, pg.num_pages = 0x300000, 10, 40
    pg.k_page_stride = pg.v_page_stride = 2 * 64 * 128

    def step(p, ws=1 << 20):
        return lib.bsa_decode_topk_paged(ctypes.byref(s), p, FAKE, FAKE, FAKE, FAKE, None, 4,
                                         bsa.FORCE_TAIL, 0.0, 0.0, None, None, FAKE, bsa.BF16,
                                         ctypes.c_void_p(0x200000), ws, None)
    assert step(None) == -1 and "pages" in err()
    pg.max_pages = 9
    assert step(ctypes.byref(pg)) == -1 and "max_pages" in err()
    pg.max_pages, pg.num_pages = 10, 0
    assert step(ctypes.byref(pg)) == -1 and "num_pages" in err()
    pg.num_pages, pg.k_page_stride = 40, 2 * 64 * 128 + 4
    assert step(ctypes.byref(pg)) == -2 and "multiples" in err()
    pg.k_page_stride = 2 * 64 * 128
    tbl = pg.table
    pg.table = None
    assert lib.bsa_summarize_blocks_paged(ctypes.byref(s), ctypes.byref(pg), FAKE, None, FAKE,
                                          FAKE, None) == -1 and "table" in err()
    pg.table = tbl
    assert lib.bsa_summarize_blocks_paged(ctypes.byref(s), ctypes.byref(pg), FAKE, None, None,
                                          FAKE, None) == -1 and "blk" in err()


def backward(s, k_max=4, o_dtype=None, g_dtype=None, lse=FAKE, dO=FAKE, ws_bytes=None,
             sm_scale=0.0, wsel=None, sigma=0.0, dwsel=None):
    n = (lib.bsa_workspace_size(bsa.OP_ATTEND_BACKWARD, ctypes.byref(s), k_max)
         if ws_bytes is None else ws_bytes)
    return lib.bsa_attend_backward(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE,
                                   s.dtype if o_dtype is None else o_dtype, dO, lse, FAKE, FAKE,
                                   k_max, sm_scale, wsel, sigma, dwsel, FAKE, FAKE, FAKE,
                                   s.dtype if g_dtype is None else g_dtype,
                                   ctypes.c_void_p(0x200000), n, None)


def route_backward(s, width=6, alpha=1.5, ws_bytes=None, dwsel=FAKE, g_dtype=None):
    n = (lib.bsa_workspace_size(bsa.OP_ROUTE_ENTMAX_BACKWARD, ctypes.byref(s), 0)
         if ws_bytes is None else ws_bytes)
    return lib.bsa_route_entmax_backward(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, width,
                                         dwsel, alpha, 1.0, 0.0, FAKE, FAKE,
                                         s.dtype if g_dtype is None else g_dtype,
                                         ctypes.c_void_p(0x200000), n, None)


def test_backward_validation_and_workspace():
    s = shape(q_len=64 * 10 + 5, kv_len=64 * 10 + 5)  # 11 query and key blocks
    need = lib.bsa_workspace_size(bsa.OP_ATTEND_BACKWARD, ctypes.byref(s), 4)
    al = lambda x: (x + 255) // 256 * 256
    nrow = nblk = 11
    per = 4 * 5 // 2 + (nrow - 4) * 4  # (row, block <= row) pairs of one KV head, k = 4
    E = 2 * per
    items = 2 * nblk + -(-E // 32)
    red = min(2 * nblk, E // 33 + 1)
    slots = E // 32 + red + 1
    units = 2 * (64 // 32)  # query heads per KV head x 32-query sub-tiles of a block
    assert need == (al(4 * 645 * 4) + al(2 * 1 * nblk * 4) + al(items * 16) + al(red * 16) + al(8)
                    + al(slots * 2 * 64 * 128 * 4) + al(2 * nrow * units * 4 * 4))
    assert backward(s, ws_bytes=need - 1) == -4
    assert backward(shape(mode=bsa.DECODE, q_len=1)) == -1 and "BSA_TOKEN" in err()
    assert backward(shape(dtype=bsa.F32)) == -2 and "bf16" in err()
    assert backward(s, lse=None) == -1 and "lse" in err()
    assert backward(s, dO=None) == -1 and "dO" in err()
    assert backward(s, g_dtype=7) == -2 and "g_dtype" in err()
    assert backward(s, sm_scale=-1.0) == -1
    assert backward(s, lse=ctypes.c_void_p(0x100002)) == -2 and "aligned" in err()
    # more key blocks than the marking kernel holds in LDS
    big = shape(q_len=64 * 16385, kv_len=64 * 16385, hq=2, hkv=1)
    assert backward(big, ws_bytes=0) == -2 and "16384" in err()
    assert lib.bsa_workspace_size(bsa.OP_ATTEND_BACKWARD, ctypes.byref(shape(mode=bsa.DECODE)), 4) == 0
    # the prior's variant is the same size for block rows
    assert lib.bsa_workspace_size(bsa.OP_ATTEND_BACKWARD_PRIOR, ctypes.byref(s), 4) == need


def test_token_backward_workspace():
    # per-token selections: the rows are the 11 64-query tiles, each listing
    # up to all 11 blocks; the tile masks, the list positions and (with a
    # prior) the per-query bias and dS sums come on top
    s = shape(q_len=64 * 10 + 5, kv_len=64 * 10 + 5, mode=bsa.TOKEN)
    al = lambda x: (x + 255) // 256 * 256
    nrow = nblk = 11
    E = 2 * sum(min(nblk, r + 1) for r in range(nrow))
    items = 2 * nblk + -(-E // 32)
    red = min(2 * nblk, E // 33 + 1)
    slots = E // 32 + red + 1
    rl = 2 * nrow * nblk
    base = (al(4 * 645 * 4) + al(2 * 1 * nblk * 4) + al(items * 16) + al(red * 16) + al(8)
            + al(slots * 2 * 64 * 128 * 4) + al(rl * 4) + al(rl * 4) + al(rl * 8) + al(2 * nrow * 4))
    need = lib.bsa_workspace_size(bsa.OP_ATTEND_BACKWARD, ctypes.byref(s), 6)
    assert need == base
    prior = lib.bsa_workspace_size(bsa.OP_ATTEND_BACKWARD_PRIOR, ctypes.byref(s), 6)
    assert prior == base + al(rl * 64 * 4) + al(rl * 1 * 64 * 4)  # G = 2: one part
    assert backward(s, k_max=6, ws_bytes=need - 1) == -4
    assert backward(s, k_max=6, wsel=FAKE, ws_bytes=prior - 1) == -4
    # more blocks than the tile masks hold
    big = shape(q_len=64 * 4097, kv_len=64 * 4097, hq=2, hkv=1, mode=bsa.TOKEN)
    assert backward(big, ws_bytes=0) == -2 and "4096" in err()


def test_backward_prior_and_routing_backward_validation():
    s = shape()
    assert backward(s, dwsel=FAKE) == -1 and "dwsel needs wsel" in err()
    assert backward(s, wsel=FAKE, sigma=float("nan")) == -1 and "sigma" in err()
    assert backward(s, k_max=81, wsel=FAKE, dwsel=FAKE) == -2 and "80" in err()
    assert backward(s, wsel=ctypes.c_void_p(0x100002)) == -2 and "aligned" in err()
    need = lib.bsa_workspace_size(bsa.OP_ROUTE_ENTMAX_BACKWARD, ctypes.byref(s), 0)
    al = lambda x: (x + 255) // 256 * 256
    # q-hat, dz (4 rows x 4 blocks), dL/dq-hat and the heads' parts of dL/dS
    assert need == 3 * al(1 * 4 * 4 * 128 * 4) + al(1 * 4 * 4 * 4 * 4)
    assert route_backward(s, ws_bytes=need - 1) == -4
    assert route_backward(shape(mode=bsa.DECODE, q_len=1)) == -1 and "BSA_TOKEN" in err()
    # token rows: q-hat, dL/dq-hat and dz per (head, token); the heads' dS
    # parts per block
    t = shape(mode=bsa.TOKEN)
    tneed = lib.bsa_workspace_size(bsa.OP_ROUTE_ENTMAX_BACKWARD, ctypes.byref(t), 0)
    assert tneed == 2 * al(4 * 256 * 128 * 4) + al(4 * 256 * 4 * 4) + al(4 * 4 * 128 * 4)
    assert route_backward(t, ws_bytes=tneed - 1) == -4
    assert route_backward(s, alpha=1.0) == -1 and "alpha" in err()
    assert route_backward(s, dwsel=None) == -1 and "dwsel" in err()
    assert route_backward(s, width=0) == -1
    assert route_backward(s, g_dtype=5) == -2


def test_decode_noalloc_validation():
    """The allocation-free decode entry point validates on the host before it
    looks up its static scratch (no HIP call on these paths)."""
    def call(s, k=5, force=bsa.FORCE_TAIL, O=FAKE):
        return lib.bsa_decode_topk_noalloc(None if s is None else ctypes.byref(s), FAKE, FAKE,
                                           FAKE, FAKE, None, k, force, 0.0, 0.0, FAKE, FAKE, O,
                                           bsa.BF16, None)
    dec = dict(mode=bsa.DECODE, q_len=1, kv_len=4096)
    assert call(None) == -1 and "NULL" in err()
    assert call(shape()) == -1 and "BSA_DECODE" in err()
    assert call(shape(**dec), k=0) == -1 and "k_total" in err()
    assert call(shape(**dec), force=8) == -1
    assert call(shape(**dec), O=None) == -1


def test_entmax_attention_validation():
    """Token-level entmax attention and its backward: every argument is
    checked on the host before anything is enqueued."""
    s = shape(q_len=64 * 5 + 3, kv_len=64 * 5 + 3)

    def fwd(sh, alpha=1.5, refine=2, O=FAKE, tau=None, live=None):
        return lib.bsa_attend_entmax(ctypes.byref(sh), FAKE, FAKE, FAKE, alpha, refine, 0.0, O,
                                     sh.dtype, tau, live, None)

    def bwd(sh, alpha=1.5, tau=FAKE, live=None, ws_bytes=None):
        n = lib.bsa_workspace_size(bsa.OP_ATTEND_ENTMAX_BACKWARD, ctypes.byref(sh), 0)
        return lib.bsa_attend_entmax_backward(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, tau, live,
                                              alpha, 0.0, FAKE, FAKE, FAKE, sh.dtype,
                                              ctypes.c_void_p(0x200000),
                                              n if ws_bytes is None else ws_bytes, None)

    assert fwd(s, alpha=1.0) == -1 and "alpha" in err()
    assert fwd(s, alpha=17.0) == -2 and "alpha <= 16" in err()
    assert fwd(s, refine=25) == -1 and "refine" in err()
    assert fwd(s, O=None) == -1
    assert fwd(shape(dtype=bsa.F32)) == -2 and "bf16" in err()
    assert fwd(s, tau=ctypes.c_void_p(0x100004)) == -2 and "aligned" in err()
    big = shape(q_len=131072 + 64, kv_len=131072 + 64, hq=1, hkv=1)
    assert fwd(big) == -2 and "131072" in err()
    assert bwd(s, alpha=2.5) == -2
    assert bwd(s, tau=None) == -1 and "tau" in err()
    assert bwd(shape(q_len=320, kv_len=320, B=128)) == -2 and "block 64" in err()
    assert bwd(big) == -2 and "131072" in err()
    assert bwd(s, ws_bytes=0) == -4
