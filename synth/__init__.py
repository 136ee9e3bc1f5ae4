"""Seeded synthetic inputs for block-sparse attention, shared by the HIP-path
tests, the oracle tests and the benchmark.

This module holds workload shapes and random draws only -- none of the
method's arithmetic.  Recipe (stated once here, used everywhere):

* every tensor is cut into chunks of CHUNK tokens per (batch, head); chunk c of
  tensor stream s is drawn with ``numpy.random.default_rng(SeedSequence([seed,
  s, b, h, c])).standard_normal((rows, d), dtype=float32)``, so any slice can be
  regenerated without drawing the whole tensor; streams: q=0, k=1, v=2, u=3,
  planted key blocks=4, planted query positions=5, query-tile components=6,
  key-tile components=7, upstream gradients dO of the attention output=8
  (shaped like q, plain N(0, 1), nothing added);
* planting (the long-context retrieval structure): a unit vector
  u = g/|g|, g ~ N(0, I_d) (stream 3, fp64), a set of planted key blocks drawn
  without replacement (stream 4, identical for every KV head) whose keys get
  ``+ amp * u``, and round(frac * N) query positions (stream 5) whose queries get
  ``+ amp * u`` in every query head;
* query locality (loc_amp > 0): every tile of 64 consecutive query tokens
  shares a component c ~ N(0, I_d) per (batch, head, tile), drawn as stream 6
  with one row per tile, and its queries get ``+ loc_amp * c`` (before the
  planting), so nearby tokens route alike without routing identically;
* key locality (kloc_amp > 0): likewise every tile of 64 consecutive keys
  shares a component (stream 7, per (batch, KV head, tile)) added as
  kloc_amp * c; with query locality this gives scores a block structure (a
  query tile favours a few key tiles), as attention over real text has;
* query scale (q_scale != 1): queries are multiplied by q_scale after the
  locality component and before the planting, which sharpens the score
  distribution the way trained attention heads are sharper than random ones;
* bf16 tensors are the round-to-nearest-even bf16 of the fp32 values.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 4096
STREAM_Q, STREAM_K, STREAM_V, STREAM_U, STREAM_PK, STREAM_PQ, STREAM_QL, STREAM_KL, STREAM_DO = \
    0, 1, 2, 3, 4, 5, 6, 7, 8
QTILE = 64  # query tokens sharing one locality component

FORCE_DIAG = 1
FORCE_FIRST = 2
FORCE_TAIL = 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str  # "f32" or "bf16"
    batch: int
    hq: int
    hkv: int
    n: int  # prefill: sequence length N; decode: cache length L
    d: int
    B: int
    mode: str  # "prefill", "token" (prefill routed per query token) or "decode"
    router: str  # "topk", "entmax", or "entmax_attn" (token-level entmax attention, no routing)
    k_total: int = 0
    force: int = 0
    alpha: float = 1.5
    gamma: float = 1.0
    cap: int = 64
    n_bins: int = 16
    max_iter: int = 8
    seed: int = 0
    planted_blocks: int = 0
    planted_query_frac: float = 0.0
    amp: float = 3.0
    kv_lens: tuple = ()  # decode only; empty -> all equal to n
    loc_amp: float = 0.0  # query-tile component amplitude
    sigma: float = 0.0  # prior strength of the fine softmax (entmax routing); 0: plain softmax
    q_scale: float = 1.0  # queries multiplied by this (score temperature), before planting
    kloc_amp: float = 0.0  # key-tile component amplitude

    @property
    def nblk(self) -> int:
        return (self.n + self.B - 1) // self.B

    @property
    def q_len(self) -> int:
        return 1 if self.mode == "decode" else self.n

    @property
    def nrow(self) -> int:
        """Routing rows: query blocks (prefill), tokens (token), 1 (decode)."""
        return {"prefill": self.nblk, "token": self.n, "decode": 1}[self.mode]

    @property
    def idx_width(self) -> int:
        if self.router == "topk":
            return self.k_total
        return self.cap + bin(self.force & 7).count("1")

    def lens(self) -> np.ndarray:
        if self.mode != "decode":
            return np.full(self.batch, self.n, np.int64)
        if self.kv_lens:
            return np.asarray(self.kv_lens, np.int64)
        return np.full(self.batch, self.n, np.int64)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads of the method's hot path.
WORKLOADS = {
    "fp32_prefill_n1k": Workload(
        "fp32_prefill_n1k", "f32", 1, 2, 2, 1024, 64, 64, "prefill", "topk",
        k_total=4, force=FORCE_DIAG, seed=0),
    "bf16_gqa_prefill_n32k": Workload(
        "bf16_gqa_prefill_n32k", "bf16", 1, 32, 8, 32768, 128, 64, "prefill", "topk",
        k_total=16, force=0, seed=1, planted_blocks=32, planted_query_frac=0.01),
    "bf16_decode_l128k": Workload(
        "bf16_decode_l128k", "bf16", 16, 32, 8, 131072, 128, 64, "decode", "topk",
        k_total=33, force=FORCE_TAIL, seed=2),
    "entmax_prefill_n64k": Workload(
        "entmax_prefill_n64k", "bf16", 1, 32, 8, 65536, 128, 64, "prefill", "entmax",
        alpha=1.5, gamma=1.0, cap=64, n_bins=16, max_iter=8, force=FORCE_DIAG, seed=3,
        planted_blocks=32, planted_query_frac=0.01),
    "bf16_long_prefill_n256k": Workload(
        "bf16_long_prefill_n256k", "bf16", 1, 16, 2, 262144, 128, 128, "prefill", "topk",
        k_total=32, force=FORCE_DIAG | FORCE_FIRST, seed=4, planted_blocks=64,
        planted_query_frac=0.01),
    # every query token routed on its own (alpha-entmax per token), queries
    # with 64-token locality; attention over the active blocks of 64-query
    # tiles with the routing weights as the softmax prior (sigma = 1)
    "token_entmax_prefill_n32k": Workload(
        "token_entmax_prefill_n32k", "bf16", 1, 32, 8, 32768, 128, 64, "token", "entmax",
        alpha=1.5, gamma=4.0, cap=32, n_bins=16, max_iter=8, force=FORCE_DIAG, seed=5,
        planted_blocks=32, planted_query_frac=0.01, loc_amp=4.0, sigma=1.0),
    # token-level alpha-entmax attention (no block routing): dense causal with
    # zero key tiles skipped; block-structured scores (query and key tiles
    # with shared components), queries sharpened by 2
    "entmax_attn_prefill_n16k": Workload(
        "entmax_attn_prefill_n16k", "bf16", 1, 32, 8, 16384, 128, 64, "prefill", "entmax_attn",
        alpha=1.5, seed=6, q_scale=2.0, loc_amp=2.0, kloc_amp=2.0, planted_blocks=32,
        planted_query_frac=0.01),
}
WORKLOAD_ORDER = list(WORKLOADS)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _chunk(seed, stream, b, h, c, rows, d):
    rng = np.random.default_rng(np.random.SeedSequence([seed, stream, b, h, c]))
    return rng.standard_normal((rows, d), dtype=np.float32)


def planted_vector(w: Workload) -> np.ndarray:
    g = np.random.default_rng(np.random.SeedSequence([w.seed, STREAM_U])).standard_normal(w.d)
    return g / np.linalg.norm(g)


def planted_key_blocks(w: Workload) -> np.ndarray:
    if w.planted_blocks <= 0:
        return np.zeros(0, np.int64)
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, STREAM_PK]))
    return np.sort(rng.choice(w.nblk, size=min(w.planted_blocks, w.nblk), replace=False))


def planted_query_positions(w: Workload) -> np.ndarray:
    nq = int(round(w.planted_query_frac * w.q_len))
    if nq <= 0:
        return np.zeros(0, np.int64)
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, STREAM_PQ]))
    return np.sort(rng.choice(w.q_len, size=nq, replace=False))


def _fill(w: Workload, stream: int, heads: int, rows: int, t0: int, t1: int, b: int, h: int,
          out: np.ndarray):
    """Draw rows [t0, t1) of (b, h) for one tensor stream into out (fp32)."""
    c0, c1 = t0 // CHUNK, (t1 - 1) // CHUNK
    for c in range(c0, c1 + 1):
        r0 = c * CHUNK
        r1 = min(r0 + CHUNK, rows)
        blk = _chunk(w.seed, stream, b, h, c, r1 - r0, w.d)
        a, e = max(t0, r0), min(t1, r1)
        out[a - t0:e - t0] = blk[a - r0:e - r0]


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def gen(w: Workload, name: str, heads=None, t0: int = 0, t1=None, batches=None):
    """Draw tensor `name` in {"q","k","v","do"} as fp32 [len(batches), len(heads), t1-t0, d],
    with planting applied ("do": the upstream gradient of the output, shaped
    like q).  Defaults: every batch, head and row."""
    if name == "q":
        nh, rows, stream = w.hq, w.q_len, STREAM_Q
    elif name == "do":
        nh, rows, stream = w.hq, w.q_len, STREAM_DO
    elif name in ("k", "v"):
        nh, rows, stream = w.hkv, w.n, STREAM_K if name == "k" else STREAM_V
    else:
        raise ValueError(name)
    heads = list(range(nh)) if heads is None else list(heads)
    batches = list(range(w.batch)) if batches is None else list(batches)
    t1 = rows if t1 is None else t1
    out = np.empty((len(batches), len(heads), t1 - t0, w.d), np.float32)
    jobs = [(bi, b, hi, h) for bi, b in enumerate(batches) for hi, h in enumerate(heads)]

    def work(job):
        bi, b, hi, h = job
        _fill(w, stream, nh, rows, t0, t1, b, h, out[bi, hi])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, jobs))
    if name == "k" and w.planted_blocks > 0:
        u = planted_vector(w).astype(np.float32)
        for j in planted_key_blocks(w):
            a, e = max(t0, j * w.B), min(t1, (j + 1) * w.B)
            if a < e:
                out[:, :, a - t0:e - t0, :] += w.amp * u
    amp, lstream = (w.loc_amp, STREAM_QL) if name == "q" else (w.kloc_amp, STREAM_KL)
    if name in ("q", "k") and amp > 0 and w.mode != "decode":
        tiles = (rows + QTILE - 1) // QTILE
        a, e = t0 // QTILE, (t1 - 1) // QTILE + 1
        for bi, b in enumerate(batches):
            for hi, h in enumerate(heads):
                c = np.empty((e - a, w.d), np.float32)
                _fill(w, lstream, nh, tiles, a, e, b, h, c)
                tok = np.arange(t0, t1) // QTILE - a
                out[bi, hi] += np.float32(amp) * c[tok]
    if name == "q" and w.q_scale != 1.0:
        out *= np.float32(w.q_scale)
    if name == "q" and w.planted_query_frac > 0 and w.mode != "decode":
        u = planted_vector(w).astype(np.float32)
        pos = planted_query_positions(w)
        pos = pos[(pos >= t0) & (pos < t1)]
        if pos.size:
            out[:, :, pos - t0, :] += w.amp * u
    return out


def gen_stored(w: Workload, name: str, **kw):
    """Like gen(), but returns (stored, exact_f32): stored is what the device
    holds (fp32 array, or bf16 bit patterns as uint16), exact_f32 its exact
    fp32 value."""
    x = gen(w, name, **kw)
    if w.dtype == "f32":
        return x, x
    bits = f32_to_bf16_bits(x)
    return bits, bf16_bits_to_f32(bits)
