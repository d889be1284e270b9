"""Seeded synthetic inputs for R-SWA decode and prefill workloads.

This module draws random numbers and rounds them to the storage precision. It holds no attention
arithmetic: the oracle side (tests, CPU baseline) and the GPU side (tests, bench) both take their
inputs from here and share nothing else.

Shapes follow the Unlimited-OCR pages: a "Base"-mode page is 256 visual tokens (GeekNews
"Unlimited OCR", DeepEncoder section), pages are joined with one <page> delimiter token each
(deep dive, multi-page input passage), the default output window is n = 128 (both pages, R-SWA
section), and teacher-forced sequences are packed to 32K tokens (GeekNews, training section).
A 16-token prompt, 16 heads and head_dim 128 are this library's choice; the pages do not state them.

Recipe (per sequence b of workload `cfg`):
  rng = numpy.random.default_rng(SeedSequence([seed, cfg, b]))
  decode:  prefix K (m,H,D), prefix V (m,H,D), output K (T,H,D), output V (T,H,D), output Q (T,H,D)
  prefill: Q (S,H,D), K (S,H,D), V (S,H,D)
  output gradient of a prefill workload: default_rng(SeedSequence([seed, cfg, 1000 + b])) draws
    dO (S,H,D) the same way
  each drawn as standard_normal float32, in that order; then, if outliers are on, for each array in
  the same order a Bernoulli(p) set of positions is drawn as geometric gaps and those entries are
  multiplied by 8. Finally bf16 workloads round every value to nearest-even bf16.
Per-workload metadata (page counts, lengths, windows of the ragged workload and of the packed
  training sequence) comes from default_rng(SeedSequence([seed, cfg])).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

NUM_HEADS = 16
HEAD_DIM = 128
TOKENS_PER_PAGE = 256
PROMPT_TOKENS = 16


# --------------------------------------------------------------------------------------------
# bf16 storage rounding (input preparation only)
# --------------------------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of stored input values ("bf16" bit patterns or "f32" floats)."""
    if dtype == "bf16":
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _apply_outliers(rng: np.random.Generator, arr: np.ndarray, p: float, factor: float) -> None:
    """Multiply a Bernoulli(p) subset of entries by `factor`, positions drawn as geometric gaps."""
    flat = arr.reshape(-1)
    n = flat.size
    pos = -1
    chunk = max(1024, int(n * p * 1.2) + 64)
    while True:
        gaps = rng.geometric(p, size=chunk)
        idx = pos + np.cumsum(gaps)
        keep = idx[idx < n]
        flat[keep] *= np.float32(factor)
        if keep.size < idx.size:
            return
        pos = int(idx[-1])


def _draw(rng: np.random.Generator, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    rng.standard_normal(out=out, dtype=np.float32)
    return out


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else x


# --------------------------------------------------------------------------------------------
# decode workloads
# --------------------------------------------------------------------------------------------
@dataclass
class DecodeWorkload:
    """Inputs for a batch of decode trajectories.

    prefix_k / prefix_v: packed [sum_b m_b][H][D] (token-major), sequence b at rows
      prefix_offset[b] .. prefix_offset[b] + m_b.
    q / k / v: [T][B][H][D]; entry [t-1, b] is the query / new key / new value of output t of
      sequence b (1-based t). Entries with t > steps[b] are zero and never used.
    Values are bf16 bit patterns (uint16) when dtype == "bf16", float32 when dtype == "f32".
    """
    name: str
    cfg: int
    dtype: str
    prefix_len: np.ndarray
    window: np.ndarray
    steps: np.ndarray
    prefix_k: np.ndarray
    prefix_v: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.prefix_len.size)

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def prefix_offset(self) -> np.ndarray:
        off = np.zeros(self.batch + 1, dtype=np.int64)
        np.cumsum(self.prefix_len, out=off[1:])
        return off

    def active(self, t: int) -> np.ndarray:
        """uint8 [B]: 1 where sequence b appends / decodes output t (1-based)."""
        return (self.steps >= t).astype(np.uint8)

    def prefix(self, b: int):
        o = self.prefix_offset
        return self.prefix_k[o[b]:o[b + 1]], self.prefix_v[o[b]:o[b + 1]]


def _decode_sequence(seed, cfg, b, m, T, T_alloc, dtype, outlier_p):
    rng = np.random.default_rng(np.random.SeedSequence([seed, cfg, b]))
    H, D = NUM_HEADS, HEAD_DIM
    arrs = [_draw(rng, (m, H, D)), _draw(rng, (m, H, D)),
            _draw(rng, (T, H, D)), _draw(rng, (T, H, D)), _draw(rng, (T, H, D))]
    if outlier_p:
        for a in arrs:
            _apply_outliers(rng, a, outlier_p, 8.0)
    return [_store(a, dtype) for a in arrs]


def make_decode(name: str, cfg: int, dtype: str, prefix_len, window, steps, seed: int = 0,
                outlier_p: float = 0.0, meta: dict | None = None) -> DecodeWorkload:
    prefix_len = np.asarray(prefix_len, dtype=np.int32)
    window = np.asarray(window, dtype=np.int32)
    steps = np.asarray(steps, dtype=np.int32)
    B = prefix_len.size
    T = int(steps.max()) if B else 0
    H, D = NUM_HEADS, HEAD_DIM
    sdt = np.uint16 if dtype == "bf16" else np.float32
    total_m = int(prefix_len.sum())
    pk = np.empty((total_m, H, D), dtype=sdt)
    pv = np.empty((total_m, H, D), dtype=sdt)
    q = np.zeros((T, B, H, D), dtype=sdt)
    k = np.zeros((T, B, H, D), dtype=sdt)
    v = np.zeros((T, B, H, D), dtype=sdt)
    off = np.zeros(B + 1, dtype=np.int64)
    np.cumsum(prefix_len, out=off[1:])

    def job(b):
        a = _decode_sequence(seed, cfg, b, int(prefix_len[b]), int(steps[b]), T, dtype, outlier_p)
        pk[off[b]:off[b + 1]] = a[0]
        pv[off[b]:off[b + 1]] = a[1]
        Tb = int(steps[b])
        k[:Tb, b] = a[2]
        v[:Tb, b] = a[3]
        q[:Tb, b] = a[4]

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(job, range(B)))
    return DecodeWorkload(name, cfg, dtype, prefix_len, window, steps, pk, pv, q, k, v,
                          dict(meta or {}, seed=seed, outlier_p=outlier_p))


def decode_config(cfg: int, seed: int = 0, *, batch: int | None = None, T: int | None = None,
                  prefix_len: int | None = None, window: int | None = None) -> DecodeWorkload:
    """The decode workloads at their stated sizes; keyword overrides give scaled-down copies
    (same recipe, smaller batch / length) for quick parity runs."""
    if cfg == 1:
        B, m, n, TT, dt, p = 1, TOKENS_PER_PAGE + PROMPT_TOKENS, 128, 512, "f32", 0.0
        name = "single-page R-SWA decode, B=1, fp32, m=272, n=128, T=512"
    elif cfg == 2:
        B, m, n, TT, dt, p = 64, TOKENS_PER_PAGE + PROMPT_TOKENS, 128, 6000, "bf16", 0.01
        name = "single-page batched R-SWA decode, B=64, bf16 + 1% x8 outliers, m=272, n=128, T=6000"
    elif cfg == 3:
        pages = 20
        B, m, n, TT, dt, p = 8, pages * TOKENS_PER_PAGE + (pages - 1) + PROMPT_TOKENS, 128, 20000, \
            "bf16", 0.0
        name = "multi-page R-SWA decode, B=8, 20 pages, m=5155, n=128, T=20000, bf16"
    elif cfg == 5:
        return varlen_config(seed, batch=batch, T_max=T)
    else:
        raise ValueError(f"no decode workload {cfg}")
    B = batch if batch is not None else B
    m = prefix_len if prefix_len is not None else m
    n = window if window is not None else n
    TT = T if T is not None else TT
    return make_decode(name, cfg, dt, [m] * B, [n] * B, [TT] * B, seed=seed, outlier_p=p,
                       meta=dict(pages=None))


def varlen_config(seed: int = 0, *, batch: int | None = None, T_max: int | None = None,
                  max_pages: int = 50) -> DecodeWorkload:
    """Ragged batch: page counts uniform in 1..50 (m = 256 pages + 16), output lengths
    log-uniform in [256, 12000], window drawn per sequence from {64, 128, 256, 512}."""
    B = 32 if batch is None else batch
    rng = np.random.default_rng(np.random.SeedSequence([seed, 5]))
    pages = rng.integers(1, max_pages + 1, size=32)
    Tb = np.rint(np.exp(rng.uniform(math.log(256.0), math.log(12000.0), size=32))).astype(np.int64)
    n = rng.choice(np.array([64, 128, 256, 512]), size=32)
    pages, Tb, n = pages[:B], Tb[:B], n[:B]
    if T_max is not None:  # scaled-down copy: keep the spread, cap the length
        Tb = np.minimum(Tb, T_max)
    m = pages * TOKENS_PER_PAGE + PROMPT_TOKENS
    name = "ragged R-SWA decode, B=32, pages U{1..50}, T log-uniform 256..12000, n in {64..512}"
    return make_decode(name, 5, "bf16", m, n, Tb, seed=seed, meta=dict(pages=pages.tolist()))


# --------------------------------------------------------------------------------------------
# prefill (teacher-forced) workloads
# --------------------------------------------------------------------------------------------
@dataclass
class PrefillWorkload:
    """Packed sequences: q / k / v are [sum S_b][H][D]; sequence b owns rows
    cu_seqlens[b] .. cu_seqlens[b+1], its first m_b rows being the prefix."""
    name: str
    dtype: str
    cu_seqlens: np.ndarray
    prefix_len: np.ndarray
    window: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    prefix_causal: bool = False

    @property
    def nseq(self) -> int:
        return int(self.prefix_len.size)

    def seq(self, b: int):
        s, e = int(self.cu_seqlens[b]), int(self.cu_seqlens[b + 1])
        return self.q[s:e], self.k[s:e], self.v[s:e]


def make_prefill(name: str, cfg: int, seqlens, prefix_len, window, seed: int = 0,
                 prefix_causal: bool = False) -> PrefillWorkload:
    seqlens = np.asarray(seqlens, dtype=np.int64)
    nseq = seqlens.size
    cu = np.zeros(nseq + 1, dtype=np.int32)
    np.cumsum(seqlens, out=cu[1:])
    total = int(cu[-1])
    H, D = NUM_HEADS, HEAD_DIM
    q = np.empty((total, H, D), dtype=np.uint16)
    k = np.empty((total, H, D), dtype=np.uint16)
    v = np.empty((total, H, D), dtype=np.uint16)

    def job(b):
        rng = np.random.default_rng(np.random.SeedSequence([seed, cfg, b]))
        S = int(seqlens[b])
        s0 = int(cu[b])
        for dst in (q, k, v):
            dst[s0:s0 + S] = bf16_bits(_draw(rng, (S, H, D)))

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(job, range(nseq)))
    return PrefillWorkload(name, "bf16", cu, np.asarray(prefix_len, dtype=np.int32),
                           np.asarray(window, dtype=np.int32), q, k, v, prefix_causal)


def prefill_config(seed: int = 0, *, S: int | None = None, prefix_len: int | None = None,
                   window: int | None = None, prefix_causal: bool = False) -> PrefillWorkload:
    """One packed 32768-token sequence: a 40-page prefix (m = 40*256 + 16 = 10256) visible in
    both directions, then 22512 output tokens under the causal window n = 128."""
    S = 32768 if S is None else S
    m = 40 * TOKENS_PER_PAGE + PROMPT_TOKENS if prefix_len is None else prefix_len
    n = 128 if window is None else window
    name = "R-SWA masked prefill, S=32768, m=10256 (40 pages), n=128, bf16"
    return make_prefill(name, 4, [S], [m], [n], seed=seed, prefix_causal=prefix_causal)


def make_output_grad(wl: PrefillWorkload, seed: int = 0, cfg: int = 6) -> np.ndarray:
    """Seeded bf16 output gradient dO [total][H][D] for a prefill workload (standard normal)."""
    total = int(wl.cu_seqlens[-1])
    H, D = NUM_HEADS, HEAD_DIM
    g = np.empty((total, H, D), dtype=np.uint16)

    def job(b):
        rng = np.random.default_rng(np.random.SeedSequence([seed, cfg, 1000 + b]))
        s0, s1 = int(wl.cu_seqlens[b]), int(wl.cu_seqlens[b + 1])
        g[s0:s1] = bf16_bits(_draw(rng, (s1 - s0, H, D)))

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(job, range(wl.nseq)))
    return g


def packed_training_config(seed: int = 0, *, S: int = 32768, window: int = 128,
                           out_per_page=(300, 700)) -> PrefillWorkload:
    """One training row of S tokens packed with prefix + output documents (GeekNews "Unlimited
    OCR", training section: single-page to multi-page documents 9:1, multi-page ones of 2 to 50
    pages, packed to 32K). Documents are drawn until S is filled: 1 page with probability 0.9,
    else a uniform page count in [2, 50]; prefix m = 256 pages + 16 prompt tokens; output length
    pages x uniform integer in out_per_page (this library's choice: the pages give no per-page
    output length). The last document is cut to fit S (its prefix too, if need be)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7]))
    lens, ms = [], []
    left = S
    while left > 0:
        pages = 1 if rng.random() < 0.9 else int(rng.integers(2, 51))
        m = pages * TOKENS_PER_PAGE + PROMPT_TOKENS
        outs = int(sum(rng.integers(out_per_page[0], out_per_page[1] + 1, size=pages)))
        L = min(m + outs, left)
        lens.append(L)
        ms.append(min(m, L))
        left -= L
    name = f"packed training row, S={S}, {len(lens)} documents, n={window}, bf16"
    return make_prefill(name, 7, lens, ms, [window] * len(lens), seed=seed)


# --------------------------------------------------------------------------------------------
# shared prefixes in a token pool (paged prefix KV)
# --------------------------------------------------------------------------------------------
@dataclass
class PagedPrefix:
    """Every document's prefix stored once in a token pool, and each sequence's page table.

    pool_k / pool_v: [pool_rows][H][D] (token-major); table: int32 [sum_b m_b], sequence b's
    prefix token j at pool row table[M_b + j], M_b = sum of the earlier m_b'; doc_of_seq[b] is the
    document sequence b decodes over."""
    pool_k: np.ndarray
    pool_v: np.ndarray
    table: np.ndarray
    doc_of_seq: np.ndarray


def make_paged_decode(name: str, cfg: int, dtype: str, doc_prefix_len, seq_doc, window, steps,
                      seed: int = 0, scatter: bool = True, spare_rows: int = 0):
    """Decode trajectories of several sequences per document. Document d's prefix K, V are drawn
    from SeedSequence([seed, cfg, 5000 + d]); sequence b's output K, V, Q from
    SeedSequence([seed, cfg, b]) as in make_decode (no prefix draws). The pool holds the documents
    back to back plus `spare_rows` unused rows; with `scatter` every token's pool row is a seeded
    permutation (SeedSequence([seed, cfg])) of that order, i.e. token-granular pages in no
    particular order. Returns (DecodeWorkload whose prefix_k / prefix_v are the gathered
    per-sequence prefixes, PagedPrefix)."""
    doc_m = np.asarray(doc_prefix_len, dtype=np.int64)
    seq_doc = np.asarray(seq_doc, dtype=np.int64)
    window = np.asarray(window, dtype=np.int32)
    steps = np.asarray(steps, dtype=np.int32)
    H, D = NUM_HEADS, HEAD_DIM
    sdt = np.uint16 if dtype == "bf16" else np.float32
    doc_off = np.zeros(doc_m.size + 1, dtype=np.int64)
    np.cumsum(doc_m, out=doc_off[1:])
    rows = int(doc_off[-1]) + spare_rows
    flat_k = np.empty((rows, H, D), dtype=sdt)
    flat_v = np.empty((rows, H, D), dtype=sdt)

    def doc_job(d):
        rng = np.random.default_rng(np.random.SeedSequence([seed, cfg, 5000 + d]))
        m = int(doc_m[d])
        flat_k[doc_off[d]:doc_off[d + 1]] = _store(_draw(rng, (m, H, D)), dtype)
        flat_v[doc_off[d]:doc_off[d + 1]] = _store(_draw(rng, (m, H, D)), dtype)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(doc_job, range(doc_m.size)))
    if spare_rows:
        rng = np.random.default_rng(np.random.SeedSequence([seed, cfg, 4999]))
        flat_k[doc_off[-1]:] = _store(_draw(rng, (spare_rows, H, D)), dtype)
        flat_v[doc_off[-1]:] = _store(_draw(rng, (spare_rows, H, D)), dtype)
    if scatter:
        slot = np.random.default_rng(np.random.SeedSequence([seed, cfg])).permutation(rows)
    else:
        slot = np.arange(rows)
    pool_k = np.empty_like(flat_k)
    pool_v = np.empty_like(flat_v)
    pool_k[slot] = flat_k
    pool_v[slot] = flat_v
    prefix_len = doc_m[seq_doc].astype(np.int32)
    table = np.concatenate([slot[doc_off[d]:doc_off[d + 1]] for d in seq_doc]).astype(np.int32) \
        if seq_doc.size else np.zeros(0, dtype=np.int32)
    wl = make_decode(name, cfg, dtype, np.zeros_like(prefix_len), window, steps, seed=seed)
    wl.prefix_len = prefix_len
    wl.prefix_k = pool_k[table]
    wl.prefix_v = pool_v[table]
    wl.meta["documents"] = int(doc_m.size)
    return wl, PagedPrefix(pool_k, pool_v, table, seq_doc)


def shared_document_config(seed: int = 0, *, docs: int = 4, per_doc: int = 16, pages: int = 20,
                           T: int = 2048) -> tuple:
    """Shared-document decode: `docs` documents of `pages` pages (m = 256 pages + pages - 1 + 16),
    `per_doc` sequences decoding over each (B = docs x per_doc), n = 128, bf16, token-granular
    pool in scattered order."""
    m = pages * TOKENS_PER_PAGE + (pages - 1) + PROMPT_TOKENS
    B = docs * per_doc
    name = (f"shared-document R-SWA decode, {docs} documents x {per_doc} sequences (B={B}), "
            f"{pages} pages (m={m}), n=128, T={T}, bf16, token-granular prefix pool")
    return make_paged_decode(name, 8, "bf16", [m] * docs, np.repeat(np.arange(docs), per_doc),
                             [128] * B, [T] * B, seed=seed, scatter=True)
