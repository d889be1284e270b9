"""Plain CPU fp64 oracle for Reference Sliding Window Attention (R-SWA).

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import, call or execute anything in this package. It imports nothing from windowed_attention_amd
and the HIP library imports nothing from here; the two sides share only the seeded inputs of the
`workloads` module.

What R-SWA computes, as the pages state it:
  * Output token t attends to the set N(t) = P u D_n(t): the whole prefix P of L_m = m tokens
    (visual tokens plus prompt, always visible) and the previous n output tokens (default n = 128).
    [deep dive "Unlimited-OCR", the N(t) code block; GeekNews "Unlimited OCR", R-SWA section]
  * The KV cache behaves as a queue of capacity m + n: each new token evicts the oldest output KV,
    so the cache holds C(T) = L_m + min(n, T) <= L_m + n rows, while standard causal attention
    holds L_m + T. [deep dive, N(t) code block; GeekNews, "KV cache management" and
    "model architecture" sections]
  * The prefix is encoded once and never changes during decoding. [GeekNews, DeepEncoder section]

Readings taken where the pages are silent or garbled:
  R1  the n-token window includes the current output token (self), so the latest query sees
      exactly the L_m + min(n, t) rows the cache holds;
  R2  "evict the (m+1)-th" means the element at 1-based queue position m + 1, i.e. the oldest
      output, removed once the queue holds more than m + n rows;
  R3  in the teacher-forced (prefill) pass the prefix is visible in both directions to prefix
      queries (flag `prefix_causal` gives the causal alternative);
  R4  prefix queries never see output tokens;
  R5  the softmax scale is 1/sqrt(d) unless given;
  R6  inputs arrive already position-encoded; there is no position arithmetic here.

Everything here is the plain definition of masked softmax attention in float64: a growing cache
that never evicts plus an explicit visibility mask. There is no blocking beyond query blocks that
keep the prefill mask small, no fusion and no reordering. `queue_decode` is an independent second
formulation (a literal Python-list queue) and `brute_*` are scalar loops for tiny shapes.
"""
from __future__ import annotations

import math

import numpy as np

RSWA = "rswa"
FULL = "full"


def default_scale(d: int) -> float:
    """Scaled dot-product attention scale 1/sqrt(d) (reading R5)."""
    return 1.0 / math.sqrt(d)


# ------------------------------------------------------------------------------------------
# cache sizes (closed forms stated on both pages)
# ------------------------------------------------------------------------------------------
def rswa_cache_rows(m: int, n: int, t: int) -> int:
    """C_R-SWA(t) = L_m + min(n, t). [deep dive, N(t) block; GeekNews, KV cache management]"""
    return m + min(n, t)


def full_cache_rows(m: int, t: int) -> int:
    """Standard causal attention keeps every row: L_m + t. [GeekNews, KV cache management]"""
    return m + t


def cache_ratio(m: int, n: int, t: int) -> float:
    """rho(t) = C_R-SWA(t) / C_full(t); tends to 0 as t grows. [GeekNews, KV cache management]"""
    return rswa_cache_rows(m, n, t) / full_cache_rows(m, t)


# ------------------------------------------------------------------------------------------
# visibility masks
# ------------------------------------------------------------------------------------------
def decode_visible(m: int, n: int, t: int, mode: str = RSWA) -> np.ndarray:
    """Boolean mask over the growing cache rows [0, m + t) for output t (1-based).

    Row j < m is prefix (always visible). Row j >= m holds output index i = j - m (0-based), i.e.
    output token i + 1. R-SWA keeps the last n outputs, the current one included (R1):
    visible iff j < m or i >= t - n. Full causal: every row is visible.
    """
    j = np.arange(m + t)
    if mode == FULL:
        return np.ones(m + t, dtype=bool)
    return (j < m) | (j >= m + t - n)


def prefill_visible(p, k, m: int, n: int, prefix_causal: bool = False):
    """Visibility of key position k to query position p in one packed prefix+output sequence.

    prefix key (k < m): visible to every query, except that with `prefix_causal` a prefix query
      p < m sees only k <= p (R3);
    output key (k >= m): visible only to output queries p with k <= p and p - k < n, i.e. the
      query's own window of n outputs (R1, R4).
    Works elementwise on broadcastable integer arrays.
    """
    p = np.asarray(p)
    k = np.asarray(k)
    pre = k < m
    if prefix_causal:
        pre = pre & (k <= p)
    out = (k >= m) & (k <= p) & (p - k < n)
    return pre | out


# ------------------------------------------------------------------------------------------
# attention over an explicit row set
# ------------------------------------------------------------------------------------------
def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V for one head: q [d], K [L, d], V [L, d], all float64, L >= 1."""
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    return (w @ V) / w.sum()


def decode_step(q, prefix_k, prefix_v, out_k, out_v, t: int, n: int, mode: str = RSWA,
                scale: float | None = None):
    """Attention output of output token t (1-based) for every head, and the visible-row count.

    q [H, d]; prefix_k / prefix_v [m, H, d]; out_k / out_v [>= t, H, d] with row i holding the
    key / value appended with output token i + 1. The cache is the naive growing one (prefix
    followed by every appended output, never evicted); R-SWA is applied by the explicit mask.
    """
    q = np.asarray(q, dtype=np.float64)
    H, d = q.shape
    m = prefix_k.shape[0]
    if m + t == 0:
        raise ValueError("empty key set: m = 0 and t = 0")
    scale = default_scale(d) if scale is None else scale
    K_all = np.concatenate([np.asarray(prefix_k, np.float64), np.asarray(out_k[:t], np.float64)])
    V_all = np.concatenate([np.asarray(prefix_v, np.float64), np.asarray(out_v[:t], np.float64)])
    vis = decode_visible(m, n, t, mode)
    o = np.empty((H, d), dtype=np.float64)
    for h in range(H):
        o[h] = attend(q[h], K_all[vis, h], V_all[vis, h], scale)
    return o, int(vis.sum())


def prefill(Q, K, V, m: int, n: int, prefix_causal: bool = False, scale: float | None = None,
            rows=None, block: int = 512) -> np.ndarray:
    """Masked attention of one packed sequence, Q/K/V [S, H, d] -> O [S, H, d] (float64).

    `rows` (optional) selects the query positions to compute; the result then has one row per
    selected position. Queries are processed in blocks of `block` so that the S x S mask is never
    materialised; within a block it is the plain masked softmax of `prefill_visible`.
    """
    Q = np.asarray(Q)
    S, H, d = Q.shape
    scale = default_scale(d) if scale is None else scale
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    Kf = np.asarray(K, dtype=np.float64)
    Vf = np.asarray(V, dtype=np.float64)
    out = np.empty((rows.size, H, d), dtype=np.float64)
    keys = np.arange(S)
    for s in range(0, rows.size, block):
        p = rows[s:s + block]
        vis = prefill_visible(p[:, None], keys[None, :], m, n, prefix_causal)
        kmax = int(np.nonzero(vis.any(axis=0))[0].max()) + 1
        vis = vis[:, :kmax]
        Qb = np.asarray(Q[p], dtype=np.float64)
        for h in range(H):
            z = scale * (Qb[:, h, :] @ Kf[:kmax, h, :].T)
            z = np.where(vis, z, -np.inf)
            w = np.exp(z - z.max(axis=1, keepdims=True))
            out[s:s + p.size, h, :] = (w @ Vf[:kmax, h, :]) / w.sum(axis=1, keepdims=True)
    return out


# ------------------------------------------------------------------------------------------
# literal-queue formulation (independent of the mask)
# ------------------------------------------------------------------------------------------
def queue_decode(q_seq, prefix_k, prefix_v, out_k, out_v, n: int, T: int,
                 scale: float | None = None):
    """Decode T steps with the cache held as a literal queue of capacity m + n.

    The queue starts as the prefix rows. Each step appends the new (k, v); when the queue then
    holds more than m + n rows the element at 0-based index m (1-based position m + 1, the oldest
    output, reading R2) is deleted. The query attends to every row in the queue.
    Returns (outputs [T, H, d], queue lengths [T], queue contents as output indices per step).
    """
    m = prefix_k.shape[0]
    H, d = np.asarray(q_seq[0]).shape
    scale = default_scale(d) if scale is None else scale
    queue = [("prefix", j, np.asarray(prefix_k[j], np.float64), np.asarray(prefix_v[j], np.float64))
             for j in range(m)]
    outs, lens, members = [], [], []
    for t in range(1, T + 1):
        queue.append(("out", t - 1, np.asarray(out_k[t - 1], np.float64),
                      np.asarray(out_v[t - 1], np.float64)))
        if len(queue) > m + n:
            del queue[m]
        Kq = np.stack([e[2] for e in queue])
        Vq = np.stack([e[3] for e in queue])
        qt = np.asarray(q_seq[t - 1], np.float64)
        o = np.empty((H, d))
        for h in range(H):
            o[h] = attend(qt[h], Kq[:, h, :], Vq[:, h, :], scale)
        outs.append(o)
        lens.append(len(queue))
        members.append(sorted(e[1] for e in queue if e[0] == "out"))
    return np.stack(outs) if outs else np.zeros((0, H, d)), lens, members


# ------------------------------------------------------------------------------------------
# ring realisation of the queue (what the GPU cache stores; checked bit-exactly)
# ------------------------------------------------------------------------------------------
def ring_row(m: int, n: int, j: int) -> int:
    """Cache row of output index j (0-based) in an n-slot ring placed after the m prefix rows."""
    return m + j % n


def ring_occupants(n: int, t: int) -> np.ndarray:
    """After t appends, slot s (0..n-1) holds the largest output index j < t with j % n == s,
    or -1 if no output has reached it yet (the slot still holds whatever was there before)."""
    occ = np.full(n, -1, dtype=np.int64)
    for j in range(t):
        occ[j % n] = j
    return occ


def full_row(m: int, j: int) -> int:
    """Full-causal cache row of output index j: the cache simply grows."""
    return m + j


# ------------------------------------------------------------------------------------------
# scalar brute force (tiny shapes only)
# ------------------------------------------------------------------------------------------
def brute_decode(q, prefix_k, prefix_v, out_k, out_v, t: int, n: int, mode: str = RSWA,
                 scale: float | None = None):
    """Scalar-loop decode of output t: enumerate the rows the step may see, then a textbook
    two-pass softmax with math.exp. Only for tiny shapes."""
    m = len(prefix_k)
    H = len(q)
    d = len(q[0])
    scale = default_scale(d) if scale is None else scale
    rows = []
    for j in range(m):
        rows.append((prefix_k[j], prefix_v[j]))
    first = 0 if mode == FULL else max(0, t - n)
    for i in range(first, t):
        rows.append((out_k[i], out_v[i]))
    o = [[0.0] * d for _ in range(H)]
    for h in range(H):
        zs = []
        for kr, _ in rows:
            acc = 0.0
            for c in range(d):
                acc += float(q[h][c]) * float(kr[h][c])
            zs.append(scale * acc)
        zmax = max(zs)
        ws = [math.exp(z - zmax) for z in zs]
        tot = sum(ws)
        for c in range(d):
            o[h][c] = sum(w * float(vr[h][c]) for w, (_, vr) in zip(ws, rows)) / tot
    return o, len(rows)


def brute_prefill(Q, K, V, m: int, n: int, prefix_causal: bool = False,
                  scale: float | None = None):
    """Scalar-loop prefill: each query enumerates its own key list from the stated rules
    (prefix keys, then the window of outputs ending at itself)."""
    S = len(Q)
    H = len(Q[0])
    d = len(Q[0][0])
    scale = default_scale(d) if scale is None else scale
    O = [[[0.0] * d for _ in range(H)] for _ in range(S)]
    for p in range(S):
        if p < m:
            keys = list(range(p + 1)) if prefix_causal else list(range(m))
        else:
            keys = list(range(m)) + list(range(max(m, p - n + 1), p + 1))
        for h in range(H):
            zs = []
            for k in keys:
                acc = 0.0
                for c in range(d):
                    acc += float(Q[p][h][c]) * float(K[k][h][c])
                zs.append(scale * acc)
            zmax = max(zs)
            ws = [math.exp(z - zmax) for z in zs]
            tot = sum(ws)
            for c in range(d):
                O[p][h][c] = sum(w * float(V[k][h][c]) for w, k in zip(ws, keys)) / tot
    return O


# ------------------------------------------------------------------------------------------
# teacher-forced training pass: log-sum-exp and gradients of the masked prefill
# ------------------------------------------------------------------------------------------
# The pages train the R-SWA decoder on packed 32K sequences with the encoder frozen [GeekNews,
# training section; deep dive, training setup table]. They print no backward formula; what
# follows is the chain rule applied to the masked softmax attention above, in float64:
#   Z = scale * Q K^T (invisible pairs -inf),  P = softmax_rows(Z),  O = P V,  L = sum(dO * O)
#   dV = P^T dO,  dP = dO V^T,  dZ = softmax_grad(P, dP),  dQ = scale dZ K,  dK = scale dZ^T Q.
def softmax_grad(P: np.ndarray, dP: np.ndarray) -> np.ndarray:
    """Back-propagate dP through P = softmax(Z) taken along the last axis: the Jacobian
    diag(P) - P P^T applied to dP, i.e. P * (dP - sum_j P_j dP_j)."""
    return P * (dP - (P * dP).sum(axis=-1, keepdims=True))


def prefill_lse(Q, K, m: int, n: int, prefix_causal: bool = False, scale: float | None = None,
                rows=None, block: int = 512) -> np.ndarray:
    """Natural-log log-sum-exp of each selected query's visible scaled scores, [rows, H] float64:
    lse_p = log sum_{k visible} exp(scale q_p . k_k) (max-shifted before the exp)."""
    Q = np.asarray(Q)
    S, H, d = Q.shape
    scale = default_scale(d) if scale is None else scale
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    Kf = np.asarray(K, dtype=np.float64)
    keys = np.arange(S)
    out = np.empty((rows.size, H), dtype=np.float64)
    for s in range(0, rows.size, block):
        p = rows[s:s + block]
        vis = prefill_visible(p[:, None], keys[None, :], m, n, prefix_causal)
        kmax = int(np.nonzero(vis.any(axis=0))[0].max()) + 1
        vis = vis[:, :kmax]
        Qb = np.asarray(Q[p], dtype=np.float64)
        for h in range(H):
            z = np.where(vis, scale * (Qb[:, h, :] @ Kf[:kmax, h, :].T), -np.inf)
            zmax = z.max(axis=1)
            out[s:s + p.size, h] = zmax + np.log(np.exp(z - zmax[:, None]).sum(axis=1))
    return out


def prefill_backward(Q, K, V, dO, m: int, n: int, prefix_causal: bool = False,
                     scale: float | None = None, heads=None, q_rows=None, k_rows=None,
                     block: int = 512):
    """Gradients of L = sum(dO * prefill(Q, K, V)) for one packed sequence (float64).

    Q, K, V, dO: [S, H, d]. Returns (dQ [q_rows, heads, d], dK [k_rows, heads, d],
    dV [k_rows, heads, d]) for the selected heads / query rows / key rows (default: all).
    Every query contributes to the key gradients; the sums over queries run in query blocks of
    `block` rows (an order of summation only), each block forming its scores, probabilities and
    probability gradients in full before the chain-rule products.
    """
    Q = np.asarray(Q)
    S, H, d = Q.shape
    scale = default_scale(d) if scale is None else scale
    heads = list(range(H)) if heads is None else list(heads)
    q_rows = np.arange(S) if q_rows is None else np.asarray(q_rows, dtype=np.int64)
    k_rows = np.arange(S) if k_rows is None else np.asarray(k_rows, dtype=np.int64)
    q_pos = {int(p): i for i, p in enumerate(q_rows)}
    Kf = np.asarray(K, dtype=np.float64)
    Vf = np.asarray(V, dtype=np.float64)
    dQ = np.zeros((q_rows.size, len(heads), d))
    dK = np.zeros((k_rows.size, len(heads), d))
    dV = np.zeros((k_rows.size, len(heads), d))
    keys = np.arange(S)
    for s in range(0, S, block):
        p = np.arange(s, min(S, s + block))
        vis = prefill_visible(p[:, None], keys[None, :], m, n, prefix_causal)
        kmax = int(np.nonzero(vis.any(axis=0))[0].max()) + 1
        vis = vis[:, :kmax]
        kin = k_rows[k_rows < kmax]
        kidx = np.nonzero(k_rows < kmax)[0]
        sel = [i for i, pp in enumerate(p) if int(pp) in q_pos]
        Qb = np.asarray(Q[p], dtype=np.float64)
        dOb = np.asarray(dO[p], dtype=np.float64)
        for hi, h in enumerate(heads):
            z = np.where(vis, scale * (Qb[:, h, :] @ Kf[:kmax, h, :].T), -np.inf)
            w = np.exp(z - z.max(axis=1, keepdims=True))
            P = w / w.sum(axis=1, keepdims=True)
            dP = dOb[:, h, :] @ Vf[:kmax, h, :].T
            dZ = softmax_grad(P, dP)
            if sel:
                rows_out = [q_pos[int(p[i])] for i in sel]
                dQ[rows_out, hi, :] = scale * (dZ[sel] @ Kf[:kmax, h, :])
            dK[kidx, hi, :] += scale * (dZ[:, kin].T @ Qb[:, h, :])
            dV[kidx, hi, :] += P[:, kin].T @ dOb[:, h, :]
    return dQ, dK, dV


# ------------------------------------------------------------------------------------------
# prefixes held once in a shared token pool (paged prefix KV)
# ------------------------------------------------------------------------------------------
def paged_prefix(pool, table, start: int, m: int) -> np.ndarray:
    """Prefix rows of one sequence whose prefix lives in a token pool: prefix token j is pool row
    table[start + j] (a page table with one token per page, the page size of the SGLang server
    that infer.py launches [deep dive, the SGLang launch flags]; several sequences may share rows).
    The attention over
    them is unchanged: `decode_step` with these rows as the prefix."""
    idx = np.asarray(table[start:start + m], dtype=np.int64)
    return np.asarray(pool)[idx]
