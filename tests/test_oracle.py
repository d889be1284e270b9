"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each pin is chosen so that a plausible mistake in the oracle (window off by one, wrong eviction
index, wrong scale, dropped prefix, transposed operand) fails at least one of them; the mutation
tests at the end plant such mistakes in a copy of the oracle and check that they are caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle import rswa as Orswa
from workloads import bf16_bits, bf16_to_f32


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def mask_from_golden(rows):
    return np.array([[c == "1" for c in r[0]] for r in rows])


# ---------------------------------------------------------------------------------------------
# hand-derived fixtures (tests/golden), each citing the passage it follows
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("fname,m,n,causal", [
    ("prefill_mask_m3_n2_s8_bidir.txt", 3, 2, False),
    ("prefill_mask_m3_n2_s8_prefix_causal.txt", 3, 2, True),
    ("prefill_mask_m0_n3_s8_vanilla_swa.txt", 0, 3, False),
    ("prefill_mask_m3_full_causal_s8.txt", 3, 8, True),
])
def test_prefill_mask_golden(golden, fname, m, n, causal):
    expected = mask_from_golden(golden(fname))
    S = expected.shape[0]
    got = O.prefill_visible(np.arange(S)[:, None], np.arange(S)[None, :], m, n, causal)
    np.testing.assert_array_equal(got, expected)


def test_decode_visible_golden(golden):
    for t, mask, count in golden("decode_visible_m3_n2.txt"):
        got = O.decode_visible(3, 2, int(t))
        np.testing.assert_array_equal(got, np.array([c == "1" for c in mask]))
        assert int(got.sum()) == int(count) == O.rswa_cache_rows(3, 2, int(t))


def test_ring_slots_golden(golden):
    for row in golden("ring_slots_n3.txt"):
        t = int(row[0])
        np.testing.assert_array_equal(O.ring_occupants(3, t), np.array([int(x) for x in row[1:]]))


def _cache_contents(m, n, t, mode):
    """Labels of the cache rows after t appends, built by writing output j into the row that the
    oracle's row helper names (the ring's n slots after the prefix, or the growing cache)."""
    rows = [f"P{i}" for i in range(m)] + ["-"] * (n if mode == O.RSWA else t)
    for j in range(t):
        r = O.ring_row(m, n, j) if mode == O.RSWA else O.full_row(m, j)
        rows[r] = f"o{j}"
    return rows


def test_cache_rows_golden(golden):
    """Where each output's K/V lives, for the ring and for the full-causal cache, against the
    hand-derived contents of tests/golden/cache_rows_m3_n2.txt."""
    m, n = 3, 2
    fixture = golden("cache_rows_m3_n2.txt")
    assert [int(r[0]) for r in fixture] == list(range(8))
    for t, ring, full in fixture:
        t = int(t)
        assert _cache_contents(m, n, t, O.RSWA) == ring.split(","), t
        assert _cache_contents(m, n, t, O.FULL) == full.split(","), t
        # written rows = the cache sizes the pages state: L_m + min(n, t) and L_m + t
        assert sum(x != "-" for x in ring.split(",")) == O.rswa_cache_rows(m, n, t)
        assert len(full.split(",")) == O.full_cache_rows(m, t)
        # the ring agrees with the slot occupants the other fixture pins
        occ = O.ring_occupants(n, t)
        assert [f"o{j}" if j >= 0 else "-" for j in occ] == ring.split(",")[m:]


def test_queue_golden(golden):
    m, n, H, d, T = 3, 2, 1, 2, 5
    pk, pv = rnd((m, H, d), 1), rnd((m, H, d), 2)
    ok, ov, q = rnd((T, H, d), 3), rnd((T, H, d), 4), rnd((T, H, d), 5)
    _, lens, members = O.queue_decode(q, pk, pv, ok, ov, n, T)
    for (t, idx, ln), got_members, got_len in zip(golden("queue_members_m3_n2.txt"), members, lens):
        assert got_members == [int(x) for x in idx.split(",")]
        assert got_len == int(ln)


# ---------------------------------------------------------------------------------------------
# closed forms stated on the pages
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("m", [0, 1, 5, 272])
@pytest.mark.parametrize("n", [1, 2, 128])
def test_cache_size_closed_form(m, n):
    """Visible rows at step t equal L_m + min(n, t) (R-SWA) and L_m + t (full causal)."""
    for t in range(0 if m else 1, 400):
        assert int(O.decode_visible(m, n, t).sum()) == m + min(n, t)
        assert int(O.decode_visible(m, n, t, O.FULL).sum()) == m + t


def test_cache_ratio_tends_to_zero():
    m, n = 272, 128
    prev = 1.0
    for t in [n, 2 * n, 1000, 10_000, 100_000, 10_000_000]:
        r = O.cache_ratio(m, n, t)
        assert r <= prev
        assert r == pytest.approx((m + n) / (m + t))
        prev = r
    assert prev < 1e-4
    for t in range(1, n + 1):  # before the window fills the two caches coincide
        assert O.cache_ratio(m, n, t) == 1.0


# ---------------------------------------------------------------------------------------------
# special cases that reduce to textbook / library routines
# ---------------------------------------------------------------------------------------------
def sdpa(q, K, V, mask=None, causal=False):
    """torch's scaled_dot_product_attention in float64 on the CPU; q [..., L, d]."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    msk = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(K), t(V), attn_mask=msk, is_causal=causal).numpy()


def test_window_covers_everything_equals_full_causal():
    """For t <= n R-SWA is plain causal attention over the whole cache."""
    m, n, H, d = 7, 16, 3, 8
    pk, pv = rnd((m, H, d), 10), rnd((m, H, d), 11)
    ok, ov, q = rnd((n, H, d), 12), rnd((n, H, d), 13), rnd((n, H, d), 14)
    for t in range(1, n + 1):
        o, c = O.decode_step(q[t - 1], pk, pv, ok, ov, t, n)
        o_full, _ = O.decode_step(q[t - 1], pk, pv, ok, ov, t, n, O.FULL)
        np.testing.assert_array_equal(o, o_full)
        K = np.concatenate([pk, ok[:t]]).transpose(1, 0, 2)
        V = np.concatenate([pv, ov[:t]]).transpose(1, 0, 2)
        ref = sdpa(q[t - 1][:, None, :], K, V)[:, 0, :]
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
        assert c == m + t


def test_full_mode_matches_library_at_every_step():
    m, n, H, d, T = 5, 3, 2, 16, 12
    pk, pv = rnd((m, H, d), 20), rnd((m, H, d), 21)
    ok, ov, q = rnd((T, H, d), 22), rnd((T, H, d), 23), rnd((T, H, d), 24)
    for t in range(1, T + 1):
        o, c = O.decode_step(q[t - 1], pk, pv, ok, ov, t, n, O.FULL)
        K = np.concatenate([pk, ok[:t]]).transpose(1, 0, 2)
        V = np.concatenate([pv, ov[:t]]).transpose(1, 0, 2)
        np.testing.assert_allclose(o, sdpa(q[t - 1][:, None, :], K, V)[:, 0, :], atol=1e-12)
        assert c == m + t


def torch_rswa_mask(S, m, n, prefix_causal):
    """The R-SWA prefill mask assembled from torch's triangular routines (independent of
    prefill_visible): prefix block, output rows' prefix columns, and a band of width n."""
    M = torch.zeros(S, S, dtype=torch.bool)
    ones = torch.ones(S, S, dtype=torch.bool)
    if prefix_causal:
        M[:m, :m] = torch.tril(ones[:m, :m])
    else:
        M[:m, :m] = True
    M[m:, :m] = True
    band = torch.tril(ones[m:, m:]) & torch.triu(ones[m:, m:], diagonal=-(n - 1))
    M[m:, m:] = band
    return M.numpy()


@pytest.mark.parametrize("m,n,S,causal", [(0, 4, 40, False), (9, 5, 37, False),
                                          (9, 5, 37, True), (16, 64, 70, False), (3, 100, 20, True)])
def test_prefill_matches_library(m, n, S, causal):
    H, d = 2, 16
    Q, K, V = rnd((S, H, d), 30), rnd((S, H, d), 31), rnd((S, H, d), 32)
    got = O.prefill(Q, K, V, m, n, causal, block=7)
    mask = torch_rswa_mask(S, m, n, causal)
    ref = sdpa(Q.transpose(1, 0, 2), K.transpose(1, 0, 2), V.transpose(1, 0, 2), mask=mask)
    np.testing.assert_allclose(got, ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_vanilla_swa_is_m0_and_full_causal_is_long_window():
    """m = 0 is vanilla sliding-window attention; a window >= S with a causal prefix is the
    library's causal attention."""
    S, H, d = 33, 2, 8
    Q, K, V = rnd((S, H, d), 40), rnd((S, H, d), 41), rnd((S, H, d), 42)
    T = lambda a: a.transpose(1, 0, 2)
    got = O.prefill(Q, K, V, 0, S, prefix_causal=False)
    np.testing.assert_allclose(got, T(sdpa(T(Q), T(K), T(V), causal=True)), atol=1e-12)
    got = O.prefill(Q, K, V, 5, S, prefix_causal=True)
    np.testing.assert_allclose(got, T(sdpa(T(Q), T(K), T(V), causal=True)), atol=1e-12)


def test_single_visible_key_returns_that_value_exactly():
    H, d, T = 2, 8, 9
    ok, ov, q = rnd((T, H, d), 50), rnd((T, H, d), 51), rnd((T, H, d), 52)
    empty = np.zeros((0, H, d))
    for t in range(1, T + 1):
        o, c = O.decode_step(q[t - 1], empty, empty, ok, ov, t, 1)
        assert c == 1
        np.testing.assert_array_equal(o, ov[t - 1])


def test_identical_keys_give_mean_of_visible_values():
    m, n, H, d, T = 6, 4, 2, 8, 11
    key = rnd((1, H, d), 60)
    pk = np.repeat(key, m, axis=0)
    ok = np.repeat(key, T, axis=0)
    pv, ov, q = rnd((m, H, d), 61), rnd((T, H, d), 62), rnd((T, H, d), 63)
    for t in range(1, T + 1):
        o, _ = O.decode_step(q[t - 1], pk, pv, ok, ov, t, n)
        vis_vals = np.concatenate([pv, ov[max(0, t - n):t]])
        np.testing.assert_allclose(o, vis_vals.mean(axis=0), atol=1e-13)


def test_scale_and_window_closed_form():
    """Keys chosen so that the scaled scores are ln(w_j): the output must be the w-weighted
    mean of the visible values. Pins the 1/sqrt(d) scale and the visible set together."""
    m, n, H, d, T = 5, 3, 1, 4, 9
    w_pre = np.arange(1, m + 1, dtype=np.float64)
    w_out = np.arange(1, T + 1, dtype=np.float64) * 10.0
    c = 2.0  # scale 1/sqrt(4) = 0.5, so score = 0.5 * c * k0 = k0
    pk = np.zeros((m, H, d)); pk[:, 0, 0] = np.log(w_pre)
    ok = np.zeros((T, H, d)); ok[:, 0, 0] = np.log(w_out)
    q = np.zeros((T, H, d)); q[:, 0, 0] = c
    pv, ov = rnd((m, H, d), 70), rnd((T, H, d), 71)
    for t in range(1, T + 1):
        o, _ = O.decode_step(q[t - 1], pk, pv, ok, ov, t, n)
        lo = max(0, t - n)
        w = np.concatenate([w_pre, w_out[lo:t]])
        vals = np.concatenate([pv, ov[lo:t]])[:, 0, :]
        np.testing.assert_allclose(o[0], (w[:, None] * vals).sum(0) / w.sum(), atol=1e-12)


def test_ring_order_gives_the_same_output():
    """Softmax attention is invariant under key permutation, so the ring's slot order (what the
    GPU cache stores) gives the queue's result."""
    m, n, H, d, T = 4, 5, 2, 8, 23
    pk, pv = rnd((m, H, d), 80), rnd((m, H, d), 81)
    ok, ov, q = rnd((T, H, d), 82), rnd((T, H, d), 83), rnd((T, H, d), 84)
    for t in range(1, T + 1):
        o, _ = O.decode_step(q[t - 1], pk, pv, ok, ov, t, n)
        occ = O.ring_occupants(n, t)
        live = occ[occ >= 0]
        K = np.concatenate([pk, ok[live]])
        V = np.concatenate([pv, ov[live]])
        o_ring = np.stack([O.attend(q[t - 1][h], K[:, h], V[:, h], O.default_scale(d))
                           for h in range(H)])
        np.testing.assert_allclose(o, o_ring, atol=1e-12)
        assert sorted(live.tolist()) == list(range(max(0, t - n), t))
        # the ring rows of the live outputs are distinct rows of the n-row region after the prefix
        rows = sorted(O.ring_row(m, n, int(j)) for j in live)
        assert len(set(rows)) == len(rows) and all(m <= r < m + n for r in rows)


def test_queue_equals_mask():
    m, n, H, d, T = 6, 4, 2, 8, 20
    pk, pv = rnd((m, H, d), 90), rnd((m, H, d), 91)
    ok, ov, q = rnd((T, H, d), 92), rnd((T, H, d), 93), rnd((T, H, d), 94)
    outs, lens, members = O.queue_decode(q, pk, pv, ok, ov, n, T)
    for t in range(1, T + 1):
        o, c = O.decode_step(q[t - 1], pk, pv, ok, ov, t, n)
        np.testing.assert_allclose(outs[t - 1], o, atol=1e-12)
        assert lens[t - 1] == c == m + min(n, t)
        vis = O.decode_visible(m, n, t)
        assert members[t - 1] == [j - m for j in np.nonzero(vis)[0] if j >= m]


def test_prefill_rows_equal_decode_steps():
    m, n, H, d, T = 6, 3, 2, 8, 10
    S = m + T
    Q, K, V = rnd((S, H, d), 100), rnd((S, H, d), 101), rnd((S, H, d), 102)
    P = O.prefill(Q, K, V, m, n)
    for t in range(1, T + 1):
        o, _ = O.decode_step(Q[m + t - 1], K[:m], V[:m], K[m:], V[m:], t, n)
        np.testing.assert_allclose(P[m + t - 1], o, atol=1e-12)
    rows = np.array([0, m - 1, m, S - 1])
    np.testing.assert_array_equal(O.prefill(Q, K, V, m, n, rows=rows), P[rows])


def test_empty_key_set_is_an_error():
    H, d = 1, 4
    z = np.zeros((0, H, d))
    with pytest.raises(ValueError):
        O.decode_step(np.ones((H, d)), z, z, z, z, 0, 4)


# ---------------------------------------------------------------------------------------------
# brute force on tiny shapes
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("m", [0, 1, 2, 5])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [1, 2, 4])
def test_brute_force_decode(m, n, d):
    H, T = 2, 10
    pk, pv = rnd((m, H, d), 110), rnd((m, H, d), 111)
    ok, ov, q = rnd((T, H, d), 112), rnd((T, H, d), 113), rnd((T, H, d), 114)
    for mode in (O.RSWA, O.FULL):
        for t in range(0 if m else 1, T + 1):
            if m + t == 0:
                continue
            o, c = O.decode_step(q[t - 1] if t else q[0], pk, pv, ok, ov, t, n, mode)
            ob, cb = O.brute_decode((q[t - 1] if t else q[0]).tolist(), pk.tolist(), pv.tolist(),
                                    ok.tolist(), ov.tolist(), t, n, mode)
            assert c == cb
            np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)


@pytest.mark.parametrize("m", [0, 1, 2, 5])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_prefill(m, n, causal):
    H, d, S = 2, 2, m + 7
    Q, K, V = rnd((S, H, d), 120), rnd((S, H, d), 121), rnd((S, H, d), 122)
    got = O.prefill(Q, K, V, m, n, causal, block=3)
    ref = np.array(O.brute_prefill(Q.tolist(), K.tolist(), V.tolist(), m, n, causal))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# input preparation: bf16 rounding is round-to-nearest-even
# ---------------------------------------------------------------------------------------------
def test_bf16_rounding_matches_library():
    x = np.concatenate([rnd(100_000, 130).astype(np.float32) * 37,
                        np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0],
                                 np.float32)])
    bits = bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    assert bits[-5:].tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0000]
    np.testing.assert_array_equal(bf16_to_f32(bits), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).float().numpy())


# ---------------------------------------------------------------------------------------------
# mutation checks: planted oracle mistakes must be caught by the pins above
# ---------------------------------------------------------------------------------------------
def _mask_off_by_one(m, n, t, mode=O.RSWA):  # window excludes the current token
    j = np.arange(m + t)
    if mode == O.FULL:
        return np.ones(m + t, dtype=bool)
    return (j < m) | ((j >= m + t - n - 1) & (j < m + t - 1))


def _prefill_no_prefix(p, k, m, n, prefix_causal=False):  # vanilla SWA: prefix slides away
    p, k = np.asarray(p), np.asarray(k)
    return (k <= p) & (p - k < n)


def test_mutation_window_off_by_one_is_caught(monkeypatch, golden):
    monkeypatch.setattr(Orswa, "decode_visible", _mask_off_by_one)
    monkeypatch.setattr(O, "decode_visible", _mask_off_by_one)
    with pytest.raises(AssertionError):
        test_decode_visible_golden(golden)
    with pytest.raises(AssertionError):
        test_cache_size_closed_form(5, 2)


def test_mutation_prefix_dropped_is_caught(monkeypatch, golden):
    monkeypatch.setattr(Orswa, "prefill_visible", _prefill_no_prefix)
    monkeypatch.setattr(O, "prefill_visible", _prefill_no_prefix)
    with pytest.raises(AssertionError):
        test_prefill_mask_golden(golden, "prefill_mask_m3_n2_s8_bidir.txt", 3, 2, False)
    with pytest.raises(AssertionError):
        test_prefill_matches_library(9, 5, 37, False)


def test_mutation_wrong_scale_is_caught(monkeypatch):
    monkeypatch.setattr(Orswa, "default_scale", lambda d: 1.0 / d)
    with pytest.raises(AssertionError):
        test_scale_and_window_closed_form()
    with pytest.raises(AssertionError):
        test_full_mode_matches_library_at_every_step()


def test_mutation_ring_row_off_by_one_is_caught(monkeypatch, golden):
    monkeypatch.setattr(Orswa, "ring_row", lambda m, n, j: m + (j + 1) % n)
    monkeypatch.setattr(O, "ring_row", lambda m, n, j: m + (j + 1) % n)
    with pytest.raises(AssertionError):
        test_cache_rows_golden(golden)


def test_mutation_ring_row_without_prefix_offset_is_caught(monkeypatch, golden):
    monkeypatch.setattr(O, "ring_row", lambda m, n, j: j % n)
    with pytest.raises(AssertionError):
        test_cache_rows_golden(golden)


def test_mutation_full_row_off_by_one_is_caught(monkeypatch, golden):
    monkeypatch.setattr(Orswa, "full_row", lambda m, j: m + j - 1)
    monkeypatch.setattr(O, "full_row", lambda m, j: m + j - 1)
    with pytest.raises(AssertionError):
        test_cache_rows_golden(golden)


def test_mutation_full_row_as_ring_is_caught(monkeypatch, golden):
    monkeypatch.setattr(O, "full_row", lambda m, j: m + j % 2)
    with pytest.raises(AssertionError):
        test_cache_rows_golden(golden)


def test_mutation_transposed_value_is_caught(monkeypatch):
    real = Orswa.attend
    monkeypatch.setattr(Orswa, "attend",
                        lambda q, K, V, s: real(q, K, V[::-1].copy(), s))
    with pytest.raises(AssertionError):
        test_brute_force_decode(2, 3, 4)


# ---------------------------------------------------------------------------------------------
# prefixes in a shared token pool
# ---------------------------------------------------------------------------------------------
def test_paged_prefix_identity_and_permuted_pool():
    m, H, d = 11, 2, 4
    pre = rnd((m, H, d), 90)
    np.testing.assert_array_equal(O.paged_prefix(pre, np.arange(m), 0, m), pre)
    perm = np.random.default_rng(3).permutation(m + 5)
    pool = rnd((m + 5, H, d), 91)
    pool[perm[:m]] = pre          # token j stored at slot perm[j]
    table = np.concatenate([[7, 7, 7], perm[:m]])  # another sequence's entries come first
    np.testing.assert_array_equal(O.paged_prefix(pool, table, 3, m), pre)


def test_shared_pool_rows_give_each_sequence_its_document():
    """Two sequences over one document stored once: each sees exactly the document's rows."""
    m, n, H, d, T = 6, 3, 2, 8, 5
    doc_k, doc_v = rnd((m, H, d), 92), rnd((m, H, d), 93)
    pool_k = np.concatenate([rnd((4, H, d), 94), doc_k])
    pool_v = np.concatenate([rnd((4, H, d), 95), doc_v])
    table = np.concatenate([np.arange(4, 4 + m), np.arange(4, 4 + m)])
    ok, ov, q = rnd((T, H, d), 96), rnd((T, H, d), 97), rnd((T, H, d), 98)
    for s in range(2):
        pk = O.paged_prefix(pool_k, table, s * m, m)
        pv = O.paged_prefix(pool_v, table, s * m, m)
        for t in range(1, T + 1):
            got, _ = O.decode_step(q[t - 1], pk, pv, ok, ov, t, n)
            ref, _ = O.decode_step(q[t - 1], doc_k, doc_v, ok, ov, t, n)
            np.testing.assert_array_equal(got, ref)
