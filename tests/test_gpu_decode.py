"""GPU parity of K1 (ring append / evict) and K2 (split-K decode) against the fp64 oracle.

K1 is checked bit-exactly: prefix rows, ring slots (output j in row m + j mod n), full-causal rows,
step counters and untouched canary rows. K2 is checked element by element against the oracle
fed the same stored inputs: max-abs error <= 1e-2 for bf16 inputs and <= 1e-5 for fp32 inputs,
judged on the kernel's float32 output; its bf16 output must be exactly the round-to-nearest-even
of that float32 output. Full-size workloads are checked at sampled steps, in the same launch
configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import Trajectory, sample_steps, upload
from workloads import to_f64

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-5}
CANARY = 0x5A5A


@pytest.fixture(scope="module")
def wa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import windowed_attention_amd
    return windowed_attention_amd


def oracle_out(wl, t, b, mode):
    pk, pv = wl.prefix(b)
    o, c = O.decode_step(to_f64(wl.q[t - 1, b], wl.dtype), to_f64(pk, wl.dtype),
                         to_f64(pv, wl.dtype), to_f64(wl.k[:t, b], wl.dtype),
                         to_f64(wl.v[:t, b], wl.dtype), t, int(wl.window[b]),
                         O.FULL if mode else O.RSWA)
    return o, c


def check_steps(wl, mode, got, seqs_per_step=None, seed=0):
    rng = np.random.default_rng(seed)
    worst = 0.0
    for t, out in sorted(got.items()):
        seqs = [b for b in range(wl.batch) if wl.steps[b] >= t]
        if seqs_per_step is not None and len(seqs) > seqs_per_step:
            seqs = sorted(rng.choice(seqs, size=seqs_per_step, replace=False).tolist())
        for b in seqs:
            ref, _ = oracle_out(wl, t, b, mode)
            err = float(np.abs(out[b] - ref).max())
            worst = max(worst, err)
            assert err <= TOL[wl.dtype], f"t={t} b={b}: max abs err {err}"
    return worst


def bf16_rne(x):
    return W.bf16_bits(np.asarray(x, np.float32))


# ---------------------------------------------------------------------------------------------
# K1: bit-exact ring and canaries
# ---------------------------------------------------------------------------------------------
def read_storage(storage):
    torch.cuda.synchronize()
    return storage.cpu().numpy().view(np.uint16)


def seq_blocks(wa, st, wl, mode, b, off, rows):
    H, D = 16, 128
    n_el = H * rows[b] * D
    K = st[off[b]:off[b] + n_el].reshape(H, rows[b], D)
    V = st[off[b] + n_el:off[b] + 2 * n_el].reshape(H, rows[b], D)
    return K, V


@pytest.mark.parametrize("mode", [0, 1])
def test_append_rows_bit_exact(wa, mode):
    m, n, T = [5, 0, 70], [4, 3, 64], [150, 150, 150]
    wl = W.make_decode("ring", 91, "bf16", m, n, T, seed=1)
    cap = n if mode == 0 else T
    off, rows, nbytes = wa.rswa_cache_plan(m, n if mode == 0 else None, T if mode else None,
                                           mode=mode)
    storage = torch.full((nbytes // 2,), CANARY, dtype=torch.int16, device="cuda")
    tr = Trajectory(wa, wl, mode, storage=storage)
    check_at = set(range(0, 12)) | {63, 64, 65, 66, 128, 129, 130, 149, 150}
    for t in range(0, 151):
        if t > 0:
            tr.cache.append(tr.k[t - 1], tr.v[t - 1])
        if t not in check_at:
            continue
        st = read_storage(storage)
        np.testing.assert_array_equal(tr.cache.steps(), [t, t, t])
        for b in range(3):
            K, V = seq_blocks(wa, st, wl, mode, b, off, rows)
            pk, pv = wl.prefix(b)
            np.testing.assert_array_equal(K[:, :m[b]], pk.transpose(1, 0, 2))
            np.testing.assert_array_equal(V[:, :m[b]], pv.transpose(1, 0, 2))
            if mode == 0:
                occ = O.ring_occupants(n[b], t)
                slots = [(O.ring_row(m[b], n[b], j) if j >= 0 else m[b] + s, j)
                         for s, j in enumerate(occ)]
                assert sorted(r for r, _ in slots) == list(range(m[b], m[b] + n[b]))
            else:
                slots = [(O.full_row(m[b], j), j if j < t else -1) for j in range(cap[b])]
            for r, j in slots:
                if j >= 0:
                    np.testing.assert_array_equal(K[:, r], wl.k[j, b])
                    np.testing.assert_array_equal(V[:, r], wl.v[j, b])
                else:
                    assert (K[:, r] == CANARY).all() and (V[:, r] == CANARY).all(), (t, b, r)
    # nothing outside the planned storage was written: the tensor is exactly the plan's size
    assert storage.numel() * 2 == nbytes
    tr.cache.close()


def test_active_mask_and_capacity(wa):
    m, T = [3, 4], [5, 5]
    wl = W.make_decode("cap", 92, "bf16", m, [8, 8], T, seed=2)
    tr = Trajectory(wa, wl, wa.MODE_FULL_CAUSAL)
    act = torch.tensor([1, 0], dtype=torch.uint8, device="cuda")
    for t in range(3):
        tr.cache.append(tr.k[t], tr.v[t], act)
    np.testing.assert_array_equal(tr.cache.steps(), [3, 0])
    for t in range(3):  # host mirror counts calls: 3 more fill sequence 0 past max_steps = 5
        tr.cache.append(tr.k[t], tr.v[t], act)
    with pytest.raises(wa.RswaError) as e:
        tr.cache.steps()
    assert e.value.status == -3
    # after a masked call the host no longer knows t_b: an unmasked append is enqueued, and the
    # device skips the full sequence (its counter stays) and keeps reporting the overflow
    tr.cache.append(tr.k[0], tr.v[0])
    with pytest.raises(wa.RswaError) as e:
        tr.cache.steps()
    assert e.value.status == -3
    tr.cache.close()


def test_alternating_masks_then_unmasked_appends(wa):
    """Full causal, max_steps 6: ten masked calls (alternate sequences) leave t = [5, 5]; an
    unmasked append must then go through (no spurious capacity error from the host's call count)
    and a second one must be refused on the device."""
    wl = W.make_decode("cap-alt", 95, "bf16", [3, 4], [8, 8], [6, 6], seed=5)
    tr = Trajectory(wa, wl, wa.MODE_FULL_CAUSAL)
    masks = [torch.tensor(x, dtype=torch.uint8, device="cuda") for x in ([1, 0], [0, 1])]
    for i in range(10):
        tr.cache.append(tr.k[i // 2], tr.v[i // 2], masks[i % 2])
    np.testing.assert_array_equal(tr.cache.steps(), [5, 5])
    tr.cache.append(tr.k[5], tr.v[5])
    np.testing.assert_array_equal(tr.cache.steps(), [6, 6])
    _, ko, vo, rows, st = tr.cache.query()
    np.testing.assert_array_equal(st, [6, 6])
    np.testing.assert_array_equal(rows, [3 + 6, 4 + 6])
    np.testing.assert_array_equal(vo - ko, 16 * rows * 128)
    tr.cache.append(tr.k[0], tr.v[0])  # past max_steps: skipped on the device, then reported
    with pytest.raises(wa.RswaError) as e:
        tr.cache.steps()
    assert e.value.status == -3
    tr.cache.close()


def test_empty_key_set_is_rejected(wa):
    wl = W.make_decode("empty", 93, "bf16", [0], [4], [3], seed=3)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    with pytest.raises(wa.RswaError) as e:
        tr.cache.decode(tr.q[0])
    assert e.value.status == -1
    tr.cache.close()


def test_single_visible_key_is_exact(wa):
    """m = 0, n = 1: every output must be the latest value row, bit for bit."""
    wl = W.make_decode("one", 94, "bf16", [0, 0], [1, 1], [20, 20], seed=4)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    got = tr.run(range(1, 21))
    for t, out in got.items():
        np.testing.assert_array_equal(out, W.bf16_to_f32(wl.v[t - 1]))
    tr.cache.close()


# ---------------------------------------------------------------------------------------------
# K2: small shapes, every step, several chunk settings
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("chunk", [0, 64, 128, 512])
def test_decode_small_every_step(wa, dtype, chunk):
    m, n, T = [272, 0, 37], [128, 5, 64], [300, 300, 300]
    # fp32 follows the single-page fp32 recipe (N(0,1)); bf16 the batched one (1% x8 outliers)
    wl = W.make_decode("small", 95, dtype, m, n, T, seed=5,
                       outlier_p=0.01 if dtype == "bf16" else 0.0)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    tr.cache.set_decode_split(chunk, 0)
    got = tr.run(range(1, 301))
    check_steps(wl, 0, got)
    tr.cache.close()


def test_split_layout_equal_ranges(wa):
    """A uniform batch whose 128 ranges divide the resident workgroups (1,024 on MI355X at four
    per CU) takes the split layout: every range cut into k equal pieces, merged in the launch.
    Every step against the oracle, fused and unfused, and against a forced stream-K split."""
    B, T = 8, 40
    wl = W.make_decode("split", 97, "bf16", [600] * B, [128] * B, [T] * B, seed=7)
    got = {}
    for fused in (False, True):
        tr = Trajectory(wa, wl, wa.MODE_RSWA)
        grid, launches = tr.cache.decode_plan()
        assert launches == 1
        got[fused] = tr.run(range(1, T + 1), t_end=T, fused=fused)
        tr.cache.close()
        check_steps(wl, 0, got[fused])
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    tr.cache.set_decode_split(0, 1000)  # a user grid: stream-K
    sk = tr.run(range(1, T + 1), t_end=T, fused=True)
    tr.cache.close()
    for t in range(1, T + 1):
        np.testing.assert_allclose(got[True][t], sk[t], rtol=0, atol=1e-5)
        np.testing.assert_allclose(got[False][t], sk[t], rtol=0, atol=1e-5)


@pytest.mark.parametrize("grid", [1, 7, 4096])
def test_decode_grid_sizes(wa, grid):
    m, n, T = [100, 300, 9, 64], [16, 128, 5, 64], [80, 80, 80, 80]
    wl = W.make_decode("grid", 96, "bf16", m, n, T, seed=6)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    tr.cache.set_decode_split(64, grid)
    got = tr.run([1, 5, 16, 17, 63, 64, 65, 80])
    check_steps(wl, 0, got)
    tr.cache.close()


def test_decode_full_causal_small(wa):
    m, T = [50, 0, 130], [200, 200, 200]
    wl = W.make_decode("full", 97, "bf16", m, [8, 8, 8], T, seed=7)
    tr = Trajectory(wa, wl, wa.MODE_FULL_CAUSAL)
    tr.cache.set_decode_split(64, 0)
    got = tr.run(range(1, 201, 7))
    check_steps(wl, 1, got)
    tr.cache.close()


def test_bf16_output_is_rne_of_f32_output(wa):
    wl = W.make_decode("rne", 98, "bf16", [272, 40], [128, 16], [150, 150], seed=8,
                       outlier_p=0.01)
    a = Trajectory(wa, wl, wa.MODE_RSWA)
    b = Trajectory(wa, wl, wa.MODE_RSWA)
    steps = [1, 50, 128, 129, 150]
    f32 = a.run(steps, out_dtype=torch.float32)
    bf = b.run(steps, out_dtype=torch.bfloat16)
    for t in steps:
        np.testing.assert_array_equal(W.bf16_bits(bf[t]), bf16_rne(f32[t]))
    a.cache.close()
    b.cache.close()


def test_ragged_small_one_launch(wa):
    wl = W.varlen_config(0, batch=6, T_max=400)
    # shrink the prefixes so the oracle stays quick, keep the ragged lengths / windows
    wl2 = W.make_decode("ragged-small", 99, "bf16", np.minimum(wl.prefix_len, 300), wl.window,
                        np.minimum(wl.steps, 400) - np.arange(6) * 37, seed=9)
    tr = Trajectory(wa, wl2, wa.MODE_RSWA)
    got = tr.run(sample_steps(int(wl2.T), 64, 0, extra=20))
    check_steps(wl2, 0, got)
    tr.cache.close()


# ---------------------------------------------------------------------------------------------
# K1 + K2 fused in one launch: bit-identical to append then decode
# ---------------------------------------------------------------------------------------------
FUSED_CASES = [
    # (prefix lengths, windows, steps, mode, split setting)
    ([272] * 4, [128] * 4, [300] * 4, 0, (0, 0)),          # equal ranges
    ([272, 0, 37, 600], [128, 5, 64, 16], [300, 300, 250, 120], 0, (0, 0)),  # ragged + mask
    ([100, 9], [16, 5], [200, 200], 0, (64, 7)),             # pieces forced, 7 workgroups
    ([50, 0, 130], [8, 8, 8], [150, 150, 150], 1, (0, 0)),  # full causal
    ([5155], [128], [200], 0, (0, 0)),                       # one long range over many pieces
    # live rows past the 256 MiB last-level cache: streamed steps (non-temporal loads)
    ([11000] * 3, [64] * 3, [80] * 3, 0, (0, 0)),            # equal ranges, host-known plan
    ([15000, 9000, 12000], [16, 128, 64], [70, 50, 60], 1, (0, 0)),  # full causal, masked
]


@pytest.mark.parametrize("case", range(len(FUSED_CASES)))
def test_fused_step_equals_append_then_decode(wa, case):
    m, n, T, mode, split = FUSED_CASES[case]
    wl = W.make_decode("fused", 80 + case, "bf16", m, n, T, seed=20 + case, outlier_p=0.01)
    off, rows, nbytes = wa.rswa_cache_plan(m, n if mode == 0 else None, T if mode else None,
                                           mode=mode)
    sa = torch.full((nbytes // 2,), CANARY, dtype=torch.int16, device="cuda")
    sb = torch.full((nbytes // 2,), CANARY, dtype=torch.int16, device="cuda")
    a = Trajectory(wa, wl, mode, storage=sa)
    b = Trajectory(wa, wl, mode, storage=sb)
    a.cache.set_decode_split(*split)
    b.cache.set_decode_split(*split)
    if sum(m) * 16 * 512 > 256 << 20 and len(set(m)) == 1 and mode == 0:
        # the streamed plan: each range cut into pieces over three workgroups per CU
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        ranges = len(m) * 16
        k = min(3 * cus // ranges, (m[0] + 1) // 64)
        assert b.cache.decode_plan(appending=True) == (ranges * k, 1)
    steps = range(1, wl.T + 1)
    ra = a.run(steps, raw=True)
    rb = b.run(steps, fused=True, raw=True)
    for t in steps:
        live = wl.steps >= t
        assert torch.equal(ra[t][torch.from_numpy(live).cuda()],
                           rb[t][torch.from_numpy(live).cuda()]), f"step {t}"
    assert torch.equal(sa, sb)
    np.testing.assert_array_equal(a.cache.steps(), b.cache.steps())
    np.testing.assert_array_equal(b.cache.steps(), wl.steps)
    check_steps(wl, mode, {t: rb[t].float().cpu().numpy() for t in [1, 2, 17, 64, 65, 128, 129,
                                                                   int(wl.T)] if t <= wl.T})
    a.cache.close()
    b.cache.close()


def test_fused_step_capacity(wa):
    wl = W.make_decode("cap2", 85, "bf16", [3], [8], [4], seed=25)
    tr = Trajectory(wa, wl, wa.MODE_FULL_CAUSAL)
    tr.run(range(1, 5), fused=True)
    with pytest.raises(wa.RswaError) as e:
        tr.cache.step(tr.q[0], tr.k[0], tr.v[0])
    assert e.value.status == -3
    tr.cache.close()


# ---------------------------------------------------------------------------------------------
# full-size workloads, sampled steps, benchmark launch configuration
# ---------------------------------------------------------------------------------------------
def test_cfg_single_page_fp32_all_steps(wa):
    wl = W.decode_config(1)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    got = tr.run(range(1, wl.T + 1), fused=True)
    worst = check_steps(wl, 0, got)
    print(f"single-page fp32 decode: worst max-abs error {worst:.3e} over {len(got)} steps")
    tr.cache.close()


@pytest.mark.slow
def test_cfg_batched_single_page_sampled(wa):
    wl = W.decode_config(2)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    steps = sample_steps(wl.T, 128, 272)
    got = tr.run(steps, fused=True)
    worst = check_steps(wl, 0, got, seqs_per_step=6)
    print(f"batched decode: worst max-abs error {worst:.3e} at {len(steps)} steps")
    tr.cache.close()


@pytest.mark.slow
@pytest.mark.parametrize("mode", [0, 1])
def test_cfg_multi_page_sampled(wa, mode):
    wl = W.decode_config(3)
    tr = Trajectory(wa, wl, mode)
    steps = sample_steps(wl.T, 128, 5155, full=bool(mode), crossings=12, extra=8)
    got = tr.run(steps, fused=True)
    worst = check_steps(wl, mode, got, seqs_per_step=2)
    print(f"multi-page decode mode={mode}: worst max-abs error {worst:.3e}")
    tr.cache.close()


@pytest.mark.slow
def test_cfg_ragged_sampled(wa):
    wl = W.varlen_config(0)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    steps = sample_steps(wl.T, 64, 272, extra=12)
    got = tr.run(steps, fused=True)
    worst = check_steps(wl, 0, got, seqs_per_step=3)
    print(f"ragged decode: worst max-abs error {worst:.3e}")
    tr.cache.close()


@pytest.mark.slow
@pytest.mark.parametrize("dtype,batch,m", [("f32", 4, 5155), ("bf16", 32, 1100)])
def test_streamed_steps_sampled(wa, dtype, batch, m):
    """Steps whose live rows exceed the 256 MiB last-level cache read them with non-temporal
    loads over three workgroups per CU: float32 rows in the split layout (4 sequences, 338-346 MB
    per step) and bf16 rows in the aligned layout (512 ranges, 289-297 MB), against the oracle at
    sampled steps, ring wrap included."""
    n, T = 128, 140
    wl = W.make_decode(f"streamed-{dtype}", 87, dtype, [m] * batch, [n] * batch, [T] * batch,
                       seed=27)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    ranges = batch * 16
    grid, launches = tr.cache.decode_plan(appending=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if ranges <= 3 * cus:  # the streamed plan: at most three resident workgroups per CU
        k = min(3 * cus // ranges, (m + 1) // 64)
        assert (grid, launches) == ((ranges, 1) if 2 * ranges >= 3 * cus else (ranges * k, 1))
    got = tr.run([1, 2, 64, 128, 129, 140], fused=True)
    worst = check_steps(wl, 0, got, seqs_per_step=3)
    print(f"streamed {dtype}: worst max-abs error {worst:.3e}")
    tr.cache.close()


@pytest.mark.slow
@pytest.mark.parametrize("seed", range(3))
def test_streamed_steps_fuzz(wa, seed):
    """Seeded ragged batches whose live rows exceed the last-level cache (streamed steps over
    device-derived plans): random prefix lengths, windows and step counts, some sequences
    stopping early (active mask), both modes; sampled steps against the oracle."""
    rng = np.random.default_rng(3000 + seed)
    B = int(rng.integers(3, 5))
    m = rng.integers(11500, 16000, size=B)
    n = rng.choice([16, 64, 128, 256], size=B)
    T = int(rng.integers(40, 90))
    steps = rng.integers(T // 2, T + 1, size=B)
    steps[0] = T
    assert int(m.sum()) * 16 * 512 > 256 << 20  # the steps stream
    mode = seed % 2
    wl = W.make_decode(f"streamed-fuzz-{seed}", 88, "bf16", m, n, steps, seed=4000 + seed)
    tr = Trajectory(wa, wl, mode)
    got = tr.run(sample_steps(T, int(n.min()), int(m.min()), seed=seed, extra=6, crossings=2),
                 fused=True)
    worst = check_steps(wl, mode, got, seqs_per_step=2, seed=seed)
    print(f"streamed fuzz {seed}: worst max-abs error {worst:.3e}")
    tr.cache.close()


# ---------------------------------------------------------------------------------------------
# the comparison modes of the pages: vanilla sliding window and sink tokens
# ---------------------------------------------------------------------------------------------
def test_vanilla_sliding_window_decode(wa):
    """Vanilla SWA (the pages' "progressive blurring" contrast case): no reference prefix; the
    visual tokens are appended through the ring like outputs and slide out of the window."""
    n, P, T = 48, 100, 150  # window, streamed "visual" tokens, outputs
    wl = W.make_decode("vswa", 86, "bf16", [0, 0], [n, n], [P + T, P + T], seed=26, outlier_p=0.01)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    got = tr.run(range(P + 1, P + T + 1), fused=True)  # every query after the visual tokens
    check_steps(wl, 0, got)
    # the first visual token is still visible at step n and gone from step n + 1 on: with a
    # reference prefix (R-SWA) it never leaves
    assert O.decode_visible(0, n, n)[0] and not O.decode_visible(0, n, n + 1)[0]
    tr.cache.close()


def test_sink_tokens_decode(wa):
    """Attention sinks: the first s tokens stay visible, the rest slide — R-SWA with m = s."""
    s, n, T = 4, 32, 200
    wl = W.make_decode("sink", 87, "bf16", [s, s, s], [n, n, n], [T, T, T], seed=27)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    got = tr.run(range(1, T + 1), fused=True)
    check_steps(wl, 0, got)
    tr.cache.close()


def test_maximum_batch(wa):
    """The largest batch a cache accepts (2048 sequences), ragged prefixes and windows, through
    the fused step; sampled sequences at every step against the oracle."""
    B = 2048
    rng = np.random.default_rng(31)
    m = rng.integers(0, 40, size=B)
    n = rng.integers(1, 24, size=B)
    m[0] = 0  # a sequence with no prefix
    wl = W.make_decode("maxbatch", 88, "bf16", m, n, [20] * B, seed=31)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    got = tr.run(range(1, 21), fused=True)
    check_steps(wl, 0, got, seqs_per_step=24, seed=3)
    for t in (1, 20):
        o, _ = oracle_out(wl, t, 0, 0)
        assert float(np.abs(got[t][0] - o).max()) <= TOL["bf16"]
    tr.cache.close()
    with pytest.raises(wa.RswaError):
        wa.rswa_cache_plan([4] * (B + 1), [4] * (B + 1))
