"""GPU parity of the paged / shared prefix cache (prefixes held once in a token pool, looked up
through a page table) against the fp64 oracle and against the copied-prefix cache.

A paged cache must give, bit for bit, what a cache holding copies of the same prefixes gives (the
kernels visit the same rows in the same order; only where the prefix rows are read from
differs), and must match the oracle, whose prefix is `oracle.paged_prefix` of the pool, within
the decode tolerance (max-abs 1e-2 for bf16 inputs on the float32 output).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import Trajectory, sample_steps, upload
from workloads import to_f64

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module")
def wa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import windowed_attention_amd
    return windowed_attention_amd


def oracle_paged(wl, pp, t, b, full=False):
    off = int(np.concatenate([[0], np.cumsum(wl.prefix_len)])[b])
    m = int(wl.prefix_len[b])
    f = lambda x: to_f64(x, wl.dtype)
    pk = O.paged_prefix(pp.pool_k, pp.table, off, m)
    pv = O.paged_prefix(pp.pool_v, pp.table, off, m)
    o, _ = O.decode_step(f(wl.q[t - 1, b]), f(pk), f(pv), f(wl.k[:t, b]), f(wl.v[:t, b]), t,
                         int(wl.window[b]), O.FULL if full else O.RSWA)
    return o


def small_case(seed=0, scatter=True):
    # three documents, six sequences (documents shared by up to three sequences), spare pool rows
    return W.make_paged_decode("paged-small", 9, "bf16", [300, 150, 40], [0, 1, 0, 2, 1, 0],
                               [32, 32, 64, 16, 32, 128], [120, 120, 90, 120, 60, 120],
                               seed=seed, scatter=scatter, spare_rows=37)


@pytest.mark.parametrize("scatter", [False, True])
@pytest.mark.parametrize("fused", [False, True])
def test_paged_equals_copied_prefix_bitwise(wa, scatter, fused):
    wl, pp = small_case(seed=3, scatter=scatter)
    steps = range(1, wl.T + 1)
    ref = Trajectory(wa, wl, wa.MODE_RSWA).run(steps, fused=fused, raw=True)
    got = Trajectory(wa, wl, wa.MODE_RSWA, paged=pp).run(steps, fused=fused, raw=True)
    for t in steps:
        act = torch.from_numpy(wl.active(t).astype(bool)).cuda()
        assert torch.equal(got[t][act].view(torch.int32), ref[t][act].view(torch.int32)), t


def test_paged_matches_oracle_every_step(wa):
    wl, pp = small_case(seed=4)
    got = Trajectory(wa, wl, wa.MODE_RSWA, paged=pp).run(range(1, wl.T + 1), fused=True)
    worst = 0.0
    for t, out in got.items():
        for b in range(wl.batch):
            if wl.steps[b] < t:
                continue
            err = float(np.abs(out[b] - oracle_paged(wl, pp, t, b)).max())
            worst = max(worst, err)
            assert err <= TOL, f"t={t} b={b}: {err}"
    print(f"paged small: worst max-abs error {worst:.3e}")


def test_paged_graph_replays_equal_eager_steps(wa):
    """Step graphs over a paged cache (ragged prefixes read through the page table): replays of
    the fused steps equal the same steps launched one by one, bit for bit, under a fixed grid."""
    wl, pp = small_case(seed=6)
    G, T = 4, 48
    ref_tr = Trajectory(wa, wl, wa.MODE_RSWA, paged=pp)
    ref_tr.cache.set_decode_split(0, 96)
    ref = ref_tr.run(range(1, T + 1), t_end=T, fused=True, raw=True)
    ref_tr.cache.close()
    tr = Trajectory(wa, wl, wa.MODE_RSWA, paged=pp)
    tr.cache.set_decode_split(0, 96)
    g = wa.StepGraph(tr.cache, G)
    for r in range(T // G):
        t0 = r * G
        g.q.copy_(tr.q[t0:t0 + G])
        g.k.copy_(tr.k[t0:t0 + G])
        g.v.copy_(tr.v[t0:t0 + G])
        g.launch()
        torch.cuda.synchronize()
        for i in range(G):
            t = t0 + i + 1
            act = torch.from_numpy(wl.active(t).astype(bool)).cuda()
            assert torch.equal(g.out[i][act].view(torch.int32), ref[t][act].view(torch.int32)), t
    g.close()
    tr.cache.close()


def test_paged_full_causal_equals_copied(wa):
    wl, pp = small_case(seed=5)
    steps = range(1, wl.T + 1)
    ref = Trajectory(wa, wl, wa.MODE_FULL_CAUSAL).run(steps, raw=True)
    got = Trajectory(wa, wl, wa.MODE_FULL_CAUSAL, paged=pp).run(steps, raw=True)
    for t in steps:
        act = torch.from_numpy(wl.active(t).astype(bool)).cuda()
        assert torch.equal(got[t][act].view(torch.int32), ref[t][act].view(torch.int32)), t
    for t in (1, 50, 120):
        for b in (0, 3):
            if wl.steps[b] >= t:
                o = oracle_paged(wl, pp, t, b, full=True)
                assert float(np.abs(got[t][b].cpu().numpy() - o).max()) <= TOL


def test_page_table_entry_outside_pool_is_rejected(wa):
    wl, pp = small_case(seed=7)
    bad = pp.table.copy()
    bad[5] = pp.pool_k.shape[0]  # one past the last pool row
    pool_k, pool_v = upload(pp.pool_k, "bf16"), upload(pp.pool_v, "bf16")
    for tab in (bad, np.where(np.arange(bad.size) == 9, -1, pp.table).astype(np.int32)):
        with pytest.raises(wa.RswaError) as e:
            wa.RswaCache(None, None, wl.prefix_len, wl.window, kv_dtype=torch.bfloat16,
                         pool_k=pool_k, pool_v=pool_v, prefix_table=torch.from_numpy(tab).cuda())
        assert e.value.status == -1


def test_shared_documents_full_size_sampled(wa):
    """Four 20-page documents (m = 5155) decoded by 16 sequences each (B = 64) over a scattered
    token pool, in the launch configuration the benchmark times; sampled steps and sequences
    against the oracle.

    At this size the copied-prefix cache reads 2.8 GB per step and streams its rows with three
    workgroups per CU, while the paged cache (its pool reads need the latency cover) keeps four:
    their key ranges are cut differently, so in the default launches the two agree to rounding
    (max-abs 1e-5 on outputs of order 0.05). Given the same grid, both cut the ranges alike and
    agree bit for bit."""
    wl, pp = W.shared_document_config(seed=1, T=260)
    n = 128
    steps = sample_steps(wl.T, n, int(wl.prefix_len[0]), seed=2, extra=4, crossings=4)
    got = Trajectory(wa, wl, wa.MODE_RSWA, paged=pp).run(steps, fused=True, raw=True)
    ref = Trajectory(wa, wl, wa.MODE_RSWA).run(steps, fused=True, raw=True)
    rng = np.random.default_rng(3)
    for t in steps:
        assert float((got[t] - ref[t]).abs().max()) <= 1e-5, t
        for b in rng.choice(wl.batch, size=3, replace=False):
            err = float(np.abs(got[t][b].cpu().numpy() - oracle_paged(wl, pp, t, b)).max())
            assert err <= TOL, f"t={t} b={b}: {err}"
    same = []
    for paged in (pp, None):
        tr = Trajectory(wa, wl, wa.MODE_RSWA, paged=paged)
        tr.cache.set_decode_split(0, 1000)
        same.append(tr.run(steps, fused=True, raw=True))
    for t in steps:
        assert torch.equal(same[0][t].view(torch.int32), same[1][t].view(torch.int32)), t
