"""GPU checks of the graph-captured step loop (rswa_step_graph_*): every replay, with eager work
(input-slot copies) and a synchronization between replays, must give bit for bit what the same
fused steps give when launched one by one, including when the captured steps split ranges over
pieces and merge them inside the launch, and the step counters must advance by the captured count.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import Trajectory
from workloads import to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import windowed_attention_amd
    return windowed_attention_amd


def eager(wa, wl, T, mode, split=None, out_dtype=torch.float32):
    tr = Trajectory(wa, wl, mode)
    if split:
        tr.cache.set_decode_split(*split)
    res = tr.run(range(1, T + 1), out_dtype=out_dtype, t_end=T, fused=True, raw=True)
    tr.cache.close()
    return res


def replayed(wa, wl, T, G, mode, split=None, out_dtype=torch.float32):
    tr = Trajectory(wa, wl, mode)
    if split:
        tr.cache.set_decode_split(*split)
    g = wa.StepGraph(tr.cache, G, out_dtype=out_dtype)
    res = {}
    for r in range(T // G):
        t0 = r * G
        g.q.copy_(tr.q[t0:t0 + G])
        g.k.copy_(tr.k[t0:t0 + G])
        g.v.copy_(tr.v[t0:t0 + G])
        g.launch()
        torch.cuda.synchronize()
        for i in range(G):
            res[t0 + i + 1] = g.out[i].clone()
    steps = tr.cache.steps()
    g.close()
    tr.cache.close()
    return res, steps


# The work split of a captured step is the one chosen at capture. With a fixed grid (or the
# aligned layout, one workgroup per range) it is the split an eager launch chooses at every step,
# so replays are bit-identical; an automatic stream-K split can differ while the window fills
# (same result up to float32 summation order).
@pytest.mark.parametrize("G,B,split", [(8, 4, (0, 64)), (4, 4, (16, 7)), (2, 4, (0, 32)),
                                       (8, 48, None)])
def test_replays_equal_eager_steps(wa, G, B, split):
    wl = W.make_decode("graph", 10, "bf16", [100] * B, [32] * B, [96] * B, seed=11,
                       outlier_p=0.01)
    T = 96
    ref = eager(wa, wl, T, wa.MODE_RSWA, split)
    got, steps = replayed(wa, wl, T, G, wa.MODE_RSWA, split)
    np.testing.assert_array_equal(steps, T)
    for t in range(1, T + 1):
        assert torch.equal(got[t].view(torch.int32), ref[t].view(torch.int32)), t
    for t in (1, 33, 96):  # and the oracle, at a few steps
        b = t % wl.batch
        pk, pv = wl.prefix(b)
        o, _ = O.decode_step(to_f64(wl.q[t - 1, b], "bf16"), to_f64(pk, "bf16"),
                             to_f64(pv, "bf16"), to_f64(wl.k[:t, b], "bf16"),
                             to_f64(wl.v[:t, b], "bf16"), t, 32)
        assert float(np.abs(got[t][b].cpu().numpy() - o).max()) <= 1e-2


def test_replays_equal_eager_steps_split_layout(wa):
    """Eight sequences of 600+ rows: the automatic plan cuts every range into equal pieces (eight
    per range on MI355X) both for eager steps, which take the plan from the host, and for the
    captured ones, which derive the rows on the device; replays must match eager steps bit for
    bit, and the oracle."""
    B, T, G = 8, 48, 8
    wl = W.make_decode("graph-split", 10, "bf16", [600] * B, [32] * B, [T] * B, seed=15)
    ref = eager(wa, wl, T, wa.MODE_RSWA)
    got, steps = replayed(wa, wl, T, G, wa.MODE_RSWA)
    np.testing.assert_array_equal(steps, T)
    for t in range(1, T + 1):
        assert torch.equal(got[t].view(torch.int32), ref[t].view(torch.int32)), t
    for t in (1, 33, 48):
        b = t % wl.batch
        pk, pv = wl.prefix(b)
        o, _ = O.decode_step(to_f64(wl.q[t - 1, b], "bf16"), to_f64(pk, "bf16"),
                             to_f64(pv, "bf16"), to_f64(wl.k[:t, b], "bf16"),
                             to_f64(wl.v[:t, b], "bf16"), t, 32)
        assert float(np.abs(got[t][b].cpu().numpy() - o).max()) <= 1e-2


@pytest.mark.slow
def test_replays_equal_eager_steps_streamed(wa):
    """Eight sequences of 5155 prefix rows (338-340 MB per step, beyond the last-level cache): eager
    and captured steps both stream the rows (non-temporal loads, three workgroups per CU) in the
    split layout; replays must match eager steps bit for bit, and the oracle."""
    B, T, G = 8, 48, 8
    wl = W.make_decode("graph-streamed", 10, "bf16", [5155] * B, [32] * B, [T] * B, seed=16)
    ref = eager(wa, wl, T, wa.MODE_RSWA)
    got, steps = replayed(wa, wl, T, G, wa.MODE_RSWA)
    np.testing.assert_array_equal(steps, T)
    for t in range(1, T + 1):
        assert torch.equal(got[t].view(torch.int32), ref[t].view(torch.int32)), t
    for t in (1, 33, 48):
        b = t % wl.batch
        pk, pv = wl.prefix(b)
        o, _ = O.decode_step(to_f64(wl.q[t - 1, b], "bf16"), to_f64(pk, "bf16"),
                             to_f64(pv, "bf16"), to_f64(wl.k[:t, b], "bf16"),
                             to_f64(wl.v[:t, b], "bf16"), t, 32)
        assert float(np.abs(got[t][b].cpu().numpy() - o).max()) <= 1e-2


def test_replays_switch_to_per_sequence_counts_after_a_masked_step(wa):
    """A cache whose sequences share their step count gets a graph copy that reads the one shared
    count; after an eager step with an active mask the counts differ, and later replays must take
    the copy that reads every sequence's counter. Launch by launch (same inputs, same fixed grid)
    the outputs and counters equal those of eager steps."""
    B, G = 4, 2
    wl = W.make_decode("graph-masked", 10, "bf16", [100] * B, [32] * B, [12] * B, seed=17)
    tr_ref = Trajectory(wa, wl, wa.MODE_RSWA)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    for t_ in (tr_ref, tr):
        t_.cache.set_decode_split(0, 64)
    g = wa.StepGraph(tr.cache, G)
    mask = torch.tensor([1, 0, 1, 0], dtype=torch.uint8, device="cuda")
    plan = ["g", "g", "m", "g", "g"]  # replays of G launches, one masked eager launch
    out = torch.empty((B, 16, 128), dtype=torch.float32, device="cuda")
    launch = 0
    for kind in plan:
        n = G if kind == "g" else 1
        q, k, v = tr.q[launch:launch + n], tr.k[launch:launch + n], tr.v[launch:launch + n]
        refs = []
        for i in range(n):  # the eager reference of the same launches
            act = mask if kind == "m" else None
            refs.append(tr_ref.cache.step(q[i], k[i], v[i], out.clone(), active=act).clone())
        if kind == "g":
            g.q.copy_(q)
            g.k.copy_(k)
            g.v.copy_(v)
            g.launch()
            got = [g.out[i].clone() for i in range(n)]
        else:
            got = [tr.cache.step(q[0], k[0], v[0], out.clone(), active=mask).clone()]
        torch.cuda.synchronize()
        for i in range(n):
            act = mask.bool() if kind == "m" else torch.ones(B, dtype=torch.bool, device="cuda")
            assert torch.equal(got[i][act].view(torch.int32), refs[i][act].view(torch.int32)), \
                (kind, launch + i)
        launch += n
    np.testing.assert_array_equal(tr.cache.steps(), tr_ref.cache.steps())
    np.testing.assert_array_equal(tr.cache.steps(), [9, 8, 9, 8])
    g.close()
    tr.cache.close()
    tr_ref.cache.close()


def test_replays_bf16_output_and_full_causal_capacity(wa):
    wl = W.make_decode("graph-full", 10, "bf16", [40, 40], [8, 8], [20, 20], seed=12)
    ref = eager(wa, wl, 20, wa.MODE_FULL_CAUSAL, split=(0, 16), out_dtype=torch.bfloat16)
    tr = Trajectory(wa, wl, wa.MODE_FULL_CAUSAL)
    tr.cache.set_decode_split(0, 16)  # a fixed grid: the split eager launches choose too
    g = wa.StepGraph(tr.cache, 2, out_dtype=torch.bfloat16)
    for r in range(10):
        g.q.copy_(tr.q[2 * r:2 * r + 2])
        g.k.copy_(tr.k[2 * r:2 * r + 2])
        g.v.copy_(tr.v[2 * r:2 * r + 2])
        g.launch()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(g.out[i].view(torch.int16), ref[2 * r + i + 1].view(torch.int16))
    with pytest.raises(wa.RswaError) as e:  # a replay past max_steps is refused on the host
        g.launch()
    assert e.value.status == -3
    g.close()
    tr.cache.close()


def test_odd_step_count_is_rejected(wa):
    wl = W.make_decode("graph-odd", 10, "bf16", [8], [4], [4], seed=13)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    with pytest.raises(wa.RswaError) as e:
        wa.StepGraph(tr.cache, 3)
    assert e.value.status == -1
    tr.cache.close()


def test_eager_steps_between_replays(wa):
    """An eager step, a replay, an eager step, a replay ...: the replays must read the counters
    the eager steps left (in either counter buffer) and give what all-eager steps give."""
    wl = W.make_decode("graph-mixed", 10, "bf16", [100] * 4, [32] * 4, [40] * 4, seed=14)
    split = (0, 64)
    T = 40
    ref = eager(wa, wl, T, wa.MODE_RSWA, split)
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    tr.cache.set_decode_split(*split)
    g = wa.StepGraph(tr.cache, 2)
    out = torch.empty((4, 16, 128), dtype=torch.float32, device="cuda")
    got = {}
    t = 0
    pattern = ["e", "g", "e", "g", "g", "e", "e", "g", "e"] * 3
    for kind in pattern:
        if kind == "e" and t + 1 <= T:
            tr.cache.step(tr.q[t], tr.k[t], tr.v[t], out)
            torch.cuda.synchronize()
            got[t + 1] = out.clone()
            t += 1
        elif kind == "g" and t + 2 <= T:
            g.q.copy_(tr.q[t:t + 2])
            g.k.copy_(tr.k[t:t + 2])
            g.v.copy_(tr.v[t:t + 2])
            g.launch()
            torch.cuda.synchronize()
            got[t + 1], got[t + 2] = g.out[0].clone(), g.out[1].clone()
            t += 2
    assert t >= 20
    np.testing.assert_array_equal(tr.cache.steps(), t)
    for s in range(1, t + 1):
        assert torch.equal(got[s].view(torch.int32), ref[s].view(torch.int32)), s
    # the cache refuses to go while its graph exists; the graph first, then the cache
    with pytest.raises(wa.RswaError) as e:
        tr.cache.close()
    assert e.value.status == -1
    g.close()
    tr.cache.close()
