"""GPU parity of the cache filled from a packed prefill batch (rswa_cache_create_from_prefill).

A prefill pass (prefix, then the outputs produced so far, packed per sequence) leaves exactly the
keys and values that a decode cache would hold after appending those outputs one by one. The filled
cache must therefore hold the same storage bytes and step counters as rswa_cache_create followed by
t_b appends, and every decode step after it must give the same outputs bit for bit; the first step
after the fill is also checked against the fp64 oracle (max-abs 1e-2 for bf16 inputs, 1e-5 for
float32, on the float32 output).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import kv_torch_dtype, upload
from workloads import to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import windowed_attention_amd
    return windowed_attention_amd


def packed_batch(wl, fill):
    """K / V of the prefill batch [total][H][D] (segment b = prefix_b, then outputs 1..fill_b of
    sequence b) and its cu_seqlens."""
    ks, vs, cu = [], [], [0]
    for b in range(wl.batch):
        pk, pv = wl.prefix(b)
        ks += [pk, wl.k[:fill[b], b]]
        vs += [pv, wl.v[:fill[b], b]]
        cu.append(cu[-1] + int(wl.prefix_len[b]) + int(fill[b]))
    return np.concatenate(ks), np.concatenate(vs), cu


def next_inputs(wl, fill, s):
    """Query / key / value of output fill_b + s + 1 of every sequence, as [B][H][D]."""
    idx = np.asarray(fill) + s
    bs = np.arange(wl.batch)
    return [upload(np.ascontiguousarray(a[idx, bs]), wl.dtype) for a in (wl.q, wl.k, wl.v)]


def run_case(wa, wl, fill, mode, extra=6):
    fill = np.asarray(fill, dtype=np.int64)
    assert np.all(wl.steps >= fill + extra)
    full = mode == wa.MODE_FULL_CAUSAL
    window = None if full else wl.window
    max_steps = wl.steps if full else None
    kvdt = kv_torch_dtype(wl.dtype)
    nbytes = wa.rswa_cache_bytes(wl.prefix_len, window, max_steps, kv_dtype=kvdt, mode=mode)
    st_a = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    st_b = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    k_all, v_all, cu = packed_batch(wl, fill)
    kd, vd = upload(k_all, wl.dtype), upload(v_all, wl.dtype)
    a = wa.rswa_cache_create_from_prefill(kd, vd, cu, wl.prefix_len, window, mode=mode,
                                          max_steps=max_steps, kv_dtype=kvdt, storage=st_a)
    b = wa.rswa_cache_create(upload(wl.prefix_k, wl.dtype), upload(wl.prefix_v, wl.dtype),
                             wl.prefix_len, window, mode=mode, max_steps=max_steps,
                             kv_dtype=kvdt, storage=st_b)
    equal = bool(np.all(fill == fill[0]))
    for s in range(int(fill.max())):
        act = None if equal else torch.from_numpy((fill > s).astype(np.uint8)).cuda()
        b.append(upload(wl.k[s], wl.dtype), upload(wl.v[s], wl.dtype), active=act)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.steps(), fill)
    np.testing.assert_array_equal(b.steps(), fill)
    assert torch.equal(st_a, st_b), "filled storage differs from the appended one"
    tol = 1e-2 if wl.dtype == "bf16" else 1e-5
    f = lambda x: to_f64(x, wl.dtype)
    for s in range(extra):
        q, k, v = next_inputs(wl, fill, s)
        oa = a.step(q, k, v)
        ob = b.step(q, k, v)
        assert torch.equal(oa.view(torch.int32), ob.view(torch.int32)), f"step {s}"
        if s == 0:
            out = oa.double().cpu().numpy()
            for i in range(wl.batch):
                t = int(fill[i]) + 1
                pk, pv = wl.prefix(i)
                ref, _ = O.decode_step(f(wl.q[t - 1, i]), f(pk), f(pv), f(wl.k[:t, i]),
                                       f(wl.v[:t, i]), t, int(wl.window[i]),
                                       O.FULL if full else O.RSWA)
                err = float(np.abs(out[i] - ref).max())
                assert err <= tol, f"b={i} t={t}: {err}"
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.steps(), fill + extra)
    a.close()
    b.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("full", [False, True])
def test_fill_unequal_outputs(wa, dtype, full):
    # no outputs yet, no prefix, a wrapped ring (t not a multiple of n), exactly n outputs, a ring
    # that has wrapped several times, and fewer outputs than the window
    m = [300, 0, 129, 64, 17, 200]
    n = [32, 16, 64, 128, 8, 32]
    fill = [0, 5, 200, 128, 37, 31]
    wl = W.make_decode("fill-ragged", 9, dtype, m, n, np.asarray(fill) + 8, seed=11)
    run_case(wa, wl, fill, wa.MODE_FULL_CAUSAL if full else wa.MODE_RSWA)


def test_fill_into_library_storage(wa):
    """The same fill with storage the library allocates: counters and every later decode step
    equal those of the appended cache, and the query hook reports the same layout."""
    m, n, fill = [64, 0, 200], [16, 8, 32], [40, 9, 77]
    wl = W.make_decode("fill-lib", 9, "bf16", m, n, np.asarray(fill) + 6, seed=13)
    k_all, v_all, cu = packed_batch(wl, fill)
    a = wa.rswa_cache_create_from_prefill(upload(k_all, "bf16"), upload(v_all, "bf16"), cu,
                                          wl.prefix_len, wl.window, kv_dtype=torch.bfloat16)
    b = wa.rswa_cache_create(upload(wl.prefix_k, "bf16"), upload(wl.prefix_v, "bf16"),
                             wl.prefix_len, wl.window, kv_dtype=torch.bfloat16)
    for s_ in range(max(fill)):
        act = torch.from_numpy((np.asarray(fill) > s_).astype(np.uint8)).cuda()
        b.append(upload(wl.k[s_], "bf16"), upload(wl.v[s_], "bf16"), active=act)
    _, ka, va, ra, sa = a.query()
    _, kb, vb, rb, sb = b.query()
    np.testing.assert_array_equal(ka, kb)
    np.testing.assert_array_equal(va, vb)
    np.testing.assert_array_equal(ra, rb)
    np.testing.assert_array_equal(sa, fill)
    np.testing.assert_array_equal(sb, fill)
    for s_ in range(6):
        q, k, v = next_inputs(wl, fill, s_)
        assert torch.equal(a.step(q, k, v).view(torch.int32), b.step(q, k, v).view(torch.int32))
    a.close()
    b.close()


@pytest.mark.parametrize("full", [False, True])
def test_fill_equal_outputs(wa, full):
    # equal m, n and t: decode after the fill takes the host-known plan (split pieces per range)
    B, m, n, fill = 8, 600, 128, 300
    wl = W.make_decode("fill-equal", 9, "bf16", [m] * B, [n] * B, [fill + 8] * B, seed=12)
    run_case(wa, wl, [fill] * B, wa.MODE_FULL_CAUSAL if full else wa.MODE_RSWA)


@pytest.mark.parametrize("seed", range(8))
def test_fill_fuzz(wa, seed):
    """Seeded random batches: sequence count, prefix lengths (0 included), windows down to 1,
    output counts from 0 past several ring wraps, both modes and both element types."""
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 10))
    m = rng.integers(0, 200, size=B)
    n = rng.integers(1, 48, size=B)
    fill = np.array([int(rng.integers(0, 3 * int(n[b]) + 2)) for b in range(B)])
    m[0] = max(int(m[0]), 1)  # at least one sequence with a prefix (no empty key set at t = 0)
    m[(fill == 0) & (m == 0)] = 1
    dtype = "bf16" if seed % 2 == 0 else "f32"
    full = seed % 4 >= 2
    wl = W.make_decode(f"fill-fuzz-{seed}", 9, dtype, m, n, fill + 3, seed=2000 + seed)
    run_case(wa, wl, fill, wa.MODE_FULL_CAUSAL if full else wa.MODE_RSWA, extra=3)
