"""GPU parity where byte offsets pass 4 GiB: a decode cache, a paged prefix pool and a packed
training batch larger than 2^31 bf16 elements, so that every 64-bit row offset of the append, the
prefix copy, the prefix look-up, the streamed decode, the masked prefill and the backward is taken
beyond it. Rows the kernels copy are checked bit for bit, outputs and gradients against the fp64
oracle with the tolerances of the other parity tests (decode 1e-2 max-abs for bf16 inputs; the
log-sum-exp 2e-4; gradients 1e-2 of the largest reference entry of the tensor)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import Trajectory, upload
from workloads import to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

H, D = 16, 128
FOUR_GIB = 1 << 32


@pytest.fixture(scope="module")
def wa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import windowed_attention_amd
    return windowed_attention_amd


def decode_ref(wl, t, b):
    pk, pv = wl.prefix(b)
    f = lambda x: to_f64(x, wl.dtype)
    o, _ = O.decode_step(f(wl.q[t - 1, b]), f(pk), f(pv), f(wl.k[:t, b]), f(wl.v[:t, b]), t,
                         int(wl.window[b]), O.RSWA)
    return o


def test_decode_cache_past_4gib(wa):
    """Nine sequences of 257 pages (m = 66,065), n = 128, bf16: 4.88 GB of cache. Sequence 7's V
    rows straddle 4 GiB and sequence 8 lies wholly past it. Its prefix rows and, after the ring
    has wrapped, its ring rows hold the inputs bit for bit; the step outputs of sequences 0, 7 and
    8 match the oracle before and after the wrap (the steps stream: the live rows exceed the
    last-level cache)."""
    B, m, n, T = 9, 257 * 257 + 16, 128, 130
    wl = W.make_decode("past-4gib", 90, "bf16", [m] * B, [n] * B, [T] * B, seed=31)
    off, rows, nbytes = wa.rswa_cache_plan([m] * B, [n] * B, mode=wa.MODE_RSWA)
    assert nbytes > FOUR_GIB + (nbytes // B)
    storage = torch.zeros(nbytes // 2, dtype=torch.int16, device="cuda")
    tr = Trajectory(wa, wl, wa.MODE_RSWA, storage=storage)
    _, ko, vo, R, _ = tr.cache.query()
    assert 2 * int(vo[7]) < FOUR_GIB < 2 * int(vo[7]) + 2 * H * int(R[7]) * D
    assert 2 * int(ko[8]) > FOUR_GIB
    got = tr.run([1, 128, 129, 130], fused=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(tr.cache.steps(), [T] * B)

    def block(o, b):
        r = int(R[b])
        return storage[int(o[b]):int(o[b]) + H * r * D].view(H, r, D)

    pk, pv = wl.prefix(8)
    for o, ref in ((ko, pk), (vo, pv)):
        got_pre = block(o, 8)[:, :m].cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got_pre, ref.transpose(1, 0, 2))
    occ = O.ring_occupants(n, T)
    for b in (7, 8):
        for o, src in ((ko, wl.k), (vo, wl.v)):
            ring = block(o, b)[:, m:m + n].cpu().numpy().view(np.uint16)
            for s, j in enumerate(occ):
                assert O.ring_row(m, n, j) == m + s
                np.testing.assert_array_equal(ring[:, s], src[j, b], err_msg=f"b={b} slot {s}")
    worst = 0.0
    for t, bs in ((1, (7, 8)), (129, (8,)), (130, (0, 7, 8))):
        for b in bs:
            err = float(np.abs(got[t][b] - decode_ref(wl, t, b)).max())
            worst = max(worst, err)
            assert err <= 1e-2, f"t={t} b={b}: max abs err {err}"
    print(f"decode past 4 GiB: worst max-abs error {worst:.3e}")
    tr.cache.close()


def test_paged_pool_past_4gib(wa):
    """One paged workload (two documents, four sequences, token-granular scattered pool) decoded
    over its pool placed at row 0 and over the same pool placed after 1,100,000 unused rows, so
    every prefix row looked up lies past 2^31 elements of the 4.5 GB pool: the two caches give
    the same outputs bit for bit at every step, and the far one matches the oracle."""
    wl, pp = W.make_paged_decode("paged-far", 91, "bf16", [600, 300], [0, 0, 1, 1], [64] * 4,
                                 [70] * 4, seed=32)
    base = 1_100_000
    assert base * H * D * 2 > FOUR_GIB
    rows = pp.pool_k.shape[0]
    near_k, near_v = upload(pp.pool_k, "bf16"), upload(pp.pool_v, "bf16")
    far_k = torch.zeros((base + rows, H, D), dtype=torch.bfloat16, device="cuda")
    far_v = torch.zeros_like(far_k)
    far_k[base:] = near_k
    far_v[base:] = near_v
    tab_near = torch.from_numpy(pp.table).cuda()
    tab_far = torch.from_numpy(pp.table.astype(np.int64) + base).to(torch.int32).cuda()
    mk = lambda pk, pv, tab: wa.RswaCache(None, None, wl.prefix_len, wl.window,
                                          kv_dtype=torch.bfloat16, pool_k=pk, pool_v=pv,
                                          prefix_table=tab)
    near, far = mk(near_k, near_v, tab_near), mk(far_k, far_v, tab_far)
    q, k, v = (upload(x, "bf16") for x in (wl.q, wl.k, wl.v))
    check = {1, 64, 65, 70}
    worst = 0.0
    for t in range(1, wl.T + 1):
        a = near.step(q[t - 1], k[t - 1], v[t - 1])
        b = far.step(q[t - 1], k[t - 1], v[t - 1])
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"step {t}"
        if t in check:
            out = b.double().cpu().numpy()
            for s in range(wl.batch):
                err = float(np.abs(out[s] - decode_ref(wl, t, s)).max())
                worst = max(worst, err)
                assert err <= 1e-2, f"t={t} b={s}: max abs err {err}"
    print(f"paged pool past 4 GiB: worst max-abs error {worst:.3e}")
    near.close()
    far.close()


def test_training_batch_past_4gib(wa):
    """A packed training batch of 1,054,720 tokens (4.3 GB per bf16 tensor): fifteen
    69,632-token documents, then an 8,192-token one whose rows cross 2^31 elements at its row
    4,096, then a 2,048-token one wholly past it. Forward output and log-sum-exp on sampled rows
    of the last two, and dQ, dK, dV of one head on sampled rows of the 8,192-token document and
    on every row of the last, against the oracle."""
    lens = [69_632] * 15 + [8_192, 2_048]
    m = [512] * 15 + [700, 300]
    n = [128] * 15 + [128, 64]
    pw = W.make_prefill("past-4gib", 92, lens, m, n, seed=33)
    g = W.make_output_grad(pw, seed=33)
    cu_h = pw.cu_seqlens
    assert int(cu_h[15]) * H * D < 1 << 31 < int(cu_h[16]) * H * D
    assert (1 << 31) // (H * D) - int(cu_h[15]) == 4096
    q, k, v, dout = (upload(x, "bf16") for x in (pw.q, pw.k, pw.v, g))
    cu = torch.tensor(cu_h, dtype=torch.int32, device="cuda")
    md = torch.tensor(m, dtype=torch.int32, device="cuda")
    nd = torch.tensor(n, dtype=torch.int32, device="cuda")
    out, lse = wa.rswa_prefill_fwd(q, k, v, cu, md, nd, out_dtype=torch.bfloat16)
    dq, dk, dv = wa.rswa_prefill_bwd(q, k, v, out, dout, lse, cu, md, nd,
                                     grad_dtype=torch.float32)
    torch.cuda.synchronize()
    f = lambda x: W.to_f64(x, "bf16")
    rng = np.random.default_rng(34)
    head = 5
    for b in (15, 16):
        s0, s1 = int(cu_h[b]), int(cu_h[b + 1])
        S, mb, nb = s1 - s0, m[b], n[b]
        pick = {0, mb - 1, mb, mb + 1, mb + nb, S - 1, 4095, 4096, 4097}
        pick |= set(rng.integers(0, S, size=12).tolist())
        rows = np.array(sorted(r for r in pick if 0 <= r < S))
        qs, ks, vs = pw.seq(b)
        ref_o = O.prefill(f(qs), f(ks), f(vs), mb, nb, rows=rows)
        got_o = out[s0:s1][torch.from_numpy(rows).cuda()].double().cpu().numpy()
        err = float(np.abs(got_o - ref_o).max())
        assert err <= 1e-2, f"document {b}: output max abs err {err}"
        ref_l = O.prefill_lse(f(qs), f(ks), mb, nb, rows=rows)
        got_l = lse[s0:s1][torch.from_numpy(rows).cuda()].double().cpu().numpy()
        lerr = float(np.abs(got_l - ref_l).max())
        assert lerr <= 2e-4, f"document {b}: lse max abs err {lerr}"
        grows = np.arange(S) if S <= 2048 else rows
        ref = O.prefill_backward(f(qs), f(ks), f(vs), f(g[s0:s1]), mb, nb, heads=[head],
                                 q_rows=grows, k_rows=grows)
        idx = torch.from_numpy(grows).cuda()
        for name, t, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            got = t[s0:s1][idx][:, head:head + 1].double().cpu().numpy()
            scale = max(float(np.abs(r).max()), 1e-30)
            gerr = float(np.abs(got - r).max())
            print(f"document {b} {name}: max abs err {gerr:.3e}, max |ref| {scale:.3e}")
            assert gerr <= 1e-2 * scale, f"document {b} {name}: {gerr} > 1e-2 * {scale}"
