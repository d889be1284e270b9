"""Seeded random shapes through every GPU path, against the fp64 oracle.

Each case draws its own sizes from a fixed seed: packed prefill batches (ragged documents,
prefix lengths anywhere in [0, S], windows shorter and longer than the outputs, causal and
bidirectional prefixes) for the forward with log-sum-exp and for the training backward, and
decode batches (ragged step counts, R-SWA and full-causal caches, bf16 and fp32, the fused step
and the separate append + decode, forced stream-K splits, prefixes shared through a token pool)
checked at random steps. Tolerances are the ones of the per-path tests: max-abs 1e-2 (bf16
inputs) / 1e-5 (fp32) on float32 outputs, 2e-4 on lse, 1e-2 of the largest reference entry on
each gradient.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import Trajectory, upload
from workloads import to_f64

pytestmark = pytest.mark.gpu
TOL = {"bf16": 1e-2, "f32": 1e-5}
LSE_TOL = 2e-4
GTOL = 1e-2


@pytest.fixture(scope="module")
def wa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import windowed_attention_amd
    return windowed_attention_amd


def prefill_case(seed):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 900]))
    nseq = int(rng.integers(1, 5))
    lens = rng.integers(0, 420, size=nseq)
    lens[rng.integers(0, nseq)] = max(int(lens.max()), 1)  # at least one non-empty document
    m = np.array([int(rng.integers(0, L + 1)) for L in lens])
    n = rng.choice([1, 2, 7, 16, 64, 100, 128, 300, 700], size=nseq)
    pc = bool(rng.integers(0, 2))
    return W.make_prefill(f"fuzz{seed}", 9, lens.tolist(), m.tolist(), n.tolist(), seed=seed,
                          prefix_causal=pc)


def dev_meta(pw):
    cu = torch.tensor(pw.cu_seqlens, dtype=torch.int32, device="cuda")
    m = torch.tensor(pw.prefix_len, dtype=torch.int32, device="cuda")
    n = torch.tensor(pw.window, dtype=torch.int32, device="cuda")
    return cu, m, n


@pytest.mark.parametrize("seed", range(12))
def test_fuzz_prefill_forward(wa, seed):
    pw = prefill_case(seed)
    q, k, v = upload(pw.q, "bf16"), upload(pw.k, "bf16"), upload(pw.v, "bf16")
    cu, m, n = dev_meta(pw)
    out, lse = wa.rswa_prefill_fwd(q, k, v, cu, m, n, out_dtype=torch.float32,
                                   prefix_causal=pw.prefix_causal)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    f = lambda x: to_f64(x, "bf16")
    for b in range(pw.nseq):
        s0, s1 = int(pw.cu_seqlens[b]), int(pw.cu_seqlens[b + 1])
        if s1 == s0:
            continue
        qs, ks, vs = pw.seq(b)
        mb, nb = int(pw.prefix_len[b]), int(pw.window[b])
        ref = O.prefill(f(qs), f(ks), f(vs), mb, nb, pw.prefix_causal)
        err = float(np.abs(out[s0:s1] - ref).max())
        assert err <= TOL["bf16"], f"seed {seed} doc {b} (S={s1 - s0}, m={mb}, n={nb}): {err}"
        lref = O.prefill_lse(f(qs), f(ks), mb, nb, pw.prefix_causal)
        lerr = float(np.abs(lse[s0:s1] - lref).max())
        assert lerr <= LSE_TOL, f"seed {seed} doc {b}: lse err {lerr}"


@pytest.mark.parametrize("seed", range(8))
def test_fuzz_training_backward(wa, seed):
    pw = prefill_case(100 + seed)
    g = W.make_output_grad(pw, seed=seed)
    q, k, v = upload(pw.q, "bf16"), upload(pw.k, "bf16"), upload(pw.v, "bf16")
    cu, m, n = dev_meta(pw)
    out, lse = wa.rswa_prefill_fwd(q, k, v, cu, m, n, out_dtype=torch.bfloat16,
                                   prefix_causal=pw.prefix_causal)
    grads = wa.rswa_prefill_bwd(q, k, v, out, upload(g, "bf16"), lse, cu, m, n,
                                grad_dtype=torch.float32, prefix_causal=pw.prefix_causal)
    torch.cuda.synchronize()
    got = [x.cpu().numpy() for x in grads]
    f = lambda x: to_f64(x, "bf16")
    for b in range(pw.nseq):
        s0, s1 = int(pw.cu_seqlens[b]), int(pw.cu_seqlens[b + 1])
        if s1 == s0:
            continue
        qs, ks, vs = pw.seq(b)
        refs = O.prefill_backward(f(qs), f(ks), f(vs), f(g[s0:s1]), int(pw.prefix_len[b]),
                                  int(pw.window[b]), pw.prefix_causal)
        for name, x, r in zip(("dQ", "dK", "dV"), got, refs):
            scale = max(float(np.abs(r).max()), 1e-30)
            err = float(np.abs(x[s0:s1] - r).max())
            assert err <= GTOL * scale, f"seed {seed} doc {b} {name}: {err} vs {scale}"


@pytest.mark.parametrize("seed", range(10))
def test_fuzz_decode(wa, seed):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 901]))
    B = int(rng.integers(1, 9))
    dtype = "bf16" if rng.integers(0, 3) else "f32"
    full = bool(rng.integers(0, 4) == 0)
    m = rng.integers(0, 300, size=B)
    n = rng.choice([1, 3, 16, 64, 65, 128, 200], size=B)
    steps = rng.integers(1, 160, size=B)
    wl = W.make_decode(f"fuzz{seed}", 9, dtype, m.tolist(), n.tolist(), steps.tolist(),
                       seed=seed, outlier_p=0.01)
    tr = Trajectory(wa, wl, wa.MODE_FULL_CAUSAL if full else wa.MODE_RSWA)
    if rng.integers(0, 2):  # force a stream-K split: small pieces over a small grid
        tr.cache.set_decode_split(int(rng.choice([16, 32, 64])), int(rng.integers(1, 48)))
    T = wl.T
    checks = sorted(set(rng.integers(1, T + 1, size=6).tolist()) | {1, T})
    got = tr.run(checks, fused=bool(rng.integers(0, 2)))
    tr.cache.close()
    f = lambda x: to_f64(x, dtype)
    for t in checks:
        for b in range(B):
            if wl.steps[b] < t:
                continue
            pk, pv = wl.prefix(b)
            o, _ = O.decode_step(f(wl.q[t - 1, b]), f(pk), f(pv), f(wl.k[:t, b]), f(wl.v[:t, b]),
                                 t, int(wl.window[b]), O.FULL if full else O.RSWA)
            err = float(np.abs(got[t][b] - o).max())
            assert err <= TOL[dtype], (f"seed {seed} t={t} b={b} (m={int(m[b])}, n={int(n[b])}, "
                                       f"{dtype}, {'full' if full else 'rswa'}): {err}")


@pytest.mark.parametrize("seed", range(6))
def test_fuzz_paged_decode(wa, seed):
    """Prefixes held once in a scattered token pool and shared by several sequences: every random
    checkpoint bit-identical to a cache holding copies of the same prefixes, and within the decode
    tolerance of the oracle over `oracle.paged_prefix` of the pool."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 902]))
    docs = rng.integers(0, 300, size=int(rng.integers(1, 4)))
    B = int(rng.integers(1, 7))
    seq_doc = rng.integers(0, docs.size, size=B)
    dtype = "bf16" if rng.integers(0, 3) else "f32"
    full = bool(rng.integers(0, 4) == 0)
    n = rng.choice([1, 16, 64, 128], size=B)
    steps = rng.integers(1, 130, size=B)
    wl, pp = W.make_paged_decode(f"fuzzp{seed}", 9, dtype, docs.tolist(), seq_doc.tolist(),
                                 n.tolist(), steps.tolist(), seed=seed,
                                 spare_rows=int(rng.integers(0, 40)))
    mode = wa.MODE_FULL_CAUSAL if full else wa.MODE_RSWA
    checks = sorted(set(rng.integers(1, wl.T + 1, size=5).tolist()) | {1, wl.T})
    fused = bool(rng.integers(0, 2))
    got = Trajectory(wa, wl, mode, paged=pp).run(checks, fused=fused, raw=True)
    ref = Trajectory(wa, wl, mode).run(checks, fused=fused, raw=True)
    off = np.concatenate([[0], np.cumsum(wl.prefix_len)])
    f = lambda x: to_f64(x, dtype)
    for t in checks:
        act = torch.from_numpy(wl.active(t).astype(bool)).cuda()
        assert torch.equal(got[t][act].view(torch.int32), ref[t][act].view(torch.int32)), t
        out = got[t].cpu().numpy()
        for b in range(B):
            if wl.steps[b] < t:
                continue
            mb = int(wl.prefix_len[b])
            pk = O.paged_prefix(pp.pool_k, pp.table, int(off[b]), mb)
            pv = O.paged_prefix(pp.pool_v, pp.table, int(off[b]), mb)
            o, _ = O.decode_step(f(wl.q[t - 1, b]), f(pk), f(pv), f(wl.k[:t, b]), f(wl.v[:t, b]),
                                 t, int(wl.window[b]), O.FULL if full else O.RSWA)
            err = float(np.abs(out[b] - o).max())
            assert err <= TOL[dtype], f"seed {seed} t={t} b={b}: {err}"
