"""GPU parity of the teacher-forced training pass against the fp64 oracle: the forward's
log-sum-exp and the backward's dQ, dK, dV, on packed prefix + output documents.

Tolerance. The inputs are bf16 and every sum runs in float32; the kernels round P and
dS = P * (dP - delta) to bf16 (unit roundoff 2^-8) before the products that form dV, dK and dQ,
and the forward output that delta is formed from is bf16. Each gradient element is a sum of many
such rounded terms of both signs, so its error is a fraction of 2^-8 of the size of the gradient;
the bar is max |got - ref| <= 1e-2 * max |ref| over each gradient tensor (all heads and documents
of the case), the same 1e-2 the forward output meets on unit-scale data. The log-sum-exp is
formed from float32 scores: max abs error 2e-4. A bf16 gradient must be exactly the
round-to-nearest-even of the float32 gradient (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import upload

pytestmark = pytest.mark.gpu
GTOL = 1e-2
LSE_TOL = 2e-4


@pytest.fixture(scope="module")
def wa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import windowed_attention_amd
    return windowed_attention_amd


def run_training(wa, pw, g, out_dtype=torch.bfloat16, grad_dtype=torch.float32):
    q, k, v = upload(pw.q, "bf16"), upload(pw.k, "bf16"), upload(pw.v, "bf16")
    dout = upload(g, "bf16")
    cu = torch.tensor(pw.cu_seqlens, dtype=torch.int32, device="cuda")
    m = torch.tensor(pw.prefix_len, dtype=torch.int32, device="cuda")
    n = torch.tensor(pw.window, dtype=torch.int32, device="cuda")
    out, lse = wa.rswa_prefill_fwd(q, k, v, cu, m, n, out_dtype=out_dtype,
                                   prefix_causal=pw.prefix_causal)
    dq, dk, dv = wa.rswa_prefill_bwd(q, k, v, out, dout, lse, cu, m, n, grad_dtype=grad_dtype,
                                     prefix_causal=pw.prefix_causal)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    return f(out), f(lse), f(dq), f(dk), f(dv)


def oracle_doc(pw, g, b, **kw):
    q, k, v = pw.seq(b)
    s0, s1 = int(pw.cu_seqlens[b]), int(pw.cu_seqlens[b + 1])
    f = lambda x: W.to_f64(x, "bf16")
    return O.prefill_backward(f(q), f(k), f(v), f(g[s0:s1]), int(pw.prefix_len[b]),
                              int(pw.window[b]), pw.prefix_causal, **kw)


def oracle_lse(pw, b, rows=None):
    q, k, _ = pw.seq(b)
    f = lambda x: W.to_f64(x, "bf16")
    return O.prefill_lse(f(q), f(k), int(pw.prefix_len[b]), int(pw.window[b]), pw.prefix_causal,
                         rows=rows)


def check_grads(name, got, ref):
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = float(np.abs(got - ref).max())
    print(f"{name}: max abs err {err:.3e}, max |ref| {scale:.3e}, ratio {err / scale:.3e}")
    assert err <= GTOL * scale, f"{name}: max abs err {err} > {GTOL} * {scale}"


CASES = [
    # (document lengths, prefix lengths, windows, causal prefix)
    ([300], [70], [16], False),
    ([300], [70], [16], True),
    ([257], [0], [64], False),            # vanilla sliding window (no reference prefix)
    ([200], [200], [4], False),           # prefix only
    ([333], [130], [400], False),         # window longer than the outputs: causal outputs
    ([129, 1, 0, 400, 64], [64, 1, 0, 17, 63], [128, 1, 5, 1, 2], False),  # packed, ragged
    ([640], [272], [128], False),         # single-page prefix, several tiles each side
    ([520], [300], [128], True),
    ([1100], [700], [128], False),        # long prefix: the unrolled mask-free key loops
    ([700, 330, 290], [272, 272, 16], [128, 128, 128], False),  # packed training documents
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_small_every_row(wa, case):
    lens, m, n, pc = CASES[case]
    pw = W.make_prefill("small", 4, lens, m, n, seed=40 + case, prefix_causal=pc)
    g = W.make_output_grad(pw, seed=case)
    _, lse, dq, dk, dv = run_training(wa, pw, g)
    total = int(pw.cu_seqlens[-1])
    ref = [np.zeros((total, 16, 128)) for _ in range(3)]
    for b in range(pw.nseq):
        s0, s1 = int(pw.cu_seqlens[b]), int(pw.cu_seqlens[b + 1])
        if s1 == s0:
            continue
        for r, x in zip(ref, oracle_doc(pw, g, b)):
            r[s0:s1] = x
        lerr = float(np.abs(lse[s0:s1] - oracle_lse(pw, b)).max())
        assert lerr <= LSE_TOL, f"document {b}: lse max abs err {lerr}"
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_grads(f"case {case} {name}", got, r)


def test_forward_with_lse_equals_inference_forward(wa):
    pw = W.make_prefill("fwd", 4, [500, 77], [200, 5], [64, 8], seed=60)
    q, k, v = upload(pw.q, "bf16"), upload(pw.k, "bf16"), upload(pw.v, "bf16")
    cu = torch.tensor(pw.cu_seqlens, dtype=torch.int32, device="cuda")
    m = torch.tensor(pw.prefix_len, dtype=torch.int32, device="cuda")
    n = torch.tensor(pw.window, dtype=torch.int32, device="cuda")
    for dt in (torch.float32, torch.bfloat16):
        a = wa.rswa_prefill_attn(q, k, v, cu, m, n, out_dtype=dt)
        b, _ = wa.rswa_prefill_fwd(q, k, v, cu, m, n, out_dtype=dt)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16) if dt == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if dt == torch.bfloat16 else b.view(torch.int32))


def test_bf16_gradients_are_rne_of_f32(wa):
    pw = W.make_prefill("rne", 4, [400, 90], [100, 0], [32, 16], seed=61)
    g = W.make_output_grad(pw, seed=61)
    f32 = run_training(wa, pw, g, grad_dtype=torch.float32)
    bf = run_training(wa, pw, g, grad_dtype=torch.bfloat16)
    for i in (2, 3, 4):
        np.testing.assert_array_equal(W.bf16_bits(bf[i]), W.bf16_bits(f32[i]))


def test_float32_forward_output_gives_the_same_gradients(wa):
    """delta may come from a float32 or a bf16 forward output; both stay within tolerance."""
    pw = W.make_prefill("f32out", 4, [450], [200], [64], seed=62)
    g = W.make_output_grad(pw, seed=62)
    _, _, dq, dk, dv = run_training(wa, pw, g, out_dtype=torch.float32)
    ref = oracle_doc(pw, g, 0)
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_grads(f"f32 out {name}", got, r)


def sample_rows(S, m, n, rng, extra=24):
    s = {0, 1, m - 1, m, m + 1, m + n - 1, m + n, S - 2, S - 1}
    s |= set(rng.integers(0, S, size=extra).tolist())
    return np.array(sorted(x for x in s if 0 <= x < S))


def test_backward_full_32k_sampled(wa):
    """One 32768-token document with a 40-page bidirectional prefix (m = 10256, n = 128): dQ on
    sampled query rows and dK, dV on sampled key rows of two heads, the oracle forming every
    query's contribution to those keys."""
    pw = W.prefill_config(seed=3)
    g = W.make_output_grad(pw, seed=3)
    _, lse, dq, dk, dv = run_training(wa, pw, g)
    S, m, n = 32768, int(pw.prefix_len[0]), int(pw.window[0])
    rng = np.random.default_rng(5)
    rows = sample_rows(S, m, n, rng)
    heads = [3, 12]
    rq, rk, rv = oracle_doc(pw, g, 0, heads=heads, q_rows=rows, k_rows=rows)
    check_grads("32K dq", dq[rows][:, heads], rq)
    check_grads("32K dk", dk[rows][:, heads], rk)
    check_grads("32K dv", dv[rows][:, heads], rv)
    lerr = float(np.abs(lse[rows] - oracle_lse(pw, 0, rows=rows)).max())
    assert lerr <= LSE_TOL


def test_backward_packed_training_row_sampled(wa):
    """A 32768-token training row packed with documents of their own prefix lengths: the small
    documents on every row of one head, the large one on sampled rows."""
    pw = W.packed_training_config(seed=0)
    g = W.make_output_grad(pw, seed=8)
    _, _, dq, dk, dv = run_training(wa, pw, g)
    rng = np.random.default_rng(9)
    for b in range(pw.nseq):
        s0, s1 = int(pw.cu_seqlens[b]), int(pw.cu_seqlens[b + 1])
        S, m, n = s1 - s0, int(pw.prefix_len[b]), int(pw.window[b])
        rows = np.arange(S) if S <= 2048 else sample_rows(S, m, n, rng)
        heads = [b % 16]
        ref = oracle_doc(pw, g, b, heads=heads, q_rows=rows, k_rows=rows)
        for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            check_grads(f"packed doc {b} {name}", got[s0:s1][rows][:, heads], r)


def test_work_array_holds_log2_lse_and_negated_delta(wa):
    """The work array the backward fills, head-major: [0][h][token] = lse * log2(e) and
    [1][h][token] = -delta, with delta the row sum of dO * O over the forward output as passed,
    checked against that definition on the host (float64 sums of the same bf16 values; the kernel
    sums 128 products in float32)."""
    pw = W.make_prefill("work", 4, [300, 90], [100, 0], [32, 16], seed=63)
    g = W.make_output_grad(pw, seed=63)
    q, k, v = upload(pw.q, "bf16"), upload(pw.k, "bf16"), upload(pw.v, "bf16")
    dout = upload(g, "bf16")
    cu = torch.tensor(pw.cu_seqlens, dtype=torch.int32, device="cuda")
    m = torch.tensor(pw.prefix_len, dtype=torch.int32, device="cuda")
    n = torch.tensor(pw.window, dtype=torch.int32, device="cuda")
    out, lse = wa.rswa_prefill_fwd(q, k, v, cu, m, n, out_dtype=torch.bfloat16)
    total, heads, _ = q.shape
    work = torch.full((2, heads, total), float("nan"), dtype=torch.float32, device="cuda")
    wa.rswa_prefill_bwd(q, k, v, out, dout, lse, cu, m, n, work=work)
    torch.cuda.synchronize()
    o = out.double().cpu().numpy()
    d = dout.double().cpu().numpy()
    delta = (o * d).sum(-1)
    scale = (np.abs(o) * np.abs(d)).sum(-1).max()
    w = work.double().cpu().numpy().transpose(0, 2, 1)  # [2][token][h]
    assert np.abs(w[1] + delta).max() <= 1e-5 * scale
    lse64 = lse.double().cpu().numpy()
    np.testing.assert_allclose(w[0], lse64 * np.log2(np.e), rtol=1e-6, atol=1e-6)
