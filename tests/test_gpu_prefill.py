"""GPU parity of K3 (R-SWA-masked prefill on bf16 MFMA) against the fp64 oracle.

Small packed batches are compared on every row; the full 32768-token sequence (40-page prefix,
m = 10256) on sampled rows, which the oracle computes one by one. Tolerance: max-abs error
<= 1e-2 on the float32 output (P is rounded to bf16 for the PV product); the bf16 output must be
exactly the round-to-nearest-even of the float32 output.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_common import Trajectory, upload

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module")
def wa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import windowed_attention_amd
    return windowed_attention_amd


def run_prefill(wa, pw, out_dtype=torch.float32):
    q, k, v = upload(pw.q, "bf16"), upload(pw.k, "bf16"), upload(pw.v, "bf16")
    cu = torch.tensor(pw.cu_seqlens, dtype=torch.int32, device="cuda")
    m = torch.tensor(pw.prefix_len, dtype=torch.int32, device="cuda")
    n = torch.tensor(pw.window, dtype=torch.int32, device="cuda")
    out = wa.rswa_prefill_attn(q, k, v, cu, m, n, out_dtype=out_dtype,
                               prefix_causal=pw.prefix_causal)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def oracle_seq(pw, b, rows=None):
    q, k, v = pw.seq(b)
    f = lambda x: W.to_f64(x, "bf16")
    return O.prefill(f(q), f(k), f(v), int(pw.prefix_len[b]), int(pw.window[b]),
                     pw.prefix_causal, rows=rows)


CASES = [
    # (sequence lengths, prefix lengths, windows, causal prefix)
    ([300], [70], [16], False),
    ([300], [70], [16], True),
    ([257], [0], [64], False),            # vanilla sliding window (no reference prefix)
    ([200], [200], [4], False),           # prefix only
    ([333], [130], [400], False),         # window longer than the outputs: causal outputs
    ([129, 1, 0, 400, 64], [64, 1, 0, 17, 63], [128, 1, 5, 1, 2], False),  # packed, ragged
    ([640], [272], [128], False),         # single-page prefix, several tiles each side
    ([520], [300], [128], True),
    ([1100], [700], [128], False),        # long prefix: the unrolled mask-free key loops
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_small_every_row(wa, case):
    lens, m, n, pc = CASES[case]
    pw = W.make_prefill("small", 4, lens, m, n, seed=case, prefix_causal=pc)
    got = run_prefill(wa, pw)
    for b in range(pw.nseq):
        s0, s1 = int(pw.cu_seqlens[b]), int(pw.cu_seqlens[b + 1])
        if s1 == s0:
            continue
        ref = oracle_seq(pw, b)
        err = float(np.abs(got[s0:s1] - ref).max())
        assert err <= TOL, f"sequence {b}: max abs err {err}"


def test_prefill_bf16_output_is_rne_of_f32(wa):
    pw = W.make_prefill("rne", 4, [400, 90], [100, 0], [32, 16], seed=11)
    f32 = run_prefill(wa, pw, torch.float32)
    bf = run_prefill(wa, pw, torch.bfloat16)
    np.testing.assert_array_equal(W.bf16_bits(bf), W.bf16_bits(f32))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_prefill_wide_row_offsets_match(wa, out_dtype):
    """A launch whose max_seqlen * heads * 128 reaches 2^31 forms its K / V row offsets in 64 bits
    instead of with the 24-bit multiply; both must give the same output bit for bit. (max_seqlen
    only sizes the grid: the workgroups past each sequence's end exit at once.)"""
    pw = W.make_prefill("wide", 4, [300, 129], [70, 64], [16, 128], seed=21)
    q, k, v = upload(pw.q, "bf16"), upload(pw.k, "bf16"), upload(pw.v, "bf16")
    cu = torch.tensor(pw.cu_seqlens, dtype=torch.int32, device="cuda")
    m = torch.tensor(pw.prefix_len, dtype=torch.int32, device="cuda")
    n = torch.tensor(pw.window, dtype=torch.int32, device="cuda")
    H = q.shape[1]
    wide = (1 << 31) // (H * 128)
    narrow = wa.rswa_prefill_attn(q, k, v, cu, m, n, out_dtype=out_dtype, max_seqlen=300)
    widened = wa.rswa_prefill_attn(q, k, v, cu, m, n, out_dtype=out_dtype, max_seqlen=wide)
    torch.cuda.synchronize()
    bits = torch.int32 if out_dtype == torch.float32 else torch.int16
    assert torch.equal(narrow.view(bits), widened.view(bits))
    ref = oracle_seq(pw, 0)
    assert float(np.abs(widened[:300].float().cpu().numpy() - ref).max()) <= TOL


def test_prefill_rows_match_decode_steps(wa):
    """The teacher-forced row of output t equals decode step t on the same inputs (both K3 and
    K2 against the oracle, and against each other)."""
    m, n, T = 272, 128, 300
    S = m + T
    pw = W.make_prefill("consist", 4, [S], [m], [n], seed=12)
    pre = run_prefill(wa, pw)
    wl = W.make_decode("consist", 4, "bf16", [m], [n], [T], seed=12)
    # feed the decode path the prefill sequence's own Q/K/V
    wl.prefix_k[:] = pw.k[:m]
    wl.prefix_v[:] = pw.v[:m]
    wl.q[:, 0] = pw.q[m:]
    wl.k[:, 0] = pw.k[m:]
    wl.v[:, 0] = pw.v[m:]
    tr = Trajectory(wa, wl, wa.MODE_RSWA)
    dec = tr.run(range(1, T + 1))
    tr.cache.close()
    for t in range(1, T + 1):
        assert float(np.abs(dec[t][0] - pre[m + t - 1]).max()) <= TOL
    ref = oracle_seq(pw, 0, rows=np.arange(m, S))
    assert float(np.abs(pre[m:] - ref).max()) <= TOL


@pytest.mark.slow
def test_prefill_full_sequence_sampled_rows(wa):
    pw = W.prefill_config()
    got = run_prefill(wa, pw)
    S, m = int(pw.cu_seqlens[-1]), int(pw.prefix_len[0])
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([
        [0, 1, 63, 64, 127, 128, m - 129, m - 128, m - 1, m, m + 1, m + 127, m + 128, m + 129,
         S - 129, S - 128, S - 2, S - 1],
        rng.integers(0, m, 24), rng.integers(m, S, 40)]))
    ref = oracle_seq(pw, 0, rows=rows)
    err = float(np.abs(got[rows] - ref).max())
    print(f"prefill S={S} m={m}: max abs err {err:.3e} over {rows.size} sampled rows")
    assert err <= TOL


def test_prefill_metadata_checked_on_device(wa):
    """max_seqlen below a sequence's length leaves that sequence's rows past max_seqlen unwritten:
    the kernels report it through the device error word that rswa_prefill_check() reads (and
    clears); a launch whose metadata is right reports nothing. Forward and backward."""
    pw = W.make_prefill("meta", 4, [300, 129], [70, 64], [16, 128], seed=22)
    q, k, v = upload(pw.q, "bf16"), upload(pw.k, "bf16"), upload(pw.v, "bf16")
    cu = torch.tensor(pw.cu_seqlens, dtype=torch.int32, device="cuda")
    m = torch.tensor(pw.prefix_len, dtype=torch.int32, device="cuda")
    n = torch.tensor(pw.window, dtype=torch.int32, device="cuda")
    wa.rswa_prefill_check()  # start clean (raises if an earlier test left an error behind)
    out, lse = wa.rswa_prefill_fwd(q, k, v, cu, m, n, max_seqlen=300)
    wa.rswa_prefill_check()
    wa.rswa_prefill_attn(q, k, v, cu, m, n, max_seqlen=200)  # enqueued: the host cannot know
    with pytest.raises(wa.RswaError) as e:
        wa.rswa_prefill_check()
    assert e.value.status == -1
    wa.rswa_prefill_check()  # cleared by the read
    dout = upload(W.make_output_grad(pw, seed=1), "bf16")
    wa.rswa_prefill_bwd(q, k, v, out, dout, lse, cu, m, n, max_seqlen=300)
    wa.rswa_prefill_check()
    wa.rswa_prefill_bwd(q, k, v, out, dout, lse, cu, m, n, max_seqlen=100)
    with pytest.raises(wa.RswaError) as e:
        wa.rswa_prefill_check()
    assert e.value.status == -1
    wa.rswa_prefill_check()
