"""rswa_prefill_bwd_noalloc: the training backward without a caller work array (its work rows
live in a device array inside the library). Through the C ABI it must give rswa_prefill_bwd's
gradients bit for bit, on two calls in a row (the second with a smaller input, so the array
keeps the first call's rows beyond what the second uses), and refuse sizes past its array."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import upload


@pytest.fixture(scope="module")
def wa():
    import windowed_attention_amd
    return windowed_attention_amd


def test_noalloc_rejects_sizes_past_its_array(wa):
    """Host-checked before anything is enqueued (no GPU involved): 65537 tokens x 16 heads."""
    fake = ctypes.c_void_p(0x1000)
    st = wa._lib.rswa_prefill_bwd_noalloc(fake, fake, fake, fake, wa.BF16, fake, fake, fake, fake,
                                          fake, wa.BF16, fake, fake, fake, 1, 65537, 16, 128,
                                          65537, 0, ctypes.c_float(0.0), ctypes.c_void_p(None))
    assert st == -1
    assert b"scratch" in wa._lib.rswa_last_error()


def _run_pair(wa, pw, grad_dtype):
    q, k, v = upload(pw.q, "bf16"), upload(pw.k, "bf16"), upload(pw.v, "bf16")
    dout = upload(W.make_output_grad(pw, seed=3), "bf16")
    cu = torch.tensor(pw.cu_seqlens, dtype=torch.int32, device="cuda")
    m = torch.tensor(pw.prefix_len, dtype=torch.int32, device="cuda")
    n = torch.tensor(pw.window, dtype=torch.int32, device="cuda")
    S = int(np.diff(pw.cu_seqlens).max())
    out, lse = wa.rswa_prefill_fwd(q, k, v, cu, m, n, max_seqlen=S)
    ref = wa.rswa_prefill_bwd(q, k, v, out, dout, lse, cu, m, n, grad_dtype=grad_dtype,
                              max_seqlen=S)
    got = [torch.full_like(r, float("nan")) for r in ref]
    wa.rswa_prefill_bwd_noalloc(q, k, v, out, dout, lse, cu, m, n, dq=got[0], dk=got[1],
                                dv=got[2], max_seqlen=S)
    torch.cuda.synchronize()
    wa.rswa_prefill_check()
    return ref, got


@pytest.mark.gpu
def test_noalloc_equals_backward_on_two_calls(wa):
    bits = {torch.float32: torch.int32, torch.bfloat16: torch.int16}
    first = W.make_prefill("noalloc-a", 4, [700, 129, 300], [300, 64, 0], [128, 16, 64], seed=31)
    second = W.make_prefill("noalloc-b", 4, [200, 90], [70, 0], [32, 8], seed=32)
    for pw, gdt in ((first, torch.float32), (second, torch.bfloat16)):
        ref, got = _run_pair(wa, pw, gdt)
        for name, r, g in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(r.view(bits[gdt]), g.view(bits[gdt])), name
