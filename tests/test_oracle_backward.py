"""Pins of the oracle's teacher-forced training pass (log-sum-exp and gradients), CPU only.

The gradients are pinned to things other than the oracle's own chain-rule formulas: torch's
autograd through its library attention with a mask built from torch's triangular routines,
central finite differences of the oracle's forward, exact invariants of softmax attention
(key gradients sum to zero, value gradients sum to the output gradients), closed forms for one key
and for identical keys, and packed documents equal to the documents run one at a time. The
mutation tests plant plausible mistakes in the oracle and check that these pins catch them.
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import rswa as Orswa
from test_oracle import torch_rswa_mask


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def autograd_grads(Q, K, V, dO, mask, scale=None):
    """dQ, dK, dV of sum(dO * SDPA(Q, K, V, mask)) by torch autograd, float64 CPU; arrays
    [S, H, d]; mask [S, S] bool (True = visible)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2), dtype=np.float64))
    q, k, v = (t(a).requires_grad_(True) for a in (Q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=torch.from_numpy(mask),
                                                         scale=scale)
    (o * t(dO)).sum().backward()
    return [g.grad.numpy().transpose(1, 0, 2) for g in (q, k, v)]


CASES = [(0, 4, 40, False), (9, 5, 37, False), (9, 5, 37, True), (16, 64, 70, False),
         (3, 100, 20, True), (30, 1, 33, False)]


@pytest.mark.parametrize("m,n,S,causal", CASES)
def test_backward_matches_autograd(m, n, S, causal):
    H, d = 2, 16
    Q, K, V, dO = (rnd((S, H, d), 100 + i) for i in range(4))
    got = O.prefill_backward(Q, K, V, dO, m, n, causal, block=7)
    ref = autograd_grads(Q, K, V, dO, torch_rswa_mask(S, m, n, causal))
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-11)


def test_backward_finite_differences():
    """Central differences of L = sum(dO * O) through the oracle's forward."""
    m, n, S, H, d = 3, 2, 8, 1, 4
    Q, K, V, dO = (rnd((S, H, d), 110 + i) for i in range(4))
    dQ, dK, dV = O.prefill_backward(Q, K, V, dO, m, n)
    loss = lambda q, k, v: float((O.prefill(q, k, v, m, n) * dO).sum())
    eps = 1e-6
    rng = np.random.default_rng(7)
    for which, grad in ((0, dQ), (1, dK), (2, dV)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in (S, H, d))
            args_p = [Q.copy(), K.copy(), V.copy()]
            args_m = [Q.copy(), K.copy(), V.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7, (which, idx, fd, grad[idx])


@pytest.mark.parametrize("m,n,S,causal", [(12, 5, 50, False), (12, 5, 50, True), (0, 7, 30, False)])
def test_backward_invariants(m, n, S, causal):
    """Shifting every key by one vector leaves every softmax unchanged, so the key gradients
    sum to zero; each probability row sums to one, so the value gradients sum to the output
    gradients."""
    H, d = 3, 8
    Q, K, V, dO = (rnd((S, H, d), 120 + i) for i in range(4))
    _, dK, dV = O.prefill_backward(Q, K, V, dO, m, n, causal, block=16)
    np.testing.assert_allclose(dK.sum(axis=0), 0.0, atol=1e-11)
    np.testing.assert_allclose(dV.sum(axis=0), dO.sum(axis=0), atol=1e-11)


def test_backward_single_key():
    """One token: its softmax is the constant 1, so dQ = dK = 0 and dV = dO."""
    for m in (0, 1):
        Q, K, V, dO = (rnd((1, 2, 8), 130 + i) for i in range(4))
        dQ, dK, dV = O.prefill_backward(Q, K, V, dO, m, 4)
        np.testing.assert_array_equal(dQ, 0.0)
        np.testing.assert_array_equal(dK, 0.0)
        np.testing.assert_allclose(dV, dO, atol=0)


def test_selected_rows_and_heads_are_slices_of_the_full_result():
    m, n, S, H, d = 10, 6, 45, 3, 8
    Q, K, V, dO = (rnd((S, H, d), 140 + i) for i in range(4))
    full = O.prefill_backward(Q, K, V, dO, m, n, block=9)
    qr, kr, hs = np.array([0, 9, 10, 44, 17]), np.array([3, 44, 10, 11]), [2, 0]
    part = O.prefill_backward(Q, K, V, dO, m, n, heads=hs, q_rows=qr, k_rows=kr, block=13)
    np.testing.assert_allclose(part[0], full[0][qr][:, hs], atol=1e-12)
    np.testing.assert_allclose(part[1], full[1][kr][:, hs], atol=1e-12)
    np.testing.assert_allclose(part[2], full[2][kr][:, hs], atol=1e-12)


def test_packed_documents_equal_documents_one_at_a_time():
    """Several prefix + output documents packed into one sequence, each with its own prefix
    length, attend only inside themselves: autograd over the packed sequence with a
    block-diagonal library mask equals the oracle run per document."""
    docs = [(5, 17, 4), (0, 9, 3), (11, 30, 8), (2, 2, 5)]  # (m, length, n)
    H, d = 2, 8
    S = sum(L for _, L, _ in docs)
    Q, K, V, dO = (rnd((S, H, d), 150 + i) for i in range(4))
    mask = torch.block_diag(*[torch.from_numpy(torch_rswa_mask(L, m, n, False))
                              for m, L, n in docs]).numpy()
    ref = autograd_grads(Q, K, V, dO, mask)
    off = 0
    for m, L, n in docs:
        sl = slice(off, off + L)
        got = O.prefill_backward(Q[sl], K[sl], V[sl], dO[sl], m, n)
        for g, r in zip(got, ref):
            np.testing.assert_allclose(g, r[sl], atol=1e-11)
        off += L


@pytest.mark.parametrize("m,n,S,causal", CASES[:4])
def test_lse_matches_library(m, n, S, causal):
    H, d = 2, 16
    Q, K = rnd((S, H, d), 160), rnd((S, H, d), 161)
    got = O.prefill_lse(Q, K, m, n, causal, block=5)
    z = torch.from_numpy(np.einsum("phd,khd->hpk", Q, K) / np.sqrt(d))
    z = z.masked_fill(~torch.from_numpy(torch_rswa_mask(S, m, n, causal)), -float("inf"))
    np.testing.assert_allclose(got, torch.logsumexp(z, dim=-1).numpy().T, atol=1e-12)


def test_lse_identical_keys_closed_form():
    """All keys equal: every visible score is s = scale q.k, so lse = s + log(#visible), with
    #visible = m for a prefix query (p + 1 if the prefix is causal) and m + min(n, p - m + 1) for
    output query p."""
    m, n, S, H, d = 6, 4, 20, 1, 8
    key = rnd((1, H, d), 170)
    K = np.repeat(key, S, axis=0)
    Q = rnd((S, H, d), 171)
    for causal in (False, True):
        got = O.prefill_lse(Q, K, m, n, causal)
        for p in range(S):
            cnt = (p + 1 if causal else m) if p < m else m + min(n, p - m + 1)
            s = float(Q[p, 0] @ key[0, 0]) / np.sqrt(d)
            assert abs(got[p, 0] - (s + np.log(cnt))) < 1e-12


# ---------------------------------------------------------------------------------------------
# planted mistakes: each must fail a pin above
# ---------------------------------------------------------------------------------------------
def test_mutation_softmax_correction_dropped_is_caught(monkeypatch):
    monkeypatch.setattr(Orswa, "softmax_grad", lambda P, dP: P * dP)
    with pytest.raises(AssertionError):
        test_backward_invariants(12, 5, 50, False)
    with pytest.raises(AssertionError):
        test_backward_matches_autograd(9, 5, 37, False)


def test_mutation_softmax_grad_sign_is_caught(monkeypatch):
    real = Orswa.softmax_grad
    monkeypatch.setattr(Orswa, "softmax_grad", lambda P, dP: -real(P, dP))
    with pytest.raises(AssertionError):
        test_backward_finite_differences()


def test_mutation_window_off_by_one_in_backward_is_caught(monkeypatch):
    real = Orswa.prefill_visible

    def wider(p, k, m, n, prefix_causal=False):
        return real(p, k, m, n + 1, prefix_causal)
    monkeypatch.setattr(Orswa, "prefill_visible", wider)
    with pytest.raises(AssertionError):
        test_backward_matches_autograd(9, 5, 37, False)


def test_mutation_wrong_scale_in_backward_is_caught(monkeypatch):
    monkeypatch.setattr(Orswa, "default_scale", lambda d: 1.0 / d)
    with pytest.raises(AssertionError):
        test_backward_matches_autograd(16, 64, 70, False)
    with pytest.raises(AssertionError):
        test_lse_matches_library(16, 64, 70, False)


def test_mutation_transposed_output_gradient_is_caught(monkeypatch):
    real = Orswa.prefill_backward

    def flipped(Q, K, V, dO, *a, **kw):
        return real(Q, K, V, np.ascontiguousarray(dO[:, :, ::-1]), *a, **kw)
    monkeypatch.setattr(O, "prefill_backward", flipped)
    with pytest.raises(AssertionError):
        test_backward_finite_differences()
