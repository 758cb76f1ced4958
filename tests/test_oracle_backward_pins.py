"""Pins of the FP64 oracle's backward of the indexer scores (dq, dk, dw).

Each pin is chosen so that a plausible slip in the oracle's chain rule fails it:
  * exact finite differences (rational arithmetic) of the forward definition on tiny
    inputs: any wrong term, index, transposed operand or missing weight;
  * float64 autograd of a torch transcription of the forward definition at full head
    count and dimension (a different route to the same derivative);
  * homogeneity: the score is linear in w and positively homogeneous of degree one in q
    and in k, so sum(w * dw) = sum(q * dq) = sum(k * dk) = sum(g * I) (drops of a factor
    or of the mask break one of them);
  * closed form: one head, unit weight and positive inputs make the backward three plain
    masked matrix products;
  * the ReLU derivative at 0 is 0: with every dot product <= 0 (some exactly 0) every
    gradient is exactly zero;
  * invariants: segment packing and splitting a segment's queries over two calls.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from deterministic_score_top_amd import workloads as W
from tests.bruteforce import exact_dots, exact_loss, exact_values, visible_count


def _tables(wl):
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.tolist()
    return wl.cu_seqlens_q.tolist(), wl.cu_seqlens_k.tolist(), offs


@pytest.mark.parametrize("seed", [0, 1])
def test_exact_finite_differences(seed):
    H, D = 3, 2
    wl = W.random_segments([3, 0, 2, 2], [4, 2, 3, 2], [1, 0, 5, -1], topk=2, H=H, D=D, seed=seed)
    grad = W.draw_grad(wl.T, 4, seed=seed)
    dq, dk, dw = O.backward_workload(wl, grad)
    cu_q, cu_k, offs = _tables(wl)
    q = exact_values(wl.q.reshape(wl.T, -1))
    k = exact_values(wl.k)
    w = exact_values(wl.w)
    g = exact_values(grad)
    base_dots = exact_dots(q, k, cu_q, cu_k, offs, H, D)
    assert all(v != 0 for v in base_dots.values())      # no kink at the base point
    L0 = exact_loss(q, k, w, g, cu_q, cu_k, offs, H, D)
    eps = Fraction(1, 2 ** 50)

    def check(arr, i, j, got):
        arr[i][j] += eps
        dots = exact_dots(q, k, cu_q, cu_k, offs, H, D)
        assert all((dots[key] > 0) == (v > 0) for key, v in base_dots.items())   # same linear piece
        deriv = (exact_loss(q, k, w, g, cu_q, cu_k, offs, H, D) - L0) / eps
        arr[i][j] -= eps
        assert abs(got - float(deriv)) <= 1e-12 * max(1.0, abs(float(deriv))), (i, j, got, float(deriv))

    for t in range(wl.T):
        for x in range(H * D):
            check(q, t, x, dq[t].reshape(-1)[x])
        for h in range(H):
            check(w, t, h, dw[t, h])
    for s in range(wl.Tkv):
        for d in range(D):
            check(k, s, d, dk[s, d])


def test_autograd_of_forward_definition():
    wl = W.random_segments([9, 4, 0, 6], [12, 0, 5, 20], [2, 3, 0, 16], topk=4, seed=21)
    grad = W.draw_grad(wl.T, 20, seed=21)
    dq, dk, dw = O.backward_workload(wl, grad)
    q = wl.q.double().requires_grad_(True)
    k = wl.k.double().requires_grad_(True)
    w = wl.w.double().requires_grad_(True)
    cu_q, cu_k, offs = _tables(wl)
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(wl.T):
        _, first, n = visible_count(cu_q, cu_k, offs, t)
        if n == 0:
            continue
        S = torch.einsum("hd,sd->hs", q[t], k[first:first + n])
        I = (w[t][:, None] * torch.relu(S)).sum(0)
        loss = loss + (grad[t, :n].double() * I).sum()
    loss.backward()
    assert np.allclose(dq, q.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dk, k.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dw, w.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_homogeneity_identities():
    # a negative offset (first queries see nothing), an empty segment and a segment whose
    # last keys no query sees
    wl = W.random_segments([30, 0, 25, 12], [40, 5, 33, 30], [5, 0, 40, -4], topk=4, seed=3)
    grad = W.draw_grad(wl.T, 40, seed=3)
    dq, dk, dw = O.backward_workload(wl, grad)
    q64, k64, w64 = O.from_torch(wl.q, wl.k, wl.w)
    cu_q, cu_k, offs = _tables(wl)
    total = 0.0
    seen = np.zeros(wl.Tkv, dtype=bool)
    for t in range(wl.T):
        _, first, n = visible_count(cu_q, cu_k, offs, t)
        total += float(grad[t, :n].double().numpy() @ O.row_scores(q64, k64, w64, t, first, n))
        seen[first:first + n] = True
        if n == 0:
            assert not dq[t].any() and not dw[t].any()
    for lhs in (np.sum(w64 * dw), np.sum(q64 * dq), np.sum(k64 * dk)):
        assert abs(lhs - total) <= 1e-10 * max(1.0, abs(total))
    assert not dk[~seen].any() and (~seen).sum() > 0


def test_closed_form_one_head_positive():
    wl = W.random_segments([7, 5], [9, 6], [2, 0], topk=3, H=1, D=16, seed=4)
    wl.q = wl.q.abs() + 0.25
    wl.k = wl.k.abs() + 0.25
    wl.w = torch.ones_like(wl.w)
    grad = W.draw_grad(wl.T, 9, seed=4)
    dq, dk, dw = O.backward_workload(wl, grad)
    cu_q, cu_k, offs = _tables(wl)
    Gd = np.zeros((wl.T, wl.Tkv))
    for t in range(wl.T):
        _, first, n = visible_count(cu_q, cu_k, offs, t)
        Gd[t, first:first + n] = grad[t, :n].double().numpy()
    Q = wl.q.double().numpy()[:, 0, :]
    K = wl.k.double().numpy()
    assert np.allclose(dq[:, 0, :], Gd @ K, rtol=1e-13, atol=0)
    assert np.allclose(dk, Gd.T @ Q, rtol=1e-13, atol=0)
    assert np.allclose(dw[:, 0], (Gd * (Q @ K.T)).sum(1), rtol=1e-13, atol=0)


def test_relu_derivative_at_zero_is_zero():
    wl = W.random_segments([8, 4], [10, 6], [2, 0], topk=3, H=4, D=8, seed=5)
    gen = torch.Generator().manual_seed(5)
    u = torch.randn(8, generator=gen)
    a = torch.rand(wl.T, 4, 1, generator=gen) + 0.1
    b = torch.rand(wl.Tkv, 1, generator=gen) + 0.1
    q = (a * u).to(torch.bfloat16)
    q[:, :2, 4:] = 0          # heads 0, 1: support on dims 0..3 only
    k = (-b * u).to(torch.bfloat16)
    k[: wl.Tkv // 2, :4] = 0  # half the keys orthogonal to heads 0, 1: dots exactly 0
    wl.q, wl.k = q, k
    q64, k64, _ = O.from_torch(wl.q, wl.k, wl.w)
    dots = np.einsum("thd,sd->ths", q64, k64)
    assert (dots == 0).any()
    grad = W.draw_grad(wl.T, 10, seed=5)
    cu_q, cu_k, offs = _tables(wl)
    # only visible pairs matter: check that they are all <= 0
    for t in range(wl.T):
        _, first, n = visible_count(cu_q, cu_k, offs, t)
        assert (dots[t, :, first:first + n] <= 0).all()
    dq, dk, dw = O.backward_workload(wl, grad)
    assert not dq.any() and not dk.any() and not dw.any()


def test_invariant_segment_packing_and_query_split():
    wl = W.random_segments([6, 7], [8, 9], [1, 2], topk=3, H=4, D=8, seed=12)
    grad = W.draw_grad(wl.T, 9, seed=12).double().numpy()
    dq, dk, dw = O.backward_workload(wl, grad)
    q64, k64, w64 = O.from_torch(wl.q, wl.k, wl.w)
    a = O.backward_rows(q64[:6], k64[:8], w64[:6], np.array([0, 6]), np.array([0, 8]), np.array([1]), grad[:6])
    b = O.backward_rows(q64[6:], k64[8:], w64[6:], np.array([0, 7]), np.array([0, 9]), np.array([2]), grad[6:])
    assert np.array_equal(np.concatenate([a[0], b[0]]), dq)
    assert np.array_equal(np.concatenate([a[1], b[1]]), dk)
    assert np.array_equal(np.concatenate([a[2], b[2]]), dw)
    # the second segment's queries in two calls: dq, dw rows equal, dk adds up
    c = O.backward_rows(q64[6:9], k64[8:], w64[6:9], np.array([0, 3]), np.array([0, 9]), np.array([2]), grad[6:9])
    d = O.backward_rows(q64[9:], k64[8:], w64[9:], np.array([0, 4]), np.array([0, 9]), np.array([5]), grad[9:])
    assert np.array_equal(np.concatenate([c[0], d[0]]), dq[6:])
    assert np.array_equal(np.concatenate([c[2], d[2]]), dw[6:])
    assert np.allclose(c[1] + d[1], dk[8:], rtol=1e-14, atol=1e-14)
