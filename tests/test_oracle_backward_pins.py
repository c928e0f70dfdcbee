"""Pins for the oracle's backward functions, independent of their code.

* Adjoint identities against the oracle's forward ``apply`` (itself pinned in
  test_oracle_pins.py): the routed forward is linear in x, in A, in B and in
  the per-pair gate weights separately, so for any direction V,
  <gy, apply(0, ...V...)> equals <gradient, V> exactly (up to rounding).
  A transposed operand, a wrong scale, a wrong token index or a dropped pair
  breaks one of them.
* torch.autograd (fp64, CPU) on forwards written as the pages define them:
  the weighted sum of the selected adapters' LoRA deltas; the softmax over the
  selected logits; the ReLU MLP router.
* Central finite differences of the oracle's route_topk weights and router
  logits, and closed forms (two-way softmax = logistic function).
"""
import numpy as np
import pytest
import torch

from oracle import (apply, apply_backward, dispatch, route_topk, route_topk_backward, router_backward,
                    router_logits)


def _case(seed, N, d_in, d_out, K, r, k, unrouted=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, d_in))
    gy = rng.standard_normal((N, d_out))
    A = rng.standard_normal((K, d_in, r)) * 0.3
    B = rng.standard_normal((K, r, d_out)) * 0.3
    logits = rng.standard_normal((N, K))
    idx, w, _ = route_topk(logits, k)
    idx = idx.copy()
    if unrouted > 0:
        drop = rng.random(idx.shape) < unrouted
        idx[drop] = -1
    return rng, x, gy, A, B, idx, w


SHAPES = [(7, 5, 3, 1, 2, 1), (16, 6, 9, 3, 4, 1), (19, 8, 5, 4, 3, 2), (23, 4, 7, 5, 2, 3), (11, 3, 3, 2, 1, 2)]


@pytest.mark.parametrize("N,d_in,d_out,K,r,k", SHAPES)
@pytest.mark.parametrize("unrouted", [0.0, 0.3])
def test_apply_backward_adjoint_identities(N, d_in, d_out, K, r, k, unrouted):
    rng, x, gy, A, B, idx, w = _case(N * 7 + K, N, d_in, d_out, K, r, k, unrouted)
    scale = 0.75
    counts, offsets, perm, perm_w, inv = dispatch(idx, w, K)
    dx, dA, dB, dw = apply_backward(x, gy, A, B, scale, perm, perm_w, offsets, k)
    zero = np.zeros((N, d_out))

    def inner(y):
        return float(np.sum(gy * y))

    V = rng.standard_normal(x.shape)
    assert inner(apply(zero, V, A, B, scale, perm, perm_w, offsets, k)) == pytest.approx(float(np.sum(dx * V)),
                                                                                        rel=1e-10, abs=1e-10)
    VA = rng.standard_normal(A.shape)
    assert inner(apply(zero, x, VA, B, scale, perm, perm_w, offsets, k)) == pytest.approx(float(np.sum(dA * VA)),
                                                                                         rel=1e-10, abs=1e-10)
    VB = rng.standard_normal(B.shape)
    assert inner(apply(zero, x, A, VB, scale, perm, perm_w, offsets, k)) == pytest.approx(float(np.sum(dB * VB)),
                                                                                         rel=1e-10, abs=1e-10)
    # gate weights: a direction v over pairs enters the forward through perm_w = v[perm]
    v = rng.standard_normal(N * k)
    got = inner(apply(zero, x, A, B, scale, perm, v[np.asarray(perm, np.int64)], offsets, k))
    assert got == pytest.approx(float(np.sum(dw * v)), rel=1e-10, abs=1e-10)
    # unrouted pairs carry no gradient
    assert np.all(dw[np.asarray(inv) < 0] == 0.0)


def _torch_forward(x, A, B, scale, idx, w):
    """Figure 2's weighted sum written per token slot: y_t = sum_j w_tj * scale * (x_t A_e) B_e."""
    N, k = idx.shape
    rows = []
    for t in range(N):
        acc = torch.zeros(B.shape[2], dtype=torch.float64)
        for j in range(k):
            e = int(idx[t, j])
            if e < 0:
                continue
            acc = acc + w[t, j] * scale * ((x[t] @ A[e]) @ B[e])
        rows.append(acc)
    return torch.stack(rows)


@pytest.mark.parametrize("N,d_in,d_out,K,r,k", SHAPES[:4])
def test_apply_backward_matches_autograd(N, d_in, d_out, K, r, k):
    rng, x, gy, A, B, idx, w = _case(N + 100 * k, N, d_in, d_out, K, r, k, 0.2)
    scale = 0.5
    counts, offsets, perm, perm_w, inv = dispatch(idx, w, K)
    dx, dA, dB, dw = apply_backward(x, gy, A, B, scale, perm, perm_w, offsets, k)
    xt = torch.tensor(x, requires_grad=True)
    At = torch.tensor(A, requires_grad=True)
    Bt = torch.tensor(B, requires_grad=True)
    wt = torch.tensor(np.asarray(w, np.float64).reshape(N, k), requires_grad=True)
    y = _torch_forward(xt, At, Bt, scale, np.asarray(idx).reshape(N, k), wt)
    y.backward(torch.tensor(gy))
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dA, At.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dB, Bt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dw, wt.grad.numpy().reshape(-1), rtol=1e-11, atol=1e-11)


def test_apply_backward_single_adapter_is_plain_lora_gradient():
    """K = 1, k = 1, w = 1: the textbook LoRA gradients dA = s x^T gy B^T, dB = s (xA)^T gy,
    dx = s gy B^T A^T."""
    rng = np.random.default_rng(3)
    N, d_in, d_out, r, s = 9, 6, 5, 3, 0.25
    x, gy = rng.standard_normal((N, d_in)), rng.standard_normal((N, d_out))
    A, B = rng.standard_normal((1, d_in, r)), rng.standard_normal((1, r, d_out))
    idx = np.zeros(N, np.int32)
    w = np.ones(N)
    counts, offsets, perm, perm_w, inv = dispatch(idx, w, 1)
    dx, dA, dB, dw = apply_backward(x, gy, A, B, s, perm, perm_w, offsets, 1)
    np.testing.assert_allclose(dA[0], s * np.einsum("ti,tc,jc->ij", x, gy, B[0]), rtol=1e-12)
    np.testing.assert_allclose(dB[0], s * np.einsum("ti,ij,tc->jc", x, A[0], gy), rtol=1e-12)
    np.testing.assert_allclose(dx, s * np.einsum("tc,jc,ij->ti", gy, B[0], A[0]), rtol=1e-12)


def test_apply_backward_empty_adapter_and_gy_zero():
    rng, x, gy, A, B, idx, w = _case(5, 12, 4, 4, 3, 2, 1)
    idx = np.where(idx == 1, 0, idx)  # adapter 1 gets no pair
    counts, offsets, perm, perm_w, inv = dispatch(idx, w, 3)
    dx, dA, dB, dw = apply_backward(x, gy, A, B, 1.0, perm, perm_w, offsets, 1)
    assert np.all(dA[1] == 0) and np.all(dB[1] == 0)
    dx0, dA0, dB0, dw0 = apply_backward(x, np.zeros_like(gy), A, B, 1.0, perm, perm_w, offsets, 1)
    assert not dx0.any() and not dA0.any() and not dB0.any() and not dw0.any()


@pytest.mark.parametrize("K,k", [(2, 1), (2, 2), (4, 2), (6, 3), (8, 8)])
def test_route_topk_backward_finite_differences(K, k):
    rng = np.random.default_rng(K * 10 + k)
    N = 13
    logits = rng.standard_normal((N, K)) * 2.0
    idx, w, _ = route_topk(logits, k)
    dw = rng.standard_normal((N, k))
    dl = route_topk_backward(w, idx, dw, K)
    eps = 1e-6
    fd = np.zeros((N, K))
    for e in range(K):
        lp, lm = logits.copy(), logits.copy()
        lp[:, e] += eps
        lm[:, e] -= eps
        ip, wp, _ = route_topk(lp, k)
        im, wm, _ = route_topk(lm, k)
        assert (ip == idx).all() and (im == idx).all()  # no selection change at this step
        fd[:, e] = (np.sum(dw * wp, axis=1) - np.sum(dw * wm, axis=1)) / (2 * eps)
    np.testing.assert_allclose(dl, fd, rtol=1e-6, atol=1e-8)
    # a softmax is shift invariant: each token's logit gradients sum to 0; unselected get 0
    np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-12)
    sel = np.zeros((N, K), bool)
    np.put_along_axis(sel, idx.astype(np.int64), True, axis=1)
    assert np.all(dl[~sel] == 0.0)


def test_route_topk_backward_two_way_is_logistic_derivative():
    """k = 2 of K = 2: w_0 = sigmoid(l_0 - l_1), so dL/dl_0 = w_0 w_1 (dw_0 - dw_1) = -dL/dl_1."""
    l = np.array([[0.3, -1.1], [2.0, 2.5]])
    idx, w, _ = route_topk(l, 2)
    dw = np.array([[1.5, -0.5], [0.25, 3.0]])
    dl = route_topk_backward(w, idx, dw, 2)
    sig = 1.0 / (1.0 + np.exp(-(l[:, 0] - l[:, 1])))
    expect0 = sig * (1 - sig) * (dw[:, 0] - dw[:, 1])
    np.testing.assert_allclose(dl[:, 0], expect0, rtol=1e-13)
    np.testing.assert_allclose(dl[:, 1], -expect0, rtol=1e-13)


def test_route_topk_backward_matches_autograd():
    rng = np.random.default_rng(9)
    N, K, k = 17, 7, 3
    logits = rng.standard_normal((N, K))
    idx, w, _ = route_topk(logits, k)
    dw = rng.standard_normal((N, k))
    lt = torch.tensor(logits, requires_grad=True)
    sel = torch.gather(lt, 1, torch.tensor(idx.astype(np.int64)))
    torch.softmax(sel, dim=1).backward(torch.tensor(dw))
    np.testing.assert_allclose(route_topk_backward(w, idx, dw, K), lt.grad.numpy(), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("with_b1", [True, False])
def test_router_backward_matches_autograd_and_adjoint(with_b1):
    rng = np.random.default_rng(21 + with_b1)
    N, d, H, K = 11, 9, 6, 4
    x = rng.standard_normal((N, d))
    W1 = rng.standard_normal((d, H)) * 0.5
    b1 = rng.standard_normal(H) * 0.5 if with_b1 else None
    W2 = rng.standard_normal((H, K)) * 0.5
    b2 = rng.standard_normal(K)
    dl = rng.standard_normal((N, K))
    dW1, db1, dW2, db2, dx = router_backward(x, W1, b1, W2, dl)
    xt, W1t, W2t, b2t = (torch.tensor(v, requires_grad=True) for v in (x, W1, W2, b2))
    b1t = torch.tensor(b1, requires_grad=True) if with_b1 else None
    a = xt @ W1t + (b1t if with_b1 else 0.0)
    (torch.relu(a) @ W2t + b2t).backward(torch.tensor(dl))
    for got, ref in ((dW1, W1t), (dW2, W2t), (db2, b2t), (dx, xt)):
        np.testing.assert_allclose(got, ref.grad.numpy(), rtol=1e-12, atol=1e-12)
    if with_b1:
        np.testing.assert_allclose(db1, b1t.grad.numpy(), rtol=1e-12, atol=1e-12)
    # logits are linear in W2: <dl, logits(W2 = V) - logits(W2 = 0)> = <dW2, V>
    V = rng.standard_normal(W2.shape)
    lin = router_logits(x, W1, b1, V, None) - router_logits(x, W1, b1, np.zeros_like(V), None)
    assert float(np.sum(dl * lin)) == pytest.approx(float(np.sum(dW2 * V)), rel=1e-11)
    # a finite difference on W1 (central, fp64) away from the ReLU's kink
    pre = x @ W1 + (b1 if with_b1 else 0.0)
    assert np.min(np.abs(pre)) > 1e-4
    i, j, eps = 2, 3, 1e-7
    Wp, Wm = W1.copy(), W1.copy()
    Wp[i, j] += eps
    Wm[i, j] -= eps
    fd = (np.sum(dl * router_logits(x, Wp, b1, W2, b2)) - np.sum(dl * router_logits(x, Wm, b1, W2, b2))) / (2 * eps)
    assert fd == pytest.approx(dW1[i, j], rel=1e-6, abs=1e-9)


def test_backward_chain_on_a_synthetic_stress_slice():
    """The chain dL/dw -> dL/dlogits -> router parameters against torch.autograd of the whole
    routed forward (router MLP, top-k softmax, weighted LoRA sum), the selection taken from
    the oracle."""
    rng = np.random.default_rng(31)
    N, d, H, K, k, r, d_out = 12, 8, 6, 5, 2, 3, 7
    x = rng.standard_normal((N, d))
    W1, W2 = rng.standard_normal((d, H)), rng.standard_normal((H, K))
    A, B = rng.standard_normal((K, d, r)) * 0.3, rng.standard_normal((K, r, d_out)) * 0.3
    gy = rng.standard_normal((N, d_out))
    scale = 0.5
    logits = router_logits(x, W1, None, W2, None)
    idx, w, _ = route_topk(logits, k)
    counts, offsets, perm, perm_w, inv = dispatch(idx, w, K)
    dx_l, dA, dB, dw = apply_backward(x, gy, A, B, scale, perm, perm_w, offsets, k)
    dl = route_topk_backward(w, idx, dw.reshape(N, k), K)
    dW1, db1, dW2, db2, dx_r = router_backward(x, W1, None, W2, dl)
    xt, W1t, W2t, At, Bt = (torch.tensor(v, requires_grad=True) for v in (x, W1, W2, A, B))
    lg = torch.relu(xt @ W1t) @ W2t
    wt = torch.softmax(torch.gather(lg, 1, torch.tensor(idx.astype(np.int64))), dim=1)
    y = _torch_forward(xt, At, Bt, scale, idx, wt)
    y.backward(torch.tensor(gy))
    np.testing.assert_allclose(dx_l + dx_r, xt.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dW1, W1t.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dW2, W2t.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dA, At.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dB, Bt.grad.numpy(), rtol=1e-10, atol=1e-11)
