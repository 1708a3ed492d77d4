"""Pins of the oracle's backward of the bf16 layer (no GPU).

The oracle writes the chain rule out token by token in fp32. It is checked
against a different formulation: the dense masked layer
y = sum_e M[:, e] * FFN_e(X) over all experts, in float64, differentiated by
torch's automatic differentiation (the loss is <dy, y>). Then: linearity in
dy (doubling dy doubles every gradient exactly), zero gradients for experts
no token selects, and independence of the thread count."""
import numpy as np
import pytest
import torch

import oracle


def _inputs(T, d, f, E, k, seed, unused=()):
    rng = np.random.default_rng(seed)
    bf = lambda a: oracle.f32_to_bf16_bits(np.asarray(a, np.float32)).reshape(np.shape(a))  # noqa: E731
    x = bf(rng.standard_normal((T, d)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    for e in unused:
        logits[:, e] = -1e9
    ids, w = oracle.route(logits, k, "softmax")
    w13 = [bf(rng.standard_normal((2 * f, d)) / np.sqrt(d)) for _ in range(E)]
    w2 = [bf(rng.standard_normal((d, f)) / np.sqrt(f)) for _ in range(E)]
    dy = bf(rng.standard_normal((T, d)))
    return x, ids, w, w13, w2, dy


def _dense_autograd(x, ids, w, w13, w2, dy):
    """dX, dW13, dW2, dtopk_w of <dy, y> for the dense masked layer, float64."""
    f64 = lambda b: torch.from_numpy(oracle.bf16_bits_to_f32(b).astype(np.float64))  # noqa: E731
    T, d = x.shape
    E, k = len(w13), ids.shape[1]
    X = f64(x).requires_grad_(True)
    W13 = [f64(a).requires_grad_(True) for a in w13]
    W2 = [f64(a).requires_grad_(True) for a in w2]
    M = torch.zeros(T, E, dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            M[t, ids[t, j]] = float(w[t, j])
    M.requires_grad_(True)
    y = torch.zeros(T, d, dtype=torch.float64)
    f = w13[0].shape[0] // 2
    for e in range(E):
        g = X @ W13[e][:f].T
        u = X @ W13[e][f:].T
        y = y + M[:, e:e + 1] * ((torch.nn.functional.silu(g) * u) @ W2[e].T)
    (y * f64(dy)).sum().backward()
    dtw = np.array([[M.grad[t, ids[t, j]].item() for j in range(k)] for t in range(T)])
    return X.grad.numpy(), [a.grad.numpy() for a in W13], [a.grad.numpy() for a in W2], dtw


def _close(a, b, tol):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    scale = max(np.abs(b).max(), 1e-30)
    assert np.abs(a - b).max() <= tol * scale, (np.abs(a - b).max(), scale)


@pytest.mark.parametrize("T,d,f,E,k", [(6, 32, 48, 4, 2), (5, 64, 32, 3, 3), (4, 16, 16, 1, 1)])
def test_backward_matches_autograd_of_the_dense_masked_layer(T, d, f, E, k):
    x, ids, w, w13, w2, dy = _inputs(T, d, f, E, k, seed=T + d)
    dx, dw13, dw2, dtw = oracle.moe_backward(x, ids, w, w13, w2, dy, h_exact=True)
    rx, r13, r2, rtw = _dense_autograd(x, ids, w, w13, w2, dy)
    _close(dx, rx, 1e-5)
    _close(dtw, rtw, 1e-5)
    for e in range(E):
        _close(dw13[e], r13[e], 1e-5)
        _close(dw2[e], r2[e], 1e-5)
    # the layer as run (h rounded to bf16, gradient passed through the rounding)
    dx_b, dw13_b, dw2_b, dtw_b = oracle.moe_backward(x, ids, w, w13, w2, dy)
    _close(dx_b, rx, 2e-2)
    _close(dtw_b, rtw, 2e-2)
    for e in range(E):
        _close(dw2_b[e], r2[e], 2e-2)


def test_backward_is_linear_in_dy_and_zero_for_unused_experts():
    x, ids, w, w13, w2, dy = _inputs(7, 32, 32, 5, 2, seed=3, unused=(4,))
    assert not (ids == 4).any()
    dx, dw13, dw2, dtw = oracle.moe_backward(x, ids, w, w13, w2, dy)
    dy2 = oracle.f32_to_bf16_bits(2 * oracle.bf16_bits_to_f32(dy)).reshape(dy.shape)
    dx2, dw13_2, dw2_2, dtw2 = oracle.moe_backward(x, ids, w, w13, w2, dy2)
    assert np.array_equal(dx2, 2 * dx) and np.array_equal(dtw2, 2 * dtw)
    for e in range(5):
        assert np.array_equal(dw13_2[e], 2 * dw13[e]) and np.array_equal(dw2_2[e], 2 * dw2[e])
    assert not dw13[4].any() and not dw2[4].any()


def test_backward_does_not_depend_on_the_thread_count():
    x, ids, w, w13, w2, dy = _inputs(9, 32, 48, 4, 2, seed=5)
    a = oracle.moe_backward(x, ids, w, w13, w2, dy, threads=1)
    b = oracle.moe_backward(x, ids, w, w13, w2, dy, threads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[3], b[3])
    for e in range(4):
        assert np.array_equal(a[1][e], b[1][e]) and np.array_equal(a[2][e], b[2][e])


def test_sampled_backward_matches_the_whole_backward():
    """moe_backward_sampled (per-entry, float64) against moe_backward (whole
    layer, fp32) on a small routed layer: same chain rule, same bf16 h."""
    rng = np.random.default_rng(11)
    T, d, f, E, k = 12, 64, 96, 4, 2
    x = oracle.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32)).reshape(T, d)
    dy = oracle.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32)).reshape(T, d)
    w13 = [oracle.f32_to_bf16_bits((rng.standard_normal((2 * f, d)) * d ** -0.5).astype(np.float32))
           .reshape(2 * f, d) for _ in range(E)]
    w2 = [oracle.f32_to_bf16_bits((rng.standard_normal((d, f)) * f ** -0.5).astype(np.float32))
          .reshape(d, f) for _ in range(E)]
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    rdx, r13, r2, rtw = oracle.moe_backward(x, ids, w, w13, w2, dy)
    used = sorted(set(ids.ravel().tolist()))
    at13 = [(e, r, c) for e in used for r, c in ((0, 0), (f - 1, d - 1), (f, 3), (2 * f - 1, 17))]
    at2 = [(e, m, n) for e in used for m, n in ((0, 0), (d - 1, f - 1), (5, 40))]
    s_dx, s13, s2, stw = oracle.moe_backward_sampled(x, ids, w, w13, w2, dy, dx_tokens=[0, 5, T - 1],
                                                     dw13_at=at13, dw2_at=at2,
                                                     dtw_at=list(range(T * k)), chunk=40)
    np.testing.assert_allclose(s_dx, rdx[[0, 5, T - 1]], rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(s13, [r13[e][r, c] for e, r, c in at13], rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(s2, [r2[e][m, n] for e, m, n in at2], rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(stw, rtw.ravel(), rtol=1e-4, atol=1e-5)


def test_expert_blocks_match_the_whole_backward():
    """moe_backward_expert (per expert, float64 matrix products over the
    expert's assignments) against moe_backward (whole layer, fp32, token by
    token): whole weight-gradient blocks of every expert, the routing-weight
    gradient of every assignment and every dx row (summed over experts)."""
    rng = np.random.default_rng(12)
    T, d, f, E, k = 14, 64, 96, 4, 2
    x = oracle.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32)).reshape(T, d)
    dy = oracle.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32)).reshape(T, d)
    w13 = [oracle.f32_to_bf16_bits((rng.standard_normal((2 * f, d)) * d ** -0.5).astype(np.float32))
           .reshape(2 * f, d) for _ in range(E)]
    w2 = [oracle.f32_to_bf16_bits((rng.standard_normal((d, f)) * f ** -0.5).astype(np.float32))
          .reshape(d, f) for _ in range(E)]
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 3] = -1e9   # expert 3 unused: zero blocks, no assignments
    ids, w = oracle.route(logits, k)
    rdx, r13, r2, rtw = oracle.moe_backward(x, ids, w, w13, w2, dy)
    dx = np.zeros((T, d))
    for e in range(E):
        asg = np.flatnonzero(ids.ravel() == e)
        b13, b2, dtw, share = oracle.moe_backward_expert(
            x, ids, w, e, w13[e], w2[e], dy, rows13=range(2 * f), cols13=range(d), rows2=range(d),
            cols2=range(f), full_asg=asg, chunk=40)
        np.testing.assert_allclose(b13, r13[e], rtol=1e-4, atol=1e-5)
        np.testing.assert_allclose(b2, r2[e], rtol=1e-4, atol=1e-5)
        for a in asg:
            np.testing.assert_allclose(dtw[int(a)], rtw.ravel()[a], rtol=1e-4, atol=1e-5)
            dx[a // k] += share[int(a)]
        if e == 3:
            assert asg.size == 0 and not b13.any() and not b2.any()
    np.testing.assert_allclose(dx, rdx, rtol=1e-4, atol=1e-5)
    # a sub-block picks the same entries
    b13, b2, _, _ = oracle.moe_backward_expert(x, ids, w, 1, w13[1], w2[1], dy, rows13=[5, f + 7],
                                               cols13=[0, 63], rows2=[2], cols2=[0, 95])
    np.testing.assert_allclose(b13, r13[1][np.ix_([5, f + 7], [0, 63])], rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(b2, r2[1][np.ix_([2], [0, 95])], rtol=1e-4, atol=1e-5)
