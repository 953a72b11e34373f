"""Pins of the oracle's backward (gating softmax and expert FFN).

The pages print only the forward; the backward is the derivative of that
forward.  Each pin fixes it against something other than the backward code
itself: central finite differences of the (separately pinned) forward oracle,
float64 autograd through a dense brute-force formulation of the layer (every
expert on every token, combined through a gate that is zero off the top-k),
and invariants of the softmax gradient.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _tiny(seed, T, H, I, E, k, norm=True, drop=False):
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((T, H)).astype(np.float32)
    w13 = (g.standard_normal((E, 2 * I, H)) / math.sqrt(H)).astype(np.float32)
    w2 = (g.standard_normal((E, H, I)) / math.sqrt(I)).astype(np.float32)
    logits = g.standard_normal((T, E)).astype(np.float32)
    w, ids = oracle.route(logits, k, norm)
    if drop:  # one dropped slot (id -1) exercises the invalid-slot rule
        ids = ids.copy()
        ids[0, k - 1] = -1
    dy = g.standard_normal((T, H)).astype(np.float32)
    return x, w13, w2, w, ids, dy, logits


def _loss(x, w13, w2, w, ids, dy):
    return float(np.sum(oracle.expert_ffn(x, w13, w2, w, ids, "f32") * dy.astype(np.float64)))


def _fd(f, arr, idx, h=2.0 ** -12):
    """Central difference of f in element idx of a float32 or float64 array."""
    a = arr.copy()
    plus = arr.dtype.type(arr[idx] + h)
    minus = arr.dtype.type(arr[idx] - h)
    a[idx] = plus
    fp = f(a)
    a[idx] = minus
    fm = f(a)
    return (fp - fm) / (float(plus) - float(minus))


@pytest.mark.parametrize("seed,T,H,I,E,k,drop", [(1, 3, 4, 3, 3, 2, True), (2, 4, 5, 2, 4, 3, False)])
def test_ffn_backward_matches_finite_differences(seed, T, H, I, E, k, drop):
    x, w13, w2, w, ids, dy, _ = _tiny(seed, T, H, I, E, k, drop=drop)
    g = oracle.expert_ffn_backward(x, w13, w2, w, ids, dy, "f32", weights=True)
    scale = max(np.abs(v).max() for v in g.values())
    tol = 1e-6 * scale
    for idx in np.ndindex(x.shape):
        fd = _fd(lambda a: _loss(a, w13, w2, w, ids, dy), x, idx)
        assert abs(fd - g["grad_hidden"][idx]) <= tol, ("hidden", idx)
    for idx in np.ndindex(w13.shape):
        fd = _fd(lambda a: _loss(x, a, w2, w, ids, dy), w13, idx)
        assert abs(fd - g["grad_w13"][idx]) <= tol, ("w13", idx)
    for idx in np.ndindex(w2.shape):
        fd = _fd(lambda a: _loss(x, w13, a, w, ids, dy), w2, idx)
        assert abs(fd - g["grad_w2"][idx]) <= tol, ("w2", idx)
    for idx in np.ndindex(w.shape):
        fd = _fd(lambda a: _loss(x, w13, w2, a, ids, dy), w, idx)
        assert abs(fd - g["grad_topk_w"][idx]) <= tol, ("topk_w", idx)
    if drop:
        assert g["grad_topk_w"][0, k - 1] == 0.0


def _dense_autograd(x, w13, w2, w, ids, dy):
    """float64 autograd through every expert on every token and a dense gate."""
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    k = ids.shape[1]
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    a13 = torch.tensor(w13, dtype=torch.float64, requires_grad=True)
    a2 = torch.tensor(w2, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    gate = torch.zeros((T, E), dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            if 0 <= ids[t, j] < E:
                gate = gate + torch.nn.functional.one_hot(
                    torch.tensor(int(ids[t, j])), E).to(torch.float64)[None, :] * \
                    (torch.arange(T)[:, None] == t).to(torch.float64) * wt[t, j]
    out = torch.zeros((T, H), dtype=torch.float64)
    for e in range(E):
        gu = torch.nn.functional.linear(xt, a13[e])
        act = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
        out = out + gate[:, e:e + 1] * torch.nn.functional.linear(act, a2[e])
    (out * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    return {"grad_hidden": xt.grad.numpy(), "grad_w13": a13.grad.numpy(),
            "grad_w2": a2.grad.numpy(), "grad_topk_w": wt.grad.numpy()}


@pytest.mark.parametrize("seed,T,H,I,E,k,drop", [(3, 6, 16, 24, 5, 2, True), (4, 5, 8, 8, 3, 3, False),
                                                  (5, 4, 8, 16, 1, 1, False)])
def test_ffn_backward_matches_dense_autograd(seed, T, H, I, E, k, drop):
    x, w13, w2, w, ids, dy, _ = _tiny(seed, T, H, I, E, k, drop=drop)
    g = oracle.expert_ffn_backward(x, w13, w2, w, ids, dy, "f32", weights=True)
    ref = _dense_autograd(x, w13, w2, w, ids, dy)
    for name in ref:
        np.testing.assert_allclose(g[name], ref[name], rtol=1e-10, atol=1e-12, err_msg=name)


def test_ffn_backward_token_subset_and_entries_agree_with_full():
    T, H, I, E, k = 11, 12, 10, 4, 2
    x, w13, w2, w, ids, dy, _ = _tiny(7, T, H, I, E, k, drop=True)
    full = oracle.expert_ffn_backward(x, w13, w2, w, ids, dy, "f32", weights=True)
    tok = [7, 0, 7, 3]
    sub = oracle.expert_ffn_backward(x, w13, w2, w, ids, dy, "f32", tokens=tok, threads=3)
    np.testing.assert_array_equal(sub["grad_hidden"], full["grad_hidden"][tok])
    np.testing.assert_array_equal(sub["grad_topk_w"], full["grad_topk_w"][tok])
    rows13 = [(e, c) for e in range(E) for c in (0, I - 1, I, 2 * I - 1, 3)]
    cols2 = [(e, i) for e in range(E) for i in (0, I - 1, 4)]
    r13, c2 = oracle.expert_wgrad_entries(x, w13, w2, w, ids, dy, "f32", rows13, cols2, threads=4)
    for q, (e, c) in enumerate(rows13):
        np.testing.assert_allclose(r13[q], full["grad_w13"][e, c], rtol=1e-12, atol=1e-14)
    for q, (e, i) in enumerate(cols2):
        np.testing.assert_allclose(c2[q], full["grad_w2"][e, :, i], rtol=1e-12, atol=1e-14)


def test_ffn_backward_bf16_inputs_decode_exactly():
    """bf16 bit patterns go through the backward as the float32 values they encode."""
    T, H, I, E, k = 5, 8, 8, 3, 2
    x, w13, w2, w, ids, dy, _ = _tiny(8, T, H, I, E, k)
    to_b = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    to_f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    xb, w13b, w2b, dyb = (to_b(a) for a in (x, w13, w2, dy))
    gb = oracle.expert_ffn_backward(xb, w13b, w2b, w, ids, dyb, "bf16", weights=True)
    gf = oracle.expert_ffn_backward(to_f(xb), to_f(w13b), to_f(w2b), w, ids, to_f(dyb), "f32",
                                    weights=True)
    for name in gf:
        np.testing.assert_array_equal(gb[name], gf[name])


def test_ffn_backward_unused_expert_gets_zero_weight_gradient():
    T, H, I, E, k = 6, 8, 8, 5, 2
    x, w13, w2, w, ids, dy, _ = _tiny(9, T, H, I, E, k)
    # Re-point every slot of expert 4 to another expert not already in its row.
    for t in range(T):
        for j in range(k):
            if ids[t, j] == 4:
                ids[t, j] = next(e for e in range(4) if e not in ids[t])
    g = oracle.expert_ffn_backward(x, w13, w2, w, ids, dy, "f32", weights=True)
    assert np.all(g["grad_w13"][4] == 0) and np.all(g["grad_w2"][4] == 0)
    assert np.abs(g["grad_w13"][ids[0, 0]]).max() > 0


# --------------------------------------------------------------------------
# Gating softmax backward
# --------------------------------------------------------------------------

@pytest.mark.parametrize("norm", [True, False])
@pytest.mark.parametrize("T,E,k", [(5, 8, 2), (3, 6, 6), (4, 64, 8)])
def test_route_backward_matches_finite_differences(T, E, k, norm):
    g = np.random.Generator(np.random.PCG64(T * 100 + E + k))
    logits = g.standard_normal((T, E)).astype(np.float32)
    w, ids = oracle.route(logits, k, norm)
    gw = g.standard_normal((T, k))
    grad = oracle.route_backward(logits, ids, gw, norm)

    def f(a):
        w2, ids2 = oracle.route(a, k, norm)
        assert np.array_equal(ids2, ids)  # the selection is fixed under tiny steps
        return float(np.sum(w2 * gw))

    for idx in np.ndindex(logits.shape):
        fd = _fd(f, logits, idx, h=2.0 ** -14)
        assert abs(fd - grad[idx]) <= 1e-6, idx


@pytest.mark.parametrize("norm", [True, False])
def test_route_backward_matches_torch_softmax_autograd(norm):
    g = np.random.Generator(np.random.PCG64(21))
    T, E, k = 7, 16, 4
    logits = g.standard_normal((T, E)).astype(np.float32)
    w, ids = oracle.route(logits, k, norm)
    gw = g.standard_normal((T, k))
    lt = torch.tensor(logits, dtype=torch.float64, requires_grad=True)
    it = torch.tensor(ids, dtype=torch.int64)
    if norm:
        wt = torch.softmax(torch.gather(lt, 1, it), dim=1)
    else:
        wt = torch.gather(torch.softmax(lt, dim=1), 1, it)
    (wt * torch.tensor(gw)).sum().backward()
    np.testing.assert_allclose(oracle.route_backward(logits, ids, gw, norm), lt.grad.numpy(),
                               rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("norm", [True, False])
def test_route_backward_invariants(norm):
    g = np.random.Generator(np.random.PCG64(22))
    T, E, k = 9, 12, 3
    logits = g.standard_normal((T, E)).astype(np.float32)
    w, ids = oracle.route(logits, k, norm)
    gw = g.standard_normal((T, k))
    grad = oracle.route_backward(logits, ids, gw, norm)
    # A softmax gradient sums to zero over its inputs.
    np.testing.assert_allclose(grad.sum(axis=1), 0.0, atol=1e-14)
    # Equal upstream gradients on every slot: under norm the weights sum to 1,
    # so nothing changes and the gradient vanishes.
    same = oracle.route_backward(logits, ids, np.ones((T, k)), norm)
    if norm:
        sel = np.zeros((T, E), bool)
        np.put_along_axis(sel, ids, True, axis=1)
        assert np.all(grad[~sel] == 0)
        np.testing.assert_allclose(same, 0.0, atol=1e-15)


# --------------------------------------------------------------------------
# Group-limited selection backward
# --------------------------------------------------------------------------

@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("method", ["group_limited_greedy", "noaux_tc"])
def test_route_grouped_backward_matches_finite_differences(method, renorm):
    g = np.random.Generator(np.random.PCG64(31 + renorm))
    T, E, k, ng, tg = 6, 16, 3, 4, 2
    scores = (1.0 / (1.0 + np.exp(-g.standard_normal((T, E))))).astype(np.float32)
    bias = (0.1 * g.standard_normal(E)).astype(np.float32)
    w, ids = oracle.route_grouped(scores, k, ng, tg, method, bias=bias, renormalize=renorm)
    gw = g.standard_normal((T, k))
    grad = oracle.route_grouped_backward(scores, ids, gw, renorm)

    def f(a):
        w2, ids2 = oracle.route_grouped(a, k, ng, tg, method, bias=bias, renormalize=renorm)
        assert np.array_equal(ids2, ids)  # the selection is fixed under tiny steps
        return float(np.sum(w2 * gw))

    for idx in np.ndindex(scores.shape):
        fd = _fd(f, scores, idx, h=2.0 ** -14)
        assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), idx


def test_route_grouped_backward_invariants():
    g = np.random.Generator(np.random.PCG64(33))
    T, E, k = 8, 32, 4
    scores = (1.0 / (1.0 + np.exp(-g.standard_normal((T, E))))).astype(np.float32)
    w, ids = oracle.route_grouped(scores, k, 8, 3, "noaux_tc", bias=np.zeros(E, np.float32),
                                  renormalize=True)
    gw = g.standard_normal((T, k))
    grad = oracle.route_grouped_backward(scores, ids, gw, True)
    # Renormalised weights are scale invariant, so the gradient is orthogonal
    # to the scores (Euler); unselected experts get exactly zero.
    np.testing.assert_allclose(np.sum(grad * scores, axis=1), 0.0, atol=1e-12)
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, ids, True, axis=1)
    assert np.all(grad[~sel] == 0)
    plain = oracle.route_grouped_backward(scores, ids, gw, False)
    np.testing.assert_array_equal(np.take_along_axis(plain, ids, axis=1), gw)


# --------------------------------------------------------------------------
# Router GEMM backward
# --------------------------------------------------------------------------

def test_router_backward_matches_finite_differences_and_matmul():
    g = np.random.Generator(np.random.PCG64(41))
    T, H, E = 5, 8, 6
    x = g.standard_normal((T, H)).astype(np.float32)
    wg = (g.standard_normal((E, H)) / math.sqrt(H)).astype(np.float32)
    gl = g.standard_normal((T, E))
    gh, gw = oracle.router_backward(x, wg, gl, "f32")

    def f_x(a):
        return float(np.sum(oracle.router_logits(a, wg, "f32") * gl))

    def f_w(a):
        return float(np.sum(oracle.router_logits(x, a, "f32") * gl))

    for idx in np.ndindex(x.shape):
        assert abs(_fd(f_x, x, idx) - gh[idx]) <= 1e-7, idx
    for idx in np.ndindex(wg.shape):
        assert abs(_fd(f_w, wg, idx) - gw[idx]) <= 1e-7, idx
    # the plain definitions as float64 library products
    np.testing.assert_allclose(gh, gl @ wg.astype(np.float64), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gw, gl.T @ x.astype(np.float64), rtol=1e-12, atol=1e-13)
