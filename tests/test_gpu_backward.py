"""GPU parity of the backward calls against the CPU oracle (through the C ABI).

Tolerances (derived from the arithmetic): the bf16 backward rounds exactly one
operand of each bf16 product to bfloat16 (w act for the w2 gradient,
d_gate/d_up for the w13 and hidden gradients; grad_out, hidden and the weights
are exact bf16 inputs) and accumulates in float32.  That rounding moves each
product term by at most u = 2^-9 relative, which gives an error RMS of about
1.7e-3 of the output's RMS and a largest error near u x the largest output
(a normwise bound: elements whose terms cancel can carry several percent of
the RMS, so no element-wise bound at the RMS scale holds).  Each gradient
must satisfy
    RMS(error) <= 4e-3 x RMS(oracle)   and   max |error| <= 4u x max |oracle|.
grad_topk_w = <G, act> is formed from exact inputs with float32 sums:
max |error| <= 1e-4 x max |oracle|.  The gating backward is float32
throughout: max |error| <= 1e-5 x max |oracle|.
"""

import math

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle

import mixture_experts_routing_moe_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda"
RMS_TOL = 4e-3
MAX_TOL = 4 * 2.0 ** -9
TOPKW_TOL = 1e-4


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def check_grad(name, got, ref, max_tol=MAX_TOL, rms_tol=RMS_TOL):
    """max |err| <= max_tol x max |ref| and RMS(err) <= rms_tol x RMS(ref)."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), name
    rms = math.sqrt(float(np.mean(ref ** 2)))
    err = got - ref
    emax = float(np.abs(err).max()) / float(np.abs(ref).max())
    erms = math.sqrt(float(np.mean(err ** 2))) / rms
    assert emax <= max_tol and erms <= rms_tol, \
        f"{name}: max err {emax:.3e} x max|ref|, rms err {erms:.3e} x RMS"
    return emax, erms


# --------------------------------------------------------------------------
# Gating softmax backward
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(1000, 64, 8), (37, 8, 2), (5, 130, 6), (16, 256, 8),
                                   (3, 1024, 64), (2, 1, 1), (64, 70, 64)])
@pytest.mark.parametrize("norm", [True, False])
def test_route_backward(T, E, k, norm):
    g = np.random.Generator(np.random.PCG64(T * 7 + E + k))
    logits = g.standard_normal((T, E)).astype(np.float32)
    gw = g.standard_normal((T, k)).astype(np.float32)
    ld = dev(logits)
    tw, tids = moe.moe_route(ld, k, norm)
    ow, oids = oracle.route(logits, k, norm)
    np.testing.assert_array_equal(tids.cpu().numpy(), oids)
    got = moe.moe_route_backward(ld, tids, tw, dev(gw), norm).cpu().numpy().astype(np.float64)
    ref = oracle.route_backward(logits, oids, gw.astype(np.float64), norm)
    scale = max(float(np.abs(ref).max()), 1e-30)
    assert np.abs(got - ref).max() <= 1e-5 * scale
    if norm:  # unselected experts get exactly zero
        sel = np.zeros((T, E), bool)
        np.put_along_axis(sel, oids, True, axis=1)
        assert np.all(got[~sel] == 0)


def test_route_backward_empty():
    z = torch.empty((0, 8), dtype=torch.float32, device=DEV)
    zi = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    zw = torch.empty((0, 2), dtype=torch.float32, device=DEV)
    out = moe.moe_route_backward(z, zi, zw, zw, True)
    assert out.shape == (0, 8)


# --------------------------------------------------------------------------
# Expert FFN backward
# --------------------------------------------------------------------------

def _rand_case(seed, T, H, I, E, k, skew=0.0, inv=0.0):
    g = np.random.Generator(np.random.PCG64(seed))
    x = mi.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    w13 = mi.f32_to_bf16_bits((g.standard_normal((E, 2 * I, H)) / math.sqrt(H)).astype(np.float32))
    w2 = mi.f32_to_bf16_bits((g.standard_normal((E, H, I)) / math.sqrt(I)).astype(np.float32))
    dy = mi.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    logits = g.standard_normal((T, E)).astype(np.float32)
    logits += (skew * np.arange(E, dtype=np.float32))[None, :]
    w, ids = oracle.route(logits, k, True)
    if inv > 0:
        ids = np.where(g.random(ids.shape) < inv, -1, ids).astype(np.int32)
    return x, w13, w2, w.astype(np.float32), ids, dy


def _bwd_gpu(x, w13, w2, w32, ids, dy):
    E = w13.shape[0]
    a = moe.moe_align(dev(ids), E)
    out = moe.moe_expert_ffn_backward(dev_bf16(x), dev_bf16(w13), dev_bf16(w2), dev(w32), a,
                                      dev_bf16(dy))
    return {n: t.cpu().numpy() for n, t in out.items()}


@pytest.mark.parametrize("T,H,I,E,k,skew,inv", [
    (300, 128, 192, 8, 2, 0.0, 0.0),
    (200, 256, 64, 5, 3, 0.0, 0.0),
    (77, 64, 64, 3, 3, 0.0, 0.0),
    (513, 192, 320, 16, 4, 0.5, 0.0),   # skew: experts with no row
    (260, 128, 128, 12, 3, 0.0, 0.2),   # dropped slots (id -1)
    (1, 128, 128, 8, 2, 0.0, 0.0),
    (400, 64, 256, 2, 1, 2.0, 0.0),
    (50, 64, 64, 1, 1, 0.0, 0.0),       # one expert
    (100, 64, 128, 256, 8, 0.0, 0.0),   # many experts, most with a few rows or none
])
def test_ffn_backward(T, H, I, E, k, skew, inv):
    x, w13, w2, w32, ids, dy = _rand_case(T + H + I + E, T, H, I, E, k, skew, inv)
    got = _bwd_gpu(x, w13, w2, w32, ids, dy)
    ref = oracle.expert_ffn_backward(x, w13, w2, w32.astype(np.float64), ids, dy, "bf16",
                                     weights=True)
    for name in ("grad_hidden", "grad_w13", "grad_w2"):
        check_grad(name, got[name], ref[name])
    check_grad("grad_topk_w", got["grad_topk_w"], ref["grad_topk_w"], TOPKW_TOL, TOPKW_TOL)
    # Slots with an invalid id get exactly 0; experts no slot names get zero gradients.
    assert np.all(got["grad_topk_w"][ids < 0] == 0)
    used = np.zeros(E, bool)
    used[ids[ids >= 0]] = True
    assert np.all(got["grad_w13"][~used] == 0) and np.all(got["grad_w2"][~used] == 0)


@pytest.mark.parametrize("T,H,I,E,k,inv", [(4, 64, 128, 8, 2, 0.0), (50, 128, 64, 5, 3, 0.0),
                                            (30, 64, 64, 3, 3, 0.2), (1, 64, 64, 1, 1, 0.0)])
def test_ffn_backward_f32(T, H, I, E, k, inv):
    """float32 layers: float32 throughout, so RMS(err) <= 1e-5 x RMS and
    max |err| <= 1e-4 x max |oracle| for every gradient."""
    g = np.random.Generator(np.random.PCG64(T * 11 + E))
    x = g.standard_normal((T, H)).astype(np.float32)
    w13 = (g.standard_normal((E, 2 * I, H)) / math.sqrt(H)).astype(np.float32)
    w2 = (g.standard_normal((E, H, I)) / math.sqrt(I)).astype(np.float32)
    dy = g.standard_normal((T, H)).astype(np.float32)
    w, ids = oracle.route(g.standard_normal((T, E)).astype(np.float32), k, True)
    if inv > 0:
        ids = np.where(g.random(ids.shape) < inv, -1, ids).astype(np.int32)
    w32 = w.astype(np.float32)
    a = moe.moe_align(dev(ids), E)
    got = moe.moe_expert_ffn_backward(dev(x), dev(w13), dev(w2), dev(w32), a, dev(dy))
    ref = oracle.expert_ffn_backward(x, w13, w2, w32.astype(np.float64), ids, dy, "f32",
                                     weights=True)
    for name in ("grad_hidden", "grad_w13", "grad_w2", "grad_topk_w"):
        check_grad(name, got[name].cpu().numpy(), ref[name], 1e-4, 1e-5)
    assert np.all(got["grad_topk_w"].cpu().numpy()[ids < 0] == 0)


@pytest.mark.parametrize("T,H,I,E,k,skew,inv", [(300, 128, 192, 8, 2, 0.0, 0.0),
                                                (513, 192, 320, 16, 4, 0.5, 0.1),
                                                (700, 64, 1408, 4, 2, 1.0, 0.0),
                                                (90, 320, 64, 3, 3, 0.0, 0.0)])
def test_ffn_backward_kmajor_weights(monkeypatch, T, H, I, E, k, skew, inv):
    """G = dy . w2 and d_hidden = [d_gate ; d_up] . w13 read w2 and w13 as
    stored (the grouped kernel transposes in its LDS reads) and G reads
    grad_out's rows in place through the token ids: the same products, term
    for term and in the same order, as the path that first copies the weights
    transposed and gathers grad_out, so every gradient is bit-identical to
    it."""
    x, w13, w2, w32, ids, dy = _rand_case(T * 3 + I, T, H, I, E, k, skew, inv)
    print(f"kmajor backward T={T} H={H} I={I} E={E} k={k}", flush=True)
    got = _bwd_gpu(x, w13, w2, w32, ids, dy)
    monkeypatch.setenv("MOE_BWD_TRANSPOSED_WEIGHTS", "1")
    ref = _bwd_gpu(x, w13, w2, w32, ids, dy)
    monkeypatch.delenv("MOE_BWD_TRANSPOSED_WEIGHTS")
    for name in got:
        np.testing.assert_array_equal(got[name].view(np.uint32), ref[name].view(np.uint32),
                                      err_msg=name)


@pytest.mark.parametrize("T,H,I,E,k,skew,inv", [(300, 128, 192, 8, 2, 0.0, 0.0),
                                                (513, 192, 320, 16, 4, 0.5, 0.1),
                                                (700, 64, 1408, 4, 2, 1.0, 0.0),
                                                (90, 320, 64, 3, 3, 0.0, 0.0),
                                                (1000, 448, 128, 5, 1, 2.0, 0.0)])
def test_ffn_backward_kmajor_wgrad(monkeypatch, T, H, I, E, k, skew, inv):
    """The weight gradients read w act and [d_gate ; d_up] as stored, per
    position (the K-major weight-gradient kernel, each expert's segment tail
    read as zeros; dw13 stored through the transposing epilogue): the same
    products over the same k order as the path that transposes all four
    operands first, so every gradient is bit-identical to it."""
    x, w13, w2, w32, ids, dy = _rand_case(T * 7 + H, T, H, I, E, k, skew, inv)
    print(f"kmajor wgrad T={T} H={H} I={I} E={E} k={k}", flush=True)
    got = _bwd_gpu(x, w13, w2, w32, ids, dy)
    monkeypatch.setenv("MOE_BWD_TRANSPOSED_OPERANDS", "1")
    ref = _bwd_gpu(x, w13, w2, w32, ids, dy)
    monkeypatch.delenv("MOE_BWD_TRANSPOSED_OPERANDS")
    for name in got:
        np.testing.assert_array_equal(got[name].view(np.uint32), ref[name].view(np.uint32),
                                      err_msg=name)


@pytest.mark.parametrize("T,H,I,E,k,skew,inv", [(300, 128, 192, 8, 2, 0.0, 0.0),
                                                (513, 192, 320, 16, 4, 0.5, 0.1),
                                                (700, 64, 1408, 4, 2, 1.0, 0.0),
                                                (90, 320, 64, 3, 3, 0.0, 0.0),
                                                (1000, 448, 128, 5, 1, 2.0, 0.0)])
def test_ffn_backward_fused_act(monkeypatch, T, H, I, E, k, skew, inv):
    """The SiLU-and-mul backward in the gate/up recompute's epilogue (the FC1
    kernel's accumulators, the same products in the same k order as the FC2
    form that stores gate/up for bwd_act_kernel, and x^T transposed from x
    through each padded position's token rather than from a gathered copy):
    gradients of hidden, w13 and w2 bit-identical to the separate path; the
    routing-weight gradient is the same sum over a row's columns in another
    order (per column tile, then the tiles in order)."""
    x, w13, w2, w32, ids, dy = _rand_case(T * 11 + I, T, H, I, E, k, skew, inv)
    print(f"fused act backward T={T} H={H} I={I} E={E} k={k}", flush=True)
    got = _bwd_gpu(x, w13, w2, w32, ids, dy)
    monkeypatch.setenv("MOE_BWD_UNFUSED_ACT", "1")
    ref = _bwd_gpu(x, w13, w2, w32, ids, dy)
    monkeypatch.delenv("MOE_BWD_UNFUSED_ACT")
    for name in got:
        if name == "grad_topk_w":
            scale = float(np.abs(ref[name]).max())
            np.testing.assert_allclose(got[name], ref[name], rtol=0, atol=1e-5 * scale)
            assert np.all(got[name][ids < 0] == 0)
        else:
            np.testing.assert_array_equal(got[name].view(np.uint32), ref[name].view(np.uint32),
                                          err_msg=name)


def test_ffn_backward_deterministic():
    x, w13, w2, w32, ids, dy = _rand_case(5, 300, 128, 192, 8, 2)
    a = _bwd_gpu(x, w13, w2, w32, ids, dy)
    b = _bwd_gpu(x, w13, w2, w32, ids, dy)
    for name in a:
        np.testing.assert_array_equal(a[name], b[name])


def test_ffn_backward_empty():
    E, H, I = 4, 64, 64
    x = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    w13 = torch.zeros((E, 2 * I, H), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((E, H, I), dtype=torch.bfloat16, device=DEV)
    tw = torch.empty((0, 2), dtype=torch.float32, device=DEV)
    a = moe.moe_align(torch.empty((0, 2), dtype=torch.int32, device=DEV), E)
    out = moe.moe_expert_ffn_backward(x, w13, w2, tw, a, x)
    assert out["grad_hidden"].shape == (0, H)


# --------------------------------------------------------------------------
# Full-size workloads, in the configuration bench.py times (backward_<name>):
# sampled tokens, sampled weight-gradient rows and columns, plus properties of
# every element.
# --------------------------------------------------------------------------

def _sample(T, ids, E, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    toks = set(g.choice(T, size=6, replace=False).tolist()) | {0, T - 1}
    counts = np.bincount(ids.reshape(-1), minlength=E)
    used = np.nonzero(counts)[0]
    # the most and the least loaded experts that have rows, and two random ones
    picks = {int(used[np.argmax(counts[used])]), int(used[np.argmin(counts[used])])}
    picks |= set(int(e) for e in g.choice(used, size=min(2, len(used)), replace=False))
    return np.array(sorted(toks), np.int64), sorted(picks), counts


@pytest.mark.parametrize("name", ["mixtral", "finegrained"])
def test_backward_full_size(name):
    w = mi.WORKLOADS[name]
    T, H, I, E, k = w.T, w.H, w.I, w.E, w.k
    inp = mi.layer_inputs(w)
    gout = mi.grad_output(w)
    ld = dev(inp["logits"])
    tw, tids = moe.moe_route(ld, k, w.norm)
    ow, oids = oracle.route(inp["logits"], k, w.norm)
    np.testing.assert_array_equal(tids.cpu().numpy(), oids)
    a = moe.moe_align(tids, E)
    g = moe.moe_expert_ffn_backward(dev_bf16(inp["hidden"]), dev_bf16(inp["w13"]),
                                    dev_bf16(inp["w2"]), tw, a, dev_bf16(gout))
    gl = moe.moe_route_backward(ld, tids, tw, g["grad_topk_w"], w.norm)
    toks, experts, counts = _sample(T, oids, E, T + E)
    # Every element finite; experts no slot names get exactly zero gradients.
    for n in ("grad_hidden", "grad_topk_w"):
        assert bool(torch.isfinite(g[n]).all()), n
    unused = torch.from_numpy(counts == 0).to(DEV)
    for n in ("grad_w13", "grad_w2"):
        assert bool(torch.isfinite(g[n]).all()), n
        if bool(unused.any()):
            assert bool((g[n][unused] == 0).all()), n
    assert bool(torch.isfinite(gl).all())

    ref = oracle.expert_ffn_backward(inp["hidden"], inp["w13"], inp["w2"], ow, oids, gout,
                                     "bf16", tokens=toks)
    check_grad("grad_hidden", g["grad_hidden"][toks].cpu().numpy(), ref["grad_hidden"])
    check_grad("grad_topk_w", g["grad_topk_w"][toks].cpu().numpy(), ref["grad_topk_w"],
               TOPKW_TOL, TOPKW_TOL)
    rows13 = [(e, c) for e in experts for c in (0, I - 1, I, 2 * I - 1, I // 3)]
    cols2 = [(e, i) for e in experts for i in (0, I - 1, I // 2)]
    r13, c2 = oracle.expert_wgrad_entries(inp["hidden"], inp["w13"], inp["w2"], ow, oids, gout,
                                          "bf16", rows13, cols2)
    got13 = np.stack([g["grad_w13"][e, c].cpu().numpy() for e, c in rows13])
    got2 = np.stack([g["grad_w2"][e, :, i].cpu().numpy() for e, i in cols2])
    check_grad("grad_w13 rows", got13, r13)
    check_grad("grad_w2 columns", got2, c2)
    # The gating backward on the sampled rows, from the oracle's own weight gradient.
    rl = oracle.route_backward(inp["logits"][toks], oids[toks], ref["grad_topk_w"], w.norm)
    gl_s = gl[torch.from_numpy(toks).to(DEV)].cpu().numpy().astype(np.float64)
    assert np.abs(gl_s - rl).max() <= 1e-3 * np.abs(rl).max()


def test_backward_graph_replay():
    """Route + align + layer backward captured as one HIP graph: replays with
    different grad_out, with other GPU work between them, equal eager runs
    of the same calls bit for bit (the calls allocate, sync and memset
    nothing)."""
    T, H, I, E, k = 300, 128, 192, 8, 2
    x, w13, w2, _, _, _ = _rand_case(77, T, H, I, E, k)
    xd, w13d, w2d = dev_bf16(x), dev_bf16(w13), dev_bf16(w2)
    g = np.random.Generator(np.random.PCG64(78))
    logits = dev(g.standard_normal((T, E)).astype(np.float32))
    dys = [dev_bf16(mi.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32)))
           for _ in range(3)]
    static_dy = dys[0].clone()

    def bufs():
        f32 = dict(dtype=torch.float32, device=DEV)
        a = {"counts": torch.empty(E, dtype=torch.int32, device=DEV),
             "offsets": torch.empty(E + 1, dtype=torch.int32, device=DEV),
             "sorted_token_ids": torch.empty(T * k, dtype=torch.int32, device=DEV),
             "sorted_slot_ids": torch.empty(T * k, dtype=torch.int32, device=DEV),
             "slot_to_sorted": torch.empty(T * k, dtype=torch.int32, device=DEV)}
        return {"tw": torch.empty((T, k), **f32),
                "ids": torch.empty((T, k), dtype=torch.int32, device=DEV),
                "aligned": a,
                "align_ws": torch.empty(moe.moe_align_workspace_size(T, k, E), dtype=torch.uint8,
                                        device=DEV),
                "grads": {"grad_hidden": torch.empty((T, H), **f32),
                          "grad_w13": torch.empty((E, 2 * I, H), **f32),
                          "grad_w2": torch.empty((E, H, I), **f32),
                          "grad_topk_w": torch.empty((T, k), **f32)},
                "gl": torch.empty((T, E), **f32),
                "ws": torch.empty(moe.moe_expert_ffn_backward_workspace_size(T, H, I, E, k),
                                  dtype=torch.uint8, device=DEV)}

    def step(b, dy):
        moe.moe_route(logits, k, True, b["tw"], b["ids"])
        moe.moe_align(b["ids"], E, b["aligned"], b["align_ws"])
        moe.moe_expert_ffn_backward(xd, w13d, w2d, b["tw"], b["aligned"], dy, b["grads"], b["ws"])
        moe.moe_route_backward(logits, b["ids"], b["tw"], b["grads"]["grad_topk_w"], True, b["gl"])

    cap = bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(cap, static_dy)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(cap, static_dy)
    eager = bufs()
    for r in (1, 2, 0, 1):
        static_dy.copy_(dys[r])
        graph.replay()
        torch.cuda.synchronize()
        got = {n: t.clone() for n, t in cap["grads"].items()}
        got_gl = cap["gl"].clone()
        torch.matmul(xd.float(), xd.float().t()).sum().item()
        step(eager, dys[r])
        torch.cuda.synchronize()
        for n in got:
            assert torch.equal(got[n], eager["grads"][n]), (r, n)
        assert torch.equal(got_gl, eager["gl"]), r


@pytest.mark.parametrize("counts", [(63, 64, 65, 128, 0, 1), (64, 0, 0, 129, 191, 2)])
def test_ffn_backward_segment_boundaries(counts):
    """Expert row counts on and around the weight gradients' 64-position
    segment padding (and empty experts between them), k = 1."""
    E, H, I, k = len(counts), 128, 192, 1
    T = sum(counts)
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])[:, None]
    g = np.random.Generator(np.random.PCG64(T))
    ids = ids[g.permutation(T)]  # tokens of one expert are not contiguous
    x = mi.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    w13 = mi.f32_to_bf16_bits((g.standard_normal((E, 2 * I, H)) / math.sqrt(H)).astype(np.float32))
    w2 = mi.f32_to_bf16_bits((g.standard_normal((E, H, I)) / math.sqrt(I)).astype(np.float32))
    dy = mi.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    w32 = g.uniform(0.2, 1.0, (T, k)).astype(np.float32)
    got = _bwd_gpu(x, w13, w2, w32, ids, dy)
    ref = oracle.expert_ffn_backward(x, w13, w2, w32.astype(np.float64), ids, dy, "bf16",
                                     weights=True)
    for name in ("grad_hidden", "grad_w13", "grad_w2"):
        check_grad(name, got[name], ref[name])
    check_grad("grad_topk_w", got["grad_topk_w"], ref["grad_topk_w"], TOPKW_TOL, TOPKW_TOL)
    for e, c in enumerate(counts):
        if c == 0:
            assert np.all(got["grad_w13"][e] == 0) and np.all(got["grad_w2"][e] == 0)
        else:  # each expert's slice on its own scale
            check_grad(f"grad_w13[{e}]", got["grad_w13"][e], ref["grad_w13"][e])
            check_grad(f"grad_w2[{e}]", got["grad_w2"][e], ref["grad_w2"][e])


# --------------------------------------------------------------------------
# Group-limited selection backward
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", sorted(mi.GROUPED))
def test_route_grouped_backward_workloads(name):
    """Full-size group-limited workloads: float32 throughout, max |err| <= 1e-5 x max."""
    w = mi.GROUPED[name]
    scores = mi.grouped_scores(w)
    bias = mi.correction_bias(w)
    sd = dev(scores)
    bd = None if bias is None else dev(bias)
    tw, tids = moe.moe_route_grouped(sd, w.k, w.n_group, w.topk_group, w.method, bd, w.renorm)
    ow, oids = oracle.route_grouped(scores, w.k, w.n_group, w.topk_group, w.method, bias=bias,
                                    renormalize=w.renorm)
    np.testing.assert_array_equal(tids.cpu().numpy(), oids)
    g = np.random.Generator(np.random.PCG64(w.wid)).standard_normal((w.T, w.k)).astype(np.float32)
    got = moe.moe_route_grouped_backward(sd, tids, tw, dev(g), w.renorm).cpu().numpy()
    ref = oracle.route_grouped_backward(scores, oids, g.astype(np.float64), w.renorm)
    assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()
    sel = np.zeros(ref.shape, bool)
    np.put_along_axis(sel, oids, True, axis=1)
    assert np.all(got[~sel] == 0)


@pytest.mark.parametrize("T,E,k,renorm", [(5, 130, 6, True), (77, 8, 8, False), (3, 256, 64, True)])
def test_route_grouped_backward_shapes(T, E, k, renorm):
    g = np.random.Generator(np.random.PCG64(T + E + k))
    scores = (1.0 / (1.0 + np.exp(-g.standard_normal((T, E))))).astype(np.float32)
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = np.take_along_axis(scores, ids, axis=1).astype(np.float64)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    gw = g.standard_normal((T, k)).astype(np.float32)
    got = moe.moe_route_grouped_backward(dev(scores), dev(ids), dev(w.astype(np.float32)),
                                         dev(gw), renorm).cpu().numpy()
    ref = oracle.route_grouped_backward(scores, ids, gw.astype(np.float64), renorm)
    assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()


def test_layer_backward_chains_the_two_calls():
    """moe_layer_backward = moe_expert_ffn_backward then moe_route_backward."""
    T, H, I, E, k = 64, 128, 128, 8, 2
    x, w13, w2, _, _, dy = _rand_case(91, T, H, I, E, k)
    logits = np.random.Generator(np.random.PCG64(92)).standard_normal((T, E)).astype(np.float32)
    xd, w13d, w2d, dyd = dev_bf16(x), dev_bf16(w13), dev_bf16(w2), dev_bf16(dy)
    out, tw, tids, a = moe.moe_layer(xd, w13d, w2d, dev(logits), k, True, decode=False)
    g = moe.moe_layer_backward(xd, w13d, w2d, dev(logits), tw, tids, a, dyd, True)
    ref = moe.moe_expert_ffn_backward(xd, w13d, w2d, tw, a, dyd)
    for n in ref:
        assert torch.equal(g[n], ref[n]), n
    rl = moe.moe_route_backward(dev(logits), tids, tw, ref["grad_topk_w"], True)
    assert torch.equal(g["grad_logits"], rl)


# --------------------------------------------------------------------------
# Router GEMM backward
# --------------------------------------------------------------------------

def _router_bwd_check(x, wg, gl):
    gh, gw = moe.moe_router_backward(dev_bf16(x), dev_bf16(wg), dev(gl))
    rh, rw = oracle.router_backward(x, wg, gl.astype(np.float64), "bf16")
    # float32 sums of exact bf16 x float32 products: relative error ~ E or T ulps
    for name, got, ref in (("grad_hidden", gh, rh), ("grad_w_gate", gw, rw)):
        got = got.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), name
        assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max(), name


@pytest.mark.parametrize("T,H,E", [(1, 64, 1), (300, 128, 64), (77, 192, 130), (513, 64, 8)])
def test_router_backward_shapes(T, H, E):
    g = np.random.Generator(np.random.PCG64(T + H + E))
    x = mi.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    wg = mi.f32_to_bf16_bits((g.standard_normal((E, H)) / math.sqrt(H)).astype(np.float32))
    gl = g.standard_normal((T, E)).astype(np.float32)
    _router_bwd_check(x, wg, gl)


@pytest.mark.parametrize("name", ["finegrained", "mixtral"])
def test_router_backward_workloads(name):
    """The router workloads' full shapes, with the logits' gradient of a
    routing-weight gradient through moe_route_backward."""
    w = mi.WORKLOADS[name]
    x = mi.normal_bf16(w.wid, mi.S_HIDDEN, w.T * w.H, 1.0).reshape(w.T, w.H)
    wg = mi.router_weights(w)
    g = np.random.Generator(np.random.PCG64(w.wid))
    gl = g.standard_normal((w.T, w.E)).astype(np.float32)
    _router_bwd_check(x, wg, gl)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ffn_backward_all_slots_dropped(dtype):
    """Every id -1: no aligned position; every gradient is exactly zero."""
    T, H, I, E, k = 10, 64, 64, 4, 2
    g = np.random.Generator(np.random.PCG64(5))
    ids = np.full((T, k), -1, np.int32)
    x, w13, w2, dy = (g.standard_normal(s).astype(np.float32)
                      for s in ((T, H), (E, 2 * I, H), (E, H, I), (T, H)))
    if dtype == "bf16":
        x, w13, w2, dy = (dev_bf16(mi.f32_to_bf16_bits(a)) for a in (x, w13, w2, dy))
    else:
        x, w13, w2, dy = (dev(a) for a in (x, w13, w2, dy))
    a = moe.moe_align(dev(ids), E)
    # Fill the outputs with NaN first: every element must be written.
    f32 = dict(dtype=torch.float32, device=DEV)
    out = {"grad_hidden": torch.full((T, H), float("nan"), **f32),
           "grad_w13": torch.full((E, 2 * I, H), float("nan"), **f32),
           "grad_w2": torch.full((E, H, I), float("nan"), **f32),
           "grad_topk_w": torch.full((T, k), float("nan"), **f32)}
    got = moe.moe_expert_ffn_backward(x, w13, w2, dev(np.ones((T, k), np.float32)), a, dy, out)
    for n, t in got.items():
        assert bool((t == 0).all()), n
