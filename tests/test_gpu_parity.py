"""GPU parity: libmoe (HIP, through the C ABI) against the CPU oracle.

Integer outputs (ids, counts, offsets, sorted ids, multihot, position maps)
must match bit for bit; routing weights within 1e-6 relative.  Layer output,
with RMS that of the oracle's output:

* float32 layers: max-abs error <= 1e-4 x RMS.
* bfloat16 layers: the combine is run a second time writing float32 from the
  same y, and that pre-rounding output must be within max-abs 2e-2 x RMS of
  the oracle; the bf16 output must equal its round-to-nearest-even bit for
  bit; and the bf16 output itself must be within 2e-2 x RMS plus half a bf16
  ulp of the oracle value (rounding an exact result to bf16 already moves
  these heavy-tailed outputs by up to ~2.4% of RMS, so the final rounding is
  allowed on top of the budget).

Full-size prefill layers are checked on sampled tokens (the oracle is
evaluated per token) plus properties of every token.
"""

import math

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle

import mixture_experts_routing_moe_amd as moe  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_BF16 = 2e-2
TOL_F32 = 1e-4
WEIGHT_RTOL = 1e-6


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def host(t):
    if t.dtype == torch.bfloat16:
        return mi.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def assert_weights_close(w_gpu, w_ref):
    w_gpu = w_gpu.astype(np.float64)
    rel = np.abs(w_gpu - w_ref) / np.maximum(np.abs(w_ref), 1e-30)
    assert rel.max() <= WEIGHT_RTOL, f"max rel err {rel.max():.3e}"


def assert_layer_close(out_gpu, out_ref, tol):
    rms = math.sqrt(float(np.mean(out_ref ** 2)))
    err = float(np.max(np.abs(out_gpu.astype(np.float64) - out_ref)))
    assert np.all(np.isfinite(out_gpu))
    assert err <= tol * rms, f"max abs err {err:.4e} > {tol} x rms {rms:.4e}"
    return err / rms


def half_ulp_bf16(v):
    """Half a bfloat16 ulp at |v| (8 significant bits)."""
    a = np.maximum(np.abs(v), np.finfo(np.float32).tiny)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 8)


def assert_bf16_layer(out_bf16, out_f32, out_ref):
    """The three bf16 checks of the module docstring."""
    rel = assert_layer_close(out_f32, out_ref, TOL_BF16)
    rne = mi.bf16_bits_to_f32(mi.f32_to_bf16_bits(out_f32))
    np.testing.assert_array_equal(out_bf16.view(np.uint32), rne.view(np.uint32))
    rms = math.sqrt(float(np.mean(out_ref ** 2)))
    excess = np.abs(out_bf16.astype(np.float64) - out_ref) - half_ulp_bf16(out_ref)
    assert excess.max() <= TOL_BF16 * rms, f"bf16 output off by {excess.max():.3e} + 1/2 ulp"
    return rel


def _nan_filled(shape, dtype):
    """A device buffer whose every element is NaN (bf16 / f32 all-ones bits), so an
    element the library fails to write shows up downstream as a non-finite output."""
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def run_ffn(x, w13, w2, tw, a, k, decode):
    """All FFN phases through the C ABI -> (out bf16 as f32, pre-rounding out f32).

    Every intermediate (act, y, the one-call workspace) and every output starts
    as NaN, so a tile the GEMMs leave unwritten reaches the output as NaN."""
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    act = moe.moe_ffn_gate_up(x, w13, a, k, decode, act=_nan_filled((T * k, I), x.dtype))
    sp = moe.moe_ffn_down_splits(moe.MOE_BF16 if x.dtype == torch.bfloat16 else moe.MOE_F32,
                                 T, H, I, E, k, decode)
    yshape = (T * k, H) if sp == 1 else (sp, T * k, H)
    y = moe.moe_ffn_down(act, w2, a, T, k, decode, y=_nan_filled(yshape, torch.float32))
    out = moe.moe_combine(y, tw, a["slot_to_sorted"], x.dtype, out=_nan_filled((T, H), x.dtype))
    out32 = moe.moe_combine(y, tw, a["slot_to_sorted"], torch.float32,
                            out=_nan_filled((T, H), torch.float32))
    dt = moe.MOE_BF16 if x.dtype == torch.bfloat16 else moe.MOE_F32
    ws = torch.full((max(1, moe.moe_expert_ffn_workspace_size(dt, T, H, I, E, k)),), 0xFF,
                    dtype=torch.uint8, device=DEV)
    one_call = moe.moe_expert_ffn(x, w13, w2, tw, a, decode=decode,
                                  out=_nan_filled((T, H), x.dtype), workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(one_call.view(torch.int16) if one_call.dtype == torch.bfloat16 else one_call,
                       out.view(torch.int16) if out.dtype == torch.bfloat16 else out)
    return host(out), host(out32)


# --------------------------------------------------------------------------
# Route
# --------------------------------------------------------------------------

def _route_check(x, k, norm):
    w, ids = moe.moe_route(dev(x), k, norm)
    torch.cuda.synchronize()
    ow, oids = oracle.route(x, k, norm)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    assert_weights_close(w.cpu().numpy(), ow)


@pytest.mark.parametrize("name", ["tiny", "routing", "mixtral", "finegrained", "decode1",
                                  "decode32"])
@pytest.mark.parametrize("norm", [True, False])
def test_route_workloads(name, norm):
    w = mi.WORKLOADS[name]
    _route_check(mi.gating_logits(w), w.k, norm)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (17, 5, 5), (33, 130, 7), (65, 300, 9),
                                   (10, 1024, 64), (1000, 64, 8), (257, 64, 64), (3, 64, 1),
                                   (129, 200, 3), (50, 600, 20)])
@pytest.mark.parametrize("ties", [False, True])
def test_route_shapes_and_ties(T, E, k, ties):
    g = np.random.Generator(np.random.PCG64(T * 7919 + E * 31 + k))
    x = g.standard_normal((T, E)).astype(np.float32)
    if ties:
        x = np.round(x * 2).astype(np.float32)
    for norm in (True, False):
        _route_check(x, k, norm)


def test_route_all_equal_rows():
    x = np.zeros((5, 64), np.float32)
    w, ids = moe.moe_route(dev(x), 8, True)
    assert ids.cpu().numpy().tolist() == [list(range(8))] * 5
    np.testing.assert_allclose(w.cpu().numpy(), 1 / 8, rtol=1e-7)


def test_route_empty():
    w, ids = moe.moe_route(torch.empty((0, 8), dtype=torch.float32, device=DEV), 2)
    assert w.shape == (0, 2)


# --------------------------------------------------------------------------
# Router GEMM + route
# --------------------------------------------------------------------------

def _router_check(x, wg, k, norm):
    """x [T,H], wg [E,H] bf16 bits.  Logits within the fp32-accumulation bound
    of the exact dot products; ids and weights exactly moe_route's selection on
    the logits the kernel wrote (oracle route on them), and equal to the
    oracle's selection on exact logits wherever the top-(k+1) gaps exceed
    twice the bound."""
    T, H = x.shape
    logits, w, ids = moe.moe_router_route(dev_bf16(x), dev_bf16(wg), k, norm)
    torch.cuda.synchronize()
    gl = logits.cpu().numpy()
    ref = oracle.router_logits(x, wg, "bf16")
    # bf16 x bf16 products are exact in fp32; at most H/32 + 8 roundings of
    # partial sums, each <= 2^-24 of the running magnitude <= sum |x w|.
    absdot = np.abs(mi.bf16_bits_to_f32(x)).astype(np.float64) @ \
        np.abs(mi.bf16_bits_to_f32(wg)).astype(np.float64).T
    bound = (H / 32 + 8) * 2.0 ** -24 * absdot
    assert np.all(np.abs(gl - ref) <= bound), f"logit err {np.max(np.abs(gl - ref) / bound):.3f} x bound"
    ow, oids = oracle.route(gl, k, norm)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    assert_weights_close(w.cpu().numpy(), ow)
    E = wg.shape[0]
    if k < E:
        srt = np.sort(ref, axis=1)[:, ::-1][:, :k + 1]
        rb = bound.max(axis=1, keepdims=True)
        clear = np.all(srt[:, :-1] - srt[:, 1:] > 2 * rb, axis=1)
        _, eids = oracle.route(ref.astype(np.float32), k, norm)
        np.testing.assert_array_equal(ids.cpu().numpy()[clear], eids[clear])
        assert clear.mean() > 0.5, f"only {clear.mean():.2f} of rows have clear margins"


@pytest.mark.parametrize("T,H,E,k", [(1, 64, 8, 2), (33, 128, 64, 8), (300, 256, 16, 4),
                                     (515, 192, 40, 6), (100, 64, 30, 3), (64, 128, 100, 8),
                                     (70, 256, 64, 20), (9000, 64, 64, 8), (8200, 128, 8, 2),
                                     (40, 4160, 16, 4), (2100, 4224, 8, 2)])
@pytest.mark.parametrize("norm", [True, False])
def test_router_route_shapes(T, H, E, k, norm):
    g = np.random.Generator(np.random.PCG64(T + H + E * 3 + k))
    x = mi.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    wg = mi.f32_to_bf16_bits((g.standard_normal((E, H)) / math.sqrt(H)).astype(np.float32))
    print(f"router T={T} H={H} E={E} k={k} norm={norm}", flush=True)
    _router_check(x, wg, k, norm)


@pytest.mark.parametrize("name", ["mixtral", "finegrained", "decode32"])
def test_router_route_workloads(name):
    w = mi.WORKLOADS[name]
    print(f"router workload {name}", flush=True)
    x = mi.normal_bf16(w.wid, mi.S_HIDDEN, w.T * w.H, 1.0).reshape(w.T, w.H)
    _router_check(x, mi.router_weights(w), w.k, w.norm)


def test_router_route_empty():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    wg = torch.zeros((8, 64), dtype=torch.bfloat16, device=DEV)
    lg, w, ids = moe.moe_router_route(x, wg, 2)
    assert lg.shape == (0, 8) and ids.shape == (0, 2)


# --------------------------------------------------------------------------
# Group-limited routing (group_limited_greedy / noaux_tc)
# --------------------------------------------------------------------------

def _grouped_check(s, k, n_group, topk_group, method, bias, renorm, scores_dev=None):
    sd = dev(s) if scores_dev is None else scores_dev
    bd = None if bias is None else dev(bias)
    w, ids = moe.moe_route_grouped(sd, k, n_group, topk_group, method, bd, renorm)
    torch.cuda.synchronize()
    ow, oids = oracle.route_grouped(s, k, n_group, topk_group, method, bias=bias,
                                    renormalize=renorm)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    if renorm:
        assert_weights_close(w.cpu().numpy(), ow)
    else:  # the scores themselves, copied
        np.testing.assert_array_equal(w.cpu().numpy().astype(np.float64), ow)


@pytest.mark.parametrize("name", sorted(mi.GROUPED))
@pytest.mark.parametrize("renorm", [False, True])
def test_route_grouped_workloads(name, renorm):
    w = mi.GROUPED[name]
    print(f"grouped routing workload {name} T={w.T} E={w.E} renorm={renorm}", flush=True)
    _grouped_check(mi.grouped_scores(w), w.k, w.n_group, w.topk_group, w.method,
                   mi.correction_bias(w), renorm)


_GROUPED_SHAPES = [
    (333, 16, 4, 2, 3), (70, 64, 8, 3, 8), (1, 64, 64, 64, 64), (129, 90, 9, 4, 7),
    (257, 96, 4, 1, 24), (200, 160, 8, 3, 6), (64, 256, 1, 1, 8), (100, 256, 8, 8, 64),
    (77, 384, 12, 5, 16), (40, 1024, 64, 7, 14), (33, 1000, 8, 2, 50),
    # 16-lanes-per-row kernel: E % 16 == 0, E <= 256, n_group | 16, k <= 16
    (500, 128, 16, 5, 16), (65, 48, 2, 1, 5), (301, 256, 4, 2, 8), (90, 32, 16, 3, 4),
    (1031, 256, 8, 4, 8), (7, 160, 8, 3, 6), (130, 64, 2, 2, 16), (66, 208, 16, 16, 9)]


# noaux_tc scores a group by its two best experts, so it needs groups of two or more.
@pytest.mark.parametrize("T,E,n_group,topk_group,k,method", [
    (*shape, m) for shape in _GROUPED_SHAPES for m in ("group_limited_greedy", "noaux_tc")
    if m == "group_limited_greedy" or shape[1] // shape[2] >= 2])
@pytest.mark.parametrize("ties", [False, True])
def test_route_grouped_shapes(T, E, n_group, topk_group, k, method, ties):
    g = np.random.Generator(np.random.PCG64(T * 7 + E + n_group + k))
    s = g.random((T, E)).astype(np.float32)
    b = (g.standard_normal(E) * 0.1).astype(np.float32) if method == "noaux_tc" else None
    if ties:  # few distinct values: equal scores, equal group scores
        s = (np.round(s * 4) / 4).astype(np.float32)
        if b is not None:
            b = (np.round(b * 4) / 4).astype(np.float32)
    print(f"grouped T={T} E={E} n_group={n_group} topk_group={topk_group} k={k} {method} "
          f"ties={ties}", flush=True)
    for renorm in (False, True):
        _grouped_check(s, k, n_group, topk_group, method, b, renorm)


@pytest.mark.parametrize("T,E,n_group,topk_group,k,method", [
    (1031, 256, 8, 4, 8, "noaux_tc"), (700, 160, 8, 3, 6, "group_limited_greedy"),
    (65, 48, 2, 1, 5, "noaux_tc"), (90, 32, 16, 3, 4, "group_limited_greedy"),
    (129, 90, 9, 4, 7, "noaux_tc"), (40, 384, 12, 5, 16, "group_limited_greedy")])
@pytest.mark.parametrize("renorm", [False, True])
def test_route_grouped_multihot(T, E, n_group, topk_group, k, method, renorm):
    """The selection's [T, E] maps, written by the selection kernel (or, off its
    fast path, by the converter after it), equal moe_indices_to_multihot of the
    selection's own ids and weights bit for bit."""
    g = np.random.Generator(np.random.PCG64(T + E + k))
    s = g.random((T, E)).astype(np.float32)
    b = dev((g.standard_normal(E) * 0.1).astype(np.float32)) if method == "noaux_tc" else None
    w, ids, mh, pim, pos = moe.moe_route_grouped(dev(s), k, n_group, topk_group, method, b,
                                                 renorm, multihot=True)
    w2, ids2 = moe.moe_route_grouped(dev(s), k, n_group, topk_group, method, b, renorm)
    rmh, rpim, rpos = moe.moe_indices_to_multihot(ids, w, E)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w.view(torch.int32), w2.view(torch.int32))
    assert torch.equal(mh, rmh) and torch.equal(pos, rpos)
    assert torch.equal(pim.view(torch.int32), rpim.view(torch.int32))
    _, oids = oracle.route_grouped(s, k, n_group, topk_group, method,
                                   bias=None if b is None else b.cpu().numpy(), renormalize=renorm)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)


def test_route_grouped_unaligned_rows():
    # Scores starting 4 bytes past a 16-byte boundary take the scalar loads.
    w = mi.GROUPED["grouped_noaux"]
    s = mi.grouped_scores(w, T=300)
    flat = torch.zeros(s.size + 1, dtype=torch.float32, device=DEV)
    flat[1:] = dev(s.reshape(-1))
    sd = flat[1:].view(300, w.E)
    assert sd.data_ptr() % 16 == 4
    _grouped_check(s, w.k, w.n_group, w.topk_group, w.method, mi.correction_bias(w), True,
                   scores_dev=sd)


def test_route_grouped_empty():
    w, ids = moe.moe_route_grouped(torch.empty((0, 64), dtype=torch.float32, device=DEV), 4, 8,
                                   2, "group_limited_greedy")
    assert w.shape == (0, 4) and ids.shape == (0, 4)


# --------------------------------------------------------------------------
# Align
# --------------------------------------------------------------------------

def _align_check(ids, E):
    a = moe.moe_align(dev(ids), E)
    torch.cuda.synchronize()
    ref = oracle.align(ids, E)
    for key in ("counts", "offsets", "sorted_token_ids", "sorted_slot_ids", "slot_to_sorted"):
        np.testing.assert_array_equal(a[key].cpu().numpy(), ref[key], err_msg=key)
    return a


@pytest.mark.parametrize("name", ["tiny", "routing", "mixtral", "finegrained", "decode1",
                                  "decode32"])
def test_align_workloads(name):
    w = mi.WORKLOADS[name]
    _, ids = oracle.route(mi.gating_logits(w), w.k, True)
    _align_check(ids, w.E)


@pytest.mark.parametrize("T,E,k,inv", [(1, 4, 4, 0.0), (1, 1, 1, 0.0), (300, 1, 1, 0.0),
                                       (777, 13, 3, 0.1), (4096, 64, 8, 0.05),
                                       (100, 1024, 16, 0.2), (5000, 200, 6, 0.0),
                                       (20000, 64, 8, 0.0), (333, 8, 8, 0.5)])
def test_align_random_ids(T, E, k, inv):
    _align_check(mi.random_ids(T * 3 + E + k, T, E, k, invalid_frac=inv), E)


def test_align_skewed_and_all_invalid():
    ids = np.tile(np.array([[3, 0, 5]], np.int32), (3000, 1))
    _align_check(ids, 8)
    a = _align_check(np.full((50, 2), -1, np.int32), 4)
    assert a["offsets"].cpu().numpy().tolist() == [0] * 5


def test_align_empty():
    a = moe.moe_align(torch.empty((0, 2), dtype=torch.int32, device=DEV), 6)
    torch.cuda.synchronize()
    assert a["offsets"].cpu().numpy().tolist() == [0] * 7
    assert a["counts"].cpu().numpy().tolist() == [0] * 6


def test_align_deterministic():
    ids = mi.random_ids(5, 20000, 64, 8)
    a1 = moe.moe_align(dev(ids), 64)
    a2 = moe.moe_align(dev(ids), 64)
    torch.cuda.synchronize()
    for key in a1:
        assert torch.equal(a1[key], a2[key])


@pytest.mark.parametrize("T,E,k,inv", [(300, 64, 8, 0.0), (1000, 8, 2, 0.05), (77, 256, 8, 0.1),
                                       (33, 30, 3, 0.0)])
def test_indices_to_multihot_backward(T, E, k, inv):
    """The converter's backward on a dense random gradient (nonzero where no
    expert was selected, unlike any forward output) equals the oracle's
    inverse conversion of that gradient bit for bit."""
    ids = mi.random_ids(T + E, T, E, k, invalid_frac=inv)
    probs = mi.random_probs(T + 1, T, k)
    _, _, pos = moe.moe_indices_to_multihot(dev(ids), dev(probs), E)
    grad = np.random.Generator(np.random.PCG64(T * E)).standard_normal((T, E)).astype(np.float32)
    got = moe.moe_indices_to_multihot_backward(dev(grad), pos, k)
    torch.cuda.synchronize()
    ref, _ = oracle.multihot_to_indices(grad, pos.cpu().numpy(), k)
    np.testing.assert_array_equal(got.cpu().numpy().view(np.int32), ref.view(np.int32))


# --------------------------------------------------------------------------
# Route + align in one call
# --------------------------------------------------------------------------

ALIGN_KEYS = ("counts", "offsets", "sorted_token_ids", "sorted_slot_ids", "slot_to_sorted")


@pytest.mark.parametrize("T,E,k", [(1, 64, 8), (32, 64, 8), (64, 64, 8), (0, 64, 8), (5, 8, 2),
                                   (100, 60, 5), (16384, 64, 8), (4096, 8, 2), (3000, 64, 6),
                                   (777, 100, 4), (300, 64, 20), (9000, 36, 4),
                                   (4096, 64, 16), (12000, 62, 8), (8192, 64, 8),
                                   (8, 64, 8), (64, 16, 1), (3, 64, 16), (9, 20, 7)])
@pytest.mark.parametrize("mh", [False, True])
def test_route_align_matches_separate_calls(T, E, k, mh):
    g = np.random.Generator(np.random.PCG64(T * 3 + E + k))
    x = g.standard_normal((T, E)).astype(np.float32)
    if T > 0:
        x[:, : min(E, 5)] = np.round(x[:, : min(E, 5)])  # some equal logits
    xd = dev(x)
    print(f"route_align T={T} E={E} k={k} multihot={mh} "
          f"fused={moe.moe_route_align_fused(T, E, k)}", flush=True)
    got = moe.moe_route_align(xd, k, True, with_multihot=mh)
    if mh:
        sep = dict(zip(("topk_w", "topk_ids", "multihot", "probs_in_multihot", "position_map"),
                       moe.moe_route_multihot(xd, k, True)))
    else:
        sep = dict(zip(("topk_w", "topk_ids"), moe.moe_route(xd, k, True)))
    sep.update(moe.moe_align(sep["topk_ids"], E))
    torch.cuda.synchronize()
    for key in sep:
        a, b = got[key], sep[key]
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b), key
    ow, oids = oracle.route(x, k, True)
    np.testing.assert_array_equal(got["topk_ids"].cpu().numpy(), oids)
    ref = oracle.align(oids, E)
    for key in ALIGN_KEYS:
        np.testing.assert_array_equal(got[key].cpu().numpy(), ref[key], err_msg=key)


@pytest.mark.parametrize("T,E,k", [(1, 64, 8), (32, 64, 8), (64, 64, 8), (0, 64, 8), (5, 8, 2),
                                   (100, 60, 5), (16384, 64, 8), (4096, 8, 2), (3000, 64, 6),
                                   (777, 100, 4), (300, 64, 20), (9000, 36, 4),
                                   (4096, 64, 16), (12000, 62, 8), (8192, 64, 8),
                                   (8, 64, 8), (64, 16, 1), (3, 64, 16), (9, 20, 7),
                                   (40000, 64, 8)])
def test_route_align_inverse_matches_separate_calls(T, E, k):
    """moe_route_align_inverse (the multihot maps converted back to indices in
    the route + align launches where they are fused) equals moe_route_multihot,
    moe_align and moe_multihot_to_indices called one after the other, bit for
    bit, and the conversion returns the routing's own ids and weights."""
    g = np.random.Generator(np.random.PCG64(T * 5 + E + k))
    x = g.standard_normal((T, E)).astype(np.float32)
    if T > 0:
        x[:, : min(E, 5)] = np.round(x[:, : min(E, 5)])  # some equal logits
    xd = dev(x)
    print(f"route_align_inverse T={T} E={E} k={k} fused={moe.moe_route_align_fused(T, E, k)}",
          flush=True)
    got = moe.moe_route_align_inverse(xd, k, True)
    sep = dict(zip(("topk_w", "topk_ids", "multihot", "probs_in_multihot", "position_map"),
                   moe.moe_route_multihot(xd, k, True)))
    sep.update(moe.moe_align(sep["topk_ids"], E))
    sep["probs_indices"], sep["ids_from_multihot"] = moe.moe_multihot_to_indices(
        sep["probs_in_multihot"], sep["position_map"], k)
    torch.cuda.synchronize()
    for key in sep:
        a, b = got[key], sep[key]
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b), key
    assert torch.equal(got["ids_from_multihot"], got["topk_ids"])
    assert torch.equal(got["probs_indices"].view(torch.int32), got["topk_w"].view(torch.int32))


@pytest.mark.parametrize("T,E,k,H,I,inverse,norm", [
    (1, 64, 8, 2048, 1408, True, True), (1, 8, 2, 128, 128, True, True),
    (2, 64, 8, 256, 192, True, False), (3, 16, 4, 192, 320, True, True),
    (8, 12, 2, 64, 128, True, True), (16, 60, 1, 128, 64, True, True),
    (5, 61, 3, 128, 128, False, True),  # E % 4 != 0: no maps
    (4, 1, 1, 64, 64, False, True), (2, 32, 7, 256, 128, False, False),
    (5, 62, 3, 128, 128, True, True),  # maps with rows not 16-byte aligned: separate launches
    # the separate calls: more than 16 slots, E > 64
    (3, 64, 8, 128, 128, True, True), (32, 64, 8, 2048, 1408, True, True),
    (2, 128, 4, 128, 128, True, True)])
def test_route_align_gate_up_matches_separate_calls(T, E, k, H, I, inverse, norm):
    """moe_route_align_gate_up (one launch for the smallest decode batches:
    every FC1 block routes and aligns the batch itself) equals
    moe_route_align(_inverse) + moe_ffn_gate_up bit for bit: every routing
    output, the conversion back to indices and the activation rows; the
    activations also meet the oracle bar."""
    g = np.random.Generator(np.random.PCG64(T * 13 + E * 3 + k + H + I))
    logits = g.standard_normal((T, E)).astype(np.float32)
    logits[:, : min(E, 3)] = np.round(logits[:, : min(E, 3)])  # some equal logits
    x = mi.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    w13 = mi.f32_to_bf16_bits((g.standard_normal((E, 2 * I, H)) / math.sqrt(H)).astype(np.float32))
    ld, xd, w13d = dev(logits), dev_bf16(x), dev_bf16(w13)
    fused = moe.moe_route_align_gate_up_fused(T, E, k, moe.MOE_BF16, True, H, I)
    assert fused == (T * k <= 16 and E <= 64 and k <= 16)
    print(f"route_align_gate_up T={T} E={E} k={k} H={H} I={I} fused={fused}", flush=True)
    got, act = moe.moe_route_align_gate_up(ld, k, xd, w13d, norm, decode=True, inverse=inverse,
                                           act=_nan_filled((T * k, I), torch.bfloat16))
    if inverse:
        sep = moe.moe_route_align_inverse(ld, k, norm)
    else:
        sep = moe.moe_route_align(ld, k, norm)
    ref_act = moe.moe_ffn_gate_up(xd, w13d, sep, k, True, act=_nan_filled((T * k, I),
                                                                          torch.bfloat16))
    torch.cuda.synchronize()
    assert set(got) == set(sep)
    for key in sep:
        a, b = got[key], sep[key]
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b), key
    rows = int(sep["offsets"][-1])
    assert torch.equal(act[:rows].view(torch.int16), ref_act[:rows].view(torch.int16))
    # the whole decode layer on the fused call's routing and activations,
    # against the oracle
    w2 = mi.f32_to_bf16_bits((g.standard_normal((E, H, I)) / math.sqrt(I)).astype(np.float32))
    w2d = dev_bf16(w2)
    y = moe.moe_ffn_down(act, w2d, got, T, k, True)
    out = moe.moe_combine(y, got["topk_w"], got["slot_to_sorted"], torch.bfloat16)
    out32 = moe.moe_combine(y, got["topk_w"], got["slot_to_sorted"], torch.float32)
    torch.cuda.synchronize()
    ow, oids = oracle.route(logits, k, norm)
    np.testing.assert_array_equal(host(got["topk_ids"]), oids)
    ref = oracle.expert_ffn(x, w13, w2, ow.astype(np.float64), oids, "bf16")
    assert_bf16_layer(host(out), host(out32), ref)


def test_route_align_gate_up_empty():
    """T = 0: zero counts and offsets, nothing else written."""
    E, k, H, I = 16, 4, 128, 128
    ld = torch.empty((0, E), dtype=torch.float32, device=DEV)
    x = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    w13 = torch.zeros((E, 2 * I, H), dtype=torch.bfloat16, device=DEV)
    out = {"topk_w": torch.empty((0, k), dtype=torch.float32, device=DEV),
           "topk_ids": torch.empty((0, k), dtype=torch.int32, device=DEV),
           "counts": torch.full((E,), 7, dtype=torch.int32, device=DEV),
           "offsets": torch.full((E + 1,), 7, dtype=torch.int32, device=DEV),
           "sorted_token_ids": torch.empty(0, dtype=torch.int32, device=DEV),
           "sorted_slot_ids": torch.empty(0, dtype=torch.int32, device=DEV),
           "slot_to_sorted": torch.empty(0, dtype=torch.int32, device=DEV)}
    got, act = moe.moe_route_align_gate_up(ld, k, x, w13, True, decode=True, inverse=False,
                                           out=out)
    torch.cuda.synchronize()
    assert act.shape == (0, I)
    assert int(got["counts"].abs().sum()) == 0 and int(got["offsets"].abs().sum()) == 0


@pytest.mark.parametrize("T,E,k,method", [(16384, 256, 8, "noaux_tc"),
                                          (16384, 160, 6, "group_limited_greedy"),
                                          (1000, 64, 8, "noaux_tc"), (1, 256, 8, "noaux_tc"),
                                          (300, 128, 4, "group_limited_greedy"),
                                          (0, 64, 8, "noaux_tc"), (777, 96, 20, "noaux_tc")])
def test_align_inverse_matches_separate_calls(T, E, k, method):
    """moe_align_inverse (the conversion's blocks in the alignment scatter's
    launch where they fit) equals moe_align and moe_multihot_to_indices one
    after the other, bit for bit, on a group-limited routing's ids and maps;
    the conversion returns the routing's own ids and weights."""
    g = np.random.Generator(np.random.PCG64(T + E * 3 + k))
    scores = (1.0 / (1.0 + np.exp(-g.standard_normal((T, E))))).astype(np.float32)
    bias = (0.1 * g.standard_normal(E)).astype(np.float32)
    n_group = 8 if E % 8 == 0 else 4
    kk = min(k, E // n_group * 4)
    print(f"align_inverse T={T} E={E} k={kk} {method}", flush=True)
    tw = torch.empty((T, kk), dtype=torch.float32, device=DEV)
    ti = torch.empty((T, kk), dtype=torch.int32, device=DEV)
    mh = torch.empty((T, E), dtype=torch.uint8, device=DEV)
    pim = torch.empty((T, E), dtype=torch.float32, device=DEV)
    pos = torch.empty((T, E), dtype=torch.int32, device=DEV)
    moe.moe_route_grouped(dev(scores), kk, n_group, 4, method, dev(bias), True, tw, ti,
                          multihot=(mh, pim, pos))
    got = moe.moe_align_inverse(ti, E, pim, pos)
    sep = moe.moe_align(ti, E)
    sep["probs_indices"], sep["ids_from_multihot"] = moe.moe_multihot_to_indices(pim, pos, kk)
    torch.cuda.synchronize()
    for key in sep:
        a, b = got[key], sep[key]
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b), key
    assert torch.equal(got["ids_from_multihot"], ti)
    assert torch.equal(got["probs_indices"].view(torch.int32), tw.view(torch.int32))


@pytest.mark.parametrize("T,E,k,skew,inv", [(4096, 8, 2, 0.0, 0.0), (8192, 64, 8, 1.1, 0.0),
                                            (16384, 64, 8, 0.0, 0.0), (300, 128, 4, 2.0, 0.1),
                                            (1, 64, 8, 0.0, 0.0), (5000, 1024, 6, 0.5, 0.0),
                                            (0, 16, 2, 0.0, 0.0), (2000, 2, 1, 3.0, 0.0)])
def test_tile_schedule(T, E, k, skew, inv):
    """moe_tile_schedule lists every expert's m-tiles in expert order: each
    expert with c rows has ceil(c / 320) tiles of equal 32-row-fragment
    shares that cover its segment exactly, in order, none empty or over 320
    rows; and the list fits moe_tile_schedule_max."""
    g = np.random.Generator(np.random.PCG64(T + E + 7))
    score = g.random((T, E)) + skew * np.linspace(1.0, 0.0, E)  # skew: low ids favoured
    ids = np.argsort(-score, axis=1)[:, :k].astype(np.int32)
    if inv > 0:
        ids = np.where(g.random(ids.shape) < inv, -1, ids).astype(np.int32)
    a = moe.moe_align(dev(ids), E)
    mx = moe.moe_tile_schedule_max(T, k, E)
    te, trs, tre, num = moe.moe_tile_schedule(a["offsets"], mx)
    torch.cuda.synchronize()
    off = oracle.align(ids, E)["offsets"] if T else np.zeros(E + 1, np.int64)
    n = int(num.item())
    got = list(zip(te.cpu().numpy()[:n], trs.cpu().numpy()[:n], tre.cpu().numpy()[:n]))
    want = []
    for e in range(E):
        c = int(off[e + 1] - off[e])
        mt = -(-c // 320)
        q = -(-c // (32 * mt)) * 32 if mt else 0
        want += [(e, int(off[e]) + min(i * q, c), int(off[e]) + min((i + 1) * q, c))
                 for i in range(mt)]
    assert n == len(want) <= mx
    assert [tuple(int(v) for v in t) for t in got] == want
    # Coverage: the tiles of each expert tile its segment [off[e], off[e+1]).
    for e in range(E):
        rows = [(s, t) for x, s, t in want if x == e]
        assert all(0 < t - s <= 320 for s, t in rows)
        assert all(rows[i][1] == rows[i + 1][0] for i in range(len(rows) - 1))
        if rows:
            assert rows[0][0] == off[e] and rows[-1][1] == off[e + 1]
            assert max(t - s for s, t in rows) - min(t - s for s, t in rows) <= 32 * len(rows)


def test_route_align_routing_workload():
    w = mi.WORKLOADS["routing"]
    x = mi.gating_logits(w)
    got = moe.moe_route_align(dev(x), w.k, w.norm, with_multihot=True)
    torch.cuda.synchronize()
    assert moe.moe_route_align_fused(w.T, w.E, w.k)
    ow, oids = oracle.route(x, w.k, w.norm)
    np.testing.assert_array_equal(got["topk_ids"].cpu().numpy(), oids)
    assert_weights_close(got["topk_w"].cpu().numpy(), ow)
    ref = oracle.align(oids, w.E)
    for key in ALIGN_KEYS:
        np.testing.assert_array_equal(got[key].cpu().numpy(), ref[key], err_msg=key)
    mh, pim, pos = oracle.indices_to_multihot(oids, got["topk_w"].cpu().numpy(), w.E)
    np.testing.assert_array_equal(got["multihot"].cpu().numpy(), mh)
    np.testing.assert_array_equal(got["position_map"].cpu().numpy(), pos)
    np.testing.assert_array_equal(got["probs_in_multihot"].cpu().numpy().view(np.int32),
                                  pim.view(np.int32))


# --------------------------------------------------------------------------
# Multihot conversion and inverse
# --------------------------------------------------------------------------

def _multihot_check(ids, probs, E):
    k = ids.shape[1]
    mh, pim, pos = moe.moe_indices_to_multihot(dev(ids), dev(probs), E)
    back, ids_back = moe.moe_multihot_to_indices(pim, pos, k)
    torch.cuda.synchronize()
    rmh, rpim, rpos = oracle.indices_to_multihot(ids, probs, E)
    np.testing.assert_array_equal(mh.cpu().numpy(), rmh)
    np.testing.assert_array_equal(pim.cpu().numpy().view(np.int32), rpim.view(np.int32))
    np.testing.assert_array_equal(pos.cpu().numpy(), rpos)
    rback, rids = oracle.multihot_to_indices(rpim, rpos, k)
    np.testing.assert_array_equal(back.cpu().numpy().view(np.int32), rback.view(np.int32))
    np.testing.assert_array_equal(ids_back.cpu().numpy(), rids)


def test_multihot_routing_workload_roundtrip():
    w = mi.WORKLOADS["routing"]
    logits = mi.gating_logits(w)
    tw, tids = moe.moe_route(dev(logits), w.k, True)
    mh, pim, pos = moe.moe_indices_to_multihot(tids, tw, w.E)
    back, ids_back = moe.moe_multihot_to_indices(pim, pos, w.k)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int32), tw.view(torch.int32))  # bit-identical
    assert torch.equal(ids_back, tids)
    _multihot_check(tids.cpu().numpy(), tw.cpu().numpy(), w.E)


@pytest.mark.parametrize("T,E,k,inv", [(1, 4, 2, 0.0), (300, 64, 8, 0.0), (100, 6, 2, 0.25),
                                       (20, 300, 9, 0.1), (7, 1024, 64, 0.0), (513, 130, 5, 0.3),
                                       (64, 1, 1, 0.0), (333, 128, 8, 0.1), (1001, 256, 8, 0.05),
                                       (77, 160, 6, 0.0), (50, 100, 16, 0.2), (9, 68, 3, 0.0),
                                       (40, 252, 17, 0.0)])
def test_multihot_random(T, E, k, inv):
    _multihot_check(mi.random_ids(T + E, T, E, k, invalid_frac=inv), mi.random_probs(T + k, T, k),
                    E)


@pytest.mark.parametrize("T,E,k,norm,ties", [(16384, 64, 8, True, False), (1, 64, 8, True, False),
                                             (37, 8, 2, False, True), (1000, 64, 16, True, True),
                                             (5, 4, 4, True, False), (301, 12, 3, False, False),
                                             (60, 6, 2, True, False), (33, 130, 7, True, False)])
def test_route_multihot_fused(T, E, k, norm, ties):
    """moe_route_multihot: every output bit-identical to moe_route followed by
    moe_indices_to_multihot (fused kernel where E <= 64, E % 4 == 0, k <= 16;
    the two launches otherwise), ids equal to the oracle's, multihot equal to
    the oracle's conversion of the weights."""
    g = np.random.Generator(np.random.PCG64(T * 131 + E * 7 + k))
    x = g.standard_normal((T, E)).astype(np.float32)
    if ties:
        x = np.round(x * 2) / 2  # many equal logits per row
    tw, ti, mh, pim, pos = moe.moe_route_multihot(dev(x), k, norm)
    rw, ri = moe.moe_route(dev(x), k, norm)
    rmh, rpim, rpos = moe.moe_indices_to_multihot(ri, rw, E)
    torch.cuda.synchronize()
    assert moe.moe_route_multihot_fused(E, k) == (E <= 64 and E % 4 == 0 and k <= 16)
    assert torch.equal(ti, ri)
    assert torch.equal(tw.view(torch.int32), rw.view(torch.int32))
    assert torch.equal(mh, rmh)
    assert torch.equal(pim.view(torch.int32), rpim.view(torch.int32))
    assert torch.equal(pos, rpos)
    _, oids = oracle.route(x, k, norm)
    np.testing.assert_array_equal(ti.cpu().numpy(), oids)
    omh, opim, opos = oracle.indices_to_multihot(ti.cpu().numpy(), tw.cpu().numpy(), E)
    np.testing.assert_array_equal(mh.cpu().numpy(), omh)
    np.testing.assert_array_equal(pim.cpu().numpy().view(np.int32), opim.view(np.int32))
    np.testing.assert_array_equal(pos.cpu().numpy(), opos)


def test_multihot_worked_examples():
    ids = np.array([[0, 1], [1, 2]], np.int32)
    probs = np.array([[0.1, 0.2], [0.3, 0.4]], np.float32)
    mh, pim, pos = moe.moe_indices_to_multihot(dev(ids), dev(probs), 4)
    assert mh.cpu().numpy().tolist() == [[1, 1, 0, 0], [0, 1, 1, 0]]
    np.testing.assert_array_equal(pim.cpu().numpy(), np.array([[0.1, 0.2, 0, 0], [0, 0.3, 0.4, 0]],
                                                              np.float32))
    pim2 = dev(np.array([[0.7, 0.8, 0, 0], [0, 0.1, 0.9, 0]], np.float32))
    pos2 = dev(np.array([[0, 1, -1, -1], [-1, 0, 1, -1]], np.int32))
    back, _ = moe.moe_multihot_to_indices(pim2, pos2, 2)
    np.testing.assert_array_equal(back.cpu().numpy(), np.array([[0.7, 0.8], [0.1, 0.9]], np.float32))


# --------------------------------------------------------------------------
# Expert FFN + combine
# --------------------------------------------------------------------------

def _rand_layer(seed, T, H, I, E, k, dtype="bf16", skew=0.0, inv=0.0):
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((T, H)).astype(np.float32)
    w13 = (g.standard_normal((E, 2 * I, H)) / math.sqrt(H)).astype(np.float32)
    w2 = (g.standard_normal((E, H, I)) / math.sqrt(I)).astype(np.float32)
    logits = g.standard_normal((T, E)).astype(np.float32)
    logits += (skew * np.arange(E, dtype=np.float32))[None, :]
    w, ids = oracle.route(logits, k, True)
    if inv > 0:
        ids = np.where(g.random(ids.shape) < inv, -1, ids).astype(np.int32)
    if dtype == "bf16":
        x, w13, w2 = (mi.f32_to_bf16_bits(a) for a in (x, w13, w2))
    return x, w13, w2, w.astype(np.float32), ids


def _ffn_gpu(x, w13, w2, w32, ids, dtype, decode=False):
    """-> (out, pre-rounding float32 out)."""
    E = w13.shape[0]
    td = dev_bf16 if dtype == "bf16" else dev
    a = moe.moe_align(dev(ids), E)
    return run_ffn(td(x), td(w13), td(w2), dev(w32), a, ids.shape[1], decode)


@pytest.mark.parametrize("T,H,I,E,k,skew,inv", [
    (300, 128, 192, 8, 2, 0.0, 0.0),
    (1000, 256, 128, 16, 4, 0.0, 0.0),
    (77, 64, 64, 3, 3, 0.0, 0.0),
    (513, 512, 384, 64, 8, 0.3, 0.0),
    (1, 128, 128, 8, 2, 0.0, 0.0),
    (600, 320, 448, 4, 1, 2.0, 0.0),
    (260, 192, 256, 12, 3, 0.0, 0.2),
    (2048, 1024, 256, 8, 2, 1.0, 0.0),
    (1400, 128, 256, 2, 1, 0.0, 0.0),
    (2600, 64, 128, 4, 2, 0.5, 0.1),
    # An expert with more m-tiles than one band of the tile order holds, in
    # both products (8 n-tiles each): every token checked.
    (2000, 2048, 1024, 2, 1, 3.0, 0.0),
    (3000, 1024, 1408, 4, 2, 2.0, 0.05),
])
def test_ffn_bf16_prefill(T, H, I, E, k, skew, inv):
    x, w13, w2, w32, ids = _rand_layer(T + H + I + E, T, H, I, E, k, skew=skew, inv=inv)
    out, out32 = _ffn_gpu(x, w13, w2, w32, ids, "bf16")
    ref = oracle.expert_ffn(x, w13, w2, w32.astype(np.float64), ids, "bf16")
    assert_bf16_layer(out, out32, ref)


@pytest.mark.parametrize("T,H,I,E,k", [(1, 128, 128, 8, 2), (5, 256, 192, 16, 4),
                                       (32, 512, 256, 64, 8), (64, 64, 64, 8, 8),
                                       (20, 192, 320, 6, 2), (15, 128, 192, 4, 2),
                                       (16, 128, 192, 4, 2), (48, 256, 128, 32, 6)])
def test_ffn_bf16_decode(T, H, I, E, k):
    x, w13, w2, w32, ids = _rand_layer(T * 5 + H + I, T, H, I, E, k)
    out, out32 = _ffn_gpu(x, w13, w2, w32, ids, "bf16", decode=True)
    ref = oracle.expert_ffn(x, w13, w2, w32.astype(np.float64), ids, "bf16")
    assert_bf16_layer(out, out32, ref)


@pytest.mark.parametrize("T,H,I,E,k,inv,skew", [
    (1, 2048, 1408, 64, 8, 0.0, 0.0), (1, 128, 128, 8, 2, 0.0, 0.0),
    (2, 512, 1536, 16, 8, 0.0, 0.0), (4, 256, 192, 64, 8, 0.0, 0.0),
    (3, 192, 320, 6, 2, 0.3, 0.0), (16, 128, 192, 4, 2, 0.0, 0.0),
    (32, 64, 64, 40, 1, 0.5, 0.0), (1, 64, 64, 1, 1, 0.0, 0.0), (6, 320, 1024, 6, 5, 0.0, 0.0),
    (8, 128, 1536, 8, 4, 0.0, 0.0),  # both limits
    # experts with more than 16 tokens (a second block of token columns)
    (32, 128, 320, 4, 1, 0.0, 3.0), (28, 256, 448, 2, 1, 0.0, 1.0),
    (24, 192, 704, 2, 1, 0.1, 2.0), (32, 64, 1536, 1, 1, 0.0, 0.0),
    # not fused: more than 32 slots, I past the limit
    (33, 128, 128, 8, 1, 0.0, 0.0), (1, 128, 1600, 4, 2, 0.0, 0.0)])
def test_ffn_down_combine_decode(T, H, I, E, k, inv, skew):
    """moe_ffn_down_combine equals moe_ffn_down + moe_combine bit for bit on
    the decode path, fused (one launch, no y) or not, with ids dropped."""
    x, w13, w2, w32, ids = _rand_layer(T * 7 + H + I + E, T, H, I, E, k, skew=skew, inv=inv)
    cnt = np.bincount(ids[ids >= 0], minlength=E)
    xd, w13d, w2d, twd = dev_bf16(x), dev_bf16(w13), dev_bf16(w2), dev(w32)
    a = moe.moe_align(dev(ids), E)
    fused = moe.moe_ffn_down_combine_fused(moe.MOE_BF16, T, H, I, E, k, decode=True)
    assert fused == (T * k <= 32 and I <= 1536)
    if T >= 20 and k == 1 and E <= 4:
        assert cnt.max() > 16  # the case is meant to reach the second column block
    act = moe.moe_ffn_gate_up(xd, w13d, a, k, decode=True)
    y = moe.moe_ffn_down(act, w2d, a, T, k, decode=True)
    two = moe.moe_combine(y, twd, a["slot_to_sorted"], torch.bfloat16,
                          out=_nan_filled((T, H), torch.bfloat16))
    one = moe.moe_ffn_down_combine(act, w2d, twd, a, T, k, decode=True,
                                   out=_nan_filled((T, H), torch.bfloat16))
    again = moe.moe_ffn_down_combine(act, w2d, twd, a, T, k, decode=True)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))
    assert torch.equal(again.view(torch.int16), two.view(torch.int16))
    ref = oracle.expert_ffn(x, w13, w2, w32.astype(np.float64), ids, "bf16")
    out32 = moe.moe_combine(y, twd, a["slot_to_sorted"], torch.float32)
    torch.cuda.synchronize()
    assert_bf16_layer(host(one), host(out32), ref)


@pytest.mark.parametrize("T,H,I,E,k", [(4, 64, 128, 8, 2), (50, 128, 64, 5, 3), (1, 64, 64, 1, 1)])
def test_ffn_f32(T, H, I, E, k):
    x, w13, w2, w32, ids = _rand_layer(T + 3 * H, T, H, I, E, k, dtype="f32")
    out, _ = _ffn_gpu(x, w13, w2, w32, ids, "f32")
    ref = oracle.expert_ffn(x, w13, w2, w32.astype(np.float64), ids, "f32")
    assert_layer_close(out, ref, TOL_F32)


def test_tiny_workload_layer_f32():
    w = mi.WORKLOADS["tiny"]
    inp = mi.layer_inputs(w)
    out, tw, tids, _ = moe.moe_layer(dev(inp["hidden"]), dev(inp["w13"]), dev(inp["w2"]),
                                     dev(inp["logits"]), w.k, w.norm, decode=False)
    torch.cuda.synchronize()
    ref = oracle.layer(inp, w.k, w.norm, "f32")
    np.testing.assert_array_equal(tids.cpu().numpy(), ref["topk_ids"])
    assert_layer_close(host(out), ref["out"], TOL_F32)


def _full_layer(name, decode, sample=None):
    w = mi.WORKLOADS[name]
    inp = mi.layer_inputs(w)
    x, w13, w2 = dev_bf16(inp["hidden"]), dev_bf16(inp["w13"]), dev_bf16(inp["w2"])
    tw, tids = moe.moe_route(dev(inp["logits"]), w.k, w.norm)
    a = moe.moe_align(tids, w.E)
    got, got32 = run_ffn(x, w13, w2, tw, a, w.k, decode)
    ow, oids = oracle.route(inp["logits"], w.k, w.norm)
    np.testing.assert_array_equal(tids.cpu().numpy(), oids)
    assert_weights_close(tw.cpu().numpy(), ow)
    toks = np.arange(w.T) if sample is None else sample(w.T, oids, w.E)
    print(f"{name}: oracle on {len(toks)} of {w.T} tokens", flush=True)
    ref = oracle.expert_ffn(inp["hidden"], inp["w13"], inp["w2"], ow, oids, "bf16", tokens=toks)
    rel = assert_bf16_layer(got[toks], got32[toks], ref)
    print(f"{name}: max |error| / RMS = {rel:.3g}", flush=True)
    assert np.all(np.isfinite(got))
    return got, rel


def _fragment_tokens(T, ids, E):
    """Tokens whose rows cover every 32-row fragment of every expert segment.

    The grouped GEMMs cut an expert's segment of the aligned order into m-tiles
    whose first rows sit at multiples of 32 from the segment start, and a tile's
    waves own 32-row fragments from there; whatever the tile height, each
    fragment of each (expert, m-tile, n-tile) is then hit by the rows at
    segment offsets 32 j and 32 j + 31 (and the segment's last row).  A token's
    output row spans every n-tile of both products, so these tokens check every
    tile of FC1 and FC2.  Plus the first and last token."""
    a = oracle.align(ids, E)
    off, sti = a["offsets"], a["sorted_token_ids"]
    picks = {0, T - 1}
    for e in range(E):
        o0, o1 = int(off[e]), int(off[e + 1])
        if o1 == o0:
            continue
        pos = np.arange(o0, o1, 32)
        pos = np.concatenate([pos, np.minimum(pos + 31, o1 - 1), [o1 - 1]])
        picks.update(int(t) for t in sti[pos])
    return np.array(sorted(picks), np.int64)


def test_mixtral_layer_full_size():
    _full_layer("mixtral", False, sample=_fragment_tokens)


def test_finegrained_layer_full_size():
    _full_layer("finegrained", False, sample=_fragment_tokens)


@pytest.mark.parametrize("name", ["decode1", "decode32"])
def test_decode_layer_full_size(name):
    got, _ = _full_layer(name, True)
    got_prefill, _ = _full_layer(name, False)
    # Both paths round act and y once to bf16 from fp32 sums of the same terms.
    np.testing.assert_allclose(got, got_prefill, rtol=0, atol=2e-2 * np.sqrt(np.mean(got ** 2)))


@pytest.mark.parametrize("T,H,I,E,k,skew,inv", [(300, 128, 192, 8, 2, 0.0, 0.0),
                                                (513, 512, 384, 64, 8, 0.3, 0.0),
                                                (260, 192, 256, 12, 3, 0.0, 0.2)])
def test_ffn_bf16_prefill_pointer_path(monkeypatch, T, H, I, E, k, skew, inv):
    """The grouped GEMMs' 64-bit pointer path (taken for operands of 2 GiB or
    more; forced here) against the oracle, and equal to the default path."""
    x, w13, w2, w32, ids = _rand_layer(T + H + I + E, T, H, I, E, k, skew=skew, inv=inv)
    base, base32 = _ffn_gpu(x, w13, w2, w32, ids, "bf16")
    monkeypatch.setenv("MOE_GEMM_POINTER_PATH", "1")
    out, out32 = _ffn_gpu(x, w13, w2, w32, ids, "bf16")
    monkeypatch.delenv("MOE_GEMM_POINTER_PATH")
    ref = oracle.expert_ffn(x, w13, w2, w32.astype(np.float64), ids, "bf16")
    assert_bf16_layer(out, out32, ref)
    np.testing.assert_array_equal(out32.view(np.uint32), base32.view(np.uint32))


@pytest.mark.parametrize("T,H,I,E,k,skew", [(700, 256, 1024, 8, 2, 0.0),
                                            (300, 512, 2048, 16, 4, 1.0)])
def test_ffn_bf16_down_k_slices(T, H, I, E, k, skew):
    """FC2 cut into K slices: the planes sum to the one-slice product (up to
    float32 reassociation), the combined output meets the oracle bar, and
    the result is the same on every run."""
    x, w13, w2, w32, ids = _rand_layer(T + 11 * I, T, H, I, E, k, skew=skew)
    xd, w13d, w2d, twd = dev_bf16(x), dev_bf16(w13), dev_bf16(w2), dev(w32)
    a = moe.moe_align(dev(ids), E)
    act = moe.moe_ffn_gate_up(xd, w13d, a, k)
    y1 = moe.moe_ffn_down(act, w2d, a, T, k, splits=1)
    ref = oracle.expert_ffn(x, w13, w2, w32.astype(np.float64), ids, "bf16")
    rows = int(a["offsets"][-1])
    base = y1[:rows].double()
    scale = float(base.pow(2).mean().sqrt())
    for sp in (2, 4):
        y = moe.moe_ffn_down(act, w2d, a, T, k, splits=sp)
        assert y.shape == (sp, T * k, H)
        err = float((y[:, :rows].double().sum(0) - base).abs().max())
        assert err <= 1e-5 * scale, f"{sp} slices: {err:.3e} vs rms {scale:.3e}"
        out = moe.moe_combine(y, twd, a["slot_to_sorted"], torch.bfloat16)
        out32 = moe.moe_combine(y, twd, a["slot_to_sorted"], torch.float32)
        again = moe.moe_combine(moe.moe_ffn_down(act, w2d, a, T, k, splits=sp), twd,
                                a["slot_to_sorted"], torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(out32, again)
        assert_bf16_layer(host(out), host(out32), ref)


def test_layer_deterministic():
    x, w13, w2, w32, ids = _rand_layer(9, 700, 256, 256, 16, 4, skew=0.5)
    a, a32 = _ffn_gpu(x, w13, w2, w32, ids, "bf16")
    b, b32 = _ffn_gpu(x, w13, w2, w32, ids, "bf16")
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    np.testing.assert_array_equal(a32.view(np.uint32), b32.view(np.uint32))


# --------------------------------------------------------------------------
# One layer step captured as a HIP graph (the library allocates, syncs and
# memsets nothing, so every call is capturable)
# --------------------------------------------------------------------------

def _layer_into(bufs, logits, x, w13, w2, k, decode, fused=False):
    T, E = logits.shape
    if fused:  # route + multihot + align in one call, as the benchmark step runs them
        out = {"topk_w": bufs["tw"], "topk_ids": bufs["ids"], **bufs["aligned"],
               "multihot": bufs["mh"], "probs_in_multihot": bufs["pim"],
               "position_map": bufs["pos"]}
        if decode:  # with FC1 in the same call (one launch for the smallest batches)
            moe.moe_route_align_gate_up(logits, k, x, w13, True, decode=True, inverse=False,
                                        out=out, act=bufs["act"], workspace=bufs["ws"])
        else:
            moe.moe_route_align(logits, k, True, with_multihot=True, out=out,
                                workspace=bufs["ws"])
            moe.moe_ffn_gate_up(x, w13, bufs["aligned"], k, decode, bufs["act"])
    else:
        moe.moe_route(logits, k, True, bufs["tw"], bufs["ids"])
        moe.moe_align(bufs["ids"], E, bufs["aligned"], bufs["ws"])
        moe.moe_ffn_gate_up(x, w13, bufs["aligned"], k, decode, bufs["act"])
    if fused:  # FC2 + combine in one call (one launch for the smallest decode batches)
        moe.moe_ffn_down_combine(bufs["act"], w2, bufs["tw"], bufs["aligned"], T, k, decode,
                                 bufs["y"], bufs["out"])
        return
    moe.moe_ffn_down(bufs["act"], w2, bufs["aligned"], T, k, decode, bufs["y"])
    moe.moe_combine(bufs["y"], bufs["tw"], bufs["aligned"]["slot_to_sorted"], torch.bfloat16,
                    bufs["out"])


def _layer_bufs(T, H, I, E, k, decode):
    sp = moe.moe_ffn_down_splits(moe.MOE_BF16, T, H, I, E, k, decode)
    return {
        "tw": torch.empty((T, k), dtype=torch.float32, device=DEV),
        "ids": torch.empty((T, k), dtype=torch.int32, device=DEV),
        "aligned": {n: torch.empty(m, dtype=torch.int32, device=DEV) for n, m in
                    (("counts", E), ("offsets", E + 1), ("sorted_token_ids", T * k),
                     ("sorted_slot_ids", T * k), ("slot_to_sorted", T * k))},
        "ws": torch.empty(max(1, moe.moe_align_workspace_size(T, k, E)), dtype=torch.uint8,
                          device=DEV),
        "act": torch.empty((T * k, I), dtype=torch.bfloat16, device=DEV),
        "y": torch.empty((sp, T * k, H), dtype=torch.float32, device=DEV),
        "out": torch.empty((T, H), dtype=torch.bfloat16, device=DEV),
        "mh": torch.empty((T, E), dtype=torch.uint8, device=DEV),
        "pim": torch.empty((T, E), dtype=torch.float32, device=DEV),
        "pos": torch.empty((T, E), dtype=torch.int32, device=DEV),
    }


@pytest.mark.parametrize("T,H,I,E,k,decode", [(1, 256, 256, 16, 4, True),
                                              (32, 512, 384, 64, 8, True),
                                              (300, 256, 2048, 8, 2, False),
                                              (2048, 256, 256, 64, 8, False)])
@pytest.mark.parametrize("fused", [False, True])
def test_layer_graph_replay(T, H, I, E, k, decode, fused):
    """Replays of a captured step, with other GPU work between them, equal
    eager runs of the same step bit for bit, for several inputs."""
    x, w13, w2, _, _ = _rand_layer(T * 3 + I, T, H, I, E, k)
    xd, w13d, w2d = dev_bf16(x), dev_bf16(w13), dev_bf16(w2)
    g = np.random.Generator(np.random.PCG64(T + E))
    draws = [dev(g.standard_normal((T, E)).astype(np.float32)) for _ in range(4)]
    static = torch.empty_like(draws[0])
    static.copy_(draws[0])
    bufs = _layer_bufs(T, H, I, E, k, decode)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _layer_into(bufs, static, xd, w13d, w2d, k, decode, fused)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _layer_into(bufs, static, xd, w13d, w2d, k, decode, fused)
    eager = _layer_bufs(T, H, I, E, k, decode)
    for r in (1, 2, 0, 3, 1):
        static.copy_(draws[r])
        graph.replay()
        torch.cuda.synchronize()
        got = bufs["out"].clone()
        got_ids = bufs["ids"].clone()
        # unrelated eager work, then the eager step on the same input
        torch.matmul(xd.float(), xd.float().t()).sum().item()
        _layer_into(eager, draws[r], xd, w13d, w2d, k, decode, fused)
        torch.cuda.synchronize()
        assert torch.equal(got_ids, eager["ids"])
        assert torch.equal(got.view(torch.int16), eager["out"].view(torch.int16))


def test_grouped_routing_graph_replay():
    """The grouped routing step (selection with its multihot maps, align,
    inverse) replayed from a captured graph equals eager runs bit for bit."""
    w = mi.GROUPED["grouped_noaux"]
    T, E, k = 2048, w.E, w.k
    draws = [dev(mi.grouped_scores(w, T=T, draw=r)) for r in range(3)]
    bias = dev(mi.correction_bias(w))

    def bufs():
        return {"tw": torch.empty((T, k), dtype=torch.float32, device=DEV),
                "ids": torch.empty((T, k), dtype=torch.int32, device=DEV),
                "mh": (torch.empty((T, E), dtype=torch.uint8, device=DEV),
                       torch.empty((T, E), dtype=torch.float32, device=DEV),
                       torch.empty((T, E), dtype=torch.int32, device=DEV)),
                "ws": torch.empty(max(1, moe.moe_align_workspace_size(T, k, E)),
                                  dtype=torch.uint8, device=DEV),
                "back": (torch.empty((T, k), dtype=torch.float32, device=DEV),
                         torch.empty((T, k), dtype=torch.int32, device=DEV))}

    def step(b, scores):
        moe.moe_route_grouped(scores, k, w.n_group, w.topk_group, w.method, bias, w.renorm,
                              b["tw"], b["ids"], multihot=b["mh"])
        b["aligned"] = moe.moe_align(b["ids"], E, b.get("aligned"), b["ws"])
        moe.moe_multihot_to_indices(b["mh"][1], b["mh"][2], k, out=b["back"])

    static = torch.empty_like(draws[0])
    static.copy_(draws[0])
    gb, eb = bufs(), bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(gb, static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gb, static)
    for r in (1, 2, 0, 1):
        static.copy_(draws[r])
        graph.replay()
        torch.cuda.synchronize()
        got = {key: gb["aligned"][key].clone() for key in ALIGN_KEYS}
        got_back = gb["back"][1].clone()
        step(eb, draws[r])
        torch.cuda.synchronize()
        for key in ALIGN_KEYS:
            assert torch.equal(got[key], eb["aligned"][key]), key
        assert torch.equal(got_back, eb["back"][1])
        assert torch.equal(got_back, eb["ids"])
