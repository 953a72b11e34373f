"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every expected value is either
printed on a page (fixtures under tests/golden/, each citing its passage), a
closed form, a textbook / library routine on a special case, an invariant, or
a brute force that computes the same quantity a different way.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import moe_inputs as mi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Route (top-k + softmax weights)
# --------------------------------------------------------------------------

def _sort_topk(x, k):
    """Full stable sort: value descending, ties by ascending index."""
    E = x.shape[1]
    out = np.empty((x.shape[0], k), np.int32)
    for t in range(x.shape[0]):
        order = np.lexsort((np.arange(E), -x[t].astype(np.float64)))
        out[t] = order[:k]
    return out


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (50, 64, 8), (17, 5, 5), (9, 1, 1), (33, 130, 7)])
@pytest.mark.parametrize("ties", [False, True])
def test_route_ids_match_full_sort(T, E, k, ties):
    g = np.random.Generator(np.random.PCG64(T * 131 + E + k))
    x = g.standard_normal((T, E)).astype(np.float32)
    if ties:  # few distinct values -> many equal pairs per row
        x = np.round(x * 2).astype(np.float32)
    for norm in (True, False):
        _, ids = oracle.route(x, k, norm)
        np.testing.assert_array_equal(ids, _sort_topk(x, k))


def test_route_crafted_rows():
    _, ids = oracle.route(np.zeros((1, 6), np.float32), 3)
    assert ids.tolist() == [[0, 1, 2]]  # all equal -> lowest indices, ascending
    _, ids = oracle.route(np.array([[1, 3, 3, 2]], np.float32), 2)
    assert ids.tolist() == [[1, 2]]  # tie at the top: lower index first
    _, ids = oracle.route(np.array([[-5, -1, -3, -1e30]], np.float32), 4)
    assert ids.tolist() == [[1, 2, 0, 3]]


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (16, 16), (7, 1)])
def test_route_norm_weights(E, k):
    g = np.random.Generator(np.random.PCG64(E * 7 + k))
    x = (g.standard_normal((40, E)) * 3).astype(np.float32)
    w, ids = oracle.route(x, k, True)
    assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)  # descending with the logits
    sel = np.take_along_axis(x.astype(np.float64), ids, 1)
    ref = scipy.special.softmax(sel, axis=1)  # library softmax over the k picked
    np.testing.assert_allclose(w, ref, rtol=1e-13, atol=0)
    if k == 1:
        assert np.all(w == 1.0)
    if k == E:  # renormalised top-E == full softmax, reordered
        full = scipy.special.softmax(x.astype(np.float64), axis=1)
        np.testing.assert_allclose(w, np.take_along_axis(full, ids, 1), rtol=1e-13)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (5, 5)])
def test_route_full_softmax_weights(E, k):
    g = np.random.Generator(np.random.PCG64(100 + E))
    x = (g.standard_normal((40, E)) * 2).astype(np.float32)
    w, ids = oracle.route(x, k, False)
    full = scipy.special.softmax(x.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids, 1), rtol=1e-13)
    if k == E:
        assert np.all(np.abs(w.sum(1) - 1) < 1e-12)


def test_route_shift_invariance():
    # Adding a constant to a row changes neither selection nor weights.
    g = np.random.Generator(np.random.PCG64(5))
    x = g.standard_normal((30, 16)).astype(np.float32)
    w0, i0 = oracle.route(x, 4, True)
    w1, i1 = oracle.route((x + np.float32(0.5)).astype(np.float32), 4, True)
    np.testing.assert_array_equal(i0, i1)
    np.testing.assert_allclose(w0, w1, rtol=1e-6)


# --------------------------------------------------------------------------
# Router logits (the linear gate before routing)
# --------------------------------------------------------------------------

def test_router_logits_one_hot_rows_pick_weight_columns():
    # A token that is the unit vector e_h has logits W[:, h], exactly.
    g = np.random.Generator(np.random.PCG64(81))
    H, E = 64, 12
    w = mi.f32_to_bf16_bits(g.standard_normal((E, H)).astype(np.float32))
    x = np.zeros((H, H), np.float32)
    x[np.arange(H), np.arange(H)] = 1.0
    got = oracle.router_logits(mi.f32_to_bf16_bits(x), w, "bf16")
    np.testing.assert_array_equal(got, mi.bf16_bits_to_f32(w).astype(np.float64).T)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_router_logits_match_library_matmul(dtype):
    g = np.random.Generator(np.random.PCG64(82))
    T, H, E = 37, 256, 20
    x = g.standard_normal((T, H)).astype(np.float32)
    w = (g.standard_normal((E, H)) / 16).astype(np.float32)
    if dtype == "bf16":
        xb, wb = mi.f32_to_bf16_bits(x), mi.f32_to_bf16_bits(w)
        x, w = mi.bf16_bits_to_f32(xb), mi.bf16_bits_to_f32(wb)
        got = oracle.router_logits(xb, wb, "bf16")
    else:
        got = oracle.router_logits(x, w, "f32")
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


# --------------------------------------------------------------------------
# Group-limited routing (group_limited_greedy / noaux_tc)
# --------------------------------------------------------------------------

def _grouped_bruteforce(scores, bias, k, n_group, topk_group, method):
    """Same selection by whole-array sorting instead of insertion: group scores
    from a sort of each group, groups and experts ranked with np.lexsort
    (value descending, lower index first)."""
    T, E = scores.shape
    gs = E // n_group
    choice = scores if bias is None else (scores + bias[None, :]).astype(np.float32)
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        grp = choice[t].reshape(n_group, gs)
        if method == "noaux_tc":
            srt = np.sort(grp, axis=1)
            gsc = (srt[:, -1] + srt[:, -2]).astype(np.float32)  # float32 add
        else:
            gsc = grp.max(axis=1)
        keep = np.lexsort((np.arange(n_group), -gsc.astype(np.float64)))[:topk_group]
        cand = np.concatenate([np.arange(g * gs, (g + 1) * gs) for g in keep])
        order = np.lexsort((cand, -choice[t, cand].astype(np.float64)))
        ids[t] = cand[order[:k]]
    return ids


def test_grouped_crafted_rows_tell_the_methods_apart():
    # Four groups of two.  Group maxima: 0.9, 0.5, 0.2, 0.3 -> greedy keeps
    # group 0 and selects experts 0, 1.  Sums of the top two: 0.9, 1.0, 0.3,
    # 0.35 -> noaux_tc keeps group 1; its two equal scores come out lower id
    # first.
    s = np.array([[0.90, 0.00, 0.50, 0.50, 0.10, 0.20, 0.30, 0.05]], np.float32)
    w, ids = oracle.route_grouped(s, 2, 4, 1, "group_limited_greedy")
    assert ids.tolist() == [[0, 1]]
    assert w.tolist() == [[float(np.float32(0.9)), 0.0]]
    w, ids = oracle.route_grouped(s, 2, 4, 1, "noaux_tc", bias=np.zeros(8, np.float32))
    assert ids.tolist() == [[2, 3]] and w.tolist() == [[0.5, 0.5]]
    # With two groups kept greedy takes groups 0 and 1 and then the best two
    # experts of those: 0 (0.9), then 2 and 3 tie at 0.5 -> 2.
    _, ids = oracle.route_grouped(s, 2, 4, 2, "group_limited_greedy")
    assert ids.tolist() == [[0, 2]]


def test_grouped_bias_steers_choice_but_not_weights():
    # Two groups of four.  Unbiased top-two sums: 1.1 vs 1.07 -> group 0.  A
    # +0.1 bias on experts 4, 5 lifts group 1 to 1.27 -> experts 4, 5, whose
    # weights are their UNbiased scores; renormalised they sum to 1.
    s = np.array([[0.6, 0.5, 0.1, 0.1, 0.55, 0.52, 0.2, 0.2]], np.float32)
    zero = np.zeros(8, np.float32)
    b = np.array([0, 0, 0, 0, 0.1, 0.1, 0, 0], np.float32)
    w, ids = oracle.route_grouped(s, 2, 2, 1, "noaux_tc", bias=zero)
    assert ids.tolist() == [[0, 1]]
    w, ids = oracle.route_grouped(s, 2, 2, 1, "noaux_tc", bias=b)
    assert ids.tolist() == [[4, 5]]
    assert w.tolist() == [[float(np.float32(0.55)), float(np.float32(0.52))]]
    w, _ = oracle.route_grouped(s, 2, 2, 1, "noaux_tc", bias=b, renormalize=True)
    a, c = float(np.float32(0.55)), float(np.float32(0.52))
    np.testing.assert_allclose(w[0], [a / (a + c), c / (a + c)], rtol=1e-15)


@pytest.mark.parametrize("method", ["group_limited_greedy", "noaux_tc"])
def test_grouped_all_groups_kept_is_plain_topk(method):
    # topk_group = n_group masks nothing: the selection is the plain top-k of
    # the choice scores (full sort), the weights the scores at those ids.
    g = np.random.Generator(np.random.PCG64(71))
    s = g.random((40, 64)).astype(np.float32)
    b = (g.standard_normal(64) * 0.1).astype(np.float32) if method == "noaux_tc" else None
    w, ids = oracle.route_grouped(s, 6, 8, 8, method, bias=b)
    choice = s if b is None else (s + b[None, :]).astype(np.float32)
    np.testing.assert_array_equal(ids, _sort_topk(choice, 6))
    np.testing.assert_array_equal(w, np.take_along_axis(s, ids, 1).astype(np.float64))


def test_grouped_singleton_groups_is_plain_topk():
    # Groups of one expert: greedy's group scores are the scores themselves,
    # so keeping the k best groups and then the k best experts is plain top-k.
    g = np.random.Generator(np.random.PCG64(72))
    s = g.random((30, 16)).astype(np.float32)
    _, ids = oracle.route_grouped(s, 4, 16, 4, "group_limited_greedy")
    np.testing.assert_array_equal(ids, _sort_topk(s, 4))


def test_grouped_all_equal_row():
    s = np.full((1, 32), 0.25, np.float32)
    for method, b in (("group_limited_greedy", None), ("noaux_tc", np.zeros(32, np.float32))):
        _, ids = oracle.route_grouped(s, 5, 8, 3, method, bias=b)
        assert ids.tolist() == [[0, 1, 2, 3, 4]]  # groups 0..2 kept, lowest ids first


@pytest.mark.parametrize("method,E,n_group,topk_group,k", [
    ("noaux_tc", 256, 8, 4, 8), ("group_limited_greedy", 160, 8, 3, 6),
    ("noaux_tc", 64, 4, 2, 6), ("group_limited_greedy", 64, 16, 5, 9)])
@pytest.mark.parametrize("ties", [False, True])
def test_grouped_matches_sort_bruteforce(method, E, n_group, topk_group, k, ties):
    g = np.random.Generator(np.random.PCG64(E + n_group * 7 + k))
    s = g.random((48, E)).astype(np.float32)
    if ties:
        s = (np.round(s * 6) / 6).astype(np.float32)
    b = (g.standard_normal(E) * 0.1).astype(np.float32) if method == "noaux_tc" else None
    if ties and b is not None:
        b = (np.round(b * 8) / 8).astype(np.float32)
    for renorm in (False, True):
        w, ids = oracle.route_grouped(s, k, n_group, topk_group, method, bias=b,
                                      renormalize=renorm)
        np.testing.assert_array_equal(ids, _grouped_bruteforce(s, b, k, n_group, topk_group,
                                                               method))
        raw = np.take_along_axis(s, ids, 1).astype(np.float64)
        if renorm:
            np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)
            np.testing.assert_allclose(w, raw / raw.sum(1, keepdims=True), rtol=1e-15)
        else:
            np.testing.assert_array_equal(w, raw)
        # Every selected expert lies in one of at most topk_group groups.
        assert max(len(set((ids[t] // (E // n_group)).tolist())) for t in range(len(ids))) \
            <= topk_group


def test_grouped_rejects_bad_shapes():
    s = np.zeros((2, 12), np.float32)
    with pytest.raises(ValueError):
        oracle.route_grouped(s, 2, 5, 1, "group_limited_greedy")  # 12 % 5 != 0
    with pytest.raises(ValueError):
        oracle.route_grouped(s, 7, 4, 2, "group_limited_greedy")  # k > 2 groups x 3
    with pytest.raises(ValueError):
        oracle.route_grouped(s, 2, 4, 2, "noaux_tc")  # noaux_tc needs the bias
    with pytest.raises(ValueError):
        oracle.route_grouped(s, 1, 12, 2, "noaux_tc", bias=np.zeros(12, np.float32))  # groups of 1


def test_grouped_workload_inputs():
    for w in mi.GROUPED.values():
        s = mi.grouped_scores(w, T=64)
        assert s.shape == (64, w.E) and s.dtype == np.float32
        assert (s > 0).all() and (s < 1).all()
        b = mi.correction_bias(w)
        assert (b is None) == (w.method != "noaux_tc")
        _, ids = oracle.route_grouped(s, w.k, w.n_group, w.topk_group, w.method, bias=b)
        np.testing.assert_array_equal(ids, _grouped_bruteforce(s, b, w.k, w.n_group,
                                                               w.topk_group, w.method))


# --------------------------------------------------------------------------
# Alignment (cumsum, indptr, indices)
# --------------------------------------------------------------------------

def test_cumsum_worked_example():
    ex = _golden("mlc_moe_cumsum_example.json")
    ids = np.array(ex["expert_indices"], np.int32)
    cs = oracle.moe_cumsum(ids, ex["E"])
    assert cs.reshape(ex["E"], ex["T"]).tolist() == ex["cumsum_E_by_T"]


def test_align_worked_example():
    ex = _golden("mlc_moe_cumsum_example.json")
    ids = np.array(ex["expert_indices"], np.int32)
    T, k, E = ex["T"], ex["k"], ex["E"]
    cs = np.array(ex["cumsum_E_by_T"], np.int64).reshape(-1)
    a = oracle.align(ids, E)
    # get_indptr's documented numpy equivalent, applied to the printed cumsum
    indptr = [0] + [int(cs[i * T - 1]) for i in range(1, E + 1)]
    assert a["offsets"].tolist() == indptr == [0, 1, 3, 5, 6, 7, 8]
    assert a["counts"].tolist() == [1, 2, 2, 1, 1, 1]
    # get_indices' scatter rule, applied to the printed cumsum
    rev = [None] * (T * k)
    tok = [None] * (T * k)
    for b in range(T):
        for j in range(k):
            p = int(cs[ids[b, j] * T + b]) - 1
            rev[p] = b * k + j
            tok[p] = b
    assert a["sorted_slot_ids"].tolist() == rev == [0, 1, 2, 3, 6, 4, 5, 7]
    assert a["sorted_token_ids"].tolist() == tok == [0, 0, 1, 1, 3, 2, 2, 3]


def _check_align_against_stable_sort(ids, E, a):
    T, k = ids.shape
    flat = ids.reshape(-1)
    valid = np.nonzero((flat >= 0) & (flat < E))[0]
    order = valid[np.argsort(flat[valid], kind="stable")]  # library stable sort
    nv = len(valid)
    np.testing.assert_array_equal(a["counts"], np.bincount(flat[valid], minlength=E))
    assert a["offsets"][0] == 0 and a["offsets"][-1] == nv
    np.testing.assert_array_equal(np.diff(a["offsets"]), a["counts"])
    np.testing.assert_array_equal(a["sorted_slot_ids"][:nv], order)
    np.testing.assert_array_equal(a["sorted_token_ids"][:nv], order // k)
    assert np.all(a["sorted_slot_ids"][nv:] == -1) and np.all(a["sorted_token_ids"][nv:] == -1)
    s2s = np.full(T * k, -1, np.int64)
    s2s[order] = np.arange(nv)
    np.testing.assert_array_equal(a["slot_to_sorted"], s2s)
    for e in range(E):  # ascending tokens inside every segment
        seg = a["sorted_token_ids"][a["offsets"][e]:a["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)


@pytest.mark.parametrize("T,E,k,inv", [(1000, 64, 8, 0.0), (333, 8, 2, 0.0), (257, 13, 3, 0.1),
                                       (1, 4, 4, 0.0), (50, 1, 1, 0.0), (64, 200, 6, 0.2)])
def test_align_matches_stable_sort(T, E, k, inv):
    ids = mi.random_ids(T * 10 + E, T, E, k, invalid_frac=inv)
    a = oracle.align(ids, E)
    _check_align_against_stable_sort(ids, E, a)
    if inv == 0:
        assert a["offsets"][-1] == T * k
        for t in range(T):  # every token appears exactly k times
            assert np.count_nonzero(a["sorted_token_ids"] == t) == k


def test_align_skewed_with_zero_counts():
    ids = np.tile(np.array([[3, 0, 5]], np.int32), (20, 1))
    a = oracle.align(ids, 8)
    assert a["counts"].tolist() == [20, 0, 0, 20, 0, 20, 0, 0]
    _check_align_against_stable_sort(ids, 8, a)


def test_align_empty():
    a = oracle.align(np.zeros((0, 4), np.int32), 6)
    assert a["offsets"].tolist() == [0] * 7 and a["counts"].tolist() == [0] * 6


def test_align_routing_workload_invariants():
    w = mi.WORKLOADS["routing"]
    _, ids = oracle.route(mi.gating_logits(w), w.k, True)
    a = oracle.align(ids, w.E)
    assert a["offsets"][-1] == w.T * w.k
    _check_align_against_stable_sort(ids, w.E, a)


# --------------------------------------------------------------------------
# Multihot conversion and its inverse
# --------------------------------------------------------------------------

def test_multihot_worked_example():
    ex = _golden("megatron_indices_to_multihot_example.json")
    ids = np.array(ex["indices"], np.int32)
    probs = np.array(ex["probs_in_indices"], np.float32)
    mh, pim, pos = oracle.indices_to_multihot(ids, probs, ex["E"])
    assert mh.tolist() == ex["multihot"]
    np.testing.assert_array_equal(pim, np.array(ex["probs_in_multihot"], np.float32))
    printed = np.array(ex["multihot_indices_printed"])
    assert np.array_equal(mh == 1, printed == 1)
    assert pos.tolist() == [[0, 1, -1, -1], [-1, 0, 1, -1]]


def test_inverse_worked_example():
    ex = _golden("megatron_multihot_to_indices_example.json")
    pim = np.array(ex["probs_in_multihot"], np.float32)
    pos = np.array(ex["position_map"], np.int32)
    probs, ids = oracle.multihot_to_indices(pim, pos, ex["k"])
    np.testing.assert_array_equal(probs, np.array(ex["probs_indices"], np.float32))
    assert ids.tolist() == [[0, 1], [1, 2]]
    assert np.array_equal(np.array(ex["position_map_printed"]) != -1, pos != -1)


@pytest.mark.parametrize("T,E,k,inv", [(300, 64, 8, 0.0), (100, 6, 2, 0.25), (20, 300, 9, 0.1)])
def test_multihot_roundtrip_and_dense(T, E, k, inv):
    ids = mi.random_ids(T + E, T, E, k, invalid_frac=inv)
    probs = mi.random_probs(T + k, T, k)
    mh, pim, pos = oracle.indices_to_multihot(ids, probs, E)
    valid = (ids >= 0) & (ids < E)
    # dense brute force: column e of row t is set iff e is a valid id of the row
    for t in range(T):
        for e in range(E):
            js = [j for j in range(k) if ids[t, j] == e]
            assert mh[t, e] == (1 if js else 0)
            assert pos[t, e] == (js[0] if js else -1)
            assert pim[t, e] == (probs[t, js[0]] if js else 0.0)
    back, ids_back = oracle.multihot_to_indices(pim, pos, k)
    np.testing.assert_array_equal(back, np.where(valid, probs, 0).astype(np.float32))
    np.testing.assert_array_equal(ids_back, np.where(valid, ids, -1))


@pytest.mark.parametrize("T,E,k,inv", [(37, 8, 2, 0.0), (64, 64, 8, 0.1), (9, 5, 5, 0.0)])
def test_converter_backward_is_the_adjoint(T, E, k, inv):
    # [mgt] IndicesToMultihot.backward runs the inverse conversion on the
    # gradient.  For fixed ids the forward's probability map F: probs [T,k] ->
    # probs_in_multihot [T,E] is linear, so its backward B must be the adjoint:
    # <F(p), g> = <p, B(g)> for every p and every gradient g, including
    # gradients that are nonzero where no expert was selected.
    ids = mi.random_ids(T * 7 + E, T, E, k, invalid_frac=inv)
    g = np.random.Generator(np.random.PCG64(T + 3 * E))
    for _ in range(3):
        p = g.standard_normal((T, k)).astype(np.float32)
        grad = g.standard_normal((T, E)).astype(np.float32)
        _, fp, pos = oracle.indices_to_multihot(ids, p, E)
        bg, _ = oracle.multihot_to_indices(grad, pos, k)
        lhs = float(np.sum(fp.astype(np.float64) * grad.astype(np.float64)))
        rhs = float(np.sum(p.astype(np.float64) * bg.astype(np.float64)))
        assert abs(lhs - rhs) <= 1e-9 * (1 + abs(lhs))
    # Slots with an invalid id receive no gradient.
    assert np.all(bg[ids < 0] == 0) and np.all(bg[ids >= E] == 0)


# --------------------------------------------------------------------------
# Expert FFN + weighted combine
# --------------------------------------------------------------------------

def _dense_bruteforce(x, w13, w2, gate):
    """Every expert on every token, combined through a dense [T,E] gate (0 off top-k)."""
    E, I2, H = w13.shape
    I = I2 // 2
    gu = np.einsum("th,eih->tei", x, w13)  # [T,E,2I]
    act = gu[..., :I] / (1 + np.exp(-gu[..., :I])) * gu[..., I:]
    y = np.einsum("tei,ehi->teh", act, w2)
    return np.einsum("te,teh->th", gate, y)


def _tiny(seed, T, H, I, E, k, norm=True):
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((T, H)).astype(np.float32)
    w13 = (g.standard_normal((E, 2 * I, H)) / math.sqrt(H)).astype(np.float32)
    w2 = (g.standard_normal((E, H, I)) / math.sqrt(I)).astype(np.float32)
    logits = g.standard_normal((T, E)).astype(np.float32)
    w, ids = oracle.route(logits, k, norm)
    return x, w13, w2, w, ids


@pytest.mark.parametrize("T,H,I,E,k", [(4, 64, 128, 8, 2), (9, 16, 24, 5, 3), (3, 8, 8, 4, 4)])
def test_ffn_matches_dense_bruteforce(T, H, I, E, k):
    x, w13, w2, w, ids = _tiny(T + H + I, T, H, I, E, k)
    out = oracle.expert_ffn(x, w13, w2, w, ids, "f32")
    gate = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            gate[t, ids[t, j]] = w[t, j]
    ref = _dense_bruteforce(x.astype(np.float64), w13.astype(np.float64), w2.astype(np.float64), gate)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_ffn_single_expert_is_swiglu_mlp():
    x, w13, w2, w, ids = _tiny(11, 6, 32, 48, 1, 1)
    assert np.all(w == 1.0) and np.all(ids == 0)
    out = oracle.expert_ffn(x, w13, w2, w, ids, "f32")
    xt = torch.from_numpy(x.astype(np.float64))
    gu = torch.nn.functional.linear(xt, torch.from_numpy(w13[0].astype(np.float64)))
    a = torch.nn.functional.silu(gu[:, :48]) * gu[:, 48:]
    ref = torch.nn.functional.linear(a, torch.from_numpy(w2[0].astype(np.float64))).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_ffn_shared_weights_reduce_to_one_mlp():
    # All experts equal + renormalised weights (sum 1) -> out = FFN(x).
    x, w13, w2, w, ids = _tiny(12, 5, 16, 32, 6, 3)
    w13[:] = w13[0]
    w2[:] = w2[0]
    out = oracle.expert_ffn(x, w13, w2, w, ids, "f32")
    single = oracle.expert_ffn(x, w13[:1], w2[:1], np.ones((5, 1)), np.zeros((5, 1), np.int32), "f32")
    np.testing.assert_allclose(out, single, rtol=1e-11, atol=1e-12)


def test_ffn_unselected_experts_are_not_read():
    x, w13, w2, w, ids = _tiny(13, 4, 16, 16, 8, 2)
    used = set(ids.reshape(-1).tolist())
    ref = oracle.expert_ffn(x, w13, w2, w, ids, "f32")
    for e in range(8):
        if e not in used:
            w13[e] = np.nan
            w2[e] = np.nan
    out = oracle.expert_ffn(x, w13, w2, w, ids, "f32")
    np.testing.assert_array_equal(out, ref)
    # invalid ids contribute nothing
    ids2 = ids.copy()
    ids2[:, 1] = -1
    out2 = oracle.expert_ffn(x, w13, w2, w, ids2, "f32")
    ids3 = ids.copy()[:, :1]
    out3 = oracle.expert_ffn(x, w13, w2, w[:, :1], ids3, "f32")
    np.testing.assert_array_equal(out2, out3)


def test_ffn_duplicate_rows_and_token_subset():
    x, w13, w2, w, ids = _tiny(14, 6, 16, 16, 4, 2)
    x[3] = x[1]
    ids[3] = ids[1]
    w[3] = w[1]
    out = oracle.expert_ffn(x, w13, w2, w, ids, "f32")
    np.testing.assert_array_equal(out[3], out[1])
    sub = oracle.expert_ffn(x, w13, w2, w, ids, "f32", tokens=[5, 0, 3])
    np.testing.assert_array_equal(sub, out[[5, 0, 3]])


def test_ffn_bf16_inputs_decode_exactly():
    x, w13, w2, w, ids = _tiny(15, 3, 32, 64, 4, 2)
    xb, w13b, w2b = (mi.f32_to_bf16_bits(a) for a in (x, w13, w2))
    out = oracle.expert_ffn(xb, w13b, w2b, w, ids, "bf16")
    ref = oracle.expert_ffn(mi.bf16_bits_to_f32(xb), mi.bf16_bits_to_f32(w13b),
                            mi.bf16_bits_to_f32(w2b), w, ids, "f32")
    np.testing.assert_array_equal(out, ref)
    gate = np.zeros((3, 4))
    for t in range(3):
        for j in range(2):
            gate[t, ids[t, j]] = w[t, j]
    dense = _dense_bruteforce(mi.bf16_bits_to_f32(xb).astype(np.float64),
                              mi.bf16_bits_to_f32(w13b).astype(np.float64),
                              mi.bf16_bits_to_f32(w2b).astype(np.float64), gate)
    np.testing.assert_allclose(out, dense, rtol=1e-11, atol=1e-12)


def test_tiny_workload_layer():
    w = mi.WORKLOADS["tiny"]
    inp = mi.layer_inputs(w)
    res = oracle.layer(inp, w.k, w.norm, w.dtype)
    assert res["out"].shape == (w.T, w.H)
    for t in range(w.T):  # "ties rejected" rows
        assert len(np.unique(inp["logits"][t])) == w.E
    rms = math.sqrt(float(np.mean(res["out"] ** 2)))
    assert 0.05 < rms < 5


# --------------------------------------------------------------------------
# Input generator
# --------------------------------------------------------------------------

def test_inputs_deterministic_and_thread_independent():
    a = mi.normal_bf16(9, 2, 3 * mi.CHUNK + 5, 0.1, threads=1)
    b = mi.normal_bf16(9, 2, 3 * mi.CHUNK + 5, 0.1, threads=8)
    np.testing.assert_array_equal(a, b)
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3], np.float32)
    # RNE: 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> 1+2^-6
    assert mi.bf16_bits_to_f32(mi.f32_to_bf16_bits(x)).tolist()[:4] == [1.0, 1.0, 1.015625, -2.5]


def test_finegrained_bias_gives_zero_count_experts():
    w = mi.WORKLOADS["finegrained"]
    _, ids = oracle.route(mi.gating_logits(w), w.k, True)
    counts = np.bincount(ids.reshape(-1), minlength=w.E)
    assert np.count_nonzero(counts == 0) >= 2
    assert counts.max() > 4 * counts.mean()
