"""CPU oracle of the MoE layer forward and backward (numpy front end over moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this package.  The product library never does,
and this package never imports the product library.

Every function returns float64 results (or exact integers) computed by the
plain C loops in ``moe_oracle.c``; see that file for which passage of the
pages each step follows.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc into libmoe_oracle.so (next to it)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               "-Wall", "-Werror", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        lib.oracle_route.argtypes = [vp, i64, i32, i32, i32, vp, vp]
        lib.oracle_router_logits.argtypes = [i32, vp, vp, i64, i32, i32, vp]
        lib.oracle_route_grouped.argtypes = [vp, vp, i64, i32, i32, i32, i32, i32, i32, vp, vp]
        lib.oracle_moe_cumsum.argtypes = [vp, i64, i32, i32, vp]
        lib.oracle_align.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp]
        lib.oracle_indices_to_multihot.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp]
        lib.oracle_multihot_to_indices.argtypes = [vp, vp, i64, i32, i32, vp, vp]
        lib.oracle_expert_ffn.argtypes = [i32, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32,
                                          vp, i64, vp, i32]
        lib.oracle_route_backward.argtypes = [vp, vp, i64, i32, i32, i32, vp, vp]
        lib.oracle_route_grouped_backward.argtypes = [vp, vp, i64, i32, i32, i32, vp, vp]
        lib.oracle_router_backward.argtypes = [i32, vp, vp, vp, i64, i32, i32, vp, vp]
        lib.oracle_expert_ffn_backward.argtypes = [i32, vp, vp, vp, vp, vp, vp, i64, i32, i32,
                                                   i32, i32, vp, i64, vp, vp, vp, vp, i32]
        lib.oracle_expert_wgrad_entries.argtypes = [i32, vp, vp, vp, vp, vp, vp, i64, i32, i32,
                                                    i32, i32, i64, vp, vp, vp, i64, vp, vp, vp,
                                                    i32]
        for f in (lib.oracle_route, lib.oracle_router_logits, lib.oracle_route_grouped, lib.oracle_moe_cumsum, lib.oracle_align,
                  lib.oracle_indices_to_multihot, lib.oracle_multihot_to_indices,
                  lib.oracle_expert_ffn, lib.oracle_route_backward,
                  lib.oracle_route_grouped_backward, lib.oracle_router_backward,
                  lib.oracle_expert_ffn_backward, lib.oracle_expert_wgrad_entries):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def route(logits: np.ndarray, k: int, norm_topk_prob: bool = True):
    """Top-k experts per row and their softmax weights -> (w [T,k] f64, ids [T,k] i32)."""
    x = _c(logits, np.float32)
    T, E = x.shape
    w = np.empty((T, k), np.float64)
    ids = np.empty((T, k), np.int32)
    _check(_load().oracle_route(_p(x), T, E, k, int(bool(norm_topk_prob)), _p(w), _p(ids)), "route")
    return w, ids


def router_logits(hidden: np.ndarray, w_gate: np.ndarray, dtype: str) -> np.ndarray:
    """logits [T,E] f64 = hidden [T,H] . w_gate[E,H]^T ("f32": float32 arrays,
    "bf16": uint16 bit patterns)."""
    dt = {"f32": 0, "bf16": 1}[dtype]
    npdt = np.float32 if dt == 0 else np.uint16
    x = _c(hidden, npdt)
    w = _c(w_gate, npdt)
    T, H = x.shape
    E, H2 = w.shape
    assert H2 == H
    out = np.empty((T, E), np.float64)
    _check(_load().oracle_router_logits(dt, _p(x), _p(w), T, H, E, _p(out)), "router_logits")
    return out


GROUP_METHODS = {"group_limited_greedy": 0, "noaux_tc": 1}


def route_grouped(scores: np.ndarray, k: int, n_group: int, topk_group: int, method: str,
                  bias: np.ndarray | None = None, renormalize: bool = False):
    """Group-limited top-k (greedy or noaux_tc) -> (w [T,k] f64, ids [T,k] i32)."""
    x = _c(scores, np.float32)
    T, E = x.shape
    m = GROUP_METHODS[method]
    b = None if bias is None else _c(bias, np.float32)
    if b is not None:
        assert b.shape == (E,)
    w = np.empty((T, k), np.float64)
    ids = np.empty((T, k), np.int32)
    _check(_load().oracle_route_grouped(_p(x), _p(b) if b is not None else None, T, E, k,
                                        n_group, topk_group, m, int(bool(renormalize)), _p(w),
                                        _p(ids)), "route_grouped")
    return w, ids


def moe_cumsum(ids: np.ndarray, E: int) -> np.ndarray:
    """The dense transposed inclusive cumsum of the expert mask, [E*T] int32."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    cs = np.empty(E * T, np.int32)
    _check(_load().oracle_moe_cumsum(_p(ids), T, k, E, _p(cs)), "moe_cumsum")
    return cs


def align(ids: np.ndarray, E: int) -> dict:
    """Expert counts, exclusive offsets, sorted token / slot ids and the inverse map."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    n = T * k
    out = {
        "counts": np.empty(E, np.int32),
        "offsets": np.empty(E + 1, np.int32),
        "sorted_token_ids": np.empty(n, np.int32),
        "sorted_slot_ids": np.empty(n, np.int32),
        "slot_to_sorted": np.empty(n, np.int32),
    }
    _check(_load().oracle_align(_p(ids), T, k, E, _p(out["counts"]), _p(out["offsets"]),
                                _p(out["sorted_token_ids"]), _p(out["sorted_slot_ids"]),
                                _p(out["slot_to_sorted"])), "align")
    return out


def indices_to_multihot(ids: np.ndarray, probs: np.ndarray, E: int):
    """-> (multihot [T,E] u8, probs_in_multihot [T,E] f32, position_map [T,E] i32)."""
    ids = _c(ids, np.int32)
    probs = _c(probs, np.float32)
    T, k = ids.shape
    mh = np.empty((T, E), np.uint8)
    pim = np.empty((T, E), np.float32)
    pos = np.empty((T, E), np.int32)
    _check(_load().oracle_indices_to_multihot(_p(ids), _p(probs), T, k, E, _p(mh), _p(pim),
                                              _p(pos)), "indices_to_multihot")
    return mh, pim, pos


def multihot_to_indices(probs_in_multihot: np.ndarray, position_map: np.ndarray, k: int):
    """-> (probs_indices [T,k] f32, ids [T,k] i32)."""
    pim = _c(probs_in_multihot, np.float32)
    pos = _c(position_map, np.int32)
    T, E = pim.shape
    probs = np.empty((T, k), np.float32)
    ids = np.empty((T, k), np.int32)
    _check(_load().oracle_multihot_to_indices(_p(pim), _p(pos), T, E, k, _p(probs), _p(ids)),
           "multihot_to_indices")
    return probs, ids


def expert_ffn(hidden: np.ndarray, w13: np.ndarray, w2: np.ndarray, topk_w: np.ndarray,
               topk_ids: np.ndarray, dtype: str, tokens=None, threads: int | None = None):
    """Expert FFN + weighted combine in float64 -> out [len(tokens) or T, H].

    dtype "f32": hidden / weights are float32 arrays; "bf16": uint16 bit patterns.
    """
    dt = {"f32": 0, "bf16": 1}[dtype]
    npdt = np.float32 if dt == 0 else np.uint16
    hidden = _c(hidden, npdt)
    w13 = _c(w13, npdt)
    w2 = _c(w2, npdt)
    T, H = hidden.shape
    E, I2, H2 = w13.shape
    I = I2 // 2
    assert H2 == H and w2.shape == (E, H, I)
    ids = _c(topk_ids, np.int32)
    w = _c(topk_w, np.float64)
    k = ids.shape[1]
    if tokens is None:
        tok = None
        ntok = T
    else:
        tok = _c(tokens, np.int64)
        ntok = len(tok)
    out = np.empty((ntok, H), np.float64)
    nthr = threads if threads else (os.cpu_count() or 1)
    _check(_load().oracle_expert_ffn(dt, _p(hidden), _p(w13), _p(w2), _p(w), _p(ids), T, H, I,
                                     E, k, _p(tok) if tok is not None else None, ntok, _p(out),
                                     nthr), "expert_ffn")
    return out


def layer(inp: dict, k: int, norm_topk_prob: bool, dtype: str, tokens=None,
          threads: int | None = None) -> dict:
    """Route + align + FFN/combine on one workload's inputs (float64 results)."""
    w, ids = route(inp["logits"], k, norm_topk_prob)
    out = {"topk_w": w, "topk_ids": ids}
    if "hidden" in inp:
        out["out"] = expert_ffn(inp["hidden"], inp["w13"], inp["w2"], w, ids, dtype,
                                tokens=tokens, threads=threads)
    return out


def route_backward(logits: np.ndarray, topk_ids: np.ndarray, grad_topk_w: np.ndarray,
                   norm_topk_prob: bool = True) -> np.ndarray:
    """Gradient of the gating softmax weights w.r.t. the logits -> [T, E] float64."""
    x = _c(logits, np.float32)
    ids = _c(topk_ids, np.int32)
    g = _c(grad_topk_w, np.float64)
    T, E = x.shape
    k = ids.shape[1]
    out = np.empty((T, E), np.float64)
    _check(_load().oracle_route_backward(_p(x), _p(ids), T, E, k, int(bool(norm_topk_prob)),
                                         _p(g), _p(out)), "route_backward")
    return out


def route_grouped_backward(scores: np.ndarray, topk_ids: np.ndarray, grad_topk_w: np.ndarray,
                           renormalize: bool = False) -> np.ndarray:
    """Gradient of the group-limited selection's weights w.r.t. the scores -> [T, E] f64."""
    x = _c(scores, np.float32)
    ids = _c(topk_ids, np.int32)
    g = _c(grad_topk_w, np.float64)
    T, E = x.shape
    k = ids.shape[1]
    out = np.empty((T, E), np.float64)
    _check(_load().oracle_route_grouped_backward(_p(x), _p(ids), T, E, k, int(bool(renormalize)),
                                                 _p(g), _p(out)), "route_grouped_backward")
    return out


def router_backward(hidden: np.ndarray, w_gate: np.ndarray, grad_logits: np.ndarray,
                    dtype: str):
    """Backward of router_logits -> (grad_hidden [T, H], grad_w_gate [E, H]) float64."""
    dt = {"f32": 0, "bf16": 1}[dtype]
    npdt = np.float32 if dt == 0 else np.uint16
    x = _c(hidden, npdt)
    w = _c(w_gate, npdt)
    g = _c(grad_logits, np.float64)
    T, H = x.shape
    E = w.shape[0]
    gh = np.empty((T, H), np.float64)
    gw = np.empty((E, H), np.float64)
    _check(_load().oracle_router_backward(dt, _p(x), _p(w), _p(g), T, H, E, _p(gh), _p(gw)),
           "router_backward")
    return gh, gw


def _ffn_operands(hidden, w13, w2, topk_w, topk_ids, grad_out, dtype):
    dt = {"f32": 0, "bf16": 1}[dtype]
    npdt = np.float32 if dt == 0 else np.uint16
    hidden, w13, w2, grad_out = (_c(a, npdt) for a in (hidden, w13, w2, grad_out))
    T, H = hidden.shape
    E, I2, H2 = w13.shape
    I = I2 // 2
    assert H2 == H and w2.shape == (E, H, I) and grad_out.shape == (T, H)
    ids = _c(topk_ids, np.int32)
    w = _c(topk_w, np.float64)
    return dt, hidden, w13, w2, w, ids, grad_out, T, H, I, E, ids.shape[1]


def expert_ffn_backward(hidden, w13, w2, topk_w, topk_ids, grad_out, dtype: str,
                        tokens=None, weights: bool = False, threads: int | None = None) -> dict:
    """Backward of expert_ffn in float64.

    Returns grad_hidden [n, H] and grad_topk_w [n, k] for the listed tokens (all T if
    None); with weights=True (all tokens only) also grad_w13 [E, 2I, H] and
    grad_w2 [E, H, I].
    """
    dt, hidden, w13, w2, w, ids, dy, T, H, I, E, k = _ffn_operands(
        hidden, w13, w2, topk_w, topk_ids, grad_out, dtype)
    assert not (weights and tokens is not None)
    tok = None if tokens is None else _c(tokens, np.int64)
    n = T if tok is None else len(tok)
    out = {"grad_hidden": np.empty((n, H), np.float64),
           "grad_topk_w": np.empty((n, k), np.float64)}
    if weights:
        out["grad_w13"] = np.empty((E, 2 * I, H), np.float64)
        out["grad_w2"] = np.empty((E, H, I), np.float64)
    nthr = threads if threads else (os.cpu_count() or 1)
    _check(_load().oracle_expert_ffn_backward(
        dt, _p(hidden), _p(w13), _p(w2), _p(w), _p(ids), _p(dy), T, H, I, E, k,
        _p(tok) if tok is not None else None, n, _p(out["grad_hidden"]),
        _p(out["grad_topk_w"]), _p(out["grad_w13"]) if weights else None,
        _p(out["grad_w2"]) if weights else None, nthr), "expert_ffn_backward")
    return out


def expert_wgrad_entries(hidden, w13, w2, topk_w, topk_ids, grad_out, dtype: str,
                         rows13=(), cols2=(), threads: int | None = None):
    """Rows of grad_w13 and columns of grad_w2 from their definitions.

    rows13: (e, c) pairs -> [len, H] rows c of grad_w13[e]; cols2: (e, i) pairs ->
    [len, H] columns i of grad_w2[e].
    """
    dt, hidden, w13, w2, w, ids, dy, T, H, I, E, k = _ffn_operands(
        hidden, w13, w2, topk_w, topk_ids, grad_out, dtype)
    r13 = _c(np.array(rows13, np.int32).reshape(-1, 2), np.int32)
    c2 = _c(np.array(cols2, np.int32).reshape(-1, 2), np.int32)
    e13, cc13 = _c(r13[:, 0], np.int32), _c(r13[:, 1], np.int32)
    e2, ii2 = _c(c2[:, 0], np.int32), _c(c2[:, 1], np.int32)
    row13 = np.empty((len(r13), H), np.float64)
    col2 = np.empty((len(c2), H), np.float64)
    nthr = threads if threads else (os.cpu_count() or 1)
    _check(_load().oracle_expert_wgrad_entries(
        dt, _p(hidden), _p(w13), _p(w2), _p(w), _p(ids), _p(dy), T, H, I, E, k,
        len(r13), _p(e13), _p(cc13), _p(row13), len(c2), _p(e2), _p(ii2), _p(col2), nthr),
        "expert_wgrad_entries")
    return row13, col2
