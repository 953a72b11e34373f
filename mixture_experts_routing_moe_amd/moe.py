"""torch-tensor front end of libmoe (same names as the C ABI in include/moe.h).

Tensors must live on the current HIP device and be contiguous; outputs are
allocated here with torch when not given.  Work is enqueued on torch's current
stream and nothing synchronises.  bfloat16 tensors are passed as torch.bfloat16
(their bits are the library's bf16 values).
"""

from __future__ import annotations

import torch

from . import _lib
from ._lib import MOE_BF16, MOE_F32, check, lib


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libmoe works on device tensors only")
        if not t.is_contiguous():
            raise ValueError("libmoe needs contiguous tensors")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def moe_route(logits: torch.Tensor, k: int, norm_topk_prob: bool = True, topk_w=None,
              topk_ids=None):
    """Top-k experts per row + softmax weights -> (topk_w [T,k] f32, topk_ids [T,k] i32)."""
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be [T, E] float32")
    T, E = logits.shape
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    _dev(logits, topk_w, topk_ids)
    check(lib().moe_route(_ptr(logits), T, E, k, int(bool(norm_topk_prob)), _ptr(topk_w),
                          _ptr(topk_ids), _stream()), "moe_route")
    return topk_w, topk_ids


def moe_router_route(hidden: torch.Tensor, w_gate: torch.Tensor, k: int,
                     norm_topk_prob: bool = True, out=None):
    """Router GEMM + gating top-k: logits = hidden . w_gate^T (bf16 in, fp32
    out), then moe_route on them -> (logits [T,E] f32, topk_w [T,k] f32,
    topk_ids [T,k] i32)."""
    if hidden.dim() != 2 or w_gate.dim() != 2 or hidden.shape[1] != w_gate.shape[1]:
        raise ValueError("hidden [T, H] and w_gate [E, H]")
    if hidden.dtype != w_gate.dtype:
        raise ValueError("hidden and w_gate must have the same dtype")
    T, H = hidden.shape
    E = w_gate.shape[0]
    dev = hidden.device
    if out is None:
        out = (torch.empty((T, E), dtype=torch.float32, device=dev),
               torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((T, k), dtype=torch.int32, device=dev))
    logits, tw, ti = out
    _dev(hidden, w_gate, logits, tw, ti)
    check(lib().moe_router_route(_dtype_code(hidden), _ptr(hidden), _ptr(w_gate), T, H, E, k,
                                 int(bool(norm_topk_prob)), _ptr(logits), _ptr(tw), _ptr(ti),
                                 _stream()), "moe_router_route")
    return logits, tw, ti


GROUP_METHODS = {"group_limited_greedy": _lib.MOE_GROUP_LIMITED_GREEDY,
                 "noaux_tc": _lib.MOE_NOAUX_TC}


def moe_route_grouped(scores: torch.Tensor, k: int, n_group: int, topk_group: int,
                      method: str = "noaux_tc", e_score_correction_bias=None,
                      renormalize: bool = False, topk_w=None, topk_ids=None, multihot=None):
    """Group-limited top-k (group_limited_greedy / noaux_tc) over [T, E] float32
    scores -> (topk_w [T,k] f32, topk_ids [T,k] i32).  multihot: True (allocate)
    or a (multihot, probs_in_multihot, position_map) tuple of [T, E] outputs,
    which the call also fills and appends to the result."""
    if scores.dtype != torch.float32 or scores.dim() != 2:
        raise ValueError("scores must be [T, E] float32")
    if method not in GROUP_METHODS:
        raise ValueError(f"method must be one of {sorted(GROUP_METHODS)}")
    T, E = scores.shape
    b = e_score_correction_bias
    if b is not None and (b.dtype != torch.float32 or b.shape != (E,)):
        raise ValueError("e_score_correction_bias must be [E] float32")
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=scores.device)
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    if multihot is True:
        multihot = (torch.empty((T, E), dtype=torch.uint8, device=scores.device),
                    torch.empty((T, E), dtype=torch.float32, device=scores.device),
                    torch.empty((T, E), dtype=torch.int32, device=scores.device))
    mh = multihot if multihot else (None, None, None)
    _dev(scores, b, topk_w, topk_ids, *mh)
    check(lib().moe_route_grouped(_ptr(scores), _ptr(b), T, E, k, n_group, topk_group,
                                  GROUP_METHODS[method], int(bool(renormalize)), _ptr(topk_w),
                                  _ptr(topk_ids), _ptr(mh[0]), _ptr(mh[1]), _ptr(mh[2]),
                                  _stream()), "moe_route_grouped")
    if multihot:
        return (topk_w, topk_ids, *multihot)
    return topk_w, topk_ids


def moe_route_multihot(logits: torch.Tensor, k: int, norm_topk_prob: bool = True, out=None):
    """moe_route + moe_indices_to_multihot of its output, one pass where the
    library fuses them -> (topk_w, topk_ids, multihot, probs_in_multihot,
    position_map)."""
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be [T, E] float32")
    T, E = logits.shape
    dev = logits.device
    if out is None:
        out = (torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((T, k), dtype=torch.int32, device=dev),
               torch.empty((T, E), dtype=torch.uint8, device=dev),
               torch.empty((T, E), dtype=torch.float32, device=dev),
               torch.empty((T, E), dtype=torch.int32, device=dev))
    tw, ti, mh, pim, pos = out
    _dev(logits, tw, ti, mh, pim, pos)
    check(lib().moe_route_multihot(_ptr(logits), T, E, k, int(bool(norm_topk_prob)), _ptr(tw),
                                   _ptr(ti), _ptr(mh), _ptr(pim), _ptr(pos), _stream()),
          "moe_route_multihot")
    return tw, ti, mh, pim, pos


def moe_route_multihot_fused(E: int, k: int) -> bool:
    return bool(lib().moe_route_multihot_fused(E, k))


def moe_align_workspace_size(T: int, k: int, E: int) -> int:
    return int(lib().moe_align_workspace_size(T, k, E))


def moe_align(topk_ids: torch.Tensor, E: int, out: dict | None = None,
              workspace: torch.Tensor | None = None) -> dict:
    """Expert counts, offsets, sorted token / slot ids and the inverse map (all int32)."""
    if topk_ids.dtype != torch.int32 or topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T, k] int32")
    T, k = topk_ids.shape
    dev = topk_ids.device
    n = T * k
    if out is None:
        out = {
            "counts": torch.empty(E, dtype=torch.int32, device=dev),
            "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "sorted_token_ids": torch.empty(n, dtype=torch.int32, device=dev),
            "sorted_slot_ids": torch.empty(n, dtype=torch.int32, device=dev),
            "slot_to_sorted": torch.empty(n, dtype=torch.int32, device=dev),
        }
    if workspace is None:
        workspace = torch.empty(max(1, moe_align_workspace_size(T, k, E)), dtype=torch.uint8,
                                device=dev)
    _dev(topk_ids, workspace, *out.values())
    check(lib().moe_align(_ptr(topk_ids), T, k, E, _ptr(out["counts"]), _ptr(out["offsets"]),
                          _ptr(out["sorted_token_ids"]), _ptr(out["sorted_slot_ids"]),
                          _ptr(out["slot_to_sorted"]), _ptr(workspace), workspace.numel(),
                          _stream()), "moe_align")
    return out


def moe_align_inverse(topk_ids: torch.Tensor, E: int, probs_in_multihot: torch.Tensor,
                      position_map: torch.Tensor, out: dict | None = None,
                      workspace: torch.Tensor | None = None) -> dict:
    """moe_align, then moe_multihot_to_indices on the given maps, in one call ->
    the dict of moe_align plus probs_indices [T, k] f32 and ids_from_multihot
    [T, k] i32."""
    if topk_ids.dtype != torch.int32 or topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T, k] int32")
    T, k = topk_ids.shape
    if (probs_in_multihot.dtype != torch.float32 or position_map.dtype != torch.int32
            or tuple(probs_in_multihot.shape) != (T, E)
            or tuple(position_map.shape) != (T, E)):
        raise ValueError("probs_in_multihot [T, E] float32 and position_map [T, E] int32")
    dev = topk_ids.device
    n = T * k
    if out is None:
        out = {
            "counts": torch.empty(E, dtype=torch.int32, device=dev),
            "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "sorted_token_ids": torch.empty(n, dtype=torch.int32, device=dev),
            "sorted_slot_ids": torch.empty(n, dtype=torch.int32, device=dev),
            "slot_to_sorted": torch.empty(n, dtype=torch.int32, device=dev),
            "probs_indices": torch.empty((T, k), dtype=torch.float32, device=dev),
            "ids_from_multihot": torch.empty((T, k), dtype=torch.int32, device=dev),
        }
    if workspace is None:
        workspace = torch.empty(max(1, moe_align_workspace_size(T, k, E)), dtype=torch.uint8,
                                device=dev)
    _dev(topk_ids, probs_in_multihot, position_map, workspace, *out.values())
    check(lib().moe_align_inverse(_ptr(topk_ids), T, k, E, _ptr(out["counts"]),
                                  _ptr(out["offsets"]), _ptr(out["sorted_token_ids"]),
                                  _ptr(out["sorted_slot_ids"]), _ptr(out["slot_to_sorted"]),
                                  _ptr(probs_in_multihot), _ptr(position_map),
                                  _ptr(out["probs_indices"]), _ptr(out["ids_from_multihot"]),
                                  _ptr(workspace), workspace.numel(), _stream()),
          "moe_align_inverse")
    return out


def moe_route_align_fused(T: int, E: int, k: int) -> bool:
    return bool(lib().moe_route_align_fused(T, E, k))


def _route_align_outputs(logits, k, with_multihot, out):
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be [T, E] float32")
    T, E = logits.shape
    dev = logits.device
    n = T * k
    if out is None:
        out = {
            "topk_w": torch.empty((T, k), dtype=torch.float32, device=dev),
            "topk_ids": torch.empty((T, k), dtype=torch.int32, device=dev),
            "counts": torch.empty(E, dtype=torch.int32, device=dev),
            "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "sorted_token_ids": torch.empty(n, dtype=torch.int32, device=dev),
            "sorted_slot_ids": torch.empty(n, dtype=torch.int32, device=dev),
            "slot_to_sorted": torch.empty(n, dtype=torch.int32, device=dev),
        }
        if with_multihot:
            out["multihot"] = torch.empty((T, E), dtype=torch.uint8, device=dev)
            out["probs_in_multihot"] = torch.empty((T, E), dtype=torch.float32, device=dev)
            out["position_map"] = torch.empty((T, E), dtype=torch.int32, device=dev)
    return T, E, out


def _route_align_ptrs(out):
    return (_ptr(out["topk_w"]), _ptr(out["topk_ids"]), _ptr(out.get("multihot")),
            _ptr(out.get("probs_in_multihot")), _ptr(out.get("position_map")),
            _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["sorted_token_ids"]),
            _ptr(out["sorted_slot_ids"]), _ptr(out["slot_to_sorted"]))


def moe_route_align(logits: torch.Tensor, k: int, norm_topk_prob: bool = True,
                    with_multihot: bool = False, out: dict | None = None,
                    workspace: torch.Tensor | None = None) -> dict:
    """moe_route (moe_route_multihot with with_multihot) + moe_align in one call ->
    dict with topk_w, topk_ids, the alignment outputs of moe_align and, with
    with_multihot, multihot / probs_in_multihot / position_map."""
    T, E, out = _route_align_outputs(logits, k, with_multihot, out)
    if workspace is None:
        workspace = torch.empty(max(1, moe_align_workspace_size(T, k, E)), dtype=torch.uint8,
                                device=logits.device)
    _dev(logits, workspace, *out.values())
    check(lib().moe_route_align(_ptr(logits), T, E, k, int(bool(norm_topk_prob)),
                                *_route_align_ptrs(out), _ptr(workspace), workspace.numel(),
                                _stream()), "moe_route_align")
    return out


def moe_tile_schedule_max(T: int, k: int, E: int) -> int:
    return int(lib().moe_tile_schedule_max(T, k, E))


def moe_tile_schedule(expert_offsets: torch.Tensor, max_tiles: int, out=None):
    """The grouped GEMMs' m-tile list from moe_align's offsets -> (tile_expert,
    tile_row_start, tile_row_end [max_tiles] int32, num_tiles [1] int32)."""
    if expert_offsets.dtype != torch.int32 or expert_offsets.dim() != 1:
        raise ValueError("expert_offsets must be [E+1] int32")
    E = expert_offsets.numel() - 1
    dev = expert_offsets.device
    if out is None:
        out = tuple(torch.empty(max(1, max_tiles), dtype=torch.int32, device=dev)
                    for _ in range(3)) + (torch.empty(1, dtype=torch.int32, device=dev),)
    _dev(expert_offsets, *out)
    check(lib().moe_tile_schedule(_ptr(expert_offsets), E, max_tiles, *(_ptr(t) for t in out),
                                  _stream()), "moe_tile_schedule")
    return out


def moe_route_align_inverse(logits: torch.Tensor, k: int, norm_topk_prob: bool = True,
                            out: dict | None = None,
                            workspace: torch.Tensor | None = None) -> dict:
    """moe_route_align with the multihot outputs, then moe_multihot_to_indices on
    its maps, in one call -> the dict of moe_route_align(with_multihot=True)
    plus probs_indices [T, k] f32 and ids_from_multihot [T, k] i32."""
    T, E, out = _route_align_outputs(logits, k, True, out)
    if "probs_indices" not in out:
        out["probs_indices"] = torch.empty((T, k), dtype=torch.float32, device=logits.device)
        out["ids_from_multihot"] = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if workspace is None:
        workspace = torch.empty(max(1, moe_align_workspace_size(T, k, E)), dtype=torch.uint8,
                                device=logits.device)
    _dev(logits, workspace, *out.values())
    check(lib().moe_route_align_inverse(_ptr(logits), T, E, k, int(bool(norm_topk_prob)),
                                        *_route_align_ptrs(out), _ptr(out["probs_indices"]),
                                        _ptr(out["ids_from_multihot"]), _ptr(workspace),
                                        workspace.numel(), _stream()),
          "moe_route_align_inverse")
    return out


def moe_route_align_gate_up_fused(T: int, E: int, k: int, dtype: int, decode: bool, H: int,
                                  I: int) -> bool:
    return bool(lib().moe_route_align_gate_up_fused(T, E, k, dtype, int(decode), H, I))


def moe_route_align_gate_up(logits: torch.Tensor, k: int, hidden: torch.Tensor,
                            w13: torch.Tensor, norm_topk_prob: bool = True, decode: bool = True,
                            inverse: bool = True, out: dict | None = None, act=None,
                            workspace: torch.Tensor | None = None):
    """moe_route_align_inverse (moe_route_align without `inverse`) + moe_ffn_gate_up
    in one call -> (the routing dict, act [T*k, I]); one launch for the smallest
    bf16 decode batches (moe_route_align_gate_up_fused)."""
    T, E, out = _route_align_outputs(logits, k, inverse, out)
    if inverse and "probs_indices" not in out:
        out["probs_indices"] = torch.empty((T, k), dtype=torch.float32, device=logits.device)
        out["ids_from_multihot"] = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    E2, I2, H = w13.shape
    if E2 != E or hidden.shape != (T, H):
        raise ValueError("hidden must be [T, H] and w13 [E, 2I, H]")
    I = I2 // 2
    if act is None:
        act = torch.empty((T * k, I), dtype=hidden.dtype, device=hidden.device)
    if workspace is None:
        workspace = torch.empty(max(1, moe_align_workspace_size(T, k, E)), dtype=torch.uint8,
                                device=logits.device)
    _dev(logits, workspace, hidden, w13, act, *out.values())
    check(lib().moe_route_align_gate_up(
        _ptr(logits), T, E, k, int(bool(norm_topk_prob)), *_route_align_ptrs(out),
        _ptr(out.get("probs_indices")), _ptr(out.get("ids_from_multihot")),
        _dtype_code(hidden), int(decode), _ptr(hidden), _ptr(w13), H, I, _ptr(act),
        _ptr(workspace), workspace.numel(), _stream()), "moe_route_align_gate_up")
    return out, act


def moe_route_align_noalloc(logits: torch.Tensor, k: int, norm_topk_prob: bool = True,
                            with_multihot: bool = False, out: dict | None = None) -> dict:
    """moe_route_align without a workspace: the library's own device scratch
    (shared by every call on the GPU) stands in for it.  With `out` given this
    allocates nothing."""
    T, E, out = _route_align_outputs(logits, k, with_multihot, out)
    _dev(logits, *out.values())
    check(lib().moe_route_align_noalloc(_ptr(logits), T, E, k, int(bool(norm_topk_prob)),
                                        *_route_align_ptrs(out), _stream()),
          "moe_route_align_noalloc")
    return out


def moe_indices_to_multihot_backward(grad_probs_in_multihot: torch.Tensor,
                                     position_map: torch.Tensor, k: int, out=None):
    """Gradient of moe_indices_to_multihot's probs from the gradient of its
    probs_in_multihot ([mgt] IndicesToMultihot.backward): moe_multihot_to_indices
    without the ids -> grad_probs [T, k] float32."""
    if out is not None:
        out = (out, None)
    return moe_multihot_to_indices(grad_probs_in_multihot, position_map, k, with_ids=False,
                                   out=out)[0]


def moe_indices_to_multihot(ids: torch.Tensor, probs: torch.Tensor, E: int, out=None):
    """-> (multihot [T,E] u8, probs_in_multihot [T,E] f32, position_map [T,E] i32)."""
    if ids.dtype != torch.int32 or probs.dtype != torch.float32 or ids.shape != probs.shape:
        raise ValueError("ids [T,k] int32 and probs [T,k] float32 of the same shape")
    T, k = ids.shape
    dev = ids.device
    if out is None:
        out = (torch.empty((T, E), dtype=torch.uint8, device=dev),
               torch.empty((T, E), dtype=torch.float32, device=dev),
               torch.empty((T, E), dtype=torch.int32, device=dev))
    mh, pim, pos = out
    _dev(ids, probs, mh, pim, pos)
    check(lib().moe_indices_to_multihot(_ptr(ids), _ptr(probs), T, k, E, _ptr(mh), _ptr(pim),
                                        _ptr(pos), _stream()), "moe_indices_to_multihot")
    return mh, pim, pos


def moe_multihot_to_indices(probs_in_multihot: torch.Tensor, position_map: torch.Tensor, k: int,
                            with_ids: bool = True, out=None):
    """-> (probs_indices [T,k] f32, ids [T,k] i32 or None)."""
    if probs_in_multihot.dtype != torch.float32 or position_map.dtype != torch.int32 or \
            probs_in_multihot.shape != position_map.shape:
        raise ValueError("probs_in_multihot [T,E] float32 and position_map [T,E] int32")
    T, E = probs_in_multihot.shape
    dev = probs_in_multihot.device
    if out is None:
        out = (torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((T, k), dtype=torch.int32, device=dev) if with_ids else None)
    probs, ids = out
    _dev(probs_in_multihot, position_map, probs, ids)
    check(lib().moe_multihot_to_indices(_ptr(probs_in_multihot), _ptr(position_map), T, E, k,
                                        _ptr(probs), _ptr(ids), _stream()),
          "moe_multihot_to_indices")
    return probs, ids


def moe_expert_ffn_workspace_size(dtype: int, T: int, H: int, I: int, E: int, k: int) -> int:
    return int(lib().moe_expert_ffn_workspace_size(dtype, T, H, I, E, k))


def _ffn_shapes(hidden, w13, w2):
    if hidden.dim() != 2 or w13.dim() != 3 or w2.dim() != 3:
        raise ValueError("hidden [T,H], w13 [E,2I,H], w2 [E,H,I]")
    T, H = hidden.shape
    E, I2, H2 = w13.shape
    I = I2 // 2
    if H2 != H or I2 != 2 * I or tuple(w2.shape) != (E, H, I):
        raise ValueError("inconsistent FFN shapes")
    if not (hidden.dtype == w13.dtype == w2.dtype):
        raise ValueError("hidden, w13, w2 must share a dtype")
    return T, H, I, E


def moe_expert_ffn(hidden, w13, w2, topk_w, aligned: dict, decode: bool = False, out=None,
                   workspace=None):
    """Grouped FC1 + SiLU-and-mul, FC2, weighted combine -> out [T, H] in hidden's dtype."""
    T, H, I, E = _ffn_shapes(hidden, w13, w2)
    k = topk_w.shape[1]
    dt = _dtype_code(hidden)
    if out is None:
        out = torch.empty((T, H), dtype=hidden.dtype, device=hidden.device)
    if workspace is None:
        workspace = torch.empty(max(1, moe_expert_ffn_workspace_size(dt, T, H, I, E, k)),
                                dtype=torch.uint8, device=hidden.device)
    _dev(hidden, w13, w2, topk_w, out, workspace, aligned["offsets"],
         aligned["sorted_token_ids"], aligned["slot_to_sorted"])
    fn = lib().moe_expert_ffn_decode if decode else lib().moe_expert_ffn
    check(fn(dt, _ptr(hidden), _ptr(w13), _ptr(w2), _ptr(topk_w), _ptr(aligned["offsets"]),
             _ptr(aligned["sorted_token_ids"]), _ptr(aligned["slot_to_sorted"]), T, H, I, E, k,
             _ptr(out), _ptr(workspace), workspace.numel(), _stream()),
          "moe_expert_ffn_decode" if decode else "moe_expert_ffn")
    return out


def moe_ffn_gate_up(hidden, w13, aligned: dict, k: int, decode: bool = False, act=None):
    """act [T*k, I] in the aligned order."""
    T, H = hidden.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    if act is None:
        act = torch.empty((T * k, I), dtype=hidden.dtype, device=hidden.device)
    _dev(hidden, w13, act, aligned["offsets"], aligned["sorted_token_ids"])
    check(lib().moe_ffn_gate_up(_dtype_code(hidden), int(decode), _ptr(hidden), _ptr(w13),
                                _ptr(aligned["offsets"]), _ptr(aligned["sorted_token_ids"]), T,
                                H, I, E, k, _ptr(act), _stream()), "moe_ffn_gate_up")
    return act


def moe_ffn_down_splits(dtype: int, T: int, H: int, I: int, E: int, k: int,
                        decode: bool = False) -> int:
    """K slices the library uses for the FC2 product of this shape."""
    return int(lib().moe_ffn_down_splits(dtype, int(decode), T, H, I, E, k))


def moe_ffn_down(act, w2, aligned: dict, T: int, k: int, decode: bool = False, y=None,
                 splits: int | None = None):
    """y float32 in the aligned order: [T*k, H] for one K slice, else [splits, T*k, H]
    partial planes (summed by moe_combine).  splits defaults to the library's choice
    (moe_ffn_down_splits), or to what an explicit y's shape holds."""
    E, H, I = w2.shape
    dt = _dtype_code(act)
    if splits is None:
        if y is not None:
            splits = y.shape[0] if y.dim() == 3 else 1
        else:
            splits = moe_ffn_down_splits(dt, T, H, I, E, k, decode)
    if y is None:
        shape = (T * k, H) if splits == 1 else (splits, T * k, H)
        y = torch.empty(shape, dtype=torch.float32, device=act.device)
    if y.numel() != splits * T * k * H:
        raise ValueError(f"y holds {y.numel()} floats, need {splits} x {T * k} x {H}")
    _dev(act, w2, y, aligned["offsets"])
    check(lib().moe_ffn_down(dt, int(decode), _ptr(act), _ptr(w2), _ptr(aligned["offsets"]), T,
                             H, I, E, k, splits, _ptr(y), _stream()), "moe_ffn_down")
    return y


def moe_combine(y, topk_w, slot_to_sorted, out_dtype=torch.bfloat16, out=None):
    """out [T, H] = sum_j topk_w[t, j] * (sum_s y[s, slot_to_sorted[t*k + j]]) (y float32,
    [T*k, H] or [splits, T*k, H])."""
    if y.dtype != torch.float32:
        raise ValueError("y must be float32")
    T, k = topk_w.shape
    splits = y.shape[0] if y.dim() == 3 else 1
    H = y.shape[-1]
    if y.shape[-2] != T * k:
        raise ValueError("y must have T*k rows per plane")
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=y.device)
    _dev(y, topk_w, slot_to_sorted, out)
    check(lib().moe_combine(_dtype_code(out), _ptr(y), splits, _ptr(topk_w), _ptr(slot_to_sorted),
                            T, H, k, _ptr(out), _stream()), "moe_combine")
    return out


def moe_ffn_down_combine_fused(dtype: int, T: int, H: int, I: int, E: int, k: int,
                               decode: bool = False) -> bool:
    return bool(lib().moe_ffn_down_combine_fused(dtype, int(decode), T, H, I, E, k))


def moe_ffn_down_combine(act, w2, topk_w, aligned: dict, T: int, k: int, decode: bool = False,
                         y=None, out=None, out_dtype=torch.bfloat16):
    """moe_ffn_down + moe_combine in one call (one launch for small bf16 decode
    batches, where y is not used) -> out [T, H]."""
    E, H, I = w2.shape
    dt = _dtype_code(act)
    fused = moe_ffn_down_combine_fused(dt, T, H, I, E, k, decode)
    if y is None and not fused:
        splits = moe_ffn_down_splits(dt, T, H, I, E, k, decode)
        shape = (T * k, H) if splits == 1 else (splits, T * k, H)
        y = torch.empty(shape, dtype=torch.float32, device=act.device)
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=act.device)
    _dev(act, w2, topk_w, aligned["offsets"], aligned["slot_to_sorted"], out,
         *([y] if y is not None else []))
    check(lib().moe_ffn_down_combine(dt, int(decode), _ptr(act), _ptr(w2), _ptr(topk_w),
                                     _ptr(aligned["offsets"]), _ptr(aligned["slot_to_sorted"]),
                                     T, H, I, E, k, _ptr(y), _ptr(out), _stream()),
          "moe_ffn_down_combine")
    return out


def moe_layer(hidden, w13, w2, logits, k: int, norm_topk_prob: bool = True,
              decode: bool | None = None):
    """route -> align -> expert FFN + combine.  Returns (out, topk_w, topk_ids, aligned)."""
    E = w13.shape[0]
    topk_w, topk_ids = moe_route(logits, k, norm_topk_prob)
    aligned = moe_align(topk_ids, E)
    if decode is None:
        decode = hidden.dtype == torch.bfloat16 and hidden.shape[0] <= _lib.MOE_DECODE_MAX_T
    out = moe_expert_ffn(hidden, w13, w2, topk_w, aligned, decode=decode)
    return out, topk_w, topk_ids, aligned


def moe_route_backward(logits, topk_ids, topk_w, grad_topk_w, norm_topk_prob: bool = True,
                       grad_logits=None):
    """Gradient of moe_route's weights w.r.t. the logits -> grad_logits [T, E] float32."""
    T, E = logits.shape
    k = topk_ids.shape[1]
    if grad_logits is None:
        grad_logits = torch.empty((T, E), dtype=torch.float32, device=logits.device)
    _dev(logits, topk_ids, topk_w, grad_topk_w, grad_logits)
    check(lib().moe_route_backward(_ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                                   _ptr(grad_topk_w), T, E, k, int(bool(norm_topk_prob)),
                                   _ptr(grad_logits), _stream()), "moe_route_backward")
    return grad_logits


def moe_route_grouped_backward(scores, topk_ids, topk_w, grad_topk_w, renormalize: bool = False,
                               grad_scores=None):
    """Gradient of moe_route_grouped's weights w.r.t. the scores -> [T, E] float32."""
    T, E = scores.shape
    k = topk_ids.shape[1]
    if grad_scores is None:
        grad_scores = torch.empty((T, E), dtype=torch.float32, device=scores.device)
    _dev(scores, topk_ids, topk_w, grad_topk_w, grad_scores)
    check(lib().moe_route_grouped_backward(_ptr(scores), _ptr(topk_ids), _ptr(topk_w),
                                           _ptr(grad_topk_w), T, E, k, int(bool(renormalize)),
                                           _ptr(grad_scores), _stream()),
          "moe_route_grouped_backward")
    return grad_scores


def moe_router_backward(hidden, w_gate, grad_logits, out=None, workspace=None):
    """Backward of the gate logits = hidden . w_gate^T -> (grad_hidden [T, H],
    grad_w_gate [E, H]) float32."""
    T, H = hidden.shape
    E = w_gate.shape[0]
    if out is None:
        out = (torch.empty((T, H), dtype=torch.float32, device=hidden.device),
               torch.empty((E, H), dtype=torch.float32, device=hidden.device))
    if workspace is None:
        workspace = torch.empty(max(1, int(lib().moe_router_backward_workspace_size(T, H, E))),
                                dtype=torch.uint8, device=hidden.device)
    _dev(hidden, w_gate, grad_logits, *out, workspace)
    check(lib().moe_router_backward(_dtype_code(hidden), _ptr(hidden), _ptr(w_gate),
                                    _ptr(grad_logits), T, H, E, _ptr(out[0]), _ptr(out[1]),
                                    _ptr(workspace), workspace.numel(), _stream()),
          "moe_router_backward")
    return out


def moe_expert_ffn_backward_workspace_size(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(lib().moe_expert_ffn_backward_workspace_size(T, H, I, E, k))


def moe_expert_ffn_backward(hidden, w13, w2, topk_w, aligned: dict, grad_out, out=None,
                            workspace=None):
    """Backward of moe_expert_ffn (bf16) -> dict of float32 grad_hidden [T, H],
    grad_w13 [E, 2I, H], grad_w2 [E, H, I], grad_topk_w [T, k]."""
    T, H, I, E = _ffn_shapes(hidden, w13, w2)
    k = topk_w.shape[1]
    dev = hidden.device
    if out is None:
        f32 = dict(dtype=torch.float32, device=dev)
        out = {"grad_hidden": torch.empty((T, H), **f32),
               "grad_w13": torch.empty((E, 2 * I, H), **f32),
               "grad_w2": torch.empty((E, H, I), **f32),
               "grad_topk_w": torch.empty((T, k), **f32)}
    if workspace is None:
        workspace = torch.empty(max(1, moe_expert_ffn_backward_workspace_size(T, H, I, E, k)),
                                dtype=torch.uint8, device=dev)
    _dev(hidden, w13, w2, topk_w, grad_out, workspace, aligned["offsets"],
         aligned["sorted_token_ids"], aligned["sorted_slot_ids"], aligned["slot_to_sorted"],
         *out.values())
    check(lib().moe_expert_ffn_backward(
        _dtype_code(hidden), _ptr(hidden), _ptr(w13), _ptr(w2), _ptr(topk_w),
        _ptr(aligned["offsets"]), _ptr(aligned["sorted_token_ids"]),
        _ptr(aligned["sorted_slot_ids"]), _ptr(aligned["slot_to_sorted"]), _ptr(grad_out),
        T, H, I, E, k, _ptr(out["grad_hidden"]), _ptr(out["grad_w13"]), _ptr(out["grad_w2"]),
        _ptr(out["grad_topk_w"]), _ptr(workspace), workspace.numel(), _stream()),
        "moe_expert_ffn_backward")
    return out


def moe_layer_backward(hidden, w13, w2, logits, topk_w, topk_ids, aligned: dict, grad_out,
                       norm_topk_prob: bool = True):
    """Backward of moe_layer from its saved routing: moe_expert_ffn_backward then
    moe_route_backward.  Returns grad_hidden, grad_w13, grad_w2, grad_topk_w and
    grad_logits (float32)."""
    g = moe_expert_ffn_backward(hidden, w13, w2, topk_w, aligned, grad_out)
    g["grad_logits"] = moe_route_backward(logits, topk_ids, topk_w, g["grad_topk_w"],
                                          norm_topk_prob)
    return g
