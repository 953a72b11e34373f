"""Seeded synthetic inputs for the MoE layer forward.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the CPU oracle (``oracle/``) and the HIP library are
fed from here, so the two sides always read identical bits.

Recipe (one generator per (workload, stream)):

* seed = 1000 * workload_id + stream, streams: 0 gating logits, 1 hidden,
  2 w13, 3 w2, 4 expert bias, 5 expert rank permutation, 6 router gate
  weights (w_gate [E, H], N(0, 1/H) bf16, so hidden . w_gate^T has unit
  variance like the workloads' N(0,1) logits).
* Large tensors are drawn in fixed-size chunks; chunk ``c`` of a stream uses
  ``PCG64(SeedSequence(seed, spawn_key=(c,)))``, so the bits do not depend on
  how many threads draw them.
* Normal draws are float32 (numpy's ziggurat), scaled in float32 by the
  standard deviation, then rounded to bfloat16 with round-to-nearest-even.
  ``N(0, v)`` means variance ``v``; weights have std ``1/sqrt(fan_in)``.

Workloads (ids as used in seeds):

1. tiny fp32 layer  T=4,     H=64,   I=128,   E=8,  k=2
2. routing only     T=16384,                  E=64, k=8
3. Mixtral-shaped   T=4096,  H=4096, I=14336, E=8,  k=2  (bf16)
4. fine-grained     T=8192,  H=2048, I=1408,  E=64, k=8  (bf16, skewed)
5. decode           T=1|32,  H=2048, I=1408,  E=64, k=8  (bf16, skewed)
6. grouped routing, noaux_tc              T=16384, E=256, 8 groups, 4 kept, k=8
7. grouped routing, group_limited_greedy  T=16384, E=160, 8 groups, 3 kept, k=6

The grouped-routing scores are the logistic function of N(0,1) draws
(computed in float64, rounded to float32), i.e. values in (0, 1) as a
sigmoid gate gives them; noaux_tc's correction bias is N(0, 0.1^2) per
expert, float32.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

CHUNK = 1 << 22  # elements per independently seeded chunk

S_LOGITS, S_HIDDEN, S_W13, S_W2, S_BIAS, S_RANK, S_WGATE, S_GRAD = range(8)


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    T: int
    E: int
    k: int
    H: int = 0
    I: int = 0
    dtype: str = "bf16"  # "f32" or "bf16" for hidden / weights / output
    norm: bool = True
    bias: str = "none"  # "none" | "normal0.5" | "zipf1.1"


WORKLOADS = {
    "tiny": Workload(1, "tiny", T=4, E=8, k=2, H=64, I=128, dtype="f32"),
    "routing": Workload(2, "routing", T=16384, E=64, k=8, bias="normal0.5"),
    "mixtral": Workload(3, "mixtral", T=4096, E=8, k=2, H=4096, I=14336),
    "finegrained": Workload(4, "finegrained", T=8192, E=64, k=8, H=2048, I=1408,
                            bias="zipf1.1"),
    "decode1": Workload(5, "decode1", T=1, E=64, k=8, H=2048, I=1408, bias="zipf1.1"),
    "decode32": Workload(5, "decode32", T=32, E=64, k=8, H=2048, I=1408, bias="zipf1.1"),
}


@dataclass(frozen=True)
class GroupedWorkload:
    wid: int
    name: str
    T: int
    E: int
    k: int
    n_group: int
    topk_group: int
    method: str  # "noaux_tc" | "group_limited_greedy"
    renorm: bool = False  # divide the selected scores by their sum


GROUPED = {
    "grouped_noaux": GroupedWorkload(6, "grouped_noaux", T=16384, E=256, k=8, n_group=8,
                                     topk_group=4, method="noaux_tc", renorm=True),
    "grouped_greedy": GroupedWorkload(7, "grouped_greedy", T=16384, E=160, k=6, n_group=8,
                                      topk_group=3, method="group_limited_greedy"),
}


def _seed(wid: int, stream: int) -> int:
    return 1000 * wid + stream


def generator(wid: int, stream: int, chunk: int | None = None) -> np.random.Generator:
    if chunk is None:
        return np.random.Generator(np.random.PCG64(_seed(wid, stream)))
    ss = np.random.SeedSequence(_seed(wid, stream), spawn_key=(chunk,))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(wid: int, stream: int, n: int, std: float, threads: int = 8) -> np.ndarray:
    """n float32 draws of N(0, std^2), chunked and seeded per chunk."""
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, math.ceil(n / CHUNK))
    s = np.float32(std)

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        seg = out[lo:hi]
        generator(wid, stream, c).standard_normal(out=seg, dtype=np.float32)
        if std != 1.0:
            seg *= s

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def normal_bf16(wid: int, stream: int, n: int, std: float, threads: int = 8) -> np.ndarray:
    """n bfloat16 draws (uint16 bits) of N(0, std^2), converted chunk by chunk."""
    out = np.empty(n, dtype=np.uint16)
    nchunks = max(1, math.ceil(n / CHUNK))
    s = np.float32(std)

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        seg = generator(wid, stream, c).standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            seg *= s
        out[lo:hi] = f32_to_bf16_bits(seg)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def expert_bias(w: Workload) -> np.ndarray:
    """Per-expert additive gating bias (float32, length E)."""
    E = w.E
    if w.bias == "none":
        return np.zeros(E, dtype=np.float32)
    if w.bias == "normal0.5":
        g = generator(w.wid, S_BIAS)
        return (g.standard_normal(E) * math.sqrt(0.5)).astype(np.float32)
    if w.bias == "zipf1.1":
        # Zipf(1.1) popularity over a seeded rank permutation; bias = 2 ln p_e.
        rank = generator(w.wid, S_RANK).permutation(E) + 1
        p = rank.astype(np.float64) ** -1.1
        p /= p.sum()
        return (2.0 * np.log(p)).astype(np.float32)
    raise ValueError(w.bias)


def gating_logits(w: Workload, T: int | None = None, reject_ties: bool | None = None) -> np.ndarray:
    """[T, E] float32 logits: N(0,1) plus the workload's per-expert bias."""
    T = w.T if T is None else T
    g = generator(w.wid, S_LOGITS)
    x = g.standard_normal((T, w.E)).astype(np.float32)
    if reject_ties is None:
        reject_ties = w.wid == 1
    if reject_ties:
        for t in range(T):
            while len(np.unique(x[t])) != w.E:
                x[t] = g.standard_normal(w.E).astype(np.float32)
    bias = expert_bias(w)
    if w.bias != "none":
        x = (x + bias[None, :]).astype(np.float32)
    return np.ascontiguousarray(x)


def gating_logits_draw(w: Workload, draw: int) -> np.ndarray:
    """Extra independent [T, E] logits for the same workload (draw >= 1; draw 0
    is gating_logits): N(0,1) from stream 100 + draw, plus the same bias."""
    if draw == 0:
        return gating_logits(w)
    g = generator(w.wid, 100 + draw)
    x = g.standard_normal((w.T, w.E)).astype(np.float32)
    if w.bias != "none":
        x = (x + expert_bias(w)[None, :]).astype(np.float32)
    return np.ascontiguousarray(x)


def layer_inputs(w: Workload, T: int | None = None, weights: bool = True) -> dict:
    """Every input of the layer forward for a workload.

    Returns numpy arrays: logits [T,E] f32, hidden [T,H], w13 [E,2I,H],
    w2 [E,H,I].  bf16 tensors are uint16 bit patterns; f32 ones float32.
    """
    T = w.T if T is None else T
    out = {"logits": gating_logits(w, T)}
    if w.H == 0:
        return out
    H, I, E = w.H, w.I, w.E
    if w.dtype == "f32":
        out["hidden"] = normal_f32(w.wid, S_HIDDEN, T * H, 1.0).reshape(T, H)
        if weights:
            out["w13"] = normal_f32(w.wid, S_W13, E * 2 * I * H, 1 / math.sqrt(H)).reshape(E, 2 * I, H)
            out["w2"] = normal_f32(w.wid, S_W2, E * H * I, 1 / math.sqrt(I)).reshape(E, H, I)
    else:
        out["hidden"] = normal_bf16(w.wid, S_HIDDEN, T * H, 1.0).reshape(T, H)
        if weights:
            out["w13"] = normal_bf16(w.wid, S_W13, E * 2 * I * H, 1 / math.sqrt(H)).reshape(E, 2 * I, H)
            out["w2"] = normal_bf16(w.wid, S_W2, E * H * I, 1 / math.sqrt(I)).reshape(E, H, I)
    return out


def random_ids(seed: int, T: int, E: int, k: int, invalid_frac: float = 0.0) -> np.ndarray:
    """[T,k] int32 ids, distinct per row; a fraction of slots set to -1 or >= E."""
    g = np.random.Generator(np.random.PCG64(seed))
    ids = np.argsort(g.random((T, E)), axis=1)[:, :k].astype(np.int32)
    if invalid_frac > 0:
        m = g.random((T, k)) < invalid_frac
        bad = np.where(g.random((T, k)) < 0.5, -1, E + g.integers(0, 3, (T, k)))
        ids = np.where(m, bad, ids).astype(np.int32)
    return np.ascontiguousarray(ids)


def random_probs(seed: int, T: int, k: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return np.ascontiguousarray(g.random((T, k)).astype(np.float32))


def grouped_scores(w: GroupedWorkload, T: int | None = None, draw: int = 0) -> np.ndarray:
    """[T, E] float32 scores in (0, 1): the logistic function of N(0,1) draws."""
    T = w.T if T is None else T
    g = generator(w.wid, S_LOGITS if draw == 0 else 100 + draw)
    x = g.standard_normal((T, w.E))
    return np.ascontiguousarray((1.0 / (1.0 + np.exp(-x))).astype(np.float32))


def correction_bias(w: GroupedWorkload) -> np.ndarray | None:
    """noaux_tc's per-expert score correction bias, N(0, 0.1^2) float32 (None otherwise)."""
    if w.method != "noaux_tc":
        return None
    g = generator(w.wid, S_BIAS)
    return np.ascontiguousarray((g.standard_normal(w.E) * 0.1).astype(np.float32))


def router_weights(w: Workload) -> np.ndarray:
    """The linear gate w_gate [E, H] (bf16 bits, N(0, 1/H)) for a layer workload."""
    return normal_bf16(w.wid, S_WGATE, w.E * w.H, 1 / math.sqrt(w.H)).reshape(w.E, w.H)


def grad_output(w: Workload, T: int | None = None) -> np.ndarray:
    """Gradient of the layer output for backward runs: [T, H] N(0, 1) in the layer dtype
    (bf16 as uint16 bits)."""
    T = w.T if T is None else T
    if w.dtype == "f32":
        return normal_f32(w.wid, S_GRAD, T * w.H, 1.0).reshape(T, w.H)
    return normal_bf16(w.wid, S_GRAD, T * w.H, 1.0).reshape(T, w.H)
