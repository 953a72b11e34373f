// Internal declarations shared by the libmoe HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

// The grouped GEMMs' token rows per tile (m-tile) and how an expert's rows
// are dealt to its m-tiles; the alignment's tile schedule follows the same
// rule.  An expert with cnt rows has ceil(cnt / BM) m-tiles; its rows go to
// them in equal shares rounded up to whole 32-row fragments (at most BM;
// never an empty tile: (mt - 1) q < cnt, checked for every cnt < 200000), so
// the tiles that share a weight tile do similar work.
#ifndef MOE_GEMM_BM
#define MOE_GEMM_BM 320
#endif
constexpr int kGemmBM = MOE_GEMM_BM;
__host__ __device__ inline int expert_mtiles(int cnt) { return (cnt + kGemmBM - 1) / kGemmBM; }
__host__ __device__ inline int mtile_share(int cnt, int mt) {
    return (cnt + 32 * mt - 1) / (32 * mt) * 32;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; the conversion lowers to gfx950's hardware cvt.
__device__ __forceinline__ __bf16 to_bf16(float f) { return static_cast<__bf16>(f); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (uint64_t(1) << lane_id()) - 1;
}

__device__ __forceinline__ int readlane_i(int v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}
__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// ---------------------------------------------------------------------------
// 16-lane row reductions with DPP (VALU lane permutes, no LDS crossbar): after
// xor-1, xor-2, half-row mirror and row mirror steps every lane of each
// 16-lane row holds the row's result.
// ---------------------------------------------------------------------------
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror
constexpr int kDppRor8 = 0x128;       // row_ror:8 (lane i of a row reads lane i ^ 8)

template <int ctrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, 0xF, 0xF, true);
}
template <int ctrl>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = dpp_u32<ctrl>((uint32_t)u), hi = dpp_u32<ctrl>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppMirror>(v));
    return v;
}
__device__ __forceinline__ double row16_sum_f64(double v) {
    v += dpp_f64<kDppXor1>(v);
    v += dpp_f64<kDppXor2>(v);
    v += dpp_f64<kDppHalfMirror>(v);
    v += dpp_f64<kDppMirror>(v);
    return v;
}

// Order-preserving map of a float to an unsigned key (larger float, larger
// key; every finite or infinite value maps above 0).  -0.0 and +0.0 compare
// equal as floats, so both map to the key of +0.0.
__device__ __forceinline__ uint32_t float_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// One routing row held by a 16-lane DPP row (g = lane / 16, q = lane % 16):
// lane q holds the logits v[0..3] of experts 4q .. 4q+3, `avail` marks which
// of them exist.  Selects the row's top k (value descending, the lower expert
// id first among equal values) in k rounds.  Each lane first sorts its four
// order-preserving keys (descending, the lower local index first among equal
// keys; missing experts key 0, last), so its best is always the head of its
// list; a round is a 4-step DPP maximum of the heads over the row and one
// ballot (the lowest lane holding the maximum wins, i.e. the lower expert id),
// and the winning lane pops its head.  Returns the weight of slot q (lanes
// q < k; softmax over the k selected logits if norm, else the full softmax at
// the selected expert), computed in double and rounded once.  Byte i of
// slot_of = the round (= slot) that picked local expert i (0xFF if none): the
// lane that owns an expert writes its id, so no round broadcasts the winner's
// local index.  Rows with no available expert (past T) select nothing; a key
// of 0 is never selected.
__device__ __forceinline__ float route_row16(const float v[4], uint32_t avail, int k, int norm,
                                             int g, int q, uint32_t &slot_of) {
    const uint32_t valid = avail;
    uint32_t key[4];
    int idx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        key[i] = ((avail >> i) & 1u) ? float_key(v[i]) : 0u;
        idx[i] = i;
    }
    // Sorting network on (key descending, index ascending): a total order,
    // so the result is that order whatever the comparators' sequence.
    auto cswap = [&](int a, int b) {
        const bool sw = key[b] > key[a] || (key[b] == key[a] && idx[b] < idx[a]);
        const uint32_t ka = key[a], kb = key[b];
        const int ia = idx[a], ib = idx[b];
        key[a] = sw ? kb : ka;
        key[b] = sw ? ka : kb;
        idx[a] = sw ? ib : ia;
        idx[b] = sw ? ia : ib;
    };
    cswap(0, 1);
    cswap(2, 3);
    cswap(0, 2);
    cswap(1, 3);
    cswap(1, 2);

    uint32_t sel_key = 0, kmax = 0;
    slot_of = 0xFFFFFFFFu;
    for (int r = 0; r < k; ++r) {
        const uint32_t bk = key[0];
        const uint32_t rmax = row16_max_u32(bk);
        const uint64_t cand = __ballot(bk != 0 && bk == rmax);
        const uint32_t mrow = (uint32_t)(cand >> (g * 16)) & 0xFFFFu;
        const int wl = __ffs((int)mrow) - 1;  // -1 only for rows without experts
        if (q == wl) {
            slot_of = (slot_of & ~(0xFFu << (8 * idx[0]))) | ((uint32_t)r << (8 * idx[0]));
            key[0] = key[1];
            key[1] = key[2];
            key[2] = key[3];
            key[3] = 0u;
            idx[0] = idx[1];
            idx[1] = idx[2];
            idx[2] = idx[3];
        }
        if (q == r) sel_key = rmax;
        if (r == 0) kmax = rmax;
    }

    // Weights in double, rounded once to float.
    const double mx = (double)key_float(kmax);
    const double ex = q < k ? exp((double)key_float(sel_key) - mx) : 0.0;
    double part;
    if (norm) {
        part = ex;
    } else {
        part = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if ((valid >> i) & 1u) part += exp((double)v[i] - mx);
    }
    const double sum = row16_sum_f64(part);
    return (float)(ex / sum);
}

// Stable alignment of at most kWave routing slots by one wave: slot s = lane
// holds expert s_ids[s] (LDS; -1 or >= E: dropped).  A slot's rank among the
// earlier slots of its expert comes from ceil(log2 E) ballots + popcount,
// the expert leaders record the counts in s_cnt (LDS, E entries, zero on
// entry), and lane e scans them into the exclusive offsets s_off (LDS, E + 1
// entries).  The wave's own LDS accesses are ordered, so it needs no block
// barrier; it must be the only wave touching s_cnt and s_off.  When
// `counts` is not null, also writes counts, offsets, sorted_tok, sorted_slot
// and slot_to_sorted to memory (positions past the valid slots read -1);
// when `l_sorted_tok` is not null, sorted_tok also goes there (LDS, n
// entries).  E <= kWave.
__device__ __forceinline__ void align_slots_wave(const int32_t *s_ids, int n, int k, int E,
                                                 int nbits, int32_t *s_cnt, int32_t *s_off,
                                                 int32_t *__restrict__ counts,
                                                 int32_t *__restrict__ offsets,
                                                 int32_t *__restrict__ sorted_tok,
                                                 int32_t *__restrict__ sorted_slot,
                                                 int32_t *__restrict__ slot_to_sorted,
                                                 int32_t *l_sorted_tok) {
    const int lane = lane_id();
    const int s = lane;
    const int e = s < n ? s_ids[s] : -1;
    const bool ok = (unsigned)e < (unsigned)E;
    uint64_t peers = __ballot(ok);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (e >> bit) & 1;
        const uint64_t m = __ballot(ok && set);
        peers &= set ? m : ~m;
    }
    const int rank = __popcll(peers & lanemask_lt());
    if (ok && rank == 0) s_cnt[e] = __popcll(peers);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int c = lane < E ? s_cnt[lane] : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    const int total = __shfl(incl, kWave - 1, kWave);
    s_off[lane] = incl - c;
    if (lane == 0) s_off[E] = total;
    if (counts != nullptr) {
        if (lane < E) {
            counts[lane] = c;
            offsets[lane] = incl - c;
        }
        if (lane == 0) offsets[E] = total;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (ok) {
        const int p = s_off[e] + rank;
        if (l_sorted_tok != nullptr) l_sorted_tok[p] = s / k;
        if (counts != nullptr) {
            sorted_tok[p] = s / k;
            sorted_slot[p] = s;
            slot_to_sorted[s] = p;
        }
    } else if (s < n && counts != nullptr) {
        slot_to_sorted[s] = -1;
    }
    for (int p = total + lane; p < n; p += kWave) {
        if (l_sorted_tok != nullptr) l_sorted_tok[p] = -1;
        if (counts != nullptr) {
            sorted_tok[p] = -1;
            sorted_slot[p] = -1;
        }
    }
}

// Largest k served by the 16-lanes-per-row converters.
constexpr int kKMax16 = 16;

// multihot -> indices for row t (T rows; the 16-lane group's lane q, CPL
// columns per lane, E <= 16 CPL, k <= kKMax16): slot j of the row is filled
// from the highest expert naming it -- each lane proposes 1 + its highest
// expert per slot, a 16-lane DPP max per slot picks the row's, and lane j
// fetches that expert's probability ([mgt] _multihot_to_indices_kernel).
// Every lane of the group must call it (rows t >= T write nothing).
template <int CPL>
__device__ __forceinline__ void to_indices_row16(const float *__restrict__ pim,
                                                 const int32_t *__restrict__ pos, int64_t T,
                                                 int64_t t, int E, int k,
                                                 float *__restrict__ probs,
                                                 int32_t *__restrict__ ids, int q) {
    const int c0 = CPL * q;
    const bool row_ok = t < T;
    int pp[CPL];
#pragma unroll
    for (int c = 0; c < CPL / 4; ++c) {
        int4 p4 = make_int4(-1, -1, -1, -1);
        if (row_ok && c0 + 4 * c < E) p4 = *reinterpret_cast<const int4 *>(pos + t * E + c0 + 4 * c);
        pp[4 * c] = p4.x;
        pp[4 * c + 1] = p4.y;
        pp[4 * c + 2] = p4.z;
        pp[4 * c + 3] = p4.w;
    }
    uint32_t best[kKMax16];
#pragma unroll
    for (int j = 0; j < kKMax16; ++j) {
        best[j] = 0;
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            if (pp[i] == j) best[j] = (uint32_t)(c0 + i + 1);
    }
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < kKMax16; ++j) {
        if (j < k) {
            const uint32_t b = row16_max_u32(best[j]);
            if (q == j) mine = b;
        }
    }
    if (row_ok && q < k) {
        const int e = (int)mine - 1;
        probs[t * k + q] = e >= 0 ? pim[t * E + e] : 0.0f;
        if (ids) ids[t * k + q] = e;
    }
}

// One routing row on a 16-lane DPP row (g = lane / 16, q = lane % 16): row
// t of logits [T, E] (E <= 64, k <= 16; rows t >= T write nothing), the
// selection of route_row16, topk_w / topk_ids written by lanes q < k, and
// with multihot != nullptr (E % 4 == 0, 16-byte aligned rows) the row's [E]
// multihot, probability and position-map entries: each lane records which
// round picked each of its 4 experts, fetches that slot's weight from the
// lane that computed it, and writes its 4 columns.  vec4: E == 64 and
// 16-byte aligned logits.  Returns slot_of (byte i: the slot that picked
// local expert i, 0xFF if none; all 0xFF for rows past T).
__device__ __forceinline__ uint32_t route16_row(const float *__restrict__ logits, int64_t T,
                                           int64_t t, int E, int k, int norm, int vec4,
                                           float *__restrict__ topk_w,
                                           int32_t *__restrict__ topk_ids,
                                           uint8_t *__restrict__ multihot, float *__restrict__ pim,
                                           int32_t *__restrict__ pos, int g, int q) {
    const int lane = lane_id();
    const bool row_ok = t < T;
    float v[4];
    uint32_t avail = 0;
    if (row_ok && vec4) {  // E == 64 and 16-byte aligned rows
        const float4 x = *reinterpret_cast<const float4 *>(logits + t * 64 + 4 * q);
        v[0] = x.x;
        v[1] = x.y;
        v[2] = x.z;
        v[3] = x.w;
        avail = 0xFu;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * q + i;
            v[i] = 0.0f;
            if (row_ok && e < E) {
                v[i] = logits[t * E + e];
                avail |= 1u << i;
            }
        }
    }
    uint32_t slot_of;  // byte i: round that picked local expert i (0xFF: none)
    const float wq = route_row16(v, avail, k, norm, g, q, slot_of);
    if (row_ok) {
        if (q < k) topk_w[t * k + q] = wq;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t r = (slot_of >> (8 * i)) & 0xFFu;
            if (r != 0xFFu) topk_ids[t * k + r] = 4 * q + i;
        }
    }
    if (multihot != nullptr) {
        int pj[4];
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (int)((slot_of >> (8 * i)) & 0xFFu);
            pj[i] = r == 0xFF ? -1 : r;
            // Every lane takes part in the shuffle; unpicked columns read
            // their own lane and are zeroed.
            const float w = __shfl(wq, pj[i] >= 0 ? (lane & ~15) + pj[i] : lane, kWave);
            pv[i] = pj[i] >= 0 ? w : 0.0f;
        }
        if (row_ok && 4 * q < E) {
            const uint32_t m = (uint32_t)(pj[0] >= 0) | (uint32_t)(pj[1] >= 0) << 8 |
                               (uint32_t)(pj[2] >= 0) << 16 | (uint32_t)(pj[3] >= 0) << 24;
            *reinterpret_cast<uint32_t *>(multihot + t * E + 4 * q) = m;
            *reinterpret_cast<float4 *>(pim + t * E + 4 * q) =
                make_float4(pv[0], pv[1], pv[2], pv[3]);
            *reinterpret_cast<int4 *>(pos + t * E + 4 * q) = make_int4(pj[0], pj[1], pj[2], pj[3]);
        }
    }
    return slot_of;
}

// SiLU in float32: z / (1 + e^-z).
// silu(z) = z / (1 + e^-z), with the hardware reciprocal (v_rcp_f32, about
// 1 ulp) instead of an IEEE division: the result is rounded to bf16 next,
// and the division's fix-up sequence tripled the size of the GEMM epilogues.
// z -> -inf gives -0 (the reciprocal of inf is 0), z -> +inf gives z.
__device__ __forceinline__ float silu_f(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// ---------------------------------------------------------------------------
// Launchers (each returns hipSuccess or the launch error).
// ---------------------------------------------------------------------------
hipError_t launch_route(const float *logits, int64_t T, int E, int k, int norm, float *w,
                        int32_t *ids, hipStream_t s);
// Route and indices->multihot in one pass where the fused kernel applies
// (route_multihot_fused), else the two launches.
bool route_multihot_fused(int E, int k, const uint8_t *mh, const float *pim, const int32_t *pos);
hipError_t launch_route_multihot(const float *logits, int64_t T, int E, int k, int norm,
                                 float *w, int32_t *ids, uint8_t *mh, float *pim, int32_t *pos,
                                 hipStream_t s);

// Group-limited selection; with mh != nullptr also the indices->multihot
// conversion of its output (in the same kernel on the 16-lanes-per-row path).
bool route_grouped_rows16(int E, int n_group, int k);
hipError_t launch_route_grouped(const float *scores, const float *bias, int64_t T, int E, int k,
                                int n_group, int topk_group, int noaux, int renorm, float *w,
                                int32_t *ids, uint8_t *mh, float *pim, int32_t *pos,
                                hipStream_t s);

hipError_t launch_router_route(const uint16_t *hidden, const uint16_t *wg, int64_t T, int H,
                               int E, int k, int norm, float *logits, float *w, int32_t *ids,
                               hipStream_t s);

// Gate backward: grad_hidden = g . w_gate, grad_w_gate = g^T . hidden (f32).
size_t router_backward_scratch_bytes(int64_t T, int H, int E);
hipError_t launch_router_backward(const uint16_t *hidden, const uint16_t *wg, const float *g,
                                  int64_t T, int H, int E, float *gh, float *gw, void *ws,
                                  hipStream_t s);

int align_num_blocks(int64_t n_slots, int E);
// The m-tile list of the grouped GEMMs from the aligned offsets (expert
// order, then m-tile order): tile i covers rows [row_start, row_end) of
// expert tile_expert; num_tiles gets the count (entries past max_tiles are
// not written).  E <= 1024.
hipError_t launch_tile_schedule(const int32_t *offsets, int E, int64_t max_tiles,
                                int32_t *tile_expert, int32_t *tile_row_start,
                                int32_t *tile_row_end, int32_t *num_tiles, hipStream_t s);
// With inv_w, also the [T, E] maps (pim, pos) back to indices (inv_w,
// inv_ids), in the scatter's launch where the 16-lanes-per-row form applies.
hipError_t launch_align(const int32_t *ids, int64_t T, int k, int E, int32_t *counts,
                        int32_t *offsets, int32_t *sorted_tok, int32_t *sorted_slot,
                        int32_t *slot_to_sorted, int32_t *ws, hipStream_t s,
                        const float *pim = nullptr, const int32_t *pos = nullptr,
                        float *inv_w = nullptr, int32_t *inv_ids = nullptr);

// Route (+ indices->multihot when mh != nullptr) and align in fewer launches
// where route_align_fused holds; otherwise the separate launches.  Outputs
// are those of the separate calls, bit for bit.  With inv_w (which needs the
// multihot outputs), the maps are also converted back to indices
// (launch_to_indices: inv_w, inv_ids) in the last launch where fused.
bool route_align_fused(int64_t T, int E, int k, const uint8_t *mh, const float *pim,
                       const int32_t *pos);
hipError_t launch_route_align(const float *logits, int64_t T, int E, int k, int norm, float *w,
                              int32_t *ids, uint8_t *mh, float *pim, int32_t *pos,
                              int32_t *counts, int32_t *offsets, int32_t *sorted_tok,
                              int32_t *sorted_slot, int32_t *slot_to_sorted, int32_t *ws,
                              float *inv_w, int32_t *inv_ids, hipStream_t s);

hipError_t launch_to_multihot(const int32_t *ids, const float *probs, int64_t T, int k, int E,
                              uint8_t *mh, float *pim, int32_t *pos, hipStream_t s);
hipError_t launch_to_indices(const float *pim, const int32_t *pos, int64_t T, int E, int k,
                             float *probs, int32_t *ids, hipStream_t s);

hipError_t launch_gate_up_bf16(const uint16_t *hidden, const uint16_t *w13,
                               const int32_t *offsets, const int32_t *sorted_tok, int64_t T,
                               int H, int I, int E, int k, uint16_t *act, hipStream_t s);
hipError_t launch_down_bf16(const uint16_t *act, const uint16_t *w2, const int32_t *offsets,
                            int64_t T, int H, int I, int E, int k, int ksplit, float *y,
                            hipStream_t s);
// The backward's gate/up recompute (x . w13^T on the FC1 kernel) with the
// SiLU-and-mul backward in its epilogue: from G [T k, I] f32 and the routing
// weights it writes wact [T k, I] and dh13 [T k, 2I] (bf16, aligned order)
// and gw_part [T k, gate_up_bwd_tiles(I)] f32, each row's partial sums of
// G . act per column tile (the routing-weight gradient is their sum in tile
// order).  Needs buffer addressing (gate_up_bwd_ok).
bool gate_up_bwd_ok(int64_t T, int H, int I);
int gate_up_bwd_tiles(int I);
hipError_t launch_gate_up_bwd_bf16(const uint16_t *hidden, const uint16_t *w13,
                                   const int32_t *offsets, const int32_t *sorted_tok,
                                   const int32_t *sorted_slot, const float *topk_w,
                                   const float *G, int64_t T, int H, int I, int E, int k,
                                   uint16_t *wact, uint16_t *dh13, float *gw_part,
                                   hipStream_t s);
// The FC2-form grouped product with a K-major weight w [E, K, N] (N
// contiguous): y[p, n] = sum_k a[row(p), k] w[e, k, n] for the rows p of
// expert e, float32 [T k, N], with row(p) = p (a [T k, K]) or, given
// `gather`, gather[p] (a [T, K]).  Needs buffer addressing (down_kmajor_ok).
bool down_kmajor_ok(int64_t T, int N, int K, int k);
hipError_t launch_down_kmajor_bf16(const uint16_t *a, const int32_t *gather, const uint16_t *w,
                                   const int32_t *offsets, int64_t T, int N, int K, int E, int k,
                                   float *y, hipStream_t s);
// Weight gradients C_e [M, N] f32 = sum over k in [poff[e], poff[e+1]) of
// a[m, k] b[n, k] (a [M, ld], b [N, ld] bf16, segments padded to whole
// 64-wide k-tiles) on the grouped kernel's machinery; needs buffer
// addressing (wgrad_grouped_ok).
bool wgrad_grouped_ok(int M, int N, int64_t ld);
hipError_t launch_wgrad_bf16(const uint16_t *a, const uint16_t *b, int64_t ld,
                             const int32_t *poff, int E, int M, int N, float *c, hipStream_t s);
// The same with b the per-position operand as stored, [positions, N] (N
// contiguous), expert e's k-rows being its positions [offs[e], offs[e+1])
// (read past the segment as zeros); `trans` stores C_e transposed, [N, M].
// Needs wgrad_km_ok (buffer addressing for a, N % 8 == 0, M % 4 == 0).
bool wgrad_km_ok(int M, int N, int64_t ld);
hipError_t launch_wgrad_km_bf16(const uint16_t *a, const uint16_t *b, int64_t ld,
                                const int32_t *poff, const int32_t *offs, int E, int M, int N,
                                bool trans, float *c, hipStream_t s);
// K slices the prefill FC2 uses for this shape (1 .. 4).
int down_splits(int64_t T, int H, int I, int E, int k);

hipError_t launch_gate_up_f32(const float *hidden, const float *w13, const int32_t *offsets,
                              const int32_t *sorted_tok, int64_t T, int H, int I, int E, int k,
                              float *act, hipStream_t s);
hipError_t launch_down_f32(const float *act, const float *w2, const int32_t *offsets, int64_t T,
                           int H, int I, int E, int k, float *y, hipStream_t s);

hipError_t launch_decode_gate_up_bf16(const uint16_t *hidden, const uint16_t *w13,
                                      const int32_t *offsets, const int32_t *sorted_tok,
                                      int64_t T, int H, int I, int E, int k, uint16_t *act,
                                      hipStream_t s);
hipError_t launch_decode_down_bf16(const uint16_t *act, const uint16_t *w2,
                                   const int32_t *offsets, int64_t T, int H, int I, int E, int k,
                                   float *y, hipStream_t s);
// Decode FC2 + combine in one launch (bf16 out) where
// decode_down_combine_fused holds (T k <= 32, I <= 1536, T k I <= 48 Ki
// elements): the same out as launch_decode_down_bf16 + launch_combine.
// Route + align (+ the multihot maps and their inverse) + decode FC1 in one
// launch; eligibility (T k <= 16, E <= 64, k <= 16) and launch.
bool decode_route_gate_up_fused(int64_t T, int E, int k, int H, int I);
hipError_t launch_decode_route_gate_up_bf16(
    const float *logits, int64_t T, int E, int k, int norm, float *topk_w, int32_t *topk_ids,
    uint8_t *multihot, float *pim, int32_t *pos, int32_t *counts, int32_t *offsets,
    int32_t *sorted_tok, int32_t *sorted_slot, int32_t *slot_to_sorted, float *inv_w,
    int32_t *inv_ids, const uint16_t *hidden, const uint16_t *w13, int H, int I, uint16_t *act,
    hipStream_t s);
bool decode_down_combine_fused(int64_t T, int H, int I, int E, int k);
hipError_t launch_decode_down_combine_bf16(const uint16_t *act, const uint16_t *w2,
                                           const int32_t *offsets, const float *topk_w,
                                           const int32_t *slot_to_sorted, int64_t T, int H,
                                           int I, int E, int k, uint16_t *out, hipStream_t s);

hipError_t launch_combine(moe_dtype_t dt, const float *y, int splits, const float *w,
                          const int32_t *slot_to_sorted, int64_t T, int H, int k, void *out,
                          hipStream_t s);

// Backward of the group-limited selection's weights (one wave per row).
hipError_t launch_route_grouped_backward(const float *scores, const int32_t *ids, const float *w,
                                         const float *gw, int64_t T, int E, int k, int renorm,
                                         float *out, hipStream_t s);
// Backward of the gating softmax (one wave per row).
hipError_t launch_route_backward(const float *logits, const int32_t *ids, const float *w,
                                 const float *gw, int64_t T, int E, int k, int norm, float *out,
                                 hipStream_t s);
// Expert FFN backward: scratch sizes (bf16; float32, always the smaller), then
// the launches.
size_t ffn_backward_scratch_bytes(int64_t T, int H, int I, int E, int k);
size_t ffn_backward_f32_scratch_bytes(int64_t T, int H, int I, int k);
hipError_t launch_ffn_backward_f32(const float *x, const float *w13, const float *w2,
                                   const float *topk_w, const int32_t *offsets,
                                   const int32_t *sorted_tok, const int32_t *sorted_slot,
                                   const int32_t *slot_to_sorted, const float *dy, int64_t T,
                                   int H, int I, int E, int k, float *dx, float *dw13,
                                   float *dw2, float *dw, void *ws, hipStream_t s);
hipError_t launch_ffn_backward_bf16(const uint16_t *x, const uint16_t *w13, const uint16_t *w2,
                                    const float *topk_w, const int32_t *offsets,
                                    const int32_t *sorted_tok, const int32_t *sorted_slot,
                                    const int32_t *slot_to_sorted, const uint16_t *dy,
                                    int64_t T, int H, int I, int E, int k, float *dx,
                                    float *dw13, float *dw2, float *dw, void *ws,
                                    hipStream_t s);

}  // namespace moe
