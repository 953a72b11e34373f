// Group-limited expert selection: group_limited_greedy and noaux_tc.
//
// Method: mlc-llm moe_misc.py, group_limited_greedy_topk.  The E experts of a
// row form n_group groups of E / n_group consecutive experts.  Choice scores
// are the scores (greedy) or the scores plus a per-expert correction bias
// added in float32 (noaux_tc).  A group scores its best choice score (greedy)
// or the float32 sum of its two best (noaux_tc); the topk_group best groups
// are kept, and the k best experts inside them are selected.  Both rankings
// are value descending with the lower index first on ties, as the pages'
// strict-greater insertion over ascending indices gives.  Weights are the
// scores without the bias at the selected experts, optionally divided by
// their sum.
//
// The pages run this as five separate operators (bias add, per-group top-2 or
// max, top-k over groups, a masking pass that writes a full [T, E] copy, and a
// top-k over that copy, plus a gather for noaux_tc).  Here each row is done in
// one pass from registers, and the masked [T, E] copy never exists.  Two
// kernels:
//  * route_grouped_rows16_kernel (E % 16 == 0, E <= 256, n_group dividing 16,
//    k <= 16): 4 rows per wave, 16 lanes per row, each group on whole lanes;
//    group scores merge over the group's lanes with DPP.
//  * route_grouped_kernel (any other shape): one wave per row (lane l holds
//    experts l*VPL .. l*VPL+VPL-1); the choice scores go to the wave's slice
//    of LDS and lane g reduces group g from there.
// In both, the group and expert rankings are rounds of a cross-lane argmax on
// order-preserving integer keys.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kGroupedThreads = 256;
constexpr int kGroupedWaves = kGroupedThreads / kWave;

// Maximum over the 64 lanes, returned as a wave-uniform value: 16-lane DPP
// maxima, then the four row results read into scalar registers.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = row16_max_u32(v);
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

// Orders the LDS traffic of one wave: every lane's earlier LDS writes are
// complete (and visible to the other lanes of the wave) before later reads,
// and the compiler moves no LDS access across this point.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

template <int VPL>
__global__ __launch_bounds__(kGroupedThreads) void route_grouped_kernel(
    const float *__restrict__ scores, const float *__restrict__ bias, int64_t T, int E, int k,
    int n_group, int topk_group, int noaux, int renorm, int vec4, float *__restrict__ topk_w,
    int32_t *__restrict__ topk_ids) {
    extern __shared__ float s_choice[];  // [kGroupedWaves][E]
    const int lane = lane_id();
    const int wib = threadIdx.x / kWave;
    float *row_c = s_choice + wib * E;
    const int gs = E / n_group;
    const int e0 = lane * VPL;

    // Per-lane constants: the bias of its experts and the group of each.
    float b[VPL];
    int grp[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = e0 + i;
        b[i] = (noaux && e < E) ? bias[e] : 0.0f;
        grp[i] = e < E ? e / gs : 63;
    }
    // Lane g < n_group reduces group g; it starts at a rotated position so
    // that the active lanes read different LDS banks.
    const int g_first = lane < n_group ? lane * gs : 0;
    const int g_rot = lane < n_group ? lane % gs : 0;

    const int64_t wave = (int64_t)blockIdx.x * kGroupedWaves + wib;
    const int64_t nwaves = (int64_t)gridDim.x * kGroupedWaves;
    for (int64_t t = wave; t < T; t += nwaves) {
        const float *row = scores + t * E;
        float v[VPL];
        uint32_t valid = 0;
        if (vec4) {  // E % 4 == 0, 16-byte aligned rows, VPL % 4 == 0
#pragma unroll
            for (int q = 0; q < VPL / 4; ++q) {
                float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
                if (e0 + 4 * q < E) {
                    x = *reinterpret_cast<const float4 *>(row + e0 + 4 * q);
                    valid |= 0xFu << (4 * q);
                }
                v[4 * q] = x.x;
                v[4 * q + 1] = x.y;
                v[4 * q + 2] = x.z;
                v[4 * q + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                v[i] = 0.0f;
                if (e0 + i < E) {
                    v[i] = row[e0 + i];
                    valid |= 1u << i;
                }
            }
        }
        uint32_t key[VPL];
        wave_lds_fence();  // the previous row's group reads are done
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const float c = noaux ? v[i] + b[i] : v[i];  // float32 add, as on the page
            key[i] = float_key(c);
            if ((valid >> i) & 1u) row_c[e0 + i] = c;
        }
        wave_lds_fence();

        // Group scores: lane g walks group g once (any order gives the same
        // maximum, and the same two largest values).
        uint32_t gkey = 0;
        if (lane < n_group) {
            float m1 = -INFINITY, m2 = -INFINITY;
            int j = g_rot;
            for (int n = 0; n < gs; ++n) {
                const float x = row_c[g_first + j];
                if (noaux) {
                    if (n == 0) {
                        m1 = x;
                    } else if (n == 1) {
                        m2 = x > m1 ? m1 : x;
                        m1 = x > m1 ? x : m1;
                    } else if (x > m1) {
                        m2 = m1;
                        m1 = x;
                    } else if (x > m2) {
                        m2 = x;
                    }
                } else {
                    m1 = n == 0 ? x : fmaxf(m1, x);
                }
                j = j + 1 == gs ? 0 : j + 1;
            }
            gkey = float_key(noaux ? m1 + m2 : m1);
        }
        // Keep the topk_group best groups; lanes hold ascending groups, so the
        // lowest candidate lane is the lowest group among equal scores.
        uint64_t kept = 0;
        for (int r = 0; r < topk_group; ++r) {
            const uint32_t m = wave_max_u32(gkey);
            const uint64_t cand = __ballot(gkey != 0 && gkey == m);
            const int L = __ffsll((unsigned long long)cand) - 1;
            kept |= uint64_t(1) << L;
            if (lane == L) gkey = 0;
        }

        uint32_t avail = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (((valid >> i) & 1u) && ((kept >> grp[i]) & 1u)) avail |= 1u << i;

        float sel_w = 0.0f;
        int sel_e = -1;
        for (int r = 0; r < k; ++r) {
            // Lane-local best; strict > keeps the lowest local index on ties.
            uint32_t bk = 0;
            int bi = 0;
            float bw = 0.0f;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                if (((avail >> i) & 1u) && key[i] > bk) {
                    bk = key[i];
                    bi = i;
                    bw = v[i];
                }
            }
            const uint32_t m = wave_max_u32(bk);
            // Lanes own ascending blocks of experts: the lowest candidate lane
            // holds the lowest id among equal choice scores.
            const uint64_t cand = __ballot(bk != 0 && bk == m);
            const int L = __ffsll((unsigned long long)cand) - 1;
            const int wi = readlane_i(bi, L);
            const float ww = readlane_f(bw, L);
            if (lane == L) avail &= ~(1u << bi);
            if (lane == r) {
                sel_w = ww;
                sel_e = L * VPL + wi;
            }
        }

        float w_out = sel_w;
        if (renorm) {
            // Sum in double, one rounding per weight.
            const double s = wave_sum_d(lane < k ? (double)sel_w : 0.0);
            w_out = (float)((double)sel_w / s);
        }
        if (lane < k) {
            topk_w[t * k + lane] = w_out;
            topk_ids[t * k + lane] = sel_e;
        }
    }
}

// Fast path: E % 16 == 0, E <= 256, n_group dividing 16, k <= 16.  A wave
// holds 4 rows, 16 lanes per row; lane q of a row holds the vpl = E / 16
// consecutive experts q*vpl .. q*vpl+vpl-1, so a group of E / n_group experts
// is exactly LG = 16 / n_group lanes and group scores come from a DPP merge
// over those lanes (no LDS).  Every round of either ranking is a 4-step DPP
// maximum over the row's 16 lanes on order-preserving keys plus one ballot;
// the lowest lane holding the maximum wins, which is the lowest group or
// expert id among equal values.
template <int ctrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __uint_as_float(dpp_u32<ctrl>(__float_as_uint(v)));
}

// Merge the two largest values (m1 >= m2) of this lane and of its DPP partner.
template <int ctrl>
__device__ __forceinline__ void merge_top2(float &m1, float &m2) {
    const float o1 = dpp_f32<ctrl>(m1), o2 = dpp_f32<ctrl>(m2);
    m2 = fmaxf(fminf(m1, o1), fmaxf(m2, o2));
    m1 = fmaxf(m1, o1);
}

// Order-preserving key of a choice score; adding +0.0 first turns -0.0 into
// +0.0, so equal scores get equal keys.  Every float maps above 0.
__device__ __forceinline__ uint32_t choice_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// With MH the kernel also writes the row's [E] multihot, probability and
// position-map entries (the indices->multihot conversion of its selection):
// each lane records the round that picked each of its experts, and the
// probability of a picked expert is its score (kept from the row's load) and
// renormalised exactly as the slot's weight is.  mvec: 16-byte aligned maps
// and VPL % 4 == 0 (vector stores), else scalar stores.
template <int VPL, bool NOAUX, bool MH>
__global__ __launch_bounds__(kGroupedThreads) void route_grouped_rows16_kernel(
    const float *__restrict__ scores, const float *__restrict__ bias, int64_t T, int k,
    int lg_log2, int topk_group, int renorm, int vec, float *__restrict__ topk_w,
    int32_t *__restrict__ topk_ids, uint8_t *__restrict__ multihot, float *__restrict__ pim,
    int32_t *__restrict__ pos, int mvec) {
    constexpr int E = 16 * VPL;
    constexpr int W = VPL % 4 == 0 ? 4 : (VPL % 2 == 0 ? 2 : 1);  // load width
    const int lane = lane_id();
    const int seg = lane >> 4;
    const int q = lane & 15;
    const int e0 = q * VPL;
    const int n_group = 16 >> lg_log2;
    const int my_group = q >> lg_log2;
    const bool mask_groups = topk_group < n_group;

    float b[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) b[i] = NOAUX ? bias[e0 + i] : 0.0f;

    const int64_t wave = (int64_t)blockIdx.x * kGroupedWaves + threadIdx.x / kWave;
    const int64_t nwaves = (int64_t)gridDim.x * kGroupedWaves;
    for (int64_t t0 = wave * 4; t0 < T; t0 += nwaves * 4) {
        const int64_t t = t0 + seg;
        const bool row_ok = t < T;
        const float *row = scores + t * E + e0;
        float c[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) c[i] = 0.0f;
        if (row_ok) {
            if (W > 1 && vec) {  // rows aligned to the load width
#pragma unroll
                for (int j = 0; j < VPL / W; ++j) {
                    if constexpr (W == 4) {
                        const float4 x = reinterpret_cast<const float4 *>(row)[j];
                        c[4 * j] = x.x;
                        c[4 * j + 1] = x.y;
                        c[4 * j + 2] = x.z;
                        c[4 * j + 3] = x.w;
                    } else if constexpr (W == 2) {
                        const float2 x = reinterpret_cast<const float2 *>(row)[j];
                        c[2 * j] = x.x;
                        c[2 * j + 1] = x.y;
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < VPL; ++i) c[i] = row[i];
            }
        }
        uint32_t key[VPL];
        float raw[MH ? VPL : 1];  // the scores themselves, for the maps
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            if (MH) raw[i] = c[i];
            if (NOAUX) c[i] = c[i] + b[i];  // float32 add, as on the page
            key[i] = row_ok ? choice_key(c[i]) : 0u;
        }

        if (mask_groups) {
            // This lane's largest (greedy) or two largest (noaux_tc) choice
            // scores, merged over the LG lanes of its group.
            float m1 = c[0], m2 = -INFINITY;
#pragma unroll
            for (int i = 1; i < VPL; ++i) {
                if (NOAUX) m2 = fmaxf(m2, fminf(m1, c[i]));
                m1 = fmaxf(m1, c[i]);
            }
            if (NOAUX) {
                if (lg_log2 >= 1) merge_top2<kDppXor1>(m1, m2);
                if (lg_log2 >= 2) merge_top2<kDppXor2>(m1, m2);
                if (lg_log2 >= 3) merge_top2<kDppHalfMirror>(m1, m2);
                if (lg_log2 >= 4) merge_top2<kDppMirror>(m1, m2);
            } else {
                if (lg_log2 >= 1) m1 = fmaxf(m1, dpp_f32<kDppXor1>(m1));
                if (lg_log2 >= 2) m1 = fmaxf(m1, dpp_f32<kDppXor2>(m1));
                if (lg_log2 >= 3) m1 = fmaxf(m1, dpp_f32<kDppHalfMirror>(m1));
                if (lg_log2 >= 4) m1 = fmaxf(m1, dpp_f32<kDppMirror>(m1));
            }
            uint32_t gkey = row_ok ? choice_key(NOAUX ? m1 + m2 : m1) : 0u;
            bool kept = false;
            for (int r = 0; r < topk_group; ++r) {
                const uint32_t m = row16_max_u32(gkey);
                const uint64_t cand = __ballot(gkey != 0 && gkey == m);
                const uint32_t bits = (uint32_t)(cand >> (seg * 16)) & 0xFFFFu;
                const int wg = (__ffs((int)bits) - 1) >> lg_log2;  // < 0 past T
                if (bits != 0 && my_group == wg) {
                    gkey = 0;
                    kept = true;
                }
            }
            if (!kept) {
#pragma unroll
                for (int i = 0; i < VPL; ++i) key[i] = 0u;
            }
        }

        int sel_e = -1;
        int pr[VPL];  // round that picked local expert i, -1 if none
#pragma unroll
        for (int i = 0; i < VPL; ++i) pr[i] = -1;
        for (int r = 0; r < k; ++r) {
            // Lane-local best; strict > keeps the lowest local index on ties.
            uint32_t bk = key[0];
            int bi = 0;
#pragma unroll
            for (int i = 1; i < VPL; ++i) {
                if (key[i] > bk) {
                    bk = key[i];
                    bi = i;
                }
            }
            const uint32_t m = row16_max_u32(bk);
            const uint64_t cand = __ballot(bk != 0 && bk == m);
            const uint32_t bits = (uint32_t)(cand >> (seg * 16)) & 0xFFFFu;
            const int wl = __ffs((int)bits) - 1;  // -1 only for rows past T
            const bool is_w = q == wl;
            const uint32_t wbi = row16_max_u32(is_w ? (uint32_t)bi : 0u);
            if (is_w) {
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    if (i == bi) {
                        key[i] = 0u;
                        if (MH) pr[i] = r;
                    }
                }
            }
            if (q == r) sel_e = wl * VPL + (int)wbi;
        }

        // The weight is the score (without the bias) of the selected expert,
        // read back from the row just loaded.
        const bool out = row_ok && q < k;
        float w = 0.0f;
        if (out) w = scores[t * E + sel_e];
        float w_out = w;
        double s = 1.0;
        if (renorm) {
            s = row16_sum_f64(out ? (double)w : 0.0);
            w_out = (float)((double)w / s);
        }
        if (out) {
            topk_w[t * k + q] = w_out;
            topk_ids[t * k + q] = sel_e;
        }
        if (MH && row_ok) {
            float pv[VPL];
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                pv[i] = 0.0f;
                if (pr[i] >= 0) pv[i] = renorm ? (float)((double)raw[i] / s) : raw[i];
            }
            uint8_t *mrow = multihot + t * E + e0;
            float *prow = pim + t * E + e0;
            int32_t *qrow = pos + t * E + e0;
            if constexpr (VPL % 4 == 0) {
                if (mvec) {
#pragma unroll
                    for (int j = 0; j < VPL / 4; ++j) {
                        const uint32_t m = (uint32_t)(pr[4 * j] >= 0) |
                                           (uint32_t)(pr[4 * j + 1] >= 0) << 8 |
                                           (uint32_t)(pr[4 * j + 2] >= 0) << 16 |
                                           (uint32_t)(pr[4 * j + 3] >= 0) << 24;
                        reinterpret_cast<uint32_t *>(mrow)[j] = m;
                        reinterpret_cast<float4 *>(prow)[j] =
                            make_float4(pv[4 * j], pv[4 * j + 1], pv[4 * j + 2], pv[4 * j + 3]);
                        reinterpret_cast<int4 *>(qrow)[j] =
                            make_int4(pr[4 * j], pr[4 * j + 1], pr[4 * j + 2], pr[4 * j + 3]);
                    }
                    continue;
                }
            }
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                mrow[i] = pr[i] >= 0 ? 1 : 0;
                prow[i] = pv[i];
                qrow[i] = pr[i];
            }
        }
    }
}

template <int VPL, bool NOAUX, bool MH>
hipError_t launch_rows16_t(const float *scores, const float *bias, int64_t T, int k,
                           int n_group, int topk_group, int renorm, float *w, int32_t *ids,
                           uint8_t *mh, float *pim, int32_t *pos, hipStream_t s) {
    int64_t blocks = (T + 4 * kGroupedWaves - 1) / (4 * kGroupedWaves);
    if (blocks > 16384) blocks = 16384;
    constexpr int W = VPL % 4 == 0 ? 4 : (VPL % 2 == 0 ? 2 : 1);
    const int vec = (reinterpret_cast<uintptr_t>(scores) & (4u * W - 1)) == 0;
    int lg_log2 = 0;
    while ((16 >> lg_log2) > n_group) ++lg_log2;
    const auto a16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    const int mvec = MH && VPL % 4 == 0 && a16(mh) && a16(pim) && a16(pos);
    hipLaunchKernelGGL((route_grouped_rows16_kernel<VPL, NOAUX, MH>), dim3((unsigned)blocks),
                       dim3(kGroupedThreads), 0, s, scores, bias, T, k, lg_log2, topk_group,
                       renorm, vec, w, ids, mh, pim, pos, mvec);
    return hipGetLastError();
}

template <int VPL>
hipError_t launch_rows16(const float *scores, const float *bias, int64_t T, int E, int k,
                         int n_group, int topk_group, int noaux, int renorm, float *w,
                         int32_t *ids, uint8_t *mh, float *pim, int32_t *pos, hipStream_t s) {
    if (E != 16 * VPL)
        return launch_rows16<VPL + 1>(scores, bias, T, E, k, n_group, topk_group, noaux, renorm,
                                      w, ids, mh, pim, pos, s);
    if (mh != nullptr) {
        if (noaux)
            return launch_rows16_t<VPL, true, true>(scores, bias, T, k, n_group, topk_group,
                                                    renorm, w, ids, mh, pim, pos, s);
        return launch_rows16_t<VPL, false, true>(scores, bias, T, k, n_group, topk_group, renorm,
                                                 w, ids, mh, pim, pos, s);
    }
    if (noaux)
        return launch_rows16_t<VPL, true, false>(scores, bias, T, k, n_group, topk_group, renorm,
                                                 w, ids, nullptr, nullptr, nullptr, s);
    return launch_rows16_t<VPL, false, false>(scores, bias, T, k, n_group, topk_group, renorm, w,
                                              ids, nullptr, nullptr, nullptr, s);
}
template <>
hipError_t launch_rows16<17>(const float *, const float *, int64_t, int, int, int, int, int,
                             int, float *, int32_t *, uint8_t *, float *, int32_t *,
                             hipStream_t) {
    return hipErrorInvalidValue;  // unreachable: E <= 256 is checked by the caller
}

template <int VPL>
hipError_t launch_vpl(const float *scores, const float *bias, int64_t T, int E, int k,
                      int n_group, int topk_group, int noaux, int renorm, float *w, int32_t *ids,
                      hipStream_t s) {
    int64_t blocks = (T + kGroupedWaves - 1) / kGroupedWaves;
    if (blocks > 16384) blocks = 16384;
    const int vec4 = VPL % 4 == 0 && E % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15u) == 0;
    const size_t lds = (size_t)kGroupedWaves * (size_t)E * sizeof(float);
    hipLaunchKernelGGL(route_grouped_kernel<VPL>, dim3((unsigned)blocks), dim3(kGroupedThreads),
                       lds, s, scores, bias, T, E, k, n_group, topk_group, noaux, renorm, vec4, w,
                       ids);
    return hipGetLastError();
}

}  // namespace

bool route_grouped_rows16(int E, int n_group, int k) {
    return E % 16 == 0 && E <= 256 && 16 % n_group == 0 && k <= 16;
}

hipError_t launch_route_grouped(const float *scores, const float *bias, int64_t T, int E, int k,
                                int n_group, int topk_group, int noaux, int renorm, float *w,
                                int32_t *ids, uint8_t *mh, float *pim, int32_t *pos,
                                hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (route_grouped_rows16(E, n_group, k))
        return launch_rows16<1>(scores, bias, T, E, k, n_group, topk_group, noaux, renorm, w, ids,
                                mh, pim, pos, s);
    if (mh != nullptr) {
        const hipError_t err = launch_route_grouped(scores, bias, T, E, k, n_group, topk_group,
                                                    noaux, renorm, w, ids, nullptr, nullptr,
                                                    nullptr, s);
        if (err != hipSuccess) return err;
        return launch_to_multihot(ids, w, T, k, E, mh, pim, pos, s);
    }
    if (E <= 64)
        return launch_vpl<1>(scores, bias, T, E, k, n_group, topk_group, noaux, renorm, w, ids, s);
    if (E <= 128)
        return launch_vpl<2>(scores, bias, T, E, k, n_group, topk_group, noaux, renorm, w, ids, s);
    if (E <= 256)
        return launch_vpl<4>(scores, bias, T, E, k, n_group, topk_group, noaux, renorm, w, ids, s);
    if (E <= 512)
        return launch_vpl<8>(scores, bias, T, E, k, n_group, topk_group, noaux, renorm, w, ids, s);
    return launch_vpl<16>(scores, bias, T, E, k, n_group, topk_group, noaux, renorm, w, ids, s);
}

}  // namespace moe
