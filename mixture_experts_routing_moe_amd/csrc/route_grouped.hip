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
// top-k over that copy, plus a gather for noaux_tc).  Here one wave does a
// whole row in one pass: the row is read once into registers (lane l holds
// experts l*VPL .. l*VPL+VPL-1), the choice scores go to the wave's slice of
// LDS, lane g reduces group g from there, and the group and expert rankings
// are rounds of a cross-lane argmax on order-preserving integer keys.  The
// masked [T, E] copy never exists.
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

hipError_t launch_route_grouped(const float *scores, const float *bias, int64_t T, int E, int k,
                                int n_group, int topk_group, int noaux, int renorm, float *w,
                                int32_t *ids, hipStream_t s) {
    if (T == 0) return hipSuccess;
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
