// Gating top-k + softmax weights: 16 lanes (E <= 64, k <= 16) or a whole
// wavefront per token row.
//
// Method: mlc-llm moe_misc.py, gating_topk / _gating_topk_process_value /
// gating_softmax_topk.  The selection order is value descending with equal
// values keeping the lower expert id first (the pages' strict-greater
// insertion over ascending expert ids).  The pages give one thread per row
// with a serial loop over E; here lanes hold consecutive experts of a row and
// run k rounds of a cross-lane argmax, so the row is read once, coalesced.
// The general kernel gives a row a whole wave (VPL experts per lane); the fast
// path packs 4 rows into a wave with 16 lanes per row and DPP reductions.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;

template <int VPL>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const float *__restrict__ logits, int64_t T, int E, int k, int norm,
    float *__restrict__ topk_w, int32_t *__restrict__ topk_ids) {
    const int lane = lane_id();
    const int64_t wave = (int64_t)blockIdx.x * (kRouteThreads / kWave) + threadIdx.x / kWave;
    const int64_t nwaves = (int64_t)gridDim.x * (kRouteThreads / kWave);

    for (int64_t t = wave; t < T; t += nwaves) {
        const float *row = logits + t * E;
        float v[VPL];
        uint32_t avail = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = lane * VPL + i;
            if (e < E) {
                v[i] = row[e];
                avail |= 1u << i;
            } else {
                v[i] = -INFINITY;
            }
        }
        const uint32_t valid = avail;

        float sel_v = 0.0f, vmax = 0.0f;
        int sel_i = -1;
        for (int r = 0; r < k; ++r) {
            // Lane-local best of the remaining experts; strict > keeps the
            // lowest local index among equal values.
            float bv = -INFINITY;
            int bi = -1;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                if (((avail >> i) & 1u) && (bi < 0 || v[i] > bv)) {
                    bv = v[i];
                    bi = i;
                }
            }
            const float m = wave_max_f(bi >= 0 ? bv : -INFINITY);
            // Lanes own ascending id blocks, so the lowest candidate lane
            // holds the lowest id among the maxima.
            const uint64_t cand = __ballot(bi >= 0 && bv == m);
            const int L = __ffsll((unsigned long long)cand) - 1;
            const int wi = readlane_i(bi, L);
            if (lane == L) avail &= ~(1u << bi);
            if (lane == r) {
                sel_v = m;
                sel_i = L * VPL + wi;
            }
            if (r == 0) vmax = m;
        }

        // Weights in double, rounded once to float: exact to the last bit
        // of float for any spread of logits.
        const double mx = (double)vmax;
        const double ex = lane < k ? exp((double)sel_v - mx) : 0.0;
        double part;
        if (norm) {
            part = ex;
        } else {
            part = 0.0;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if ((valid >> i) & 1u) part += exp((double)v[i] - mx);
        }
        const double s = wave_sum_d(part);
        if (lane < k) {
            topk_w[t * k + lane] = (float)(ex / s);
            topk_ids[t * k + lane] = sel_i;
        }
    }
}

// Fast path for E <= 64 and k <= 16: a wave holds 4 rows, 16 lanes per row,
// lane q of a row holding experts 4q .. 4q+3.  Every round of the top-k is a
// 4-step DPP max over the row's 16 lanes on an order-preserving unsigned key
// plus one ballot; the lowest lane holding the maximum wins, which is the
// lowest expert id among equal logits.  The lane that owns a picked expert
// writes its id; lane j computes and writes slot j's weight.
//
// With multihot != nullptr (E % 4 == 0, 16-byte aligned rows) the same pass
// also writes the row's [E] multihot, probability and position-map entries
// (the indices->multihot conversion of the selection just made): each lane
// records which round picked each of its 4 experts, fetches that slot's
// weight from the lane that computed it, and writes its 4 columns, so the
// conversion costs no second read of the ids and weights and no launch.
__global__ __launch_bounds__(kRouteThreads) void route_rows16_kernel(
    const float *__restrict__ logits, int64_t T, int E, int k, int norm, int vec4,
    float *__restrict__ topk_w, int32_t *__restrict__ topk_ids, uint8_t *__restrict__ multihot,
    float *__restrict__ pim, int32_t *__restrict__ pos) {
    const int lane = lane_id();
    const int g = lane >> 4;
    const int q = lane & 15;
    const int64_t wave = (int64_t)blockIdx.x * (kRouteThreads / kWave) + threadIdx.x / kWave;
    const int64_t nwaves = (int64_t)gridDim.x * (kRouteThreads / kWave);

    for (int64_t t0 = wave * 4; t0 < T; t0 += nwaves * 4)
        route16_row(logits, T, t0 + g, E, k, norm, vec4, topk_w, topk_ids, multihot, pim, pos, g,
                    q);
}

template <int VPL>
hipError_t launch_vpl(const float *logits, int64_t T, int E, int k, int norm, float *w,
                      int32_t *ids, hipStream_t s) {
    const int64_t waves_per_block = kRouteThreads / kWave;
    int64_t blocks = (T + waves_per_block - 1) / waves_per_block;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(route_kernel<VPL>, dim3((unsigned)blocks), dim3(kRouteThreads), 0, s,
                       logits, T, E, k, norm, w, ids);
    return hipGetLastError();
}

}  // namespace

namespace {

hipError_t launch_rows16(const float *logits, int64_t T, int E, int k, int norm, float *w,
                         int32_t *ids, uint8_t *mh, float *pim, int32_t *pos, hipStream_t s) {
    int64_t blocks = (T + 15) / 16;  // 4 waves x 4 rows per block
    if (blocks > 8192) blocks = 8192;
    const int vec4 = E == 64 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0;
    hipLaunchKernelGGL(route_rows16_kernel, dim3((unsigned)blocks), dim3(kRouteThreads), 0, s,
                       logits, T, E, k, norm, vec4, w, ids, mh, pim, pos);
    return hipGetLastError();
}

}  // namespace

bool route_multihot_fused(int E, int k, const uint8_t *mh, const float *pim,
                          const int32_t *pos) {
    const auto a16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    return E <= 64 && E % 4 == 0 && k <= 16 && a16(pim) && a16(pos) &&
           (reinterpret_cast<uintptr_t>(mh) & 3u) == 0;
}

hipError_t launch_route_multihot(const float *logits, int64_t T, int E, int k, int norm,
                                 float *w, int32_t *ids, uint8_t *mh, float *pim, int32_t *pos,
                                 hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (route_multihot_fused(E, k, mh, pim, pos))
        return launch_rows16(logits, T, E, k, norm, w, ids, mh, pim, pos, s);
    const hipError_t err = launch_route(logits, T, E, k, norm, w, ids, s);
    if (err != hipSuccess) return err;
    return launch_to_multihot(ids, w, T, k, E, mh, pim, pos, s);
}

hipError_t launch_route(const float *logits, int64_t T, int E, int k, int norm, float *w,
                        int32_t *ids, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (E <= 64 && k <= 16)
        return launch_rows16(logits, T, E, k, norm, w, ids, nullptr, nullptr, nullptr, s);
    if (E <= 64) return launch_vpl<1>(logits, T, E, k, norm, w, ids, s);
    if (E <= 128) return launch_vpl<2>(logits, T, E, k, norm, w, ids, s);
    if (E <= 256) return launch_vpl<4>(logits, T, E, k, norm, w, ids, s);
    if (E <= 512) return launch_vpl<8>(logits, T, E, k, norm, w, ids, s);
    return launch_vpl<16>(logits, T, E, k, norm, w, ids, s);
}

}  // namespace moe
