// Gating top-k + softmax weights: one wavefront per token row.
//
// Method: mlc-llm moe_misc.py, gating_topk / _gating_topk_process_value /
// gating_softmax_topk.  The selection order is value descending with equal
// values keeping the lower expert id first (the pages' strict-greater
// insertion over ascending expert ids).  The pages give one thread per row
// with a serial loop over E; here a 64-lane wave holds the row (VPL
// consecutive experts per lane) and runs k rounds of a wave-wide argmax, so
// the row is read once, coalesced, and every round costs six cross-lane max
// steps plus one ballot.
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

hipError_t launch_route(const float *logits, int64_t T, int E, int k, int norm, float *w,
                        int32_t *ids, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (E <= 64) return launch_vpl<1>(logits, T, E, k, norm, w, ids, s);
    if (E <= 128) return launch_vpl<2>(logits, T, E, k, norm, w, ids, s);
    if (E <= 256) return launch_vpl<4>(logits, T, E, k, norm, w, ids, s);
    if (E <= 512) return launch_vpl<8>(logits, T, E, k, norm, w, ids, s);
    return launch_vpl<16>(logits, T, E, k, norm, w, ids, s);
}

}  // namespace moe
