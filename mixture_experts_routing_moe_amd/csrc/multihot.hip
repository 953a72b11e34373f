// [T,k] routing <-> [T,E] multihot / probability / position-map conversion.
//
// Method: Megatron-LM fused_indices_converter.py, _indices_to_multihot_kernel
// and _multihot_to_indices_kernel.  The pages run one program per row that
// first initialises the row, waits on a barrier, then scatters the k entries.
// Here one wavefront owns a row with one lane per expert column (64 columns
// per pass), so every output element is written exactly once by its owner:
// no initialisation pass, no barrier, and every store is coalesced.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Lane e of the wave decides column e: which of the k slots (if any) named e.
__global__ __launch_bounds__(kThreads) void to_multihot_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ probs, int64_t T, int k, int E,
    uint8_t *__restrict__ multihot, float *__restrict__ pim, int32_t *__restrict__ pos) {
    const int lane = lane_id();
    const int64_t wave = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
    const int64_t nwaves = (int64_t)gridDim.x * (kThreads / kWave);
    for (int64_t t = wave; t < T; t += nwaves) {
        int my_id = -1;
        float my_p = 0.0f;
        if (lane < k) {
            my_id = ids[t * k + lane];
            my_p = probs[t * k + lane];
        }
        for (int c = 0; c < E; c += kWave) {
            const int e = c + lane;
            int pj = -1;
            float pv = 0.0f;
            for (int j = 0; j < k; ++j) {  // later slots win, as a sequential scatter
                const int idj = readlane_i(my_id, j);
                const float vj = readlane_f(my_p, j);
                if (idj == e) {
                    pj = j;
                    pv = vj;
                }
            }
            if (e < E) {
                multihot[t * E + e] = pj >= 0 ? 1 : 0;
                pim[t * E + e] = pv;
                pos[t * E + e] = pj;
            }
        }
    }
}

// Lane j of the wave produces slot j; each slot finds the expert naming it
// with one ballot per 64 experts.
__global__ __launch_bounds__(kThreads) void to_indices_kernel(
    const float *__restrict__ pim, const int32_t *__restrict__ pos, int64_t T, int E, int k,
    float *__restrict__ probs, int32_t *__restrict__ ids) {
    const int lane = lane_id();
    const int64_t wave = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
    const int64_t nwaves = (int64_t)gridDim.x * (kThreads / kWave);
    for (int64_t t = wave; t < T; t += nwaves) {
        float outp = 0.0f;
        int outid = -1;
        for (int c = 0; c < E; c += kWave) {
            const int e = c + lane;
            int p = -1;
            float v = 0.0f;
            if (e < E) {
                p = pos[t * E + e];
                v = pim[t * E + e];
            }
            for (int j = 0; j < k; ++j) {
                const uint64_t m = __ballot(p == j);
                if (m) {  // highest expert naming slot j wins
                    const int src = 63 - __clzll((long long)m);
                    const float vv = readlane_f(v, src);
                    if (lane == j) {
                        outp = vv;
                        outid = c + src;
                    }
                }
            }
        }
        if (lane < k) {
            probs[t * k + lane] = outp;
            if (ids) ids[t * k + lane] = outid;
        }
    }
}

unsigned grid_for_rows(int64_t T) {
    int64_t b = (T + kThreads / kWave - 1) / (kThreads / kWave);
    if (b > 8192) b = 8192;
    if (b < 1) b = 1;
    return (unsigned)b;
}

}  // namespace

hipError_t launch_to_multihot(const int32_t *ids, const float *probs, int64_t T, int k, int E,
                              uint8_t *mh, float *pim, int32_t *pos, hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(to_multihot_kernel, dim3(grid_for_rows(T)), dim3(kThreads), 0, s, ids,
                       probs, T, k, E, mh, pim, pos);
    return hipGetLastError();
}

hipError_t launch_to_indices(const float *pim, const int32_t *pos, int64_t T, int E, int k,
                             float *probs, int32_t *ids, hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(to_indices_kernel, dim3(grid_for_rows(T)), dim3(kThreads), 0, s, pim,
                       pos, T, E, k, probs, ids);
    return hipGetLastError();
}

}  // namespace moe
