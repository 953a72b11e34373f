// Float32 expert FFN over the aligned rows (small layers; no matrix cores).
//
// Method: project_6 moe_expert_gemm.cpp, moe_prefill_experts: for each row p
// of expert e's segment, gate_up = x . w13[e]^T, act = silu(gate) * up,
// y = act . w2[e]^T.  One thread computes one output element with a float32
// dot product; a wave covers 64 consecutive outputs of one row.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Expert whose segment [offsets[e], offsets[e+1]) holds row p: the largest e
// with offsets[e] <= p (empty segments share their offset with the next one).
__device__ int expert_of_row(const int32_t *__restrict__ offsets, int E, int p) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offsets[mid] <= p)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(kThreads) void gate_up_f32_kernel(
    const float *__restrict__ hidden, const float *__restrict__ w13,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ sorted_tok, int H, int I,
    int E, float *__restrict__ act) {
    const int p = blockIdx.x;
    if (p >= offsets[E]) return;
    const int n = blockIdx.y * kThreads + threadIdx.x;
    if (n >= I) return;
    const int e = expert_of_row(offsets, E, p);
    const float *x = hidden + (int64_t)sorted_tok[p] * H;
    const float *wg = w13 + ((int64_t)e * 2 * I + n) * H;
    const float *wu = w13 + ((int64_t)e * 2 * I + I + n) * H;
    float g = 0.0f, u = 0.0f;
    for (int h = 0; h < H; ++h) {
        g = fmaf(x[h], wg[h], g);
        u = fmaf(x[h], wu[h], u);
    }
    act[(int64_t)p * I + n] = g / (1.0f + expf(-g)) * u;
}

__global__ __launch_bounds__(kThreads) void down_f32_kernel(
    const float *__restrict__ act, const float *__restrict__ w2,
    const int32_t *__restrict__ offsets, int H, int I, int E, float *__restrict__ y) {
    const int p = blockIdx.x;
    if (p >= offsets[E]) return;
    const int h = blockIdx.y * kThreads + threadIdx.x;
    if (h >= H) return;
    const int e = expert_of_row(offsets, E, p);
    const float *a = act + (int64_t)p * I;
    const float *w = w2 + ((int64_t)e * H + h) * I;
    float acc = 0.0f;
    for (int i = 0; i < I; ++i) acc = fmaf(a[i], w[i], acc);
    y[(int64_t)p * H + h] = acc;
}

}  // namespace

hipError_t launch_gate_up_f32(const float *hidden, const float *w13, const int32_t *offsets,
                              const int32_t *sorted_tok, int64_t T, int H, int I, int E, int k,
                              float *act, hipStream_t s) {
    const int64_t rows = T * k;
    if (rows == 0) return hipSuccess;
    dim3 grid((unsigned)rows, (I + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(gate_up_f32_kernel, grid, dim3(kThreads), 0, s, hidden, w13, offsets,
                       sorted_tok, H, I, E, act);
    return hipGetLastError();
}

hipError_t launch_down_f32(const float *act, const float *w2, const int32_t *offsets, int64_t T,
                           int H, int I, int E, int k, float *y, hipStream_t s) {
    const int64_t rows = T * k;
    if (rows == 0) return hipSuccess;
    dim3 grid((unsigned)rows, (H + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(down_f32_kernel, grid, dim3(kThreads), 0, s, act, w2, offsets, H, I, E,
                       y);
    return hipGetLastError();
}

}  // namespace moe
