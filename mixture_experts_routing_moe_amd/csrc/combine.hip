// Weighted combine back to token order.
//
// Method: project_6 moe_expert_gemm.cpp, moe_prefill_experts (scale each
// expert output by its routing weight and add it into the token's row) and
// mlc-llm moe_misc.py scatter_output + moe_sum (un-permute, then sum the k
// expert outputs of a token).  Instead of a scatter-add, each token row
// gathers its k expert rows through the inverse map and sums them in slot
// order j = 0..k-1 in float32: one rounding at the end, no atomics, the same
// bits on every run.  When the FC2 product was cut into K slices, y holds one
// partial plane per slice and each expert row is first summed over the planes
// in slice order.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <typename T>
struct Vec;
constexpr int V = 8;  // columns per thread: 32 bytes of y

__device__ __forceinline__ void store8(uint16_t *p, const float *f) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = to_bf16(f[i]);
    *reinterpret_cast<bf16x8 *>(p) = v;
}
__device__ __forceinline__ void store8(float *p, const float *f) {
    reinterpret_cast<float4 *>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}

// y is float32 [splits, rows, H]; out is bf16 (uint16_t) or float32 [T, H].
// The k slots of a token are taken in batches of KB: every load of a batch
// is issued before the first is used, so a token costs one memory round
// trip per batch instead of one per slot (what bounds a decode batch, where
// a handful of blocks have nothing else to overlap).  The sums run in the
// same order as slot by slot: planes in plane order, then slots in slot
// order.
template <typename OutT>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const float *__restrict__ y, int splits, int64_t plane, const float *__restrict__ w,
    const int32_t *__restrict__ s2s, int64_t ntok, int H, int k, OutT *__restrict__ out) {
    constexpr int KB = 8;
    for (int64_t t = blockIdx.x; t < ntok; t += gridDim.x) {
        for (int h = threadIdx.x * V; h < H; h += kThreads * V) {
            float acc[V];
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] = 0.0f;
            for (int j0 = 0; j0 < k; j0 += KB) {
                int p[KB];
                float wj[KB];
                float4 lo[KB], hi[KB];
#pragma unroll
                for (int jj = 0; jj < KB; ++jj) {
                    const int j = j0 + jj;
                    p[jj] = j < k ? s2s[t * k + j] : -1;
                    wj[jj] = j < k ? w[t * k + j] : 0.0f;
                }
#pragma unroll
                for (int jj = 0; jj < KB; ++jj) {
                    lo[jj] = hi[jj] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (p[jj] >= 0) {
                        const float4 *src =
                            reinterpret_cast<const float4 *>(y + (int64_t)p[jj] * H + h);
                        lo[jj] = src[0];
                        hi[jj] = src[1];
                    }
                }
#pragma unroll
                for (int jj = 0; jj < KB; ++jj) {
                    if (p[jj] < 0) continue;
                    float v[V] = {lo[jj].x, lo[jj].y, lo[jj].z, lo[jj].w,
                                  hi[jj].x, hi[jj].y, hi[jj].z, hi[jj].w};
                    for (int sp = 1; sp < splits; ++sp) {
                        const float4 *q = reinterpret_cast<const float4 *>(
                            y + sp * plane + (int64_t)p[jj] * H + h);
                        const float4 c = q[0], d = q[1];
                        const float u[V] = {c.x, c.y, c.z, c.w, d.x, d.y, d.z, d.w};
#pragma unroll
                        for (int i = 0; i < V; ++i) v[i] += u[i];
                    }
#pragma unroll
                    for (int i = 0; i < V; ++i) acc[i] = fmaf(wj[jj], v[i], acc[i]);
                }
            }
            store8(out + t * H + h, acc);
        }
    }
}

}  // namespace

hipError_t launch_combine(moe_dtype_t dt, const float *y, int splits, const float *w,
                          const int32_t *slot_to_sorted, int64_t T, int H, int k, void *out,
                          hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int64_t plane = T * k * H;
    const unsigned grid = (unsigned)(T < 65536 ? T : 65536);
    if (dt == MOE_BF16) {
        hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, s, y, splits,
                           plane, w, slot_to_sorted, T, H, k, static_cast<uint16_t *>(out));
    } else {
        hipLaunchKernelGGL(combine_kernel<float>, dim3(grid), dim3(kThreads), 0, s, y, splits,
                           plane, w, slot_to_sorted, T, H, k, static_cast<float *>(out));
    }
    return hipGetLastError();
}

}  // namespace moe
