// Internal declarations shared by the libmoe HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

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

// SiLU in float32: z / (1 + e^-z).
__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// ---------------------------------------------------------------------------
// Launchers (each returns hipSuccess or the launch error).
// ---------------------------------------------------------------------------
hipError_t launch_route(const float *logits, int64_t T, int E, int k, int norm, float *w,
                        int32_t *ids, hipStream_t s);

int align_num_blocks(int64_t n_slots, int E);
hipError_t launch_align(const int32_t *ids, int64_t T, int k, int E, int32_t *counts,
                        int32_t *offsets, int32_t *sorted_tok, int32_t *sorted_slot,
                        int32_t *slot_to_sorted, int32_t *ws, hipStream_t s);

hipError_t launch_to_multihot(const int32_t *ids, const float *probs, int64_t T, int k, int E,
                              uint8_t *mh, float *pim, int32_t *pos, hipStream_t s);
hipError_t launch_to_indices(const float *pim, const int32_t *pos, int64_t T, int E, int k,
                             float *probs, int32_t *ids, hipStream_t s);

hipError_t launch_gate_up_bf16(const uint16_t *hidden, const uint16_t *w13,
                               const int32_t *offsets, const int32_t *sorted_tok, int64_t T,
                               int H, int I, int E, int k, uint16_t *act, hipStream_t s);
hipError_t launch_down_bf16(const uint16_t *act, const uint16_t *w2, const int32_t *offsets,
                            int64_t T, int H, int I, int E, int k, float *y, hipStream_t s);

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

hipError_t launch_combine(moe_dtype_t dt, const float *y, const float *w,
                          const int32_t *slot_to_sorted, int64_t T, int H, int k, void *out,
                          hipStream_t s);

}  // namespace moe
