// Router GEMM + gating top-k in one kernel.
//
// The step before routing: logits = hidden . w_gate^T (a linear gate, W
// stored [E, H] as every weight of this layer is stored [out, in]), then the
// gating top-k of mlc-llm moe_misc.py (gating_topk, gating_softmax_topk) on
// those logits.  The pages take the logits as given; fusing the gate into the
// routing pass means the [T, E] logits are written once (they are an output)
// and never read back.
//
// A block owns MC chunks of 16 tokens and EB blocks of 16 experts.  Its 4
// waves split H into contiguous quarters and feed MFMA 16x16x32 bf16 (gate
// rows as the A operand, tokens as B, fp32 accumulation), batching KB k-steps
// of loads before their MFMAs; the 4 partial sums meet in LDS in a fixed
// order.  Wave 0 writes the logits and an LDS copy of the tile, from which
// all 4 waves route the block's rows with the same 16-lanes-per-row
// selection as moe_route (so the ids and weights are exactly moe_route's on
// these logits).  For E > 64 or k > 16 the kernel only computes logits
// (blocks also split over experts) and moe_route's general kernel selects
// from them.
//
// What bounds it is the bytes each CU loads: besides its token rows, every
// block reads the whole gate matrix (E x H bf16, 256 KB at E = 64, H = 2048)
// from L2, and one CU streams on the order of 40-60 GB/s.  Staging the token
// tile in LDS with direct loads (all of it in flight at once), 8 or 16 waves
// per block, or one 16-token chunk per block all measured slower on the
// part.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;
constexpr int kRouterKB = 4;  // k-steps of 32 per load batch

__device__ __forceinline__ bf16x8 zero_unless(bool keep, bf16x8 v) {
    return keep ? v : bf16x8{};
}

template <int MC, int EB>
__global__ __launch_bounds__(kRouterThreads) void router_route_kernel(
    const uint16_t *__restrict__ hidden, const uint16_t *__restrict__ wg, int64_t T, int H, int E,
    int k, int norm, int do_route, float *__restrict__ logits, float *__restrict__ topk_w,
    int32_t *__restrict__ topk_ids) {
    __shared__ f32x4 red[3][MC][EB][kWave];
    __shared__ float s_log[MC * 16][EB * 16];
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int i = lane & 15;
    const int kq = lane >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * (MC * 16);
    const int e_base = blockIdx.y * (EB * 16);

    // Rows past T or E read a valid row; their results are never stored.
    const uint16_t *xr[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
        const int64_t t = min(t0 + mc * 16 + i, T - 1);
        xr[mc] = hidden + t * H + kq * 8;
    }
    const uint16_t *wr[EB];
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
        const int e = min(e_base + eb * 16 + i, E - 1);
        wr[eb] = wg + (int64_t)e * H + kq * 8;
    }
    f32x4 acc[MC][EB];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc)
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) acc[mc][eb] = f32x4{};

    const int ksteps = H / 32;
    const int per = (ksteps + 3) / 4;
    const int s0 = wave * per;
    const int s1 = min(ksteps, s0 + per);
    for (int s = s0; s < s1; s += kRouterKB) {
        bf16x8 xa[kRouterKB][MC], wa[kRouterKB][EB];
#pragma unroll
        for (int j = 0; j < kRouterKB; ++j) {
            const int ss = min(s + j, s1 - 1) * 32;
#pragma unroll
            for (int mc = 0; mc < MC; ++mc)
                xa[j][mc] = *reinterpret_cast<const bf16x8 *>(xr[mc] + ss);
#pragma unroll
            for (int eb = 0; eb < EB; ++eb)
                wa[j][eb] = *reinterpret_cast<const bf16x8 *>(wr[eb] + ss);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kRouterKB; ++j) {
            const bool in = s + j < s1;
#pragma unroll
            for (int eb = 0; eb < EB; ++eb) {
                const bf16x8 w = zero_unless(in, wa[j][eb]);
#pragma unroll
                for (int mc = 0; mc < MC; ++mc)
                    acc[mc][eb] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, xa[j][mc], acc[mc][eb], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    if (wave > 0) {
#pragma unroll
        for (int mc = 0; mc < MC; ++mc)
#pragma unroll
            for (int eb = 0; eb < EB; ++eb) red[wave - 1][mc][eb][lane] = acc[mc][eb];
    }
    __syncthreads();
    if (wave == 0) {
        // Accumulator r holds expert row 4 kq + r of the block and token column i.
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
            const int tl = mc * 16 + i;
            const int64_t t = t0 + tl;
#pragma unroll
            for (int eb = 0; eb < EB; ++eb) {
                f32x4 a = acc[mc][eb];
#pragma unroll
                for (int w = 0; w < 3; ++w) a += red[w][mc][eb][lane];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int el = eb * 16 + kq * 4 + r;
                    const int e = e_base + el;
                    s_log[tl][el] = a[r];
                    if (t < T && e < E) logits[t * E + e] = a[r];
                }
            }
        }
    }
    if (!do_route) return;  // uniform over the launch
    __syncthreads();

    const int g = lane >> 4;
    const int q = lane & 15;
#pragma unroll
    for (int p = 0; p < MC; ++p) {
        const int rl = p * 16 + wave * 4 + g;
        const int64_t t = t0 + rl;
        float v[4];
        uint32_t avail = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * q + j;
            v[j] = 0.0f;
            if (t < T && e < E) {
                v[j] = s_log[rl][e];
                avail |= 1u << j;
            }
        }
        uint32_t slot_of;
        const float wq = route_row16(v, avail, k, norm, g, q, slot_of);
        if (t < T) {
            if (q < k) topk_w[t * k + q] = wq;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t r = (slot_of >> (8 * j)) & 0xFFu;
                if (r != 0xFFu) topk_ids[t * k + r] = 4 * q + j;
            }
        }
    }
}

template <int MC, int EB>
hipError_t launch_mc_eb(const uint16_t *hidden, const uint16_t *wg, int64_t T, int H, int E,
                        int k, int norm, int do_route, float *logits, float *w, int32_t *ids,
                        hipStream_t s) {
    const int64_t bx = (T + MC * 16 - 1) / (MC * 16);
    const int by = (E + EB * 16 - 1) / (EB * 16);
    hipLaunchKernelGGL((router_route_kernel<MC, EB>), dim3((unsigned)bx, (unsigned)by),
                       dim3(kRouterThreads), 0, s, hidden, wg, T, H, E, k, norm, do_route, logits,
                       w, ids);
    return hipGetLastError();
}

template <int MC>
hipError_t launch_mc(const uint16_t *hidden, const uint16_t *wg, int64_t T, int H, int E, int k,
                     int norm, int do_route, float *logits, float *w, int32_t *ids,
                     hipStream_t s) {
    switch ((min(E, 64) + 15) / 16) {
        case 1: return launch_mc_eb<MC, 1>(hidden, wg, T, H, E, k, norm, do_route, logits, w, ids, s);
        case 2: return launch_mc_eb<MC, 2>(hidden, wg, T, H, E, k, norm, do_route, logits, w, ids, s);
        case 3: return launch_mc_eb<MC, 3>(hidden, wg, T, H, E, k, norm, do_route, logits, w, ids, s);
        default: return launch_mc_eb<MC, 4>(hidden, wg, T, H, E, k, norm, do_route, logits, w, ids, s);
    }
}


// ---------------------------------------------------------------------------
// Backward of the gate (logits = hidden . w_gate^T), float32 arithmetic on
// the bf16 operands: grad_hidden = g . w_gate, grad_w_gate = g^T . hidden with
// g = grad_logits [T, E].  E is small (tens of experts), so these are
// streaming kernels, not matrix-core products.
// ---------------------------------------------------------------------------

constexpr int kBwdTok = 8;      // tokens per grad_hidden block
constexpr int kBwdChunk = 256;  // tokens per grad_w_gate partial plane

__device__ __forceinline__ void unpack8(const uint4 &v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = bf16_bits_to_f32((uint16_t)w[j]);
        f[2 * j + 1] = bf16_bits_to_f32((uint16_t)(w[j] >> 16));
    }
}

// grad_hidden[t][h] = sum over e (ascending) of g[t][e] w_gate[e][h].  Block:
// kBwdTok tokens (their g rows staged in LDS); thread: 8 consecutive h.
__global__ __launch_bounds__(256) void router_dx_kernel(const uint16_t *__restrict__ wg,
                                                        const float *__restrict__ g, int64_t T,
                                                        int H, int E, float *__restrict__ gh) {
    extern __shared__ float sg[];  // [kBwdTok][E]
    const int64_t t0 = (int64_t)blockIdx.x * kBwdTok;
    for (int i = threadIdx.x; i < kBwdTok * E; i += blockDim.x) {
        const int tt = i / E, e = i % E;
        sg[i] = t0 + tt < T ? g[(t0 + tt) * E + e] : 0.f;
    }
    __syncthreads();
    for (int hc = threadIdx.x; hc < H / 8; hc += blockDim.x) {
        float acc[kBwdTok][8];
#pragma unroll
        for (int tt = 0; tt < kBwdTok; ++tt)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[tt][j] = 0.f;
        for (int e = 0; e < E; ++e) {
            float wf[8];
            unpack8(*reinterpret_cast<const uint4 *>(wg + (int64_t)e * H + 8 * hc), wf);
#pragma unroll
            for (int tt = 0; tt < kBwdTok; ++tt) {
                const float ge = sg[tt * E + e];
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[tt][j] = fmaf(ge, wf[j], acc[tt][j]);
            }
        }
#pragma unroll
        for (int tt = 0; tt < kBwdTok; ++tt) {
            if (t0 + tt >= T) break;
            float *o = gh + (t0 + tt) * H + 8 * hc;
            *reinterpret_cast<f32x4 *>(o) = f32x4{acc[tt][0], acc[tt][1], acc[tt][2], acc[tt][3]};
            *reinterpret_cast<f32x4 *>(o + 4) = f32x4{acc[tt][4], acc[tt][5], acc[tt][6], acc[tt][7]};
        }
    }
}

// part[c][e][h] = sum over the tokens t of chunk c (ascending) of
// g[t][e] hidden[t][h].  Block (h block, chunk c): 32 h-chunks of 8 x 8
// groups of 8 experts (groups beyond the eighth loop).
__global__ __launch_bounds__(256) void router_dw_partial_kernel(const uint16_t *__restrict__ x,
                                                                const float *__restrict__ g,
                                                                int64_t T, int H, int E,
                                                                float *__restrict__ part) {
    const int hc = blockIdx.x * 32 + (threadIdx.x & 31);
    if (hc >= H / 8) return;
    const int64_t t0 = (int64_t)blockIdx.y * kBwdChunk;
    const int64_t t1 = min(T, t0 + kBwdChunk);
    for (int eg = threadIdx.x >> 5; eg * 8 < E; eg += 8) {
        float acc[8][8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] = 0.f;
        for (int64_t t = t0; t < t1; ++t) {
            float xf[8];
            unpack8(*reinterpret_cast<const uint4 *>(x + t * H + 8 * hc), xf);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int e = eg * 8 + j;
                const float ge = e < E ? g[t * E + e] : 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[j][i] = fmaf(ge, xf[i], acc[j][i]);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = eg * 8 + j;
            if (e >= E) break;
            float *o = part + ((int64_t)blockIdx.y * E + e) * H + 8 * hc;
            *reinterpret_cast<f32x4 *>(o) = f32x4{acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
            *reinterpret_cast<f32x4 *>(o + 4) = f32x4{acc[j][4], acc[j][5], acc[j][6], acc[j][7]};
        }
    }
}

// grad_w_gate[e][h] = sum over chunks c = 0, 1, ... of part[c][e][h].
__global__ __launch_bounds__(256) void router_dw_sum_kernel(const float *__restrict__ part,
                                                            int nc, int64_t n4,
                                                            float *__restrict__ gw) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    f32x4 acc = reinterpret_cast<const f32x4 *>(part)[i];
    for (int c = 1; c < nc; ++c) acc += reinterpret_cast<const f32x4 *>(part)[(int64_t)c * n4 + i];
    reinterpret_cast<f32x4 *>(gw)[i] = acc;
}
}  // namespace

size_t router_backward_scratch_bytes(int64_t T, int H, int E) {
    const int64_t nc = (T + kBwdChunk - 1) / kBwdChunk;
    return (size_t)nc * E * H * 4;
}

hipError_t launch_router_backward(const uint16_t *hidden, const uint16_t *wg, const float *g,
                                  int64_t T, int H, int E, float *gh, float *gw, void *ws,
                                  hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipError_t err;
    hipLaunchKernelGGL(router_dx_kernel, dim3((unsigned)((T + kBwdTok - 1) / kBwdTok)), dim3(256),
                       kBwdTok * E * sizeof(float), s, wg, g, T, H, E, gh);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int nc = (int)((T + kBwdChunk - 1) / kBwdChunk);
    float *part = static_cast<float *>(ws);
    hipLaunchKernelGGL(router_dw_partial_kernel, dim3((unsigned)((H / 8 + 31) / 32), (unsigned)nc),
                       dim3(256), 0, s, hidden, g, T, H, E, part);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t n4 = (int64_t)E * H / 4;
    hipLaunchKernelGGL(router_dw_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       part, nc, n4, gw);
    return hipGetLastError();
}

hipError_t launch_router_route(const uint16_t *hidden, const uint16_t *wg, int64_t T, int H,
                               int E, int k, int norm, float *logits, float *w, int32_t *ids,
                               hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int fused = E <= 64 && k <= 16;
    // Two 16-token chunks per block (half the gate-matrix reads) once that
    // still gives a block per CU.
    const bool two = T >= 256 * 32;
    const hipError_t err = two ? launch_mc<2>(hidden, wg, T, H, E, k, norm, fused, logits, w, ids, s)
                               : launch_mc<1>(hidden, wg, T, H, E, k, norm, fused, logits, w, ids, s);
    if (err != hipSuccess || fused) return err;
    return launch_route(logits, T, E, k, norm, w, ids, s);
}

}  // namespace moe
