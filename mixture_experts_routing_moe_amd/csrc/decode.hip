// Decode expert FFN (few tokens): weight-streaming kernels.
//
// Method: project_6 moe_expert_gemm.cpp, moe_decode_experts: for each
// selected expert, gate_up = x . w13[e]^T, act = silu(gate) * up,
// y = act . w2[e]^T, then a weighted sum over the token's experts.  The page
// loops over the k experts of one token on the host, reading each id and
// weight back to the host first.  Here the expert set comes from the aligned
// offsets on the device: block row d serves the d-th expert with a non-empty
// segment, so every selected expert's weights are streamed from memory
// exactly once and applied to all tokens routed to it (up to 64), and
// unselected experts are never touched.
//
// Each block owns 16 weight rows (16 gate + 16 up rows for FC1) of one
// expert; its 4 waves split k into contiguous quarters, load their whole
// share of the weight rows up front and feed MFMA 16x16x32 bf16 (weights as
// the A operand, up to 4 chunks of 16 tokens as B; the chunk count follows
// the expert's own row count).  The 4 partial accumulators are summed
// through LDS.
//
// Weight loads come in pairs of k-steps.  The MFMA A operand of one k-step
// gives each of 16 rows 64 bytes (4 lanes x 16), so loading it directly
// makes every instruction touch 16 half cache lines; instead, instruction P
// reads rows 0-7 and instruction Q rows 8-15, each row's whole 128-byte line
// of the pair (lane i of a 16-lane row reads row i & 7, half i >> 3).  The
// two k-steps' operands are then rebuilt in registers: lanes i < 8 take P
// for the first k-step and lane i ^ 8's P for the second, lanes i >= 8 take
// lane i ^ 8's Q for the first and Q for the second (one DPP row rotate by 8
// and a select per dword).  Measured on the part: whole-line reads stream
// from HBM about 25 % faster than half-line reads of the same bytes.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;   // weight rows per block

// The d-th expert (in id order) whose segment is non-empty.
__device__ bool nth_nonempty_expert(const int32_t *__restrict__ offsets, int E, int d, int &e,
                                    int &base, int &cnt) {
    const int lane = lane_id();
    int seen = 0;
    for (int c = 0; c < E; c += kWave) {
        const int ee = c + lane;
        int off = 0, cn = 0;
        if (ee < E) {
            off = offsets[ee];
            cn = offsets[ee + 1] - off;
        }
        const uint64_t nz = __ballot(cn > 0);
        const int pc = __popcll(nz);
        if (d < seen + pc) {
            const int before = __popcll(nz & lanemask_lt());
            const uint64_t sel = __ballot(cn > 0 && before == d - seen);
            const int L = __ffsll((unsigned long long)sel) - 1;
            e = c + L;
            base = readlane_i(off, L);
            cnt = readlane_i(cn, L);
            return true;
        }
        seen += pc;
    }
    return false;
}

// Streamed weight load: read once, so non-temporal.
__device__ __forceinline__ bf16x8 ld_stream(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(p));
}

// Each wave owns a contiguous quarter of the k-step pairs of the block's
// weight rows and issues every load of a batch of kPairs pairs (weights and
// token fragments) before the first MFMA of the batch, so each lane keeps
// kPairs x 32 bytes per weight row group in flight (these kernels are bound
// by HBM).  Pairs past the wave's range load a clamped address and multiply
// a zeroed fragment, so the math carries no branches.
constexpr int kPairs = 4;

__device__ __forceinline__ bf16x8 zero_unless(bool keep, bf16x8 v) {
    return keep ? v : bf16x8{};
}

// The A operands of k-steps 2p and 2p+1 from the paired loads P (rows 0-7)
// and Q (rows 8-15); `lo` = this lane's row is below 8.
__device__ __forceinline__ void unpair(bool lo, const bf16x8 &P, const bf16x8 &Q, bf16x8 &a0,
                                       bf16x8 &a1) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 p = __builtin_bit_cast(u32x4, P), q = __builtin_bit_cast(u32x4, Q);
    u32x4 r0, r1;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t pr = dpp_u32<kDppRor8>(p[d]), qr = dpp_u32<kDppRor8>(q[d]);
        r0[d] = lo ? p[d] : qr;
        r1[d] = lo ? pr : q[d];
    }
    a0 = __builtin_bit_cast(bf16x8, r0);
    a1 = __builtin_bit_cast(bf16x8, r1);
}

// FC1 + SiLU-and-mul.  act[p, n] for n in this block's 16 rows and every
// position p of expert e's segment [base, base + cnt), in MC chunks of 16
// token columns.
template <int MC>
__device__ __forceinline__ void gate_up_rows(const uint16_t *__restrict__ hidden,
                                             const uint16_t *__restrict__ w13,
                                             const int32_t *__restrict__ sorted_tok, int H, int I,
                                             int e, int base, int cnt,
                                             uint16_t *__restrict__ act) {
    __shared__ f32x4 red[3][2][MC][kWave];
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int i = lane & 15;
    const int kq = lane >> 4;
    const int n0 = blockIdx.x * kRows;

    // Paired-load addresses: row (i & 7) of the gate (up) rows 0-7 for P,
    // 8 rows further for Q, half (i >> 3) of each 128-byte line.
    const bool lo = i < 8;
    const uint16_t *wgP = w13 + ((int64_t)e * 2 * I + n0 + (i & 7)) * H + (i >> 3) * 32 + kq * 8;
    const uint16_t *wgQ = wgP + (int64_t)8 * H;
    const uint16_t *wuP = wgP + (int64_t)I * H;
    const uint16_t *wuQ = wuP + (int64_t)8 * H;
    const uint16_t *xr[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
        // Token columns past the segment read a valid row and are never stored.
        const int m = min(mc * 16 + i, cnt - 1);
        xr[mc] = hidden + (int64_t)sorted_tok[base + m] * H + kq * 8;
    }
    f32x4 ag[MC], au[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
        ag[mc] = f32x4{};
        au[mc] = f32x4{};
    }
    const int npairs = H / 64;
    const int per = (npairs + 3) / 4;
    const int p0 = wave * per;
    const int p1 = min(npairs, p0 + per);
    for (int b = p0; b < p1; b += kPairs) {
        bf16x8 gP[kPairs], gQ[kPairs], uP[kPairs], uQ[kPairs], x[MC][2 * kPairs];
#pragma unroll
        for (int q = 0; q < kPairs; ++q) {
            const int k0 = min(b + q, npairs - 1) * 64;
            gP[q] = ld_stream(wgP + k0);
            gQ[q] = ld_stream(wgQ + k0);
            uP[q] = ld_stream(wuP + k0);
            uQ[q] = ld_stream(wuQ + k0);
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) {
                x[mc][2 * q] = *reinterpret_cast<const bf16x8 *>(xr[mc] + k0);
                x[mc][2 * q + 1] = *reinterpret_cast<const bf16x8 *>(xr[mc] + k0 + 32);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < kPairs; ++q) {
            const bool in = b + q < p1;
            bf16x8 g0, g1, u0, u1;
            unpair(lo, zero_unless(in, gP[q]), zero_unless(in, gQ[q]), g0, g1);
            unpair(lo, zero_unless(in, uP[q]), zero_unless(in, uQ[q]), u0, u1);
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) {
                ag[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g0, x[mc][2 * q], ag[mc], 0, 0, 0);
                au[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(u0, x[mc][2 * q], au[mc], 0, 0, 0);
                ag[mc] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(g1, x[mc][2 * q + 1], ag[mc], 0, 0, 0);
                au[mc] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(u1, x[mc][2 * q + 1], au[mc], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (wave > 0) {
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
            red[wave - 1][0][mc][lane] = ag[mc];
            red[wave - 1][1][mc][lane] = au[mc];
        }
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
            ag[mc] += red[w][0][mc][lane];
            au[mc] += red[w][1][mc][lane];
        }
    // Accumulator r holds weight row 4 kq + r and token column i.
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
        const int m = mc * 16 + i;
        if (m >= cnt) continue;
        bf16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = to_bf16(silu_f(ag[mc][r]) * au[mc][r]);
        *reinterpret_cast<bf16x4 *>(act + (int64_t)(base + m) * I + n0 + kq * 4) = o;
    }
}

// FC2.  y[p, h] (float32) for h in this block's 16 rows and every position p
// of expert e's segment, in MC chunks of 16 token columns.  KP pairs per
// batch: 6 for up to 32 tokens (one batch covers each wave's share of
// k = 1408), 4 for more.
template <int MC>
__device__ __forceinline__ void down_rows(const uint16_t *__restrict__ act,
                                          const uint16_t *__restrict__ w2, int H, int I, int e,
                                          int base, int cnt, float *__restrict__ y) {
    constexpr int KP = MC <= 2 ? 6 : 4;
    __shared__ f32x4 red[3][MC][kWave];
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int i = lane & 15;
    const int kq = lane >> 4;
    const int h0 = blockIdx.x * kRows;

    const bool lo = i < 8;
    const uint16_t *wP = w2 + ((int64_t)e * H + h0 + (i & 7)) * I + (i >> 3) * 32 + kq * 8;
    const uint16_t *wQ = wP + (int64_t)8 * I;
    const uint16_t *ar[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
        const int m = min(mc * 16 + i, cnt - 1);
        ar[mc] = act + (int64_t)(base + m) * I + kq * 8;
    }
    f32x4 acc[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) acc[mc] = f32x4{};
    const int npairs = I / 64;
    const int per = (npairs + 3) / 4;
    const int p0 = wave * per;
    const int p1 = min(npairs, p0 + per);
    for (int b = p0; b < p1; b += KP) {
        bf16x8 wPv[KP], wQv[KP], x[MC][2 * KP];
#pragma unroll
        for (int q = 0; q < KP; ++q) {
            const int k0 = min(b + q, npairs - 1) * 64;
            wPv[q] = ld_stream(wP + k0);
            wQv[q] = ld_stream(wQ + k0);
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) {
                x[mc][2 * q] = *reinterpret_cast<const bf16x8 *>(ar[mc] + k0);
                x[mc][2 * q + 1] = *reinterpret_cast<const bf16x8 *>(ar[mc] + k0 + 32);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < KP; ++q) {
            const bool in = b + q < p1;
            bf16x8 w0, w1;
            unpair(lo, zero_unless(in, wPv[q]), zero_unless(in, wQv[q]), w0, w1);
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) {
                acc[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, x[mc][2 * q], acc[mc], 0, 0, 0);
                acc[mc] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, x[mc][2 * q + 1], acc[mc], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (wave > 0) {
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) red[wave - 1][mc][lane] = acc[mc];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) acc[mc] += red[w][mc][lane];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
        const int m = mc * 16 + i;
        if (m >= cnt) continue;
        *reinterpret_cast<float4 *>(y + (int64_t)(base + m) * H + h0 + kq * 4) =
            make_float4(acc[mc][0], acc[mc][1], acc[mc][2], acc[mc][3]);
    }
}

// One block per (16 weight rows, non-empty expert).  The number of 16-token
// chunks is chosen per block from the expert's own row count (at most MCmax,
// which the launch sets from T): with T = 32 most experts hold 16 rows or
// fewer and take the one-chunk path.
template <int MCmax>
__global__ __launch_bounds__(kThreads) void decode_gate_up_kernel(
    const uint16_t *__restrict__ hidden, const uint16_t *__restrict__ w13,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ sorted_tok, int H, int I,
    int E, uint16_t *__restrict__ act) {
    int e, base, cnt;
    if (!nth_nonempty_expert(offsets, E, blockIdx.y, e, base, cnt)) return;
    if (MCmax == 1 || cnt <= 16)
        gate_up_rows<1>(hidden, w13, sorted_tok, H, I, e, base, cnt, act);
    else if (MCmax == 2 || cnt <= 32)
        gate_up_rows<(MCmax > 1 ? 2 : 1)>(hidden, w13, sorted_tok, H, I, e, base, cnt, act);
    else
        gate_up_rows<MCmax>(hidden, w13, sorted_tok, H, I, e, base, cnt, act);
}

template <int MCmax>
__global__ __launch_bounds__(kThreads) void decode_down_kernel(
    const uint16_t *__restrict__ act, const uint16_t *__restrict__ w2,
    const int32_t *__restrict__ offsets, int H, int I, int E, float *__restrict__ y) {
    int e, base, cnt;
    if (!nth_nonempty_expert(offsets, E, blockIdx.y, e, base, cnt)) return;
    if (MCmax == 1 || cnt <= 16)
        down_rows<1>(act, w2, H, I, e, base, cnt, y);
    else if (MCmax == 2 || cnt <= 32)
        down_rows<(MCmax > 1 ? 2 : 1)>(act, w2, H, I, e, base, cnt, y);
    else
        down_rows<MCmax>(act, w2, H, I, e, base, cnt, y);
}

int token_chunks(int64_t T) { return T <= 16 ? 1 : (T <= 32 ? 2 : 4); }

unsigned expert_rows(int64_t T, int E, int k) {
    const int64_t d = T * k < E ? T * k : E;
    return (unsigned)d;
}

}  // namespace

hipError_t launch_decode_gate_up_bf16(const uint16_t *hidden, const uint16_t *w13,
                                      const int32_t *offsets, const int32_t *sorted_tok,
                                      int64_t T, int H, int I, int E, int k, uint16_t *act,
                                      hipStream_t s) {
    if (T == 0) return hipSuccess;
    const dim3 grid(I / kRows, expert_rows(T, E, k));
    switch (token_chunks(T)) {
        case 1:
            hipLaunchKernelGGL(decode_gate_up_kernel<1>, grid, dim3(kThreads), 0, s, hidden, w13,
                               offsets, sorted_tok, H, I, E, act);
            break;
        case 2:
            hipLaunchKernelGGL(decode_gate_up_kernel<2>, grid, dim3(kThreads), 0, s, hidden, w13,
                               offsets, sorted_tok, H, I, E, act);
            break;
        default:
            hipLaunchKernelGGL(decode_gate_up_kernel<4>, grid, dim3(kThreads), 0, s, hidden, w13,
                               offsets, sorted_tok, H, I, E, act);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_decode_down_bf16(const uint16_t *act, const uint16_t *w2,
                                   const int32_t *offsets, int64_t T, int H, int I, int E, int k,
                                   float *y, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const dim3 grid(H / kRows, expert_rows(T, E, k));
    switch (token_chunks(T)) {
        case 1:
            hipLaunchKernelGGL((decode_down_kernel<1>), grid, dim3(kThreads), 0, s, act, w2,
                               offsets, H, I, E, y);
            break;
        case 2:
            hipLaunchKernelGGL((decode_down_kernel<2>), grid, dim3(kThreads), 0, s, act, w2,
                               offsets, H, I, E, y);
            break;
        default:
            hipLaunchKernelGGL((decode_down_kernel<4>), grid, dim3(kThreads), 0, s, act, w2,
                               offsets, H, I, E, y);
            break;
    }
    return hipGetLastError();
}

}  // namespace moe
