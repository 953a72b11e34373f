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

// FC1 + SiLU-and-mul.  act[p, n] for n in this block's RT x 16 rows and
// every position p of expert e's segment [base, base + cnt), in MC chunks of
// 16 token columns.  Two row tiles per block (from 16 tokens on) read the
// token rows once for 32 gate and 32 up rows; they take batches of 2 pairs
// instead of kPairs to stay within the registers.
template <int MC, int RT>
__device__ __forceinline__ void gate_up_rows(const uint16_t *__restrict__ hidden,
                                             const uint16_t *__restrict__ w13,
                                             const int32_t *__restrict__ sorted_tok, int H, int I,
                                             int e, int base, int cnt,
                                             uint16_t *__restrict__ act) {
    constexpr int KP = RT == 1 ? kPairs : 2;
    __shared__ f32x4 red[3][2][RT][MC][kWave];
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int i = lane & 15;
    const int kq = lane >> 4;
    const int n0 = blockIdx.x * kRows * RT;

    // Paired-load addresses: row (i & 7) of the gate (up) rows 0-7 for P,
    // 8 rows further for Q, half (i >> 3) of each 128-byte line.
    const bool lo = i < 8;
    const uint16_t *wgP[RT], *wgQ[RT], *wuP[RT], *wuQ[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        wgP[rt] = w13 + ((int64_t)e * 2 * I + n0 + rt * kRows + (i & 7)) * H + (i >> 3) * 32 +
                  kq * 8;
        wgQ[rt] = wgP[rt] + (int64_t)8 * H;
        wuP[rt] = wgP[rt] + (int64_t)I * H;
        wuQ[rt] = wuP[rt] + (int64_t)8 * H;
    }
    const uint16_t *xr[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
        // Token columns past the segment read a valid row and are never stored.
        const int m = min(mc * 16 + i, cnt - 1);
        xr[mc] = hidden + (int64_t)sorted_tok[base + m] * H + kq * 8;
    }
    f32x4 ag[RT][MC], au[RT][MC];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
            ag[rt][mc] = f32x4{};
            au[rt][mc] = f32x4{};
        }
    const int npairs = H / 64;
    const int per = (npairs + 3) / 4;
    const int p0 = wave * per;
    const int p1 = min(npairs, p0 + per);
    for (int b = p0; b < p1; b += KP) {
        bf16x8 gP[RT][KP], gQ[RT][KP], uP[RT][KP], uQ[RT][KP], x[MC][2 * KP];
#pragma unroll
        for (int q = 0; q < KP; ++q) {
            const int k0 = min(b + q, npairs - 1) * 64;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                gP[rt][q] = ld_stream(wgP[rt] + k0);
                gQ[rt][q] = ld_stream(wgQ[rt] + k0);
                uP[rt][q] = ld_stream(wuP[rt] + k0);
                uQ[rt][q] = ld_stream(wuQ[rt] + k0);
            }
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) {
                x[mc][2 * q] = *reinterpret_cast<const bf16x8 *>(xr[mc] + k0);
                x[mc][2 * q + 1] = *reinterpret_cast<const bf16x8 *>(xr[mc] + k0 + 32);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < KP; ++q) {
            const bool in = b + q < p1;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                bf16x8 g0, g1, u0, u1;
                unpair(lo, zero_unless(in, gP[rt][q]), zero_unless(in, gQ[rt][q]), g0, g1);
                unpair(lo, zero_unless(in, uP[rt][q]), zero_unless(in, uQ[rt][q]), u0, u1);
#pragma unroll
                for (int mc = 0; mc < MC; ++mc) {
                    ag[rt][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g0, x[mc][2 * q],
                                                                        ag[rt][mc], 0, 0, 0);
                    au[rt][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(u0, x[mc][2 * q],
                                                                        au[rt][mc], 0, 0, 0);
                    ag[rt][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g1, x[mc][2 * q + 1],
                                                                        ag[rt][mc], 0, 0, 0);
                    au[rt][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(u1, x[mc][2 * q + 1],
                                                                        au[rt][mc], 0, 0, 0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (wave > 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) {
                red[wave - 1][0][rt][mc][lane] = ag[rt][mc];
                red[wave - 1][1][rt][mc][lane] = au[rt][mc];
            }
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) {
                ag[rt][mc] += red[w][0][rt][mc][lane];
                au[rt][mc] += red[w][1][rt][mc][lane];
            }
    // Accumulator r holds weight row 4 kq + r and token column i.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
            const int m = mc * 16 + i;
            if (m >= cnt) continue;
            bf16x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                o[r] = to_bf16(silu_f(ag[rt][mc][r]) * au[rt][mc][r]);
            *reinterpret_cast<bf16x4 *>(act + (int64_t)(base + m) * I + n0 + rt * kRows +
                                        kq * 4) = o;
        }
    }
}

// FC2.  y[p, h] (float32) for h in this block's RT x 16 rows and every
// position p of expert e's segment, in MC chunks of 16 token columns.  KP
// pairs per batch: with one row tile, 6 for up to 32 tokens (one batch covers
// each wave's share of k = 1408), 4 for more; with two row tiles 3, with four
// 2.  Several row tiles per block (from 16 tokens on: four up to 32 tokens,
// two past that, where four token chunks leave registers for two) read the
// expert's activation rows once for 64 or 32 weight rows: at T = 32 those
// rows are otherwise close to half of a block's bytes.
template <int MC, int RT>
__device__ __forceinline__ void down_rows(const uint16_t *__restrict__ act,
                                          const uint16_t *__restrict__ w2, int H, int I, int e,
                                          int base, int cnt, float *__restrict__ y) {
    constexpr int KP = RT == 1 ? (MC <= 2 ? 6 : 4) : (RT == 2 ? 3 : 2);
    __shared__ f32x4 red[3][RT][MC][kWave];
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int i = lane & 15;
    const int kq = lane >> 4;
    const int h0 = blockIdx.x * kRows * RT;

    const bool lo = i < 8;
    const uint16_t *wP[RT], *wQ[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        wP[rt] = w2 + ((int64_t)e * H + h0 + rt * kRows + (i & 7)) * I + (i >> 3) * 32 + kq * 8;
        wQ[rt] = wP[rt] + (int64_t)8 * I;
    }
    const uint16_t *ar[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
        const int m = min(mc * 16 + i, cnt - 1);
        ar[mc] = act + (int64_t)(base + m) * I + kq * 8;
    }
    f32x4 acc[RT][MC];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) acc[rt][mc] = f32x4{};
    const int npairs = I / 64;
    const int per = (npairs + 3) / 4;
    const int p0 = wave * per;
    const int p1 = min(npairs, p0 + per);
    for (int b = p0; b < p1; b += KP) {
        bf16x8 wPv[RT][KP], wQv[RT][KP], x[MC][2 * KP];
#pragma unroll
        for (int q = 0; q < KP; ++q) {
            const int k0 = min(b + q, npairs - 1) * 64;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                wPv[rt][q] = ld_stream(wP[rt] + k0);
                wQv[rt][q] = ld_stream(wQ[rt] + k0);
            }
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
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                bf16x8 w0, w1;
                unpair(lo, zero_unless(in, wPv[rt][q]), zero_unless(in, wQv[rt][q]), w0, w1);
#pragma unroll
                for (int mc = 0; mc < MC; ++mc) {
                    acc[rt][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, x[mc][2 * q],
                                                                         acc[rt][mc], 0, 0, 0);
                    acc[rt][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, x[mc][2 * q + 1],
                                                                         acc[rt][mc], 0, 0, 0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (wave > 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) red[wave - 1][rt][mc][lane] = acc[rt][mc];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) acc[rt][mc] += red[w][rt][mc][lane];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
            const int m = mc * 16 + i;
            if (m >= cnt) continue;
            *reinterpret_cast<float4 *>(y + (int64_t)(base + m) * H + h0 + rt * kRows + kq * 4) =
                make_float4(acc[rt][mc][0], acc[rt][mc][1], acc[rt][mc][2], acc[rt][mc][3]);
        }
    }
}

// One block per (16 weight rows, non-empty expert).  The number of 16-token
// chunks is chosen per block from the expert's own row count (at most MCmax,
// which the launch sets from T): with T = 32 most experts hold 16 rows or
// fewer and take the one-chunk path.
template <int MCmax, int RT>
__global__ __launch_bounds__(kThreads) void decode_gate_up_kernel(
    const uint16_t *__restrict__ hidden, const uint16_t *__restrict__ w13,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ sorted_tok, int H, int I,
    int E, uint16_t *__restrict__ act) {
    int e, base, cnt;
    if (!nth_nonempty_expert(offsets, E, blockIdx.y, e, base, cnt)) return;
    if (MCmax == 1 || cnt <= 16)
        gate_up_rows<1, RT>(hidden, w13, sorted_tok, H, I, e, base, cnt, act);
    else if (MCmax == 2 || cnt <= 32)
        gate_up_rows<(MCmax > 1 ? 2 : 1), RT>(hidden, w13, sorted_tok, H, I, e, base, cnt, act);
    else
        gate_up_rows<MCmax, RT>(hidden, w13, sorted_tok, H, I, e, base, cnt, act);
}

// Route + align + FC1 in one launch for the smallest decode batches (T k <=
// kRouteGateUpSlots, E <= 64, k <= 16): every block routes the batch's rows
// itself (route16_row, the moe_route selection; wave w takes rows 4w .. 4w +
// 3) and aligns them (align_slots_wave, the moe_align order) in LDS, then
// runs FC1 for the blockIdx.y-th non-empty expert from the LDS copy of the
// aligned token ids, so no block waits for another launch's writes.  Block
// (0, 0) also writes every routing output (weights, ids, the multihot maps
// when given, the alignment) and, after its FC1 rows, converts the maps back
// to indices: the outputs of moe_route_align(_inverse) bit for bit.
__global__ __launch_bounds__(kThreads) void decode_route_gate_up_kernel(
    const float *__restrict__ logits, int T, int E, int k, int norm, int vec4, int nbits,
    float *__restrict__ topk_w, int32_t *__restrict__ topk_ids, uint8_t *__restrict__ multihot,
    float *__restrict__ pim, int32_t *__restrict__ pos, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_tok,
    int32_t *__restrict__ sorted_slot, int32_t *__restrict__ slot_to_sorted,
    float *__restrict__ inv_w, int32_t *__restrict__ inv_ids, const uint16_t *__restrict__ hidden,
    const uint16_t *__restrict__ w13, int H, int I, uint16_t *__restrict__ act) {
    __shared__ int32_t s_ids[kWave];
    __shared__ int32_t s_cnt[kWave];
    __shared__ int32_t s_off[kWave + 1];
    __shared__ int32_t s_tok[kWave];
    __shared__ float s_w[kWave];     // weights and ids of the blocks that do not
    __shared__ int32_t s_tid[kWave];  // write them out
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int g = lane >> 4;
    const int q = lane & 15;
    const int n = T * k;
    const bool writer = blockIdx.x == 0 && blockIdx.y == 0;
    if (threadIdx.x < kWave) {
        s_ids[lane] = -1;
        s_cnt[lane] = 0;
    }
    __syncthreads();
    const int t = 4 * wave + g;  // T <= 16 (T k <= 16): one row per 16-lane group
    const uint32_t slot_of =
        route16_row(logits, T, t, E, k, norm, vec4, writer ? topk_w : s_w,
                    writer ? topk_ids : s_tid, writer ? multihot : nullptr, pim, pos, g, q);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t r = (slot_of >> (8 * i)) & 0xFFu;
        if (r != 0xFFu) s_ids[t * k + (int)r] = 4 * q + i;
    }
    __syncthreads();
    if (wave == 0)
        align_slots_wave(s_ids, n, k, E, nbits, s_cnt, s_off, writer ? counts : nullptr, offsets,
                         sorted_tok, sorted_slot, slot_to_sorted, s_tok);
    __syncthreads();
    int e, base, cnt;
    if (nth_nonempty_expert(s_off, E, blockIdx.y, e, base, cnt))
        gate_up_rows<1, 1>(hidden, w13, s_tok, H, I, e, base, cnt, act);
    // With inv_w: block (0, 0) converts the maps it wrote back to indices.
    if (writer && inv_w != nullptr) {
        __syncthreads();
        to_indices_row16<4>(pim, pos, T, t, E, k, inv_w, inv_ids, q);
    }
}

// One block per (RT x 16 weight rows, non-empty expert).
template <int MCmax, int RT>
__global__ __launch_bounds__(kThreads) void decode_down_kernel(
    const uint16_t *__restrict__ act, const uint16_t *__restrict__ w2,
    const int32_t *__restrict__ offsets, int H, int I, int E, float *__restrict__ y) {
    int e, base, cnt;
    if (!nth_nonempty_expert(offsets, E, blockIdx.y, e, base, cnt)) return;
    if (MCmax == 1 || cnt <= 16)
        down_rows<1, RT>(act, w2, H, I, e, base, cnt, y);
    else if (MCmax == 2 || cnt <= 32)
        down_rows<(MCmax > 1 ? 2 : 1), RT>(act, w2, H, I, e, base, cnt, y);
    else
        down_rows<MCmax, RT>(act, w2, H, I, e, base, cnt, y);
}

// FC2 and the combine in one launch, for the smallest batches (at most
// kFusedSlots routing slots, I <= 64 kFusedPairs): block b owns output
// columns [8 b, 8 b + 8) of every token, and wave w takes the non-empty
// experts w, w + 8, ... in id order.  Each wave finds its first expert,
// issues its first activation-chunk loads, then all of that expert's
// weight loads (the 8 rows' whole lines, one 16-byte piece per lane per
// 64-wide k-step pair; rows 8-15 of the MFMA operand are zero); the block
// stages the activation rows in LDS (row pitch I + 8, so the 16 token
// columns' reads fall on distinct banks) and meets at a barrier that waits
// for LDS only, so the products start as the first pairs land.  Pair j's
// registers are refilled with the next expert's pair j as soon as they are
// consumed.  The k-steps are summed in the four quarters decode_down_kernel's
// four waves take, in the same order, and the quarter sums are added in that
// kernel's order (its batching only appends zero terms), so each y value is
// that kernel's bit pattern; y goes to LDS, and the block sums each token's
// k slots in slot order as combine_kernel does (fmaf, one rounding to bf16),
// so `out` equals the two launches' for finite activations.
constexpr int kFusedSlots = 32;
constexpr int kFusedPairs = 24;
constexpr int kFusedRows = 8;
constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = kFusedWaves * kWave;
constexpr int kStageLoads = 4;  // activation chunks per thread loaded ahead of the weights

__device__ __forceinline__ int fused_pitch(int I) { return I + 8; }

// One expert's products for the fused kernel: quarters of PER k-step pairs
// (w = 0..3 covers pairs [w PER, w PER + PER) clipped to npairs; steps past
// the last pair multiply zero weights, which adds exact zeros), quarter
// sums added in order.  kTwo: a second block of token columns (16-31).
// kRefill: each step reloads its pair's registers from wn (the next expert).
// Straight-line code, so every wait counts the loads in flight exactly.
template <int PER, bool kTwo, bool kRefill>
__device__ __forceinline__ void fused_products(bf16x8 (&P)[4 * PER], int npairs, bool lo,
                                               const uint16_t *ar0, const uint16_t *ar1,
                                               const uint16_t *wn, f32x4 &t0, f32x4 &t1) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        f32x4 c0{}, c1{};
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int j = w * PER + s;
            // npairs >= 4 PER - 3: only the last three steps can fall past
            // the last pair (a constant per unrolled step).
            const bool tail = j >= 4 * PER - 3;
            const int jc = tail ? min(j, npairs - 1) : j;
            bf16x8 w0, w1;
            unpair(lo, tail ? zero_unless(j < npairs, P[j]) : P[j], bf16x8{}, w0, w1);
            const bf16x8 x0 = *reinterpret_cast<const bf16x8 *>(ar0 + jc * 64);
            const bf16x8 x1 = *reinterpret_cast<const bf16x8 *>(ar0 + jc * 64 + 32);
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, x0, c0, 0, 0, 0);
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, x1, c0, 0, 0, 0);
            if constexpr (kTwo) {
                const bf16x8 z0 = *reinterpret_cast<const bf16x8 *>(ar1 + jc * 64);
                const bf16x8 z1 = *reinterpret_cast<const bf16x8 *>(ar1 + jc * 64 + 32);
                c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, z0, c1, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, z1, c1, 0, 0, 0);
            }
            if constexpr (kRefill) P[j] = ld_stream(wn + jc * 64);
        }
        if (w == 0) {
            t0 = c0;
            t1 = c1;
        } else {
            t0 += c0;
            t1 += c1;
        }
    }
}

template <int PER>
__device__ __forceinline__ void fused_products_any(bool two, bool refill,
                                                   bf16x8 (&P)[4 * PER], int npairs,
                                                   bool lo, const uint16_t *ar0,
                                                   const uint16_t *ar1, const uint16_t *wn,
                                                   f32x4 &t0, f32x4 &t1) {
    if (two) {
        if (refill)
            fused_products<PER, true, true>(P, npairs, lo, ar0, ar1, wn, t0, t1);
        else
            fused_products<PER, true, false>(P, npairs, lo, ar0, ar1, wn, t0, t1);
    } else {
        if (refill)
            fused_products<PER, false, true>(P, npairs, lo, ar0, ar1, wn, t0, t1);
        else
            fused_products<PER, false, false>(P, npairs, lo, ar0, ar1, wn, t0, t1);
    }
}

// PER: k-step pairs per quarter, ceil(I / 256) (1..6).
template <int PER>
__global__ __launch_bounds__(kFusedThreads) void decode_down_combine_kernel(
    const uint16_t *__restrict__ act, const uint16_t *__restrict__ w2,
    const int32_t *__restrict__ offsets, const float *__restrict__ topk_w,
    const int32_t *__restrict__ s2s, int T, int H, int I, int E, int k,
    uint16_t *__restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) uint16_t sact[];  // [rows][I + 8]
    __shared__ int32_t le[kFusedSlots], lb[kFusedSlots], lc[kFusedSlots];
    __shared__ int32_t lslot[kFusedSlots];
    __shared__ float lw[kFusedSlots];
    __shared__ float ys[kFusedSlots][kFusedRows];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int h0 = blockIdx.x * kFusedRows;
    const int rows = min(offsets[E], T * k);  // valid positions (LDS holds T k rows)
    // The combine's slot map and weights, read now rather than after the
    // products (and put in LDS once the weight loads are on their way).
    int my_slot = -1;
    float my_w = 0.0f;
    if (tid < T * k) {
        my_slot = s2s[tid];
        my_w = topk_w[tid];
    }
    const int npairs = I / 64;
    const int i = lane & 15;
    const int kq = lane >> 4;
    const bool lo = i < 8;

    // The non-empty experts in id order (listed in LDS by wave 0); every
    // wave finds its own first one.
    int nd = 0, e0 = -1;
    for (int c = 0; c < E; c += kWave) {
        const int e = c + lane;
        int off = 0, cn = 0;
        if (e < E) {
            off = offsets[e];
            cn = offsets[e + 1] - off;
        }
        const uint64_t nz = __ballot(cn > 0);
        const int d = nd + __popcll(nz & lanemask_lt());
        if (wave == 0 && cn > 0 && d < kFusedSlots) {
            le[d] = e;
            lb[d] = off;
            lc[d] = cn;
        }
        const uint64_t hit = __ballot(cn > 0 && d == wave);
        if (hit) e0 = c + __ffsll((unsigned long long)hit) - 1;
        nd += __popcll(nz);
    }
    nd = min(nd, kFusedSlots);

    // The first kStageLoads activation chunks per thread, then the first
    // expert's weights (paired loads of rows 0-7: row i & 7, half i >> 3 of
    // each line).  Every load is issued unconditionally (indexes clamped
    // into range), so the waits below count them exactly: the staging waits
    // only for its own chunks, and pair j's products wait only for pair j.
    const int chunks = I / 8;  // 16-byte chunks per row
    const int pitch = fused_pitch(I);
    const int nch = rows * chunks;
    const int last = max(nch - 1, 0);
    bf16x8 v[kStageLoads];
#pragma unroll
    for (int u = 0; u < kStageLoads; ++u)
        v[u] = *reinterpret_cast<const bf16x8 *>(
            act + (int64_t)min(tid + u * kFusedThreads, last) * 8);
    // A wave with no expert reads one 16-byte activation chunk instead.
    const uint16_t *wrow = w2 + ((int64_t)h0 + (i & 7)) * I + (i >> 3) * 32 + kq * 8;
    const uint16_t *wp = e0 >= 0 ? wrow + (int64_t)e0 * H * I : act;
    const int pstep = e0 >= 0 ? 64 : 0;
    constexpr int NP = 4 * PER;  // pair registers (quarters of PER pairs)
    bf16x8 P[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) P[j] = ld_stream(wp + min(j, npairs - 1) * pstep);
    if (tid < T * k) {
        lslot[tid] = my_slot;
        lw[tid] = my_w;
    }
#pragma unroll
    for (int u = 0; u < kStageLoads; ++u) {
        const int c = tid + u * kFusedThreads;
        if (c < nch) {
            const int r = c / chunks;
            *reinterpret_cast<bf16x8 *>(sact + r * pitch + (c - r * chunks) * 8) = v[u];
        }
    }
    for (int c = tid + kStageLoads * kFusedThreads; c < nch; c += kFusedThreads) {
        const int r = c / chunks;
        *reinterpret_cast<bf16x8 *>(sact + r * pitch + (c - r * chunks) * 8) =
            *reinterpret_cast<const bf16x8 *>(act + (int64_t)c * 8);
    }
    // LDS written (lists, slot map, activations); the weight loads stay in
    // flight across the barrier (__syncthreads would drain them).
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");

    for (int d = wave; d < nd; d += kFusedWaves) {
        const int base = lb[d], cnt = lc[d];
        const bool two = cnt > 16;  // token columns 16-31 as a second MFMA column block
        const int dn = d + kFusedWaves;
        const bool more = dn < nd;
        const uint16_t *wn = wrow + (int64_t)(more ? le[dn] : 0) * H * I;
        const uint16_t *ar0 = sact + (base + min(i, cnt - 1)) * pitch + kq * 8;
        const uint16_t *ar1 = sact + (base + min(16 + i, cnt - 1)) * pitch + kq * 8;
        f32x4 tot0, tot1;
        fused_products_any<PER>(two, more, P, npairs, lo, ar0, ar1, wn, tot0, tot1);
        // Accumulator r holds weight row 4 kq + r (rows 0-7: kq < 2) of
        // token column i (16 + i for the second block).
        if (kq < 2) {
            if (i < cnt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) ys[base + i][4 * kq + r] = tot0[r];
            }
            if (16 + i < cnt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) ys[base + 16 + i][4 * kq + r] = tot1[r];
            }
        }
    }
    __syncthreads();
    // out[t, h0 .. h0 + 7]: the token's slots in order, as combine_kernel.
    for (int t = tid; t < T; t += kFusedThreads) {
        float o[kFusedRows];
#pragma unroll
        for (int r = 0; r < kFusedRows; ++r) o[r] = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int p = lslot[t * k + j];
            if (p < 0 || p >= rows) continue;
            const float wj = lw[t * k + j];
#pragma unroll
            for (int r = 0; r < kFusedRows; ++r) o[r] = fmaf(wj, ys[p][r], o[r]);
        }
        bf16x8 v;
#pragma unroll
        for (int r = 0; r < kFusedRows; ++r) v[r] = to_bf16(o[r]);
        *reinterpret_cast<bf16x8 *>(out + (int64_t)t * H + h0) = v;
    }
}

int token_chunks(int64_t T) { return T <= 16 ? 1 : (T <= 32 ? 2 : 4); }

unsigned expert_rows(int64_t T, int E, int k) {
    const int64_t d = T * k < E ? T * k : E;
    return (unsigned)d;
}

}  // namespace

bool decode_down_combine_fused(int64_t T, int H, int I, int E, int k) {
    return T * k <= kFusedSlots && I <= 64 * kFusedPairs && H % kFusedRows == 0 && E >= 1;
}

template <int PER>
static hipError_t launch_fused(const uint16_t *act, const uint16_t *w2, const int32_t *offsets,
                        const float *topk_w, const int32_t *slot_to_sorted, int T, int H, int I,
                        int E, int k, uint16_t *out, size_t lds, hipStream_t s) {
    hipLaunchKernelGGL(decode_down_combine_kernel<PER>, dim3(H / kFusedRows),
                       dim3(kFusedThreads), lds, s, act, w2, offsets, topk_w, slot_to_sorted, T,
                       H, I, E, k, out);
    return hipGetLastError();
}

hipError_t launch_decode_down_combine_bf16(const uint16_t *act, const uint16_t *w2,
                                           const int32_t *offsets, const float *topk_w,
                                           const int32_t *slot_to_sorted, int64_t T, int H,
                                           int I, int E, int k, uint16_t *out, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (!decode_down_combine_fused(T, H, I, E, k)) return hipErrorInvalidValue;
    // Past 64 KB of dynamic LDS a kernel's limit must be raised: once, for
    // every instantiation, to the largest staging buffer the eligibility
    // rule allows.
    static const hipError_t raised = [] {
        const void *fns[] = {reinterpret_cast<const void *>(decode_down_combine_kernel<1>),
                             reinterpret_cast<const void *>(decode_down_combine_kernel<2>),
                             reinterpret_cast<const void *>(decode_down_combine_kernel<3>),
                             reinterpret_cast<const void *>(decode_down_combine_kernel<4>),
                             reinterpret_cast<const void *>(decode_down_combine_kernel<5>),
                             reinterpret_cast<const void *>(decode_down_combine_kernel<6>)};
        for (const void *fn : fns) {
            const hipError_t e = hipFuncSetAttribute(
                fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                kFusedSlots * (64 * kFusedPairs + 8) * 2);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }();
    if (raised != hipSuccess) return raised;
    const size_t lds = (size_t)T * k * (I + 8) * 2;
    const int Ti = (int)T;
    switch ((I / 64 + 3) / 4) {  // k-step pairs per quarter
        case 1: return launch_fused<1>(act, w2, offsets, topk_w, slot_to_sorted, Ti, H, I, E, k,
                                       out, lds, s);
        case 2: return launch_fused<2>(act, w2, offsets, topk_w, slot_to_sorted, Ti, H, I, E, k,
                                       out, lds, s);
        case 3: return launch_fused<3>(act, w2, offsets, topk_w, slot_to_sorted, Ti, H, I, E, k,
                                       out, lds, s);
        case 4: return launch_fused<4>(act, w2, offsets, topk_w, slot_to_sorted, Ti, H, I, E, k,
                                       out, lds, s);
        case 5: return launch_fused<5>(act, w2, offsets, topk_w, slot_to_sorted, Ti, H, I, E, k,
                                       out, lds, s);
        default: return launch_fused<6>(act, w2, offsets, topk_w, slot_to_sorted, Ti, H, I, E, k,
                                        out, lds, s);
    }
}


// Every block routes the whole batch, so the redundant routing grows with the
// blocks (I / 16 x the selected experts) times the rows: measured at E = 64,
// k = 8, H = 2048, I = 1408 (event-timed, caches flushed) one launch beats the
// two at T = 1 (23.7 against 26.2 us), ties at T = 2 and loses from T = 3
// (T = 8: 93.3 against 87.5 us; T = 32: 146 against 118 us).
constexpr int kRouteGateUpSlots = 16;

bool decode_route_gate_up_fused(int64_t T, int E, int k, int H, int I) {
    return T >= 1 && T * k <= kRouteGateUpSlots && E >= 1 && E <= 64 && k >= 1 && k <= 16 &&
           k <= E && H % 64 == 0 && I % kRows == 0;
}

hipError_t launch_decode_route_gate_up_bf16(
    const float *logits, int64_t T, int E, int k, int norm, float *topk_w, int32_t *topk_ids,
    uint8_t *multihot, float *pim, int32_t *pos, int32_t *counts, int32_t *offsets,
    int32_t *sorted_tok, int32_t *sorted_slot, int32_t *slot_to_sorted, float *inv_w,
    int32_t *inv_ids, const uint16_t *hidden, const uint16_t *w13, int H, int I, uint16_t *act,
    hipStream_t s) {
    if (!decode_route_gate_up_fused(T, E, k, H, I)) return hipErrorInvalidValue;
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const int vec4 = E == 64 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0;
    const dim3 grid(I / kRows, expert_rows(T, E, k));
    hipLaunchKernelGGL(decode_route_gate_up_kernel, grid, dim3(kThreads), 0, s, logits, (int)T, E,
                       k, norm, vec4, nbits, topk_w, topk_ids, multihot, pim, pos, counts, offsets,
                       sorted_tok, sorted_slot, slot_to_sorted, inv_w, inv_ids, hidden, w13, H, I,
                       act);
    return hipGetLastError();
}

hipError_t launch_decode_gate_up_bf16(const uint16_t *hidden, const uint16_t *w13,
                                      const int32_t *offsets, const int32_t *sorted_tok,
                                      int64_t T, int H, int I, int E, int k, uint16_t *act,
                                      hipStream_t s) {
    if (T == 0) return hipSuccess;
    // Two row tiles per block from 16 tokens on (I % 64 == 0, so I / 32
    // blocks cover I).
    const bool two = T >= 16;
    const dim3 grid(I / (kRows * (two ? 2 : 1)), expert_rows(T, E, k));
    switch (token_chunks(T) * (two ? 10 : 1)) {
        case 1:
            hipLaunchKernelGGL((decode_gate_up_kernel<1, 1>), grid, dim3(kThreads), 0, s, hidden,
                               w13, offsets, sorted_tok, H, I, E, act);
            break;
        case 10:
            hipLaunchKernelGGL((decode_gate_up_kernel<1, 2>), grid, dim3(kThreads), 0, s, hidden,
                               w13, offsets, sorted_tok, H, I, E, act);
            break;
        case 20:
            hipLaunchKernelGGL((decode_gate_up_kernel<2, 2>), grid, dim3(kThreads), 0, s, hidden,
                               w13, offsets, sorted_tok, H, I, E, act);
            break;
        default:
            hipLaunchKernelGGL((decode_gate_up_kernel<4, 2>), grid, dim3(kThreads), 0, s, hidden,
                               w13, offsets, sorted_tok, H, I, E, act);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_decode_down_bf16(const uint16_t *act, const uint16_t *w2,
                                   const int32_t *offsets, int64_t T, int H, int I, int E, int k,
                                   float *y, hipStream_t s) {
    if (T == 0) return hipSuccess;
    // Several row tiles per block once the experts hold enough tokens for
    // their activation rows to matter: four for 16 to 32 tokens, two past
    // that (H % 64 == 0, so H / 64 or H / 32 blocks cover H).
    const int rt = T < 16 ? 1 : (T <= 32 ? 4 : 2);
    const dim3 grid(H / (kRows * rt), expert_rows(T, E, k));
    switch (token_chunks(T) * 10 + rt) {
        case 11:
            hipLaunchKernelGGL((decode_down_kernel<1, 1>), grid, dim3(kThreads), 0, s, act, w2,
                               offsets, H, I, E, y);
            break;
        case 14:
            hipLaunchKernelGGL((decode_down_kernel<1, 4>), grid, dim3(kThreads), 0, s, act, w2,
                               offsets, H, I, E, y);
            break;
        case 24:
            hipLaunchKernelGGL((decode_down_kernel<2, 4>), grid, dim3(kThreads), 0, s, act, w2,
                               offsets, H, I, E, y);
            break;
        case 42:
            hipLaunchKernelGGL((decode_down_kernel<4, 2>), grid, dim3(kThreads), 0, s, act, w2,
                               offsets, H, I, E, y);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moe
