// Backward of the MoE layer: gating softmax, group-limited selection weights
// and expert FFN (bfloat16 on the matrix cores; float32 for small layers).
//
// The pages describe the forward (the multihot converters' backward aside,
// which moe_multihot_to_indices already is); these kernels apply the chain
// rule to that forward.  For a slot (t, j) with expert e, weight w, gate/up
// rows w1 = w13[e][0:I], w3 = w13[e][I:2I], and dy = grad_out[t]:
//   G      = dy . w2[e]                      (so d_act = w G)
//   grad_w = <G, act>                        (= <dy, y>)
//   d_gate = w G up s (1 + gate (1 - s)),  d_up = w G gate s,  s = sigmoid(gate)
//   grad_hidden[t] = sum over j of [d_gate ; d_up] . w13[e]
//   grad_w2[e]  = sum over slots of dy^T (w act)
//   grad_w13[e] = sum over slots of [d_gate ; d_up]^T x
//
// Layout for the matrix cores.  Every product runs on the forward's grouped
// GEMM machinery, with the contracted index contiguous in LDS:
// * G = dy . w2 and d_hidden = [d_gate ; d_up] . w13 contract over the rows
//   of w2 and w13: the FC2-form kernel's K-major variant loads the weights as
//   stored and transposes them in its LDS fragment reads (gfx950's
//   ds_read_b64_tr_b16), so they are not copied; its A rows are dy and
//   [d_gate ; d_up] in the aligned order.
// * gate/up = x . w13^T is recomputed on the FC1 kernel, whose epilogue
//   applies the SiLU-and-mul backward from the accumulators and G (writing
//   w act, [d_gate ; d_up] and per-tile partial sums of grad_w), so gate/up
//   are never stored.
// * The two weight gradients contract over each expert's rows: dy and x are
//   transposed into [columns, positions] with every expert's segment padded
//   to a whole number of k-tiles (zeros in the padding), and w act and
//   [d_gate ; d_up] are read as stored, K-major, each k-tile's rows past the
//   segment reading as zeros; dw13 is computed as x^T [d_gate ; d_up] and
//   stored transposed.
// Operands too large for the buffer addressing take the older paths: the
// weights and all four weight-gradient operands transposed into the
// workspace, gate/up stored for bwd_act_kernel, and wgrad_kernel (256 x 256
// tiles, 8 waves of 64 x 128, two LDS stages of 64-wide k-tiles).
#include <cstdlib>

#include "moe_internal.h"

namespace moe {
namespace {

#ifndef MOE_WGRAD_TILE
#define MOE_WGRAD_TILE 256
#endif
constexpr int kWT = MOE_WGRAD_TILE;  // wgrad tile rows and columns (128 or 256)
#ifndef MOE_WGRAD_BK
#define MOE_WGRAD_BK 64
#endif
#ifndef MOE_WGRAD_STAGES
#define MOE_WGRAD_STAGES 2
#endif
constexpr int kBK = MOE_WGRAD_BK;       // k per LDS stage (MFMA k-steps of 32)
constexpr int kNS = MOE_WGRAD_STAGES;   // LDS stages (1 or 2)
constexpr int kSegPad = kBK;      // positions per padded segment unit: whole k-tiles
constexpr int kLdsW = kBK + 8;    // bf16 per LDS row: 16-byte aligned, rows staggered over banks
constexpr int kCPR = kBK / 8;                  // 16-byte chunks per tile row
static_assert(kBK % 32 == 0 && (kNS == 1 || kNS == 2) && (kWT == 128 || kWT == 256),
              "whole MFMA k-steps, one or two stages, 128 or 256 tiles");

__device__ __forceinline__ uint16_t bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, to_bf16(f));
}

// Weight gradient of one expert, C_e[m, n] = sum over k in the expert's padded
// segment [poff[e], poff[e+1]) of A[m, k] B[n, k]; A [M, ld] and B [N, ld] bf16
// with k contiguous, C_e float32 [M, N] at C + e M N.  Block (tile, e): a
// BM x BN tile, WM x WN waves of (BM / WM) x (BN / WN), each a grid of MFMA
// 16x16x32 fragments.  The next k-tile is loaded into registers while the
// current LDS stage is multiplied, then written into the other stage (one
// barrier per k-tile) or, with a single stage, into the same one after a
// second barrier.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void wgrad_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, int64_t ld,
    const int32_t *__restrict__ poff, int M, int N, int n_tiles, float *__restrict__ C) {
    constexpr int NT = WM * WN * 64;
    constexpr int FA = BM / WM / 16, FB = BN / WN / 16;  // fragments per wave
    constexpr int CA = BM * kBK / 8 / NT, CB = BN * kBK / 8 / NT;  // chunks per thread
    static_assert(CA * NT * 8 == BM * kBK && CB * NT * 8 == BN * kBK, "whole chunks per thread");
    __shared__ __attribute__((aligned(16))) uint16_t sA[kNS][BM * kLdsW];
    __shared__ __attribute__((aligned(16))) uint16_t sB[kNS][BN * kLdsW];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int e = blockIdx.y;
    const int m0 = (int)(blockIdx.x / n_tiles) * BM;
    const int n0 = (int)(blockIdx.x % n_tiles) * BN;
    const int k0 = poff[e], k_end = poff[e + 1];
    float *Ce = C + (int64_t)e * M * N;

    // Chunk c = row c / kCPR of the tile, k-group c % kCPR.
    uint4 ra[CA], rb[CB];
    auto load = [&](int kt) {
#pragma unroll
        for (int q = 0; q < CA; ++q) {
            const int c = tid + NT * q;
            const int r = c / kCPR, kc = 8 * (c % kCPR);
            ra[q] = uint4{0, 0, 0, 0};
            if (m0 + r < M) ra[q] = *reinterpret_cast<const uint4 *>(A + (int64_t)(m0 + r) * ld + kt + kc);
        }
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            const int c = tid + NT * q;
            const int r = c / kCPR, kc = 8 * (c % kCPR);
            rb[q] = uint4{0, 0, 0, 0};
            if (n0 + r < N) rb[q] = *reinterpret_cast<const uint4 *>(B + (int64_t)(n0 + r) * ld + kt + kc);
        }
    };
    auto store = [&](int st) {
#pragma unroll
        for (int q = 0; q < CA; ++q) {
            const int c = tid + NT * q;
            *reinterpret_cast<uint4 *>(&sA[st][(c / kCPR) * kLdsW + 8 * (c % kCPR)]) = ra[q];
        }
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            const int c = tid + NT * q;
            *reinterpret_cast<uint4 *>(&sB[st][(c / kCPR) * kLdsW + 8 * (c % kCPR)]) = rb[q];
        }
    };

    f32x4 acc[FA][FB];
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
        for (int b = 0; b < FB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int i = lane & 15, kq = lane >> 4;
    const int wr = wm * (BM / WM), wc = wn * (BN / WN);
    int st = 0;
    if (k0 < k_end) {
        load(k0);
        store(0);
    }
    __syncthreads();
    for (int kt = k0; kt < k_end; kt += kBK) {
        const bool more = kt + kBK < k_end;
        if (more) load(kt + kBK);
#pragma unroll
        for (int ks = 0; ks < kBK; ks += 32) {
            bf16x8 af[FA], bf[FB];
#pragma unroll
            for (int f = 0; f < FA; ++f)
                af[f] = *reinterpret_cast<const bf16x8 *>(&sA[st][(wr + f * 16 + i) * kLdsW + ks + 8 * kq]);
#pragma unroll
            for (int f = 0; f < FB; ++f)
                bf[f] = *reinterpret_cast<const bf16x8 *>(&sB[st][(wc + f * 16 + i) * kLdsW + ks + 8 * kq]);
#pragma unroll
            for (int a = 0; a < FA; ++a)
#pragma unroll
                for (int b = 0; b < FB; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bf[b], acc[a][b], 0, 0, 0);
        }
        // With two stages the other one was last read before the previous
        // barrier; with one, every wave must be done reading it first.
        if (kNS == 1) __syncthreads();
        if (more) store(kNS == 1 ? 0 : st ^ 1);
        __syncthreads();
        st = kNS == 1 ? 0 : st ^ 1;
    }

    // Accumulator r of fragment (a, b): row 4 kq + r of A's fragment, column i of B's.
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
        for (int b = 0; b < FB; ++b) {
            const int n = n0 + wc + b * 16 + i;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wr + a * 16 + 4 * kq + r;
                if (m < M && n < N) Ce[(int64_t)m * N + n] = acc[a][b][r];
            }
        }
}

// dst[p] = src[tok[p]] (rows of L bf16) for every aligned position p, for
// grad_out and, when xs is given, x.  One block per position.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ dy,
                                                          const int32_t *__restrict__ tok,
                                                          const int32_t *__restrict__ offsets,
                                                          int E, int L, uint16_t *__restrict__ xs,
                                                          uint16_t *__restrict__ dys) {
    const int p = blockIdx.x;
    if (p >= offsets[E]) return;
    const int64_t t = tok[p];
    for (int c = threadIdx.x; c < L / 8; c += blockDim.x) {
        if (xs != nullptr)
            *reinterpret_cast<uint4 *>(xs + (int64_t)p * L + 8 * c) =
                *reinterpret_cast<const uint4 *>(x + t * L + 8 * c);
        *reinterpret_cast<uint4 *>(dys + (int64_t)p * L + 8 * c) =
            *reinterpret_cast<const uint4 *>(dy + t * L + 8 * c);
    }
}

// Padded segment offsets: poff[0] = 0, poff[e+1] = poff[e] + count_e rounded
// up to kSegPad.  One thread (E <= 1024).
__global__ void seg_offsets_kernel(const int32_t *__restrict__ offsets, int E,
                                   int32_t *__restrict__ poff) {
    if (threadIdx.x != 0) return;
    int acc = 0;
    poff[0] = 0;
    for (int e = 0; e < E; ++e) {
        const int cnt = offsets[e + 1] - offsets[e];
        acc += (cnt + kSegPad - 1) / kSegPad * kSegPad;
        poff[e + 1] = acc;
    }
}

// For each padded position q < nq: the aligned position it holds, or -1 for
// padding (and for q past the last segment), and that position's token (-1
// likewise).
__global__ __launch_bounds__(256) void seg_src_kernel(const int32_t *__restrict__ offsets,
                                                      const int32_t *__restrict__ poff,
                                                      const int32_t *__restrict__ sorted_tok,
                                                      int E, int nq, int32_t *__restrict__ src,
                                                      int32_t *__restrict__ tsrc) {
    const int q = blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= nq) return;
    int r = -1;
    if (q < poff[E]) {
        int lo = 0, hi = E - 1;  // the last e with poff[e] <= q
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (poff[mid] <= q) lo = mid;
            else hi = mid - 1;
        }
        const int local = q - poff[lo];
        if (local < offsets[lo + 1] - offsets[lo]) r = offsets[lo] + local;
    }
    src[q] = r;
    tsrc[q] = r >= 0 ? sorted_tok[r] : -1;
}

// Batched bf16 transpose through LDS: for batch b = blockIdx.y / (L / 64),
// out_b[l][q] = in_b[row(q)][l] with row(q) = src[q] (0 where src[q] < 0) or q
// when src is null; q < nq (a multiple of 8), l < L (a multiple of 64).  A
// block moves a 64 x 64 tile.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(
    const uint16_t *__restrict__ in, int64_t ld_in, int64_t in_bs, const int32_t *__restrict__ src,
    int nq, int L, uint16_t *__restrict__ out, int64_t ld_out, int64_t out_bs) {
    constexpr int kTW = 72;  // LDS row stride (bf16): 144 bytes keeps 16-byte stores aligned
    __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kTW];
    const int lt = L / 64;
    const int b = blockIdx.y / lt;
    const int q0 = blockIdx.x * 64, l0 = (blockIdx.y % lt) * 64;
    in += (int64_t)b * in_bs;
    out += (int64_t)b * out_bs;
    for (int c = threadIdx.x; c < 512; c += blockDim.x) {
        const int qq = c >> 3, lc = 8 * (c & 7);
        const int q = q0 + qq;
        uint4 v = uint4{0, 0, 0, 0};
        if (q < nq) {
            const int64_t r = src ? (int64_t)src[q] : (int64_t)q;
            if (r >= 0) v = *reinterpret_cast<const uint4 *>(in + r * ld_in + l0 + lc);
        }
        *reinterpret_cast<uint4 *>(tile + qq * kTW + lc) = v;
    }
    __syncthreads();
    for (int c = threadIdx.x; c < 512; c += blockDim.x) {
        const int ll = c >> 3, qc = 8 * (c & 7);
        if (q0 + qc >= nq) continue;
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
            o[h] = (uint32_t)tile[(qc + 2 * h) * kTW + ll] |
                   ((uint32_t)tile[(qc + 2 * h + 1) * kTW + ll] << 16);
        *reinterpret_cast<uint4 *>(out + (int64_t)(l0 + ll) * ld_out + q0 + qc) =
            uint4{o[0], o[1], o[2], o[3]};
    }
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    return v;
}

// Per aligned position p: from the recomputed gate/up h13[p] and G[p] =
// grad_out[t] . w2[e], write w act (bf16: the one rounded operand of the w2
// gradient's product, whose other operand grad_out is exact), the gate/up
// gradients dh13 (bf16) and grad_topk_w of the slot = <G, act> with act in
// float32, summed in a fixed order (each thread its strided units, then a
// fixed tree).
__global__ __launch_bounds__(256) void bwd_act_kernel(const float *__restrict__ h13,
                                                      const float *__restrict__ G,
                                                      const float *__restrict__ topk_w,
                                                      const int32_t *__restrict__ offsets,
                                                      const int32_t *__restrict__ sorted_slot,
                                                      int E, int I, uint16_t *__restrict__ wact,
                                                      uint16_t *__restrict__ dh13,
                                                      float *__restrict__ grad_w) {
    __shared__ float part[4];
    const int p = blockIdx.x;
    if (p >= offsets[E]) return;
    const int slot = sorted_slot[p];
    const float w = topk_w[slot];
    const float *hg = h13 + (int64_t)p * 2 * I;
    const float *gp = G + (int64_t)p * I;
    float sum = 0.f;
    for (int c = threadIdx.x; c < I / 4; c += blockDim.x) {
        const f32x4 gate = *reinterpret_cast<const f32x4 *>(hg + 4 * c);
        const f32x4 up = *reinterpret_cast<const f32x4 *>(hg + I + 4 * c);
        const f32x4 gg = *reinterpret_cast<const f32x4 *>(gp + 4 * c);
        uint16_t a16[4], dg16[4], du16[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float z = gate[r], u = up[r];
            const float s = 1.0f / (1.0f + __expf(-z));
            const float a = z * s * u;
            a16[r] = bf16_bits(w * a);
            sum += gg[r] * a;
            const float da = w * gg[r];
            dg16[r] = bf16_bits(da * u * s * (1.0f + z * (1.0f - s)));
            du16[r] = bf16_bits(da * z * s);
        }
        const int64_t o = (int64_t)p * I + 4 * c;
        const int64_t o2 = (int64_t)p * 2 * I + 4 * c;
        *reinterpret_cast<uint2 *>(wact + o) =
            uint2{a16[0] | ((uint32_t)a16[1] << 16), a16[2] | ((uint32_t)a16[3] << 16)};
        *reinterpret_cast<uint2 *>(dh13 + o2) =
            uint2{dg16[0] | ((uint32_t)dg16[1] << 16), dg16[2] | ((uint32_t)dg16[3] << 16)};
        *reinterpret_cast<uint2 *>(dh13 + o2 + I) =
            uint2{du16[0] | ((uint32_t)du16[1] << 16), du16[2] | ((uint32_t)du16[3] << 16)};
    }
    sum = wave_sum_f(sum);
    if (lane_id() == 0) part[threadIdx.x / kWave] = sum;
    __syncthreads();
    if (threadIdx.x == 0) grad_w[slot] = (part[0] + part[1]) + (part[2] + part[3]);
}

// grad_hidden[t] = sum over slots j = 0..k-1 (in order) of dx[slot_to_sorted[t,
// j]]; slots with no position (invalid id) add nothing and get grad_topk_w 0.
// With gw_part, a valid slot's grad_topk_w is also written here: the sum of
// its position's gw_tiles partial sums, wave w taking slots w, w + 4, ...:
// lane l adds tiles l, l + 64, ... in order, then the lanes' sums meet in a
// fixed butterfly.
__global__ __launch_bounds__(256) void bwd_dx_kernel(const float *__restrict__ dxs,
                                                     const int32_t *__restrict__ slot_to_sorted,
                                                     int k, int H, float *__restrict__ dx,
                                                     float *__restrict__ grad_w,
                                                     const float *__restrict__ gw_part,
                                                     int gw_tiles) {
    const int64_t t = blockIdx.x;
    const int32_t *s2s = slot_to_sorted + t * k;
    if ((int)threadIdx.x < k && s2s[threadIdx.x] < 0) grad_w[t * k + threadIdx.x] = 0.f;
    if (gw_part != nullptr) {
        for (int j = threadIdx.x / kWave; j < k; j += blockDim.x / kWave) {
            const int p = s2s[j];
            if (p < 0) continue;  // wave-uniform
            const float *g = gw_part + (int64_t)p * gw_tiles;
            float sum = 0.f;
            for (int i = lane_id(); i < gw_tiles; i += kWave) sum += g[i];
            sum = wave_sum_f(sum);
            if (lane_id() == 0) grad_w[t * k + j] = sum;
        }
    }
    for (int c = threadIdx.x; c < H / 4; c += blockDim.x) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const int p = s2s[j];
            if (p >= 0) acc += *reinterpret_cast<const f32x4 *>(dxs + (int64_t)p * H + 4 * c);
        }
        *reinterpret_cast<f32x4 *>(dx + t * H + 4 * c) = acc;
    }
}

// ---------------------------------------------------------------------------
// Float32 layers (small; no matrix cores): one thread per output element,
// float32 dot products in a fixed order, as the float32 forward.
// ---------------------------------------------------------------------------

// Expert whose segment [offsets[e], offsets[e+1]) holds position p.
__device__ int expert_at(const int32_t *__restrict__ offsets, int E, int p) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offsets[mid] <= p) lo = mid;
        else hi = mid;
    }
    return lo;
}

// h13[p] = [x . w1^T, x . w3^T] and G[p] = dy . w2[e] for unit i of position p.
__global__ __launch_bounds__(256) void f32_gate_up_g_kernel(
    const float *__restrict__ x, const float *__restrict__ w13, const float *__restrict__ w2,
    const float *__restrict__ dy, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ tok, int H, int I, int E, float *__restrict__ h13,
    float *__restrict__ G) {
    const int p = blockIdx.x;
    if (p >= offsets[E]) return;
    const int i = blockIdx.y * blockDim.x + threadIdx.x;
    if (i >= I) return;
    const int e = expert_at(offsets, E, p);
    const int64_t t = tok[p];
    const float *xr = x + t * H, *dr = dy + t * H;
    const float *wg = w13 + ((int64_t)e * 2 * I + i) * H;
    const float *wu = w13 + ((int64_t)e * 2 * I + I + i) * H;
    const float *wd = w2 + (int64_t)e * H * I + i;
    float g = 0.f, u = 0.f, gd = 0.f;
    for (int h = 0; h < H; ++h) {
        g = fmaf(xr[h], wg[h], g);
        u = fmaf(xr[h], wu[h], u);
        gd = fmaf(dr[h], wd[(int64_t)h * I], gd);
    }
    h13[(int64_t)p * 2 * I + i] = g;
    h13[(int64_t)p * 2 * I + I + i] = u;
    G[(int64_t)p * I + i] = gd;
}

// Per position: act (float32), [d_gate ; d_up] and grad_topk_w = <G, act>
// (fixed-order sum: strided per thread, then a fixed tree).
__global__ __launch_bounds__(256) void f32_act_kernel(const float *__restrict__ h13,
                                                      const float *__restrict__ G,
                                                      const float *__restrict__ topk_w,
                                                      const int32_t *__restrict__ offsets,
                                                      const int32_t *__restrict__ sorted_slot,
                                                      int E, int I, float *__restrict__ act,
                                                      float *__restrict__ d13,
                                                      float *__restrict__ grad_w) {
    __shared__ float part[4];
    const int p = blockIdx.x;
    if (p >= offsets[E]) return;
    const int slot = sorted_slot[p];
    const float w = topk_w[slot];
    float sum = 0.f;
    for (int i = threadIdx.x; i < I; i += blockDim.x) {
        const float z = h13[(int64_t)p * 2 * I + i], u = h13[(int64_t)p * 2 * I + I + i];
        const float s = 1.0f / (1.0f + expf(-z));
        const float a = z * s * u;
        const float gi = G[(int64_t)p * I + i];
        act[(int64_t)p * I + i] = a;
        sum += gi * a;
        const float da = w * gi;
        d13[(int64_t)p * 2 * I + i] = da * u * s * (1.0f + z * (1.0f - s));
        d13[(int64_t)p * 2 * I + I + i] = da * z * s;
    }
    sum = wave_sum_f(sum);
    if (lane_id() == 0) part[threadIdx.x / kWave] = sum;
    __syncthreads();
    if (threadIdx.x == 0) grad_w[slot] = (part[0] + part[1]) + (part[2] + part[3]);
}

// dxs[p][h] = sum over c < 2I of d13[p][c] w13[e][c][h].
__global__ __launch_bounds__(256) void f32_dx_kernel(const float *__restrict__ d13,
                                                     const float *__restrict__ w13,
                                                     const int32_t *__restrict__ offsets, int H,
                                                     int I, int E, float *__restrict__ dxs) {
    const int p = blockIdx.x;
    if (p >= offsets[E]) return;
    const int h = blockIdx.y * blockDim.x + threadIdx.x;
    if (h >= H) return;
    const int e = expert_at(offsets, E, p);
    const float *d = d13 + (int64_t)p * 2 * I;
    const float *w = w13 + (int64_t)e * 2 * I * H + h;
    float acc = 0.f;
    for (int c = 0; c < 2 * I; ++c) acc = fmaf(d[c], w[(int64_t)c * H], acc);
    dxs[(int64_t)p * H + h] = acc;
}

// dw2[e][h][i] = sum over the segment of (w dy[tok p][h]) act[p][i], and
// dw13[e][c][h] = sum over the segment of d13[p][c] x[tok p][h]; positions in
// ascending order.  blockIdx.x = e * rows + row, threads over the columns.
__global__ __launch_bounds__(256) void f32_wgrad_kernel(
    const float *__restrict__ x, const float *__restrict__ dy, const float *__restrict__ act,
    const float *__restrict__ d13, const float *__restrict__ topk_w,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ tok,
    const int32_t *__restrict__ sorted_slot, int H, int I, int which, float *__restrict__ out) {
    const int rows = which == 2 ? H : 2 * I;  // rows of dw2[e] / dw13[e]
    const int cols = which == 2 ? I : H;
    const int e = blockIdx.x / rows, r = blockIdx.x % rows;
    const int c = blockIdx.y * blockDim.x + threadIdx.x;
    if (c >= cols) return;
    float acc = 0.f;
    for (int p = offsets[e]; p < offsets[e + 1]; ++p) {
        const int64_t t = tok[p];
        if (which == 2)
            acc = fmaf(topk_w[sorted_slot[p]] * dy[t * H + r], act[(int64_t)p * I + c], acc);
        else
            acc = fmaf(d13[(int64_t)p * 2 * I + r], x[t * H + c], acc);
    }
    out[((int64_t)e * rows + r) * cols + c] = acc;
}

// Gating softmax backward, one wave per row.  dot = sum_j w_j g_j over the
// forward's weights.  norm: grad[e_j] = w_j (g_j - dot), 0 elsewhere.
// Otherwise grad[e] = p_e (g(e) - dot) with p the softmax over all E logits
// and g(e) the slot gradient of e if selected, else 0.
__global__ __launch_bounds__(256) void route_backward_kernel(
    const float *__restrict__ logits, const int32_t *__restrict__ ids,
    const float *__restrict__ topk_w, const float *__restrict__ gw, int64_t T, int E, int k,
    int norm, float *__restrict__ out) {
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    const int my_id = lane < k ? ids[t * k + lane] : -1;
    const float my_g = lane < k ? gw[t * k + lane] : 0.f;
    const float my_w = lane < k ? topk_w[t * k + lane] : 0.f;
    const float dot = wave_sum_f(my_w * my_g);
    const float *x = logits + t * E;
    float m = -INFINITY, s = 0.f;
    if (!norm) {
        for (int e = lane; e < E; e += kWave) m = fmaxf(m, x[e]);
        m = wave_max_f(m);
        for (int e = lane; e < E; e += kWave) s += __expf(x[e] - m);
        s = wave_sum_f(s);
    }
    // The loop runs the same number of times on every lane (the shuffles need
    // all of them).
    for (int e0 = 0; e0 < E; e0 += kWave) {
        const int e = e0 + lane;
        int j_sel = -1;
        float ge = 0.f, we = 0.f;
        for (int j = 0; j < k; ++j) {
            const int idj = __shfl(my_id, j);
            const float gj = __shfl(my_g, j), wj = __shfl(my_w, j);
            if (idj == e) {
                j_sel = j;
                ge = gj;
                we = wj;
            }
        }
        if (e < E) {
            float r;
            if (norm)
                r = j_sel >= 0 ? we * (ge - dot) : 0.f;
            else
                r = __expf(x[e] - m) / s * (ge - dot);
            out[t * E + e] = r;
        }
    }
}


// Group-limited selection backward, one wave per row: the weights are the
// selected scores (over their sum S when renormalised), so grad[e_j] = g_j,
// or (g_j - sum_i w_i g_i) / S; 0 for unselected experts.  The bias moves
// only the selection.
__global__ __launch_bounds__(256) void route_grouped_backward_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ ids,
    const float *__restrict__ topk_w, const float *__restrict__ gw, int64_t T, int E, int k,
    int renorm, float *__restrict__ out) {
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    const float *x = scores + t * E;
    const int my_id = lane < k ? ids[t * k + lane] : -1;
    const float my_g = lane < k ? gw[t * k + lane] : 0.f;
    const float my_w = lane < k ? topk_w[t * k + lane] : 0.f;
    const float dot = wave_sum_f(my_w * my_g);
    const float S = wave_sum_f(my_id >= 0 ? x[my_id] : 0.f);
    for (int e0 = 0; e0 < E; e0 += kWave) {  // same trip count on every lane
        const int e = e0 + lane;
        int j_sel = -1;
        float ge = 0.f;
        for (int j = 0; j < k; ++j) {
            const int idj = __shfl(my_id, j);
            const float gj = __shfl(my_g, j);
            if (idj == e) {
                j_sel = j;
                ge = gj;
            }
        }
        if (e < E) out[t * E + e] = j_sel < 0 ? 0.f : renorm ? (ge - dot) / S : ge;
    }
}

}  // namespace

hipError_t launch_route_grouped_backward(const float *scores, const int32_t *ids, const float *w,
                                         const float *gw, int64_t T, int E, int k, int renorm,
                                         float *out, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int rows = 256 / kWave;
    hipLaunchKernelGGL(route_grouped_backward_kernel, dim3((unsigned)((T + rows - 1) / rows)),
                       dim3(256), 0, s, scores, ids, w, gw, T, E, k, renorm, out);
    return hipGetLastError();
}

hipError_t launch_route_backward(const float *logits, const int32_t *ids, const float *w,
                                 const float *gw, int64_t T, int E, int k, int norm, float *out,
                                 hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int rows = 256 / kWave;
    hipLaunchKernelGGL(route_backward_kernel, dim3((unsigned)((T + rows - 1) / rows)), dim3(256),
                       0, s, logits, ids, w, gw, T, E, k, norm, out);
    return hipGetLastError();
}

namespace {

// Padded positions (a multiple of 64, so the transposes' tiles are whole).
int64_t padded_positions(int64_t T, int E, int k) {
    return (T * k + (int64_t)kSegPad * E + 63) / 64 * 64;
}

// G = dy . w2 and d_hidden = [d_gate ; d_up] . w13 contract over the weights'
// rows.  They read w2 and w13 as stored (the grouped kernel's K-major variant,
// which transposes in its LDS fragment reads) unless an operand is too large
// for its buffer addressing; then w2 and w13 are transposed per expert into
// the workspace first.  MOE_BWD_TRANSPOSED_WEIGHTS=1 in the environment takes
// the transposing path at any size (tests compare the two).
bool kmajor_weights(int64_t T, int H, int I, int k) {
    const char *v = std::getenv("MOE_BWD_TRANSPOSED_WEIGHTS");  // read per call (host only)
    if (v != nullptr && v[0] == '1') return false;
    return down_kmajor_ok(T, I, H, k) && down_kmajor_ok(T, H, 2 * I, k);
}

// The weight gradients read w act and [d_gate ; d_up] as stored, per position
// (the grouped weight-gradient kernel's K-major variant; dw13 is stored
// through its transposing epilogue), and only dy and x are transposed,
// unless an operand is too large for its buffer addressing.
// MOE_BWD_TRANSPOSED_OPERANDS=1 in the environment transposes all four at any
// size (tests compare the two).
bool kmajor_wgrad(int64_t T, int H, int I, int E, int k) {
    const char *v = std::getenv("MOE_BWD_TRANSPOSED_OPERANDS");  // read per call (host only)
    if (v != nullptr && v[0] == '1') return false;
    const int64_t Pp = padded_positions(T, E, k);
    return wgrad_km_ok(H, I, Pp) && wgrad_km_ok(H, 2 * I, Pp);
}

// The SiLU-and-mul backward runs in the epilogue of the gate/up recompute
// (launch_gate_up_bwd_bf16), so gate/up are never stored, unless the
// operands are too large for its buffer addressing; then the recompute writes
// them (float32) and bwd_act_kernel follows.  MOE_BWD_UNFUSED_ACT=1 in the
// environment takes the separate path at any size (tests compare the two).
bool fused_act(int64_t T, int H, int I) {
    const char *v = std::getenv("MOE_BWD_UNFUSED_ACT");  // read per call (host only)
    if (v != nullptr && v[0] == '1') return false;
    return gate_up_bwd_ok(T, H, I);
}

// With K-major weights and the fused SiLU-and-mul backward, no product reads
// x or grad_out in the aligned order: G reads grad_out through sorted_tok and
// the transposes read both through each padded position's token, so nothing
// is gathered.
bool direct_rows(int64_t T, int H, int I, int k) {
    return kmajor_weights(T, H, I, k) && fused_act(T, H, I);
}

size_t part_bytes(int64_t T, int H, int I, int E, int k, int part) {
    const size_t P = (size_t)T * (size_t)k;
    const size_t Pp = (size_t)padded_positions(T, E, k);
    size_t b = 0;
    switch (part) {
        case 0:  // h13 f32 [P, 2I], or with the fused epilogue gw_part f32 [P, tiles]
            b = fused_act(T, H, I) ? P * gate_up_bwd_tiles(I) * 4 : P * 2 * I * 4;
            break;
        case 1: b = P * I * 4; break;                   // G      f32  [P, I]
        case 2: b = P * I * 2; break;                   // wact   bf16 [P, I]
        case 3: b = P * 2 * I * 2; break;               // dh13   bf16 [P, 2I]
        case 4: b = P * H * 4; break;                   // dxs    f32  [P, H]
        case 5:  // xs bf16 [P, H], only for the separate gate/up path
            b = fused_act(T, H, I) ? 0 : P * H * 2;
            break;
        case 6:  // dys bf16 [P, H], unless the rows are read in place
            b = direct_rows(T, H, I, k) ? 0 : P * H * 2;
            break;
        case 7:  // w13t bf16 [E, H, 2I], only on the transposing path
            b = kmajor_weights(T, H, I, k) ? 0 : (size_t)E * 2 * I * H * 2;
            break;
        case 8:  // w2t bf16 [E, I, H], only on the transposing path
            b = kmajor_weights(T, H, I, k) ? 0 : (size_t)E * H * I * 2;
            break;
        case 9: b = (size_t)H * Pp * 2; break;          // dyT    bf16 [H, Pp]
        case 10:  // wactT bf16 [I, Pp], only on the transposing path
            b = kmajor_wgrad(T, H, I, E, k) ? 0 : (size_t)I * Pp * 2;
            break;
        case 11:  // dh13T bf16 [2I, Pp], only on the transposing path
            b = kmajor_wgrad(T, H, I, E, k) ? 0 : (size_t)2 * I * Pp * 2;
            break;
        case 12: b = (size_t)H * Pp * 2; break;         // xT     bf16 [H, Pp]
        case 13: b = (size_t)(E + 1) * 4; break;        // poff   int32 [E+1]
        case 14: b = Pp * 4; break;                     // src    int32 [Pp]
        case 15: b = Pp * 4; break;                     // tsrc   int32 [Pp]
    }
    return (b + 255) / 256 * 256;
}
constexpr int kParts = 16;

hipError_t transpose(const uint16_t *in, int64_t ld_in, int64_t in_bs, const int32_t *src,
                     int nq, int L, uint16_t *out, int64_t ld_out, int64_t out_bs, int batch,
                     hipStream_t s) {
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)((nq + 63) / 64), (unsigned)(L / 64 * batch)),
                       dim3(256), 0, s, in, ld_in, in_bs, src, nq, L, out, ld_out, out_bs);
    return hipGetLastError();
}

hipError_t wgrad(const uint16_t *A, const uint16_t *B, int64_t ld, const int32_t *poff, int E,
                 int M, int N, float *C, hipStream_t s) {
    // kWT = 256: 8 waves of 64 x 128; kWT = 128: 4 waves of 64 x 64.
    constexpr int WM = kWT == 256 ? 4 : 2, WN = 2;
    const int n_tiles = (N + kWT - 1) / kWT;
    const int m_tiles = (M + kWT - 1) / kWT;
    hipLaunchKernelGGL((wgrad_kernel<kWT, kWT, WM, WN>), dim3((unsigned)(m_tiles * n_tiles), (unsigned)E),
                       dim3(WM * WN * 64), 0, s, A, B, ld, poff, M, N, n_tiles, C);
    return hipGetLastError();
}

}  // namespace

size_t ffn_backward_scratch_bytes(int64_t T, int H, int I, int E, int k) {
    size_t b = 0;
    for (int part = 0; part < kParts; ++part) b += part_bytes(T, H, I, E, k, part);
    return b;
}

hipError_t launch_ffn_backward_bf16(const uint16_t *x, const uint16_t *w13, const uint16_t *w2,
                                    const float *topk_w, const int32_t *offsets,
                                    const int32_t *sorted_tok, const int32_t *sorted_slot,
                                    const int32_t *slot_to_sorted, const uint16_t *dy,
                                    int64_t T, int H, int I, int E, int k, float *dx,
                                    float *dw13, float *dw2, float *dw, void *ws,
                                    hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int64_t P = T * k;
    const int Pp = (int)padded_positions(T, E, k);
    char *part[kParts];
    char *base = static_cast<char *>(ws);
    for (int i = 0; i < kParts; ++i) {
        part[i] = base;
        base += part_bytes(T, H, I, E, k, i);
    }
    float *h13 = reinterpret_cast<float *>(part[0]);
    float *gw_part = h13;  // the same part on the fused path
    float *G = reinterpret_cast<float *>(part[1]);
    uint16_t *wact = reinterpret_cast<uint16_t *>(part[2]);
    uint16_t *dh13 = reinterpret_cast<uint16_t *>(part[3]);
    float *dxs = reinterpret_cast<float *>(part[4]);
    uint16_t *xs = reinterpret_cast<uint16_t *>(part[5]);
    uint16_t *dys = reinterpret_cast<uint16_t *>(part[6]);
    uint16_t *w13t = reinterpret_cast<uint16_t *>(part[7]);
    uint16_t *w2t = reinterpret_cast<uint16_t *>(part[8]);
    uint16_t *dyT = reinterpret_cast<uint16_t *>(part[9]);
    uint16_t *wactT = reinterpret_cast<uint16_t *>(part[10]);
    uint16_t *dh13T = reinterpret_cast<uint16_t *>(part[11]);
    uint16_t *xT = reinterpret_cast<uint16_t *>(part[12]);
    int32_t *poff = reinterpret_cast<int32_t *>(part[13]);
    int32_t *src = reinterpret_cast<int32_t *>(part[14]);
    int32_t *tsrc = reinterpret_cast<int32_t *>(part[15]);
    const bool fused = fused_act(T, H, I);
    const bool direct = direct_rows(T, H, I, k);
    hipError_t err;
#define MOE_TRY(x)                                   \
    do {                                             \
        if ((err = (x)) != hipSuccess) return err;   \
    } while (0)

    // Layout preparation: gathered rows where a product reads them in the
    // aligned order (grad_out for G on the transposed-weight path, x for the
    // separate gate/up path), per-expert transposed weights, the padded
    // segment map.
    if (!direct) {
        hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)P), dim3(256), 0, s, x, dy,
                           sorted_tok, offsets, E, H, fused ? nullptr : xs, dys);
        MOE_TRY(hipGetLastError());
    }
    const bool km = kmajor_weights(T, H, I, k);
    if (!km) {
        MOE_TRY(transpose(w13, H, (int64_t)2 * I * H, nullptr, 2 * I, H, w13t, 2 * I,
                          (int64_t)2 * I * H, E, s));
        MOE_TRY(transpose(w2, I, (int64_t)H * I, nullptr, H, I, w2t, H, (int64_t)H * I, E, s));
    }
    hipLaunchKernelGGL(seg_offsets_kernel, dim3(1), dim3(64), 0, s, offsets, E, poff);
    MOE_TRY(hipGetLastError());
    hipLaunchKernelGGL(seg_src_kernel, dim3((unsigned)((Pp + 255) / 256)), dim3(256), 0, s,
                       offsets, poff, sorted_tok, E, Pp, src, tsrc);
    MOE_TRY(hipGetLastError());

    // Row-segment products on the forward's grouped kernel: G (FC2 form;
    // grad_out's rows read in place through the token ids where nothing was
    // gathered), then gate/up recomputed (FC1 form) with the SiLU-and-mul
    // backward in its epilogue, or (FC2 form) stored for bwd_act_kernel.
    if (!km)
        MOE_TRY(launch_down_bf16(dys, w2t, offsets, T, I, H, E, k, 1, G, s));
    else if (direct)
        MOE_TRY(launch_down_kmajor_bf16(dy, sorted_tok, w2, offsets, T, I, H, E, k, G, s));
    else
        MOE_TRY(launch_down_kmajor_bf16(dys, nullptr, w2, offsets, T, I, H, E, k, G, s));
    if (fused) {
        MOE_TRY(launch_gate_up_bwd_bf16(x, w13, offsets, sorted_tok, sorted_slot, topk_w, G, T, H,
                                        I, E, k, wact, dh13, gw_part, s));
    } else {
        MOE_TRY(launch_down_bf16(xs, w13, offsets, T, 2 * I, H, E, k, 1, h13, s));  // gate/up
        hipLaunchKernelGGL(bwd_act_kernel, dim3((unsigned)P), dim3(256), 0, s, h13, G, topk_w,
                           offsets, sorted_slot, E, I, wact, dh13, dw);
        MOE_TRY(hipGetLastError());
    }
    MOE_TRY(km ? launch_down_kmajor_bf16(dh13, nullptr, w13, offsets, T, H, 2 * I, E, k, dxs, s)
               : launch_down_bf16(dh13, w13t, offsets, T, H, 2 * I, E, k, 1, dxs, s));  // d_hidden
    hipLaunchKernelGGL(bwd_dx_kernel, dim3((unsigned)T), dim3(256), 0, s, dxs, slot_to_sorted, k,
                       H, dx, dw, fused ? gw_part : nullptr, gate_up_bwd_tiles(I));
    MOE_TRY(hipGetLastError());

    // Weight gradients over the padded, transposed segments of dy and x.
    MOE_TRY(direct ? transpose(dy, H, 0, tsrc, Pp, H, dyT, Pp, 0, 1, s)
                   : transpose(dys, H, 0, src, Pp, H, dyT, Pp, 0, 1, s));
    // x^T straight from x through each padded position's token where x was
    // not gathered.
    MOE_TRY(fused ? transpose(x, H, 0, tsrc, Pp, H, xT, Pp, 0, 1, s)
                  : transpose(xs, H, 0, src, Pp, H, xT, Pp, 0, 1, s));
    if (kmajor_wgrad(T, H, I, E, k)) {
        // dw2[e] [H, I]: dy^T (w act); dw13[e] [2I, H]: ([d_gate ; d_up]^T x),
        // computed as x^T [d_gate ; d_up] and stored transposed.
        MOE_TRY(launch_wgrad_km_bf16(dyT, wact, Pp, poff, offsets, E, H, I, false, dw2, s));
        MOE_TRY(launch_wgrad_km_bf16(xT, dh13, Pp, poff, offsets, E, H, 2 * I, true, dw13, s));
        return hipSuccess;
    }
    MOE_TRY(transpose(wact, I, 0, src, Pp, I, wactT, Pp, 0, 1, s));
    MOE_TRY(transpose(dh13, 2 * I, 0, src, Pp, 2 * I, dh13T, Pp, 0, 1, s));
    // On the grouped kernel's machinery where the operands fit its buffer
    // addressing, else on wgrad_kernel.
    MOE_TRY(wgrad_grouped_ok(H, I, Pp) ? launch_wgrad_bf16(dyT, wactT, Pp, poff, E, H, I, dw2, s)
                                       : wgrad(dyT, wactT, Pp, poff, E, H, I, dw2, s));  // dw2[e] [H, I]
    MOE_TRY(wgrad_grouped_ok(2 * I, H, Pp)
                ? launch_wgrad_bf16(dh13T, xT, Pp, poff, E, 2 * I, H, dw13, s)
                : wgrad(dh13T, xT, Pp, poff, E, 2 * I, H, dw13, s));  // dw13[e] [2I, H]
#undef MOE_TRY
    return hipSuccess;
}


hipError_t launch_ffn_backward_f32(const float *x, const float *w13, const float *w2,
                                   const float *topk_w, const int32_t *offsets,
                                   const int32_t *sorted_tok, const int32_t *sorted_slot,
                                   const int32_t *slot_to_sorted, const float *dy, int64_t T,
                                   int H, int I, int E, int k, float *dx, float *dw13,
                                   float *dw2, float *dw, void *ws, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int64_t P = T * k;
    float *h13 = static_cast<float *>(ws);   // [P, 2I]
    float *G = h13 + P * 2 * I;              // [P, I]
    float *act = G + P * I;                  // [P, I]
    float *d13 = act + P * I;                // [P, 2I]
    float *dxs = d13 + P * 2 * I;            // [P, H]
    hipError_t err;
    hipLaunchKernelGGL(f32_gate_up_g_kernel, dim3((unsigned)P, (unsigned)((I + 255) / 256)),
                       dim3(256), 0, s, x, w13, w2, dy, offsets, sorted_tok, H, I, E, h13, G);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(f32_act_kernel, dim3((unsigned)P), dim3(256), 0, s, h13, G, topk_w,
                       offsets, sorted_slot, E, I, act, d13, dw);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(f32_dx_kernel, dim3((unsigned)P, (unsigned)((H + 255) / 256)), dim3(256),
                       0, s, d13, w13, offsets, H, I, E, dxs);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(bwd_dx_kernel, dim3((unsigned)T), dim3(256), 0, s, dxs, slot_to_sorted, k,
                       H, dx, dw, nullptr, 0);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(f32_wgrad_kernel, dim3((unsigned)(E * H), (unsigned)((I + 255) / 256)),
                       dim3(256), 0, s, x, dy, act, d13, topk_w, offsets, sorted_tok, sorted_slot,
                       H, I, 2, dw2);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(f32_wgrad_kernel, dim3((unsigned)(E * 2 * I), (unsigned)((H + 255) / 256)),
                       dim3(256), 0, s, x, dy, act, d13, topk_w, offsets, sorted_tok, sorted_slot,
                       H, I, 13, dw13);
    return hipGetLastError();
}

size_t ffn_backward_f32_scratch_bytes(int64_t T, int H, int I, int k) {
    return (size_t)T * k * (6 * (size_t)I + H) * 4;
}

}  // namespace moe
