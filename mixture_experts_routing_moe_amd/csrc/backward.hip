// Backward of the MoE layer: gating softmax and expert FFN.
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
// The products are grouped GEMMs over the aligned (expert-major) slot order.
// One kernel serves them all: C[m, n] = sum_k A(m, k) B(n, k) on the bf16
// matrix cores (MFMA 16x16x32, float32 accumulation), 128 x 128 tiles, 4
// waves of 64 x 64.  Operands are either stored with k contiguous (a row per
// m or n, optionally gathered through sorted_token_ids) or with k as the row
// index (m or n contiguous); the second kind is transposed on its way into
// LDS, so fragment reads are the same for both.  The expert segments lie
// either on the M side (the dgrad-style products: rows of one expert against
// that expert's weight matrix) or on the K side (the weight gradients: a
// ragged sum over the expert's rows; an expert with no row gets zeros).
//
// This is a plain, single-buffered tiling (register prefetch of the next
// k-tile, two barriers per k-tile), not the forward GEMM's tuned pipeline.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBT = 256;          // threads per GEMM block: 4 waves in 2 x 2
constexpr int kBM = 128;          // tile rows (m)
constexpr int kBN = 128;          // tile columns (n)
constexpr int kBK = 32;           // k per LDS tile (one MFMA k-step)
constexpr int kLdsW = kBK + 8;    // bf16 per LDS row: 80 bytes, 16-byte aligned rows

struct BwdGemm {
    const uint16_t *A;
    int64_t lda;
    const int32_t *a_gather;  // A row (M-segment mode) or k row (K-segment) of position p
    const uint16_t *B;
    int64_t ldb;
    int64_t b_estride;        // M-segment mode: expert e's B starts at B + e * b_estride
    const int32_t *b_gather;  // K-segment mode: B row of position p is b_gather[p]
    float *C;
    int64_t ldc;
    int64_t c_estride;        // K-segment mode: expert e's C starts at C + e * c_estride
    const int32_t *offsets;   // [E + 1] aligned segment offsets
    int E, M, N, K;
    int n_tiles;
};

// Block s of the M-segment grid -> expert e and its rows [row0, min(row0 +
// kBM, row_end)).  Expert e owns ceil(count_e / kBM) consecutive blocks; a
// running sum over the experts (64 per pass, one per lane) finds the owner.
// Every wave computes the same answer.
__device__ bool find_mslot(const int32_t *__restrict__ off, int E, int s, int &e_out, int &row0,
                           int &row_end) {
    const int lane = lane_id();
    int carry = 0;
    for (int c = 0; c < E; c += kWave) {
        const int e = c + lane;
        int o = 0, cnt = 0;
        if (e < E) {
            o = off[e];
            cnt = off[e + 1] - o;
        }
        const int mt = (cnt + kBM - 1) / kBM;
        int incl = mt;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int v = __shfl_up(incl, d);
            if (lane >= d) incl += v;
        }
        const int lo = carry + incl - mt;
        const uint64_t b = __ballot(e < E && s >= lo && s < carry + incl);
        if (b) {
            const int l = __builtin_ctzll(b);
            const int lo_l = __shfl(lo, l);
            const int o_l = __shfl(o, l);
            const int cnt_l = __shfl(cnt, l);
            e_out = c + l;
            row0 = o_l + (s - lo_l) * kBM;
            row_end = o_l + cnt_l;
            return true;
        }
        carry += __shfl(incl, kWave - 1);
    }
    return false;
}

__device__ __forceinline__ uint16_t elem16(const uint4 &v, int j) {
    const uint32_t w = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
    return (uint16_t)(w >> (16 * (j & 1)));
}

// Tile of one operand: kBM (or kBN) rows x kBK k values into LDS row-major
// [row][k].  Two 16-byte chunks per thread.
//   KC (k contiguous):  chunk c = row (c / 4), k-group (c % 4).
//   otherwise (k rows): chunk c = k row (c / 16), 8 consecutive rows (c % 16)
//                       of the tile, written transposed.
template <bool KC>
__device__ __forceinline__ void lds_store(uint16_t *s, const uint4 (&r)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int c = threadIdx.x + kBT * q;
        if (KC) {
            *reinterpret_cast<uint4 *>(s + (c >> 2) * kLdsW + 8 * (c & 3)) = r[q];
        } else {
            const int kr = c >> 4, x0 = 8 * (c & 15);
#pragma unroll
            for (int j = 0; j < 8; ++j) s[(x0 + j) * kLdsW + kr] = elem16(r[q], j);
        }
    }
}

template <bool KSEG, bool BKM>
__global__ __launch_bounds__(kBT) void bwd_gemm_kernel(BwdGemm g) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[kBM * kLdsW];
    __shared__ __attribute__((aligned(16))) uint16_t sB[kBN * kLdsW];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int e, m0, m_end, k0, k_end, n0;
    const uint16_t *Bb;
    float *Cb;
    if (KSEG) {
        e = blockIdx.y;
        m0 = (int)(blockIdx.x / g.n_tiles) * kBM;
        n0 = (int)(blockIdx.x % g.n_tiles) * kBN;
        m_end = g.M;
        k0 = g.offsets[e];
        k_end = g.offsets[e + 1];
        Bb = g.B;
        Cb = g.C + (int64_t)e * g.c_estride;
    } else {
        n0 = blockIdx.y * kBN;
        if (!find_mslot(g.offsets, g.E, blockIdx.x, e, m0, m_end)) return;  // uniform
        k0 = 0;
        k_end = g.K;
        Bb = g.B + (int64_t)e * g.b_estride;
        Cb = g.C;
    }

    uint4 ra[2], rb[2];
    auto load = [&](int kt) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = tid + kBT * q;
            ra[q] = uint4{0, 0, 0, 0};
            rb[q] = uint4{0, 0, 0, 0};
            if (!KSEG) {  // A: rows of the segment, k contiguous
                const int p = m0 + (c >> 2);
                if (p < m_end) {
                    const int64_t row = g.a_gather ? g.a_gather[p] : p;
                    ra[q] = *reinterpret_cast<const uint4 *>(g.A + row * g.lda + kt + 8 * (c & 3));
                }
            } else {  // A: k rows (positions of the segment), m contiguous
                const int p = kt + (c >> 4);
                const int m = m0 + 8 * (c & 15);
                if (p < k_end && m < g.M) {
                    const int64_t row = g.a_gather ? g.a_gather[p] : p;
                    ra[q] = *reinterpret_cast<const uint4 *>(g.A + row * g.lda + m);
                }
            }
            if (!BKM) {  // B: rows n, k contiguous
                const int n = n0 + (c >> 2);
                if (n < g.N)
                    rb[q] = *reinterpret_cast<const uint4 *>(Bb + (int64_t)n * g.ldb + kt + 8 * (c & 3));
            } else {  // B: k rows, n contiguous
                const int p = kt + (c >> 4);
                const int n = n0 + 8 * (c & 15);
                if (p < k_end && n < g.N) {
                    const int64_t row = (KSEG && g.b_gather) ? g.b_gather[p] : p;
                    rb[q] = *reinterpret_cast<const uint4 *>(Bb + row * g.ldb + n);
                }
            }
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int i = lane & 15, kq = lane >> 4;
    if (k0 < k_end) load(k0);
    for (int kt = k0; kt < k_end; kt += kBK) {
        __syncthreads();  // the previous tile's fragment reads are done
        lds_store<!KSEG>(sA, ra);
        lds_store<!BKM>(sB, rb);
        __syncthreads();
        if (kt + kBK < k_end) load(kt + kBK);
        bf16x8 af[4], bf[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            af[f] = *reinterpret_cast<const bf16x8 *>(sA + (wm * 64 + f * 16 + i) * kLdsW + 8 * kq);
            bf[f] = *reinterpret_cast<const bf16x8 *>(sB + (wn * 64 + f * 16 + i) * kLdsW + 8 * kq);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bf[b], acc[a][b], 0, 0, 0);
    }

    // Accumulator r of fragment (a, b): row 4 kq + r of A's fragment, column i of B's.
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int n = n0 + wn * 64 + b * 16 + i;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + a * 16 + 4 * kq + r;
                if (m < m_end && n < g.N) Cb[(int64_t)m * g.ldc + n] = acc[a][b][r];
            }
        }
}

__device__ __forceinline__ uint16_t bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, to_bf16(f));
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
__global__ __launch_bounds__(256) void bwd_dx_kernel(const float *__restrict__ dxs,
                                                     const int32_t *__restrict__ slot_to_sorted,
                                                     int k, int H, float *__restrict__ dx,
                                                     float *__restrict__ grad_w) {
    const int64_t t = blockIdx.x;
    const int32_t *s2s = slot_to_sorted + t * k;
    if ((int)threadIdx.x < k && s2s[threadIdx.x] < 0) grad_w[t * k + threadIdx.x] = 0.f;
    for (int c = threadIdx.x; c < H / 4; c += blockDim.x) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const int p = s2s[j];
            if (p >= 0) acc += *reinterpret_cast<const f32x4 *>(dxs + (int64_t)p * H + 4 * c);
        }
        *reinterpret_cast<f32x4 *>(dx + t * H + 4 * c) = acc;
    }
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

}  // namespace

hipError_t launch_route_backward(const float *logits, const int32_t *ids, const float *w,
                                 const float *gw, int64_t T, int E, int k, int norm, float *out,
                                 hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int rows = 256 / kWave;
    hipLaunchKernelGGL(route_backward_kernel, dim3((unsigned)((T + rows - 1) / rows)), dim3(256),
                       0, s, logits, ids, w, gw, T, E, k, norm, out);
    return hipGetLastError();
}

size_t ffn_backward_part_bytes(int64_t T, int H, int I, int k, int part) {
    const size_t P = (size_t)T * (size_t)k;
    size_t b = 0;
    switch (part) {
        case 0: b = P * 2 * I * 4; break;  // h13   f32  [P, 2I]
        case 1: b = P * I * 4; break;      // G     f32  [P, I]
        case 2: b = P * I * 2; break;      // wact  bf16 [P, I]
        case 3: b = P * 2 * I * 2; break;  // dh13  bf16 [P, 2I]
        case 4: b = P * H * 4; break;      // dxs   f32  [P, H]
    }
    return (b + 255) / 256 * 256;
}

size_t ffn_backward_scratch_bytes(int64_t T, int H, int I, int k) {
    size_t b = 0;
    for (int part = 0; part < 5; ++part) b += ffn_backward_part_bytes(T, H, I, k, part);
    return b;
}

namespace {
template <bool KSEG, bool BKM>
hipError_t launch_bwd_gemm(const BwdGemm &g, int64_t P, hipStream_t s) {
    dim3 grid;
    if (KSEG) {
        const int m_tiles = (g.M + kBM - 1) / kBM;
        grid = dim3((unsigned)(m_tiles * g.n_tiles), (unsigned)g.E);
    } else {
        grid = dim3((unsigned)((P + kBM - 1) / kBM + g.E), (unsigned)g.n_tiles);
    }
    hipLaunchKernelGGL((bwd_gemm_kernel<KSEG, BKM>), grid, dim3(kBT), 0, s, g);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_ffn_backward_bf16(const uint16_t *x, const uint16_t *w13, const uint16_t *w2,
                                    const float *topk_w, const int32_t *offsets,
                                    const int32_t *sorted_tok, const int32_t *sorted_slot,
                                    const int32_t *slot_to_sorted, const uint16_t *dy,
                                    int64_t T, int H, int I, int E, int k, float *dx,
                                    float *dw13, float *dw2, float *dw, void *ws,
                                    hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int64_t P = T * k;
    char *base = static_cast<char *>(ws);
    float *h13 = reinterpret_cast<float *>(base);
    base += ffn_backward_part_bytes(T, H, I, k, 0);
    float *G = reinterpret_cast<float *>(base);
    base += ffn_backward_part_bytes(T, H, I, k, 1);
    uint16_t *wact = reinterpret_cast<uint16_t *>(base);
    base += ffn_backward_part_bytes(T, H, I, k, 2);
    uint16_t *dh13 = reinterpret_cast<uint16_t *>(base);
    base += ffn_backward_part_bytes(T, H, I, k, 3);
    float *dxs = reinterpret_cast<float *>(base);

    hipError_t err;
    BwdGemm g{};
    g.offsets = offsets;
    g.E = E;
    // h13[p] = x[tok p] . w13[e]^T   (gate and up recomputed)
    g.A = x; g.lda = H; g.a_gather = sorted_tok;
    g.B = w13; g.ldb = H; g.b_estride = (int64_t)2 * I * H; g.b_gather = nullptr;
    g.C = h13; g.ldc = 2 * I; g.c_estride = 0;
    g.M = 0; g.N = 2 * I; g.K = H; g.n_tiles = (g.N + kBN - 1) / kBN;
    if ((err = launch_bwd_gemm<false, false>(g, P, s)) != hipSuccess) return err;
    // G[p] = dy[tok p] . w2[e]   (w2[e] is [H, I]: k = h rows, n = i contiguous)
    g.A = dy; g.lda = H; g.a_gather = sorted_tok;
    g.B = w2; g.ldb = I; g.b_estride = (int64_t)H * I;
    g.C = G; g.ldc = I;
    g.N = I; g.K = H; g.n_tiles = (g.N + kBN - 1) / kBN;
    if ((err = launch_bwd_gemm<false, true>(g, P, s)) != hipSuccess) return err;

    hipLaunchKernelGGL(bwd_act_kernel, dim3((unsigned)P), dim3(256), 0, s, h13, G, topk_w,
                       offsets, sorted_slot, E, I, wact, dh13, dw);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    // dxs[p] = dh13[p] . w13[e]   (w13[e] is [2I, H]: k = c rows, n = h contiguous)
    g.A = dh13; g.lda = 2 * I; g.a_gather = nullptr;
    g.B = w13; g.ldb = H; g.b_estride = (int64_t)2 * I * H;
    g.C = dxs; g.ldc = H;
    g.N = H; g.K = 2 * I; g.n_tiles = (g.N + kBN - 1) / kBN;
    if ((err = launch_bwd_gemm<false, true>(g, P, s)) != hipSuccess) return err;
    hipLaunchKernelGGL(bwd_dx_kernel, dim3((unsigned)T), dim3(256), 0, s, dxs, slot_to_sorted, k,
                       H, dx, dw);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    // dw2[e][h, i] = sum over the segment of dy[tok p, h] (w act)[p, i]
    BwdGemm w{};
    w.offsets = offsets;
    w.E = E;
    w.A = dy; w.lda = H; w.a_gather = sorted_tok;
    w.B = wact; w.ldb = I; w.b_gather = nullptr;
    w.C = dw2; w.ldc = I; w.c_estride = (int64_t)H * I;
    w.M = H; w.N = I; w.n_tiles = (w.N + kBN - 1) / kBN;
    if ((err = launch_bwd_gemm<true, true>(w, P, s)) != hipSuccess) return err;
    // dw13[e][c, h] = sum over the segment of dh13[p, c] x[tok p, h]
    w.A = dh13; w.lda = 2 * I; w.a_gather = nullptr;
    w.B = x; w.ldb = H; w.b_gather = sorted_tok;
    w.C = dw13; w.ldc = H; w.c_estride = (int64_t)2 * I * H;
    w.M = 2 * I; w.N = H; w.n_tiles = (w.N + kBN - 1) / kBN;
    return launch_bwd_gemm<true, true>(w, P, s);
}

}  // namespace moe
