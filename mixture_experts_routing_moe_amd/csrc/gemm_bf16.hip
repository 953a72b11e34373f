// Grouped bf16 expert GEMMs on the CDNA4 matrix cores (prefill path).
//
// Method: project_6 moe_expert_gemm.cpp, moe_prefill_experts: per expert,
// the rows routed to it go through FC1 (x . w13[e]^T), SiLU-and-mul, FC2
// (act . w2[e]^T).  The page runs one vendor GEMM per expert from a host
// loop that reads each expert's row count back to the host.  Here one launch
// per FC covers every expert: the grid enumerates (m-slot, n-tile) pairs and
// each block finds its expert and row range on the device from the aligned
// offsets, so nothing is read back and empty experts cost nothing.
//
// Tile: 256 (rows) x 256 (weight rows) x 64 (k), 4 waves in a 2 x 2 layout,
// each wave 128 x 128 = 4 x 4 MFMA 32x32x16 bf16 tiles with float32
// accumulators.  Operand tiles go from global memory straight into LDS
// (global_load_lds, no staging registers), double buffered (2 x 64 KB), the
// next k-tile in flight while the current one feeds the matrix cores; 16-byte
// chunks are XOR-swizzled by row so the fragment reads are free of bank
// conflicts.
//
// The weight tile is the MFMA "A" operand and the token tile the "B" operand,
// so each lane's accumulators hold 4 consecutive output columns of one row
// (8-byte bf16 / 16-byte float32 stores).  For FC1 a block's 256 weight rows
// are 128 gate rows and the 128 matching up rows, and every wave holds
// matching gate and up fragments, so silu(gate) * up is applied in registers
// and only the activation is written.  FC2's output y stays float32: the layer
// output is rounded once, in the combine.
//
// Rows of a partial tile past the expert's segment load a clamped row and
// are never stored; weight rows past N are clamped the same way.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 256;  // token rows per tile
constexpr int BN = 256;  // weight rows per tile
constexpr int BK = 64;   // k per stage
constexpr int kGroupM = 4;
constexpr int kStage = (BM + BN) * BK;  // bf16 elements per LDS stage

struct MTile {
    int e, row0, row_end;
};

// m-slot -> (expert, rows): expert e owns ceil(count_e / BM) consecutive
// m-slots; a running sum over the experts (64 per pass, one per lane) finds
// the owner.  Every wave computes the same answer, so no LDS is needed.
__device__ bool find_m_tile(const int32_t *__restrict__ offsets, int E, int ms, MTile &t) {
    const int lane = lane_id();
    int carry = 0;
    for (int c = 0; c < E; c += kWave) {
        const int e = c + lane;
        int off = 0, cnt = 0;
        if (e < E) {
            off = offsets[e];
            cnt = offsets[e + 1] - off;
        }
        const int tiles = (cnt + BM - 1) / BM;
        int incl = tiles;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += y;
        }
        incl += carry;
        const int excl = incl - tiles;
        const uint64_t hit = __ballot(tiles > 0 && ms >= excl && ms < incl);
        if (hit) {
            const int L = __ffsll((unsigned long long)hit) - 1;
            const int ex = readlane_i(excl, L);
            const int o0 = readlane_i(off, L);
            const int cn = readlane_i(cnt, L);
            t.e = c + L;
            t.row0 = o0 + (ms - ex) * BM;
            t.row_end = min(t.row0 + BM, o0 + cn);
            return true;
        }
        carry = readlane_i(incl, kWave - 1);
    }
    return false;
}

typedef __attribute__((address_space(3))) void lds_void;

// Issue one k-tile of both operands straight into an LDS stage (gfx950
// global_load_lds_dwordx4: lane L's 16 bytes land at base + 16 L).  Wave w
// fills rows [64 w, 64 w + 64) of each tile, 8 rows per instruction; the
// source chunk of each lane is pre-permuted so that the stage comes out
// XOR-swizzled (chunk c of row r at position c ^ (r & 7)).
__device__ __forceinline__ void issue_stage(uint16_t *stage, const uint16_t *const (&aptr)[8],
                                            const uint16_t *const (&bptr)[8], int k0,
                                            int wave) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint16_t *da = stage + (wave * 64 + i * 8) * BK;
        uint16_t *db = stage + (BM + wave * 64 + i * 8) * BK;
        __builtin_amdgcn_global_load_lds(aptr[i] + k0, (lds_void *)da, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(bptr[i] + k0, (lds_void *)db, 16, 0, 0);
    }
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One LDS stage through the matrix cores: 4 k-steps of 16, each 4 weight
// fragments x 4 token fragments of MFMA 32x32x16.
__device__ __forceinline__ void mma_stage(f32x16 (&acc)[4][4], const uint16_t *s,
                                          const int (&nrow)[4], int xrow, int lr, int lk,
                                          int lane) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        const int ch = ((ks * 2 + lk) ^ (lane & 7)) * 8;
        bf16x8 wf[4], xf[4];
#pragma unroll
        for (int f = 0; f < 4; ++f)
            wf[f] = *reinterpret_cast<const bf16x8 *>(s + (BM + nrow[f] + lr) * BK + ch);
#pragma unroll
        for (int g = 0; g < 4; ++g)
            xf[g] = *reinterpret_cast<const bf16x8 *>(s + (xrow + g * 32) * BK + ch);
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[f], xf[g], acc[f][g], 0,
                                                                    0, 0);
    }
}

// kGateUp: A = hidden [T, K] gathered through `gather`, W = w13 [E, 2N, K],
//          C = act [rows, N] bf16 = silu(gate) * up.
// else:    A = act [rows, K], W = w2 [E, N, K], C = y [rows, N] float32.
template <bool kGateUp>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bf16_kernel(
    const uint16_t *__restrict__ A, const int32_t *__restrict__ gather,
    const uint16_t *__restrict__ W, const int32_t *__restrict__ offsets, void *__restrict__ Cv,
    int E, int K, int N, int m_slots, int n_tiles) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStage];

    // Block -> tile.  Workgroups are dealt round-robin to the 8 XCDs, so
    // block b is given tile index (b % 8) * (grid / 8) + b / 8: each XCD
    // works through one contiguous range of tiles, and within it groups of
    // kGroupM m-slots sweep the n-tiles together, sharing weight tiles (and
    // token tiles) in that XCD's L2.
    const int nblk = gridDim.x;
    const int bid = blockIdx.x;
    const int L = (bid & 7) * (nblk >> 3) + (bid >> 3);
    if (L >= m_slots * n_tiles) return;
    const int per_group = kGroupM * n_tiles;
    const int group = L / per_group;
    const int first_m = group * kGroupM;
    const int gsz = min(m_slots - first_m, kGroupM);
    const int within = L - group * per_group;
    const int ms = first_m + within % gsz;
    const int nt = within / gsz;

    MTile tile;
    if (!find_m_tile(offsets, E, ms, tile)) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // Operand rows of this lane: row 64 wave + 8 i + (lane >> 3) of each tile,
    // global chunk (lane & 7) ^ (lane >> 3) of that row (see issue_stage).
    const int rr = lane >> 3;
    const int c8 = ((lane & 7) ^ rr) * 8;
    const uint16_t *aptr[8];
    const uint16_t *bptr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = wave * 64 + i * 8 + rr;
        const int p = min(tile.row0 + r, tile.row_end - 1);
        const int arow = kGateUp ? gather[p] : p;
        aptr[i] = A + (int64_t)arow * K + c8;
        int wrow;
        if (kGateUp) {
            const int n = min(nt * (BN / 2) + (r & (BN / 2 - 1)), N - 1);
            wrow = r < BN / 2 ? n : N + n;
        } else {
            wrow = min(nt * BN + r, N - 1);
        }
        bptr[i] = W + ((int64_t)tile.e * (kGateUp ? 2 * N : N) + wrow) * K + c8;
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[f][g] = f32x16{};

    const int wn = wave & 1;
    const int wm = wave >> 1;
    const int lr = lane & 31;
    const int lk = lane >> 5;
    // LDS rows (within the weight tile) of this wave's 4 weight fragments.
    int nrow[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        if (kGateUp)
            nrow[f] = f < 2 ? wn * 64 + f * 32 : BN / 2 + wn * 64 + (f - 2) * 32;
        else
            nrow[f] = wn * 128 + f * 32;
    }
    const int xrow = wm * 128 + lr;

    const int nk = K / BK;
    issue_stage(smem, aptr, bptr, 0, wave);
    wait_loads();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        // The next k-tile streams into the other stage while this one feeds
        // the matrix cores; sched_barrier keeps the issue ahead of the math.
        if (kt + 1 < nk) issue_stage(smem + ((kt + 1) & 1) * kStage, aptr, bptr, (kt + 1) * BK,
                                     wave);
        __builtin_amdgcn_sched_barrier(0);
        mma_stage(acc, smem + (kt & 1) * kStage, nrow, xrow, lr, lk, lane);
        __builtin_amdgcn_sched_barrier(0);
        wait_loads();
        __syncthreads();
    }

    // Accumulator r of a 32x32 tile holds row 8 (r / 4) + 4 lk + (r % 4) of
    // the weight side and column lr of the token side.
    if (kGateUp) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int p = tile.row0 + wm * 128 + g * 32 + lr;
                if (p >= tile.row_end) continue;
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int n = nt * (BN / 2) + wn * 64 + f * 32 + rg * 8 + lk * 4;
                    if (n >= N) continue;
                    bf16x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        o[q] = to_bf16(silu_f(acc[f][g][rg * 4 + q]) * acc[f + 2][g][rg * 4 + q]);
                    *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(Cv) + (int64_t)p * N +
                                                n) = o;
                }
            }
        }
    } else {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int p = tile.row0 + wm * 128 + g * 32 + lr;
                if (p >= tile.row_end) continue;
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int n = nt * BN + wn * 128 + f * 32 + rg * 8 + lk * 4;
                    if (n >= N) continue;
                    const f32x16 &a = acc[f][g];
                    *reinterpret_cast<float4 *>(static_cast<float *>(Cv) + (int64_t)p * N + n) =
                        make_float4(a[rg * 4], a[rg * 4 + 1], a[rg * 4 + 2], a[rg * 4 + 3]);
                }
            }
        }
    }
}

int m_slot_bound(int64_t rows, int E) {
    const int64_t nz = rows < E ? rows : E;
    return (int)((rows + BM - 1) / BM + nz);
}

unsigned grid_of(int m_slots, int n_tiles) {
    const int64_t total = (int64_t)m_slots * n_tiles;
    return (unsigned)((total + 7) / 8 * 8);
}

}  // namespace

hipError_t launch_gate_up_bf16(const uint16_t *hidden, const uint16_t *w13,
                               const int32_t *offsets, const int32_t *sorted_tok, int64_t T,
                               int H, int I, int E, int k, uint16_t *act, hipStream_t s) {
    const int64_t rows = T * k;
    if (rows == 0) return hipSuccess;
    const int m_slots = m_slot_bound(rows, E);
    const int n_tiles = (I + BN / 2 - 1) / (BN / 2);
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<true>, dim3(grid_of(m_slots, n_tiles)),
                       dim3(kThreads), 0, s, hidden, sorted_tok, w13, offsets, act, E, H, I,
                       m_slots, n_tiles);
    return hipGetLastError();
}

hipError_t launch_down_bf16(const uint16_t *act, const uint16_t *w2, const int32_t *offsets,
                            int64_t T, int H, int I, int E, int k, float *y, hipStream_t s) {
    const int64_t rows = T * k;
    if (rows == 0) return hipSuccess;
    const int m_slots = m_slot_bound(rows, E);
    const int n_tiles = (H + BN - 1) / BN;
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<false>, dim3(grid_of(m_slots, n_tiles)),
                       dim3(kThreads), 0, s, act, nullptr, w2, offsets, y, E, I, H, m_slots,
                       n_tiles);
    return hipGetLastError();
}

}  // namespace moe
