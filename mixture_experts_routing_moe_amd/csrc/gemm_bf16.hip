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
// Tile: 320 token rows x 256 weight rows, 8 waves (2 per SIMD, so one wave's
// waits hide behind the other's matrix-core work) in a 4 x 2 layout, each
// wave 64 weight rows x 160 token rows = 2 x 5 MFMA 32x32x16 bf16 tiles with
// float32 accumulators.  320 rows rather than 256: the operand loads bound
// these kernels, and an expert with a little over 1024 rows (the Mixtral
// shape's typical count) then takes 4 m-tiles instead of 5, so its weights
// are streamed through the chip 4 times instead of 5.  Operands go from global memory straight into LDS
// (gfx950 global_load_lds_dwordx4, no staging registers), double buffered, the
// next k-tile in flight while the current one feeds the matrix cores;
// fragments are double buffered in registers and their LDS reads interleaved
// with the MFMAs; 16-byte chunks are XOR-swizzled so fragment reads are
// bank-conflict free.
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
// are never stored, and the MFMAs of token fragments that hold none of the
// expert's rows are not issued (the loop is instantiated per count of valid
// fragments, so the hot loop carries no branches); weight rows past N are
// clamped the same way.
#include <cmath>
#include <cstdlib>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = kGemmBM;  // token rows per tile (moe_internal.h)
constexpr int BN = 256;  // weight rows per tile
#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 64
#endif
#ifndef MOE_GEMM_STAGES
#define MOE_GEMM_STAGES 2
#endif
constexpr int BK = MOE_GEMM_BK;           // k elements per LDS stage
constexpr int NS = MOE_GEMM_STAGES;       // LDS stages in the ring
constexpr int KS = BK / 16;               // 16-wide k-steps per stage
#ifndef MOE_GEMM_WN
#define MOE_GEMM_WN 4
#endif
#ifndef MOE_GEMM_WM
#define MOE_GEMM_WM 2
#endif
constexpr int WN = MOE_GEMM_WN;  // waves along the weight rows
constexpr int WM = MOE_GEMM_WM;  // waves along the token rows
constexpr int kWaves = WN * WM;
constexpr int kThreads = 64 * kWaves;
constexpr int NF = BN / WN / 32;  // weight fragments per wave
constexpr int MF = BM / WM / 32;  // token fragments per wave
constexpr int kXcdChunk = 32;  // CUs per XCD: tiles an XCD runs at once
constexpr int kBandMTiles = 4;  // m-tiles per band of the tile order (at least)
// LDS: the NS token stages, then the NS weight stages, so every fragment
// address is a per-lane base plus a constant below 64 KiB (the ds_read offset
// field).
constexpr int kTokStage = BM * BK;          // bf16 elements per token stage
constexpr int kWStage = BN * BK;            // bf16 elements per weight stage
constexpr int kWOff = NS * kTokStage;       // first weight stage
constexpr int kLds = kWOff + NS * kWStage;  // bf16 elements in all
constexpr int kChunks = BK / 8;                // 16-byte chunks per row
constexpr int kRowsPerLoad = 64 / kChunks;     // rows one wave instruction fills
constexpr int kTokRowsPerWave = BM / kWaves;   // token rows each wave loads per k-tile
constexpr int kWRowsPerWave = BN / kWaves;     // weight rows each wave loads per k-tile
constexpr int NLA = kTokRowsPerWave / kRowsPerLoad;  // token load instructions per wave
constexpr int NLB = kWRowsPerWave / kRowsPerLoad;    // weight load instructions per wave
constexpr int kRowsPerWindow = 128 / BK;       // rows sharing one 256-byte bank window
static_assert(kLds * 2 <= 160 * 1024, "LDS exceeds 160 KB");
static_assert(NF % 2 == 0, "gate and up fragments come in pairs");
static_assert(MF >= 1 && MF <= 5, "the k loop is dispatched on 0..5 valid token fragments");
static_assert(NLA * kRowsPerLoad * kWaves == BM && NLB * kRowsPerLoad * kWaves == BN,
              "whole load instructions per wave");
static_assert(NS >= 2 && KS % 2 == 0, "a ring of at least two stages, an even count of k-steps");
static_assert(((NS - 1) * kWStage + BN * BK) * 2 <= 65536 &&
                  ((NS - 1) * kTokStage + (MF - 1) * 32 * BK) * 2 < 65536,
              "fragment offsets fit the ds_read field");
constexpr int kLoadsPerStage = NLA + NLB;  // load instructions per lane per stage
static_assert((NS - 2) * kLoadsPerStage <= 63, "vmcnt holds at most 63");

typedef __attribute__((address_space(3))) void lds_void;

struct MTile {
    int e, row0, row_end;
};

// Tile j of an expert with mt m-tiles (0 <= j < mt * n_tiles) -> (m-tile i,
// n-tile nt): bands of a m-tiles, each band's tiles n-tile-major, so the
// kXcdChunk tiles an XCD runs together span about a m-tiles x kXcdChunk / a
// n-tiles and share both operands in its L2 (with all m-tiles of a big expert
// under one n-tile, its token rows were re-read for every n-tile).
__device__ __forceinline__ void band_tile(int j, int mt, int n_tiles, int &i, int &nt) {
    const int a = min(mt, max(kBandMTiles, kXcdChunk / n_tiles));
    const int b = j / (a * n_tiles);
    const int r = j - b * a * n_tiles;
    const int ab = min(a, mt - b * a);
    nt = r / ab;
    i = b * a + (r - nt * ab);
}

// Tile index -> (expert, rows, n-tile).  Expert e owns mt_e = ceil(count_e /
// BM) m-tiles, and its mt_e * n_tiles tiles form one contiguous range of the
// tile index, in bands of m-tiles (below).  The segment is dealt to the
// m-tiles in near-equal whole fragments (1040 rows: 3 x 288 + 176) instead
// of 3 x 320 + 80, so the tiles sharing a weight tile do similar work and
// stay in step (measured faster for both GEMMs).  A running sum of mt_e over
// the experts (64 per pass, one per lane) finds the owner.  Every wave
// computes the same answer, so no LDS is needed.
__device__ bool find_tile(const int32_t *__restrict__ offsets, int E, int L, int n_tiles,
                          MTile &t, int &nt) {
    const int lane = lane_id();
    int carry = 0;
    for (int c = 0; c < E; c += kWave) {
        const int e = c + lane;
        int off = 0, cnt = 0;
        if (e < E) {
            off = offsets[e];
            cnt = offsets[e + 1] - off;
        }
        const int tiles = expert_mtiles(cnt);
        int incl = tiles;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += y;
        }
        incl += carry;
        const int excl = incl - tiles;
        const uint64_t hit =
            __ballot(tiles > 0 && L >= excl * n_tiles && L < incl * n_tiles);
        if (hit) {
            const int src = __ffsll((unsigned long long)hit) - 1;
            const int ex = readlane_i(excl, src);
            const int mt = readlane_i(tiles, src);
            const int o0 = readlane_i(off, src);
            const int cn = readlane_i(cnt, src);
            int i;
            band_tile(L - ex * n_tiles, mt, n_tiles, i, nt);
            t.e = c + src;
            const int q = mtile_share(cn, mt);  // rows per m-tile
            t.row0 = o0 + min(i * q, cn);
            t.row_end = o0 + min((i + 1) * q, cn);
            return t.row0 < t.row_end;
        }
        carry = readlane_i(incl, kWave - 1);
    }
    return false;
}

// Total m-tiles sum_e ceil(count_e / BM) (every lane gets it).
__device__ int count_mtiles(const int32_t *__restrict__ offsets, int E) {
    const int lane = lane_id();
    int total = 0;
    for (int c = 0; c < E; c += kWave) {
        const int e = c + lane;
        const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
        int tiles = expert_mtiles(cnt);
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) tiles += __shfl_xor(tiles, o, kWave);
        total += tiles;
    }
    return total;
}

// LDS layout of a stage: token rows [0, BM) then weight rows [BM, BM + BN),
// each BK bf16 = kChunks chunks of 16 bytes; chunk c of row r is stored at
// position c ^ swz(r).  A ds_read_b128 serves 16 lanes per cycle from 64
// banks (a 256-byte window); a fragment read has 16 consecutive rows at one
// logical chunk, and rows r, r + kRowsPerWindow, ... share window offsets, so
// swz must differ across them: swz(r) = (r / kRowsPerWindow) % kChunks.
__device__ __forceinline__ int swz(int r) { return (r / kRowsPerWindow) % kChunks; }

// Operand addressing.  kBuf: a buffer resource per operand (scalar
// registers), a 32-bit byte offset per lane and row, and the k position as the
// scalar offset, so issuing a k-tile's loads takes no vector arithmetic (the
// load path measured 2-8 % faster than with 64-bit per-lane pointers).  It
// needs each operand under 2^31 bytes; larger ones take the pointer path.
template <bool kBuf>
struct Ops;
template <>
struct Ops<true> {
    __amdgpu_buffer_rsrc_t a, b;    // token / weight operand (this expert)
    int kb;                         // first k of this K slice
    int na;                         // token loads that hold a row of the tile
    uint32_t aoff[NLA], boff[NLB];  // byte offsets of this lane's rows and chunk
};
template <>
struct Ops<false> {
    const uint16_t *a[NLA], *b[NLB];  // this lane's rows and chunk, from the slice's first k
    int na;                           // token loads that hold a row of the tile
};

// Buffer-addressed operands with the weight stored K-major (per expert
// [K, N], N contiguous: w2 and w13 as stored, for the backward's products that
// contract over their rows).  A stage's weight tile holds its BK k-rows of BN
// columns as 16-byte chunks of 8 columns; chunk c of k-row k sits at slot
// 32 k + (c ^ 4 (k % 4)) of the stage, so one DMA instruction fills two whole
// k-rows (64 consecutive slots, lane-linear as the DMA writes) and the
// transposing fragment reads (load_frags below) hit 16 distinct 16-byte bank
// groups per half-wave.
struct OpsKm {
    __amdgpu_buffer_rsrc_t a, b;    // token / weight operand (this expert)
    int kb;                         // first k of this K slice
    int na;                         // token loads that hold a row of the tile
    int ldw;                        // N, elements per weight k-row
    uint32_t aoff[NLA], boff[NLB];  // byte offsets of this lane's token rows / weight chunks
};
static_assert(BN == 256 && BK == 64 && NLB * kWaves * 2 == BK,
              "the K-major weight layout: 32 chunks per k-row, two k-rows per DMA instruction");

// The same K-major weight-side layout for an operand whose k-rows are a
// ragged range of rows of a row-major [rows, ldw] matrix (the backward's
// per-position operands, one expert's segment): each k-tile's loads go
// through a buffer resource that starts at the k-tile's first row and ends
// at the range's end, so k-rows past the range read as zeros.  The token
// operand is addressed as in Ops<true>.
struct OpsKmR {
    __amdgpu_buffer_rsrc_t a;       // token operand
    const uint16_t *bp;             // first row of the range
    int kb;                         // first k of the token operand
    int na;                         // token loads that hold a row of the tile
    int ldw;                        // elements per row of the ranged operand
    int rows;                       // rows in the range
    uint32_t aoff[NLA], boff[NLB];  // byte offsets of this lane's token rows / chunks
};

// Token load i of a wave is issued only if its rows reach into the tile
// (i < na, wave-uniform): rows past the expert's segment are never stored, so
// their LDS rows may hold anything, and skipping them cuts the load traffic
// that bounds these kernels (a partial m-tile's rows).  With more than two
// stages the waits count loads per stage, so every load is issued.
template <typename OpsT>
__device__ __forceinline__ bool tok_load(const OpsT &op, int i) {
    return i < NLA && (NS > 2 || i < op.na);
}

// Buffer resource word 3 for raw (unstructured) buffer access on gfx9-class
// parts: 32-bit data format, no swizzle or index stride.
constexpr int kBufferWord3 = 0x00020000;

// Issue one k-tile of both operands straight into an LDS stage (global /
// buffer load to LDS, 16 bytes per lane: lane L's bytes land at base + 16 L,
// i.e. row L / kChunks, position L % kChunks of the instruction's rows).
// `wave` is the (scalar) wave index: the wave's rows of each operand start
// at wave * k{Tok,W}RowsPerWave.
template <int S>
__device__ __forceinline__ void issue_stage(uint16_t *smem, const Ops<true> &op, int k0,
                                            int wave) {
    const uint32_t so = 2u * (uint32_t)(op.kb + k0);
#pragma unroll
    for (int i = 0; i < (NLA > NLB ? NLA : NLB); ++i) {
        if (tok_load(op, i)) {
            uint16_t *da = smem + S * kTokStage + (wave * kTokRowsPerWave + i * kRowsPerLoad) * BK;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(op.a, (lds_void *)da, 16, op.aoff[i], so, 0,
                                                     0);
        }
        if (i < NLB) {
            uint16_t *db =
                smem + kWOff + S * kWStage + (wave * kWRowsPerWave + i * kRowsPerLoad) * BK;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(op.b, (lds_void *)db, 16, op.boff[i], so, 0,
                                                     0);
        }
    }
}
template <int S>
__device__ __forceinline__ void issue_stage(uint16_t *smem, const OpsKm &op, int k0, int wave) {
    const uint32_t so = 2u * (uint32_t)(op.kb + k0);
    const uint32_t sow = so * (uint32_t)op.ldw;  // k-tile start of the K-major weight
#pragma unroll
    for (int i = 0; i < (NLA > NLB ? NLA : NLB); ++i) {
        if (tok_load(op, i)) {
            uint16_t *da = smem + S * kTokStage + (wave * kTokRowsPerWave + i * kRowsPerLoad) * BK;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(op.a, (lds_void *)da, 16, op.aoff[i], so, 0,
                                                     0);
        }
        if (i < NLB) {
            uint16_t *db = smem + kWOff + S * kWStage + (wave * NLB + i) * 512;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(op.b, (lds_void *)db, 16, op.boff[i], sow, 0,
                                                     0);
        }
    }
}
template <int S>
__device__ __forceinline__ void issue_stage(uint16_t *smem, const OpsKmR &op, int k0, int wave) {
    const uint32_t so = 2u * (uint32_t)(op.kb + k0);
    // At most BK rows of the range from k0 on (a 32-bit record count).
    const int left = min(BK, max(0, op.rows - k0));
    const __amdgpu_buffer_rsrc_t b = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(op.bp + (int64_t)k0 * op.ldw), (short)0, left * op.ldw * 2, kBufferWord3);
#pragma unroll
    for (int i = 0; i < (NLA > NLB ? NLA : NLB); ++i) {
        if (tok_load(op, i)) {
            uint16_t *da = smem + S * kTokStage + (wave * kTokRowsPerWave + i * kRowsPerLoad) * BK;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(op.a, (lds_void *)da, 16, op.aoff[i], so, 0,
                                                     0);
        }
        if (i < NLB) {
            uint16_t *db = smem + kWOff + S * kWStage + (wave * NLB + i) * 512;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(b, (lds_void *)db, 16, op.boff[i], 0, 0, 0);
        }
    }
}
template <int S>
__device__ __forceinline__ void issue_stage(uint16_t *smem, const Ops<false> &op, int k0,
                                            int wave) {
#pragma unroll
    for (int i = 0; i < (NLA > NLB ? NLA : NLB); ++i) {
        if (tok_load(op, i)) {
            uint16_t *da = smem + S * kTokStage + (wave * kTokRowsPerWave + i * kRowsPerLoad) * BK;
            __builtin_amdgcn_global_load_lds(op.a[i] + k0, (lds_void *)da, 16, 0, 0);
        }
        if (i < NLB) {
            uint16_t *db =
                smem + kWOff + S * kWStage + (wave * kWRowsPerWave + i * kRowsPerLoad) * BK;
            __builtin_amdgcn_global_load_lds(op.b[i] + k0, (lds_void *)db, 16, 0, 0);
        }
    }
}

// Where a k-tile's loads are issued.  Early: at the top of the k-tile that
// precedes it, into the stage the previous barrier freed; the loads write
// LDS, so the compiler first waits for the fragment reads issued after that
// barrier.  Late: right after the barrier, before those reads, with nothing
// to wait for; the reads then queue behind the loads.  Measured on the part:
// late takes 3.5-6 % off FC2 (fine-grained and Mixtral-shaped layers) and
// adds 3 % to fine-grained FC1 (Mixtral-shaped FC1: -1 %), so FC2 issues late.
template <bool kGateUp>
constexpr bool late_issue() {
    return !kGateUp;
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// also drain the loads still in flight for later stages).  Callers wait for
// the loads they need first; every LDS read of the previous stage has
// completed because the MFMAs that consume it were issued before.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Fragments of one 16-wide k-step: NF weight fragments and MV token
// fragments, one ds_read_b128 each (row + lr, 16-byte chunk 2 ks + lk,
// swizzled; fragment rows start at multiples of 32, so swz(row) = swz(lr)).
// Token fragments MV..MF-1 hold no row of the expert and are skipped.
template <int MV>
struct Frags {
    bf16x8 w[NF], x[MV > 0 ? MV : 1];
};

// Per-lane byte addresses in LDS of this lane's first weight and token
// fragment rows at k-step j of stage 0; the stage, the fragment and the
// weight half are compile-time offsets on top.
struct FragAddr {
    uint32_t w[KS], x[KS];
};

// Row of weight fragment f within the wave's rows: FC1 holds gate fragments
// then the matching up fragments BN/2 rows further.
template <bool kGateUp>
constexpr int frag_row(int f) {
    return kGateUp ? (f < NF / 2 ? 0 : BN / 2) + (f % (NF / 2)) * 32 : f * 32;
}

template <int S, int J, int MV, bool kGateUp>
__device__ __forceinline__ void load_frags(Frags<MV> &fr, const char *lds, const FragAddr &fa) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
        fr.w[f] = *reinterpret_cast<const bf16x8 *>(
            lds + fa.w[J] + (S * kWStage + frag_row<kGateUp>(f) * BK) * 2);
#pragma unroll
    for (int g = 0; g < MV; ++g)
        fr.x[g] = *reinterpret_cast<const bf16x8 *>(lds + fa.x[J] + (S * kTokStage + g * 32 * BK) * 2);
}

// K-major weights: per lane, the LDS byte address of its first transposing
// read for each weight fragment of the wave (stage 0, k-step 0); the stage,
// the k-step and the second read are compile-time offsets on top.
struct FragAddrKm {
    uint32_t w[NF], x[KS];
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// A 32x32x16 A-operand fragment (lane l: weight column l % 32, k 8 (l / 32) ..
// + 7 of the k-step) from the K-major tile: two ds_read_b64_tr_b16.  In each
// 16-lane group the read hands lane i element i % 4 of the 8 bytes that lane
// 4 q + i / 4 addresses, as its q-th value; so with lane s of group g
// addressing k-row 8 (g / 2) + 4 h + s / 4, columns 16 (g % 2) + 4 (s % 4) ..
// + 3, lane s receives column 16 (g % 2) + s at those four k-rows.
template <int S, int J, int MV, bool kGateUp>
__device__ __forceinline__ void load_frags(Frags<MV> &fr, const char *lds, const FragAddrKm &fa) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const char *p = lds + fa.w[f] + S * kWStage * 2 + 16 * J * 512;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p + 4 * 512));
        fr.w[f] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int g = 0; g < MV; ++g)
        fr.x[g] = *reinterpret_cast<const bf16x8 *>(lds + fa.x[J] + (S * kTokStage + g * 32 * BK) * 2);
}

template <int MV>
__device__ __forceinline__ void mma_frags(f32x16 (&acc)[NF][MF], const Frags<MV> &fr) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int g = 0; g < MV; ++g)
            acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.w[f], fr.x[g], acc[f][g], 0, 0,
                                                                0);
}

// Scheduling masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Order the code since the last sched_barrier as: one fragment read, then
// NF*MV/(NF+MV) MFMAs, repeated, then the remaining MFMAs -- the reads of the
// next k-step travel behind this k-step's matrix-core work.
template <int MV>
__device__ __forceinline__ void interleave() {
    constexpr int nr = NF + MV, nm = NF * MV;
#pragma unroll
    for (int i = 0; i < nr; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, nm / nr > 0 ? nm / nr : 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, nm, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// Wait until at most `later` k-tiles' loads of this wave are in flight
// (0 <= later <= NS - 2, wave-uniform; negative means none) and every LDS
// read of this wave has returned.
template <int n>
__device__ __forceinline__ void wait_landed(int later) {
    if constexpr (n > 0) {
        if (later >= n) {
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(n * kLoadsPerStage) : "memory");
            return;
        }
        wait_landed<n - 1>(later);
    } else {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    }
}

// k-steps 1 .. KS-1 of stage S but the last: the reads for k-step j+1 are
// issued during the MFMAs of k-step j (fragments double-buffered).
template <int S, int J, int MV, bool kGateUp, typename FA>
__device__ __forceinline__ void k_steps(f32x16 (&acc)[NF][MF], Frags<MV> (&fr)[2], const char *lds,
                                        const FA &fa) {
    if constexpr (J + 1 < KS) {
        load_frags<S, J + 1, MV, kGateUp>(fr[(J + 1) & 1], lds, fa);
        mma_frags(acc, fr[J & 1]);
        interleave<MV>();
        k_steps<S, J + 1, MV, kGateUp>(acc, fr, lds, fa);
    }
}

// One k-tile of the k loop: k-tile kt from stage S.  k-tile kt + NS - 1 is
// issued into the stage freed by the previous k-tile's barrier, then the KS
// k-steps run; before the last k-step every wave waits until k-tile kt + 1
// has landed (later k-tiles stay in flight) and its own LDS reads are back,
// and one barrier makes k-tile kt + 1 visible to all waves and frees stage S;
// the fragments of k-tile kt + 1's first k-step are then read from its stage
// under the last k-step's MFMAs (after the last k-tile that stage holds data
// nobody uses).  Stage indices are compile-time, so the loop computes no
// addresses.
template <int S, int MV, bool kGateUp, typename OpsT, typename FA>
__device__ __forceinline__ void k_tile(f32x16 (&acc)[NF][MF], Frags<MV> (&fr)[2], uint16_t *smem,
                                       const OpsT &op, int kt, int nk, int wv, const FA &fa) {
    const char *lds = reinterpret_cast<const char *>(smem);
    if (!late_issue<kGateUp>() && kt + NS - 1 < nk)
        issue_stage<(S + NS - 1) % NS>(smem, op, (kt + NS - 1) * BK, wv);
    __builtin_amdgcn_sched_barrier(0);
    k_steps<S, 0, MV, kGateUp>(acc, fr, lds, fa);
    wait_landed<NS - 2>(min(nk - 2 - kt, NS - 2));
    stage_barrier();
    // Late issue: stage S is free from here on and no LDS read of this wave
    // is outstanding, so k-tile kt + NS goes out without waiting for any.
    if (late_issue<kGateUp>() && kt + NS < nk) issue_stage<S>(smem, op, (kt + NS) * BK, wv);
    load_frags<(S + 1) % NS, 0, MV, kGateUp>(fr[0], lds, fa);
    mma_frags(acc, fr[(KS - 1) & 1]);
    interleave<MV>();
}

template <int S, int MV, bool kGateUp, typename OpsT, typename FA>
__device__ __forceinline__ void k_tiles(f32x16 (&acc)[NF][MF], Frags<MV> (&fr)[2], uint16_t *smem,
                                        const OpsT &op, int kt, int nk, int wv, const FA &fa) {
    if constexpr (S < NS) {
        if (kt < nk) {
            k_tile<S, MV, kGateUp>(acc, fr, smem, op, kt, nk, wv, fa);
            k_tiles<S + 1, MV, kGateUp>(acc, fr, smem, op, kt + 1, nk, wv, fa);
        }
    }
}

template <int S, typename OpsT>
__device__ __forceinline__ void issue_first(uint16_t *smem, const OpsT &op, int nk, int wv) {
    if constexpr (S + 1 < NS) {
        if (S < nk) issue_stage<S>(smem, op, S * BK, wv);
        issue_first<S + 1>(smem, op, nk, wv);
    }
}

template <int MV, bool kGateUp, typename OpsT, typename FA>
__device__ __forceinline__ void k_loop(f32x16 (&acc)[NF][MF], uint16_t *smem, const OpsT &op,
                                       int nk, int wv, const FA &fa) {
    issue_first<0>(smem, op, nk, wv);
    wait_landed<NS - 2>(min(nk - 1, NS - 2));
    stage_barrier();
    if (late_issue<kGateUp>() && NS - 1 < nk) issue_stage<NS - 1>(smem, op, (NS - 1) * BK, wv);
    Frags<MV> fr[2];
    load_frags<0, 0, MV, kGateUp>(fr[0], reinterpret_cast<const char *>(smem), fa);
    int kt = 0;
    // Whole rounds of the ring with every stage index a constant, then the
    // remaining k-tiles.
    for (; kt + NS <= nk; kt += NS)
        k_tiles<0, MV, kGateUp>(acc, fr, smem, op, kt, nk, wv, fa);
    k_tiles<0, MV, kGateUp>(acc, fr, smem, op, kt, nk, wv, fa);
}

// A float32 epilogue store, non-temporal (streamed past the caches) with kNT:
// for outputs larger than the caches or not read again soon (fine-grained
// FC2 -3 %, the backward's products and weight gradients -1.5 to -2.3 %; the
// Mixtral-shaped FC2 output, which the combine reads back from the Infinity
// Cache, keeps plain stores: its combine ran 5 us slower after non-temporal
// ones).
// (A compile-time choice: a runtime one let the compiler merge the two
// stores into a plain one.)
template <bool kNT>
__device__ __forceinline__ void store_f32x4(float *p, const float4 &v) {
    if constexpr (kNT)
        __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4 *>(p));
    else
        *reinterpret_cast<float4 *>(p) = v;
}

// Operands of the FC1-form epilogue that applies the SiLU-and-mul backward
// to the recomputed gate/up (kBwd): per aligned position p and column c < N,
// from gate z and up u (the accumulators), G[p, c] and the slot's routing
// weight w = topk_w[sorted_slot[p]], with s = sigmoid(z) and a = z s u:
//   wact[p, c]       = bf16(w a)
//   dh13[p, c]       = bf16(w G u s (1 + z (1 - s)))      (d_gate)
//   dh13[p, N + c]   = bf16(w G z s)                      (d_up)
//   gw_part[p, nt]   = sum over the tile's columns c of G[p, c] a
// (n-tile nt of the launch; the routing-weight gradient is the sum of a
// row's parts in n-tile order, taken later).
struct BwdAct {
    const float *G;
    const float *topk_w;
    const int32_t *sorted_slot;
    uint16_t *wact, *dh13;
    float *gw_part;
    int n_tiles;
};

// The k loop and the epilogue of one tile whose waves hold MV valid token
// fragments.  Each MV has its accumulators to itself: declared outside the
// dispatch on MV, one set shared by the five loop versions measured slower
// (the register allocator copies it between them).
//
// kTrans (FC2 form): C is stored transposed, element (token-side row p,
// weight-side row n) at C[n * plane + p]; p's extent must be a multiple of 4.
template <int MV, bool kGateUp, bool kTrans = false, bool kBwd = false, bool kStream = true,
          typename OpsT, typename FA>
__device__ __forceinline__ void run_tile(uint16_t *smem, const OpsT &op, int nk, int wv,
                                         const FA &fa, const MTile &tile, int nt, int wn,
                                         int wm, int lr, int lk, int N, int ks, int64_t plane,
                                         void *__restrict__ Cv, const BwdAct &bw = BwdAct{}) {
    f32x16 acc[NF][MF];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int g = 0; g < MF; ++g) acc[f][g] = f32x16{};

    k_loop<MV, kGateUp>(acc, smem, op, nk, wv, fa);

    // Accumulator r of a 32x32 tile holds row 8 (r / 4) + 4 lk + (r % 4) of
    // the weight side and column lr of the token side.
    if constexpr (kGateUp && kBwd) {
        // SiLU-and-mul backward (BwdAct), fragment by fragment through this
        // wave's LDS slice: G's 32 x 32 block is loaded as whole 128-byte rows
        // and read back in the accumulators' layout (lane (lr, lk): row lr,
        // columns 8 rg + 4 lk .. + 3); the three bf16 results go the other
        // way and are stored as 64-byte rows.  The row sums of G . act of the
        // 4 waves sharing the rows meet in LDS and are added in wave order.
        static_assert(NF == 2, "one gate and one up fragment per wave");
        constexpr int kGP = 36;  // G slice pitch (floats)
        constexpr int kOP = 40;  // result slice pitch (bf16)
        constexpr int kSlice = 32 * kGP + 3 * 32 * kOP / 2;  // floats per wave
        float *gs = reinterpret_cast<float *>(smem) + wv * kSlice;
        uint16_t *os = reinterpret_cast<uint16_t *>(gs + 32 * kGP);
        float *red = reinterpret_cast<float *>(smem) + kWaves * kSlice;  // [WM][MF][32][WN]
        static_assert((kWaves * kSlice + WM * MF * 32 * WN) * 4 <= kLds * 2, "epilogue LDS");
        const int lane = lr + 32 * lk;
        const int c0 = nt * (BN / 2) + wn * (BN / 2 / WN);  // the wave's first column
        const bool cval = c0 < N;  // N % 32 == 0: the wave's 32 columns all valid or none
        uint16_t *const dst[3] = {bw.wact, bw.dh13, bw.dh13 + N};
        const int64_t ld[3] = {N, 2 * (int64_t)N, 2 * (int64_t)N};
#pragma unroll
        for (int g = 0; g < MV; ++g) {
            const int pb = tile.row0 + wm * (BM / WM) + g * 32;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 8 * i + (lane >> 3), cc = 4 * (lane & 7);
                f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
                if (pb + rr < tile.row_end && cval)
                    v = *reinterpret_cast<const f32x4 *>(bw.G + (int64_t)(pb + rr) * N + c0 + cc);
                *reinterpret_cast<f32x4 *>(gs + rr * kGP + cc) = v;
            }
            const int p = pb + lr;
            const bool ok = p < tile.row_end && cval;
            const float w = p < tile.row_end ? bw.topk_w[bw.sorted_slot[p]] : 0.f;
            float sum = 0.f;
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int c = rg * 8 + lk * 4;
                const f32x4 gg = *reinterpret_cast<const f32x4 *>(gs + lr * kGP + c);
                uint16_t r16[3][4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float z = acc[0][g][rg * 4 + q], u = acc[1][g][rg * 4 + q];
                    const float sg = 1.0f / (1.0f + __expf(-z));
                    const float a = z * sg * u;
                    r16[0][q] = __builtin_bit_cast(uint16_t, to_bf16(w * a));
                    sum += ok ? gg[q] * a : 0.f;
                    const float da = w * gg[q];
                    r16[1][q] = __builtin_bit_cast(uint16_t,
                                                   to_bf16(da * u * sg * (1.0f + z * (1.0f - sg))));
                    r16[2][q] = __builtin_bit_cast(uint16_t, to_bf16(da * z * sg));
                }
#pragma unroll
                for (int o = 0; o < 3; ++o)
                    *reinterpret_cast<uint2 *>(os + (o * 32 + lr) * kOP + c) =
                        uint2{r16[o][0] | ((uint32_t)r16[o][1] << 16),
                              r16[o][2] | ((uint32_t)r16[o][3] << 16)};
            }
#pragma unroll
            for (int o = 0; o < 3; ++o) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int rr = 16 * j + (lane >> 2), cc = 8 * (lane & 3);
                    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(os + (o * 32 + rr) * kOP + cc);
                    if (pb + rr < tile.row_end && cval)
                        *reinterpret_cast<bf16x8 *>(dst[o] + (int64_t)(pb + rr) * ld[o] + c0 + cc) =
                            v;
                }
            }
            sum += __shfl_xor(sum, 32);
            if (lk == 0) red[((wm * MF + g) * 32 + lr) * WN + wn] = sum;
        }
        __syncthreads();
        const int tid = threadIdx.x;
        if (tid < BM) {
            const int p = tile.row0 + tid;
            if (p < tile.row_end) {
                const float *r = red + ((tid / (BM / WM)) * MF + (tid % (BM / WM)) / 32) * 32 * WN +
                                 (tid % 32) * WN;
                float t = r[0];
#pragma unroll
                for (int i = 1; i < WN; ++i) t += r[i];
                bw.gw_part[(int64_t)p * bw.n_tiles + nt] = t;
            }
        }
    } else if (kGateUp) {
        // The block's activation tile (BM rows x BN / 2 columns, bf16) is
        // gathered in LDS from all waves, then stored as whole rows: each
        // instruction writes 4 rows x 256 bytes (straight from the
        // accumulators each instruction put 16 bytes into each of 32 rows:
        // measured 1-3 % slower).  Every wave runs the one barrier, whatever
        // its count of valid fragments.
        constexpr int kP = BN / 2 + 8;  // row pitch (bf16)
        uint16_t *ep = smem;
#pragma unroll
        for (int f = 0; f < NF / 2; ++f) {
#pragma unroll
            for (int g = 0; g < MV; ++g) {
                const int r = wm * (BM / WM) + g * 32 + lr;
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    bf16x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        o[q] = to_bf16(silu_f(acc[f][g][rg * 4 + q]) *
                                       acc[f + NF / 2][g][rg * 4 + q]);
                    *reinterpret_cast<bf16x4 *>(ep + r * kP + wn * (BN / 2 / WN) + f * 32 +
                                                rg * 8 + lk * 4) = o;
                }
            }
        }
        __syncthreads();
        const int tid = threadIdx.x;
        const int c = (tid & 15) * 8;
        const int n = nt * (BN / 2) + c;
#pragma unroll
        for (int r0 = 0; r0 < BM; r0 += kThreads / 16) {
            const int r = r0 + tid / 16;
            const int p = tile.row0 + r;
            if (p < tile.row_end && n < N)
                *reinterpret_cast<bf16x8 *>(static_cast<uint16_t *>(Cv) + (int64_t)p * N + n) =
                    *reinterpret_cast<const bf16x8 *>(ep + r * kP + c);
        }
    } else {
        // Each 32 x 32 fragment goes through this wave's slice of LDS (the
        // stages are free once the k loop's last barrier is passed): written
        // as the accumulators hold it, read back so that lane l holds 4
        // consecutive columns of row l / 8, and stored as 8 whole 128-byte
        // rows per instruction (written straight from the accumulators, each
        // instruction put 32 bytes into each of 32 rows: measured 3-5 %
        // slower on FC2 and the backward's products).  Row pitch 36 floats:
        // conflict-free writes.
        constexpr int kP = 36;
        float *ep = reinterpret_cast<float *>(smem) + wv * 32 * kP;
        float *C = static_cast<float *>(Cv) + (kTrans ? 0 : ks * plane);
        const int lane = lr + 32 * lk;
        const int rl = lane >> 3, cl = (lane & 7) * 4;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
#pragma unroll
            for (int g = 0; g < MV; ++g) {
                const f32x16 &a = acc[f][g];
#pragma unroll
                for (int rg = 0; rg < 4; ++rg)
                    *reinterpret_cast<float4 *>(ep + lr * kP + rg * 8 + lk * 4) =
                        make_float4(a[rg * 4], a[rg * 4 + 1], a[rg * 4 + 2], a[rg * 4 + 3]);
                const int p0 = tile.row0 + wm * (BM / WM) + g * 32;
                if constexpr (kTrans) {
                    // Lane l: weight-side row 8 i + l / 8 of the fragment,
                    // token-side rows 4 (l % 8) .. + 3 (a column of the slice).
                    const int p = p0 + cl;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int w = 8 * i + rl;
                        const float4 v = make_float4(ep[cl * kP + w], ep[(cl + 1) * kP + w],
                                                     ep[(cl + 2) * kP + w], ep[(cl + 3) * kP + w]);
                        const int n = nt * BN + wn * (BN / WN) + f * 32 + w;
                        if (p < tile.row_end && n < N)
                            store_f32x4<kStream>(C + (int64_t)n * plane + p, v);
                    }
                } else {
                    const int n = nt * BN + wn * (BN / WN) + f * 32 + cl;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float4 v =
                            *reinterpret_cast<const float4 *>(ep + (8 * i + rl) * kP + cl);
                        const int p = p0 + 8 * i + rl;
                        if (p < tile.row_end && n < N)
                            store_f32x4<kStream>(C + (int64_t)p * N + n, v);
                    }
                }
            }
        }
    }
}

// kGateUp: A = hidden [T, K] gathered through `gather`, W = w13 [E, 2N, K],
//          C = act [rows, N] bf16 = silu(gate) * up.
// else:    A = act [rows, K], W = w2 [E, N, K], C = y [rows, N] float32;
//          with ksplit > 1, K is cut into ksplit equal slices and slice s
//          writes its partial sums to plane s of y (planes `plane` floats
//          apart).
//
// kBuf selects the operand addressing (Ops); a_bytes is the token operand's
// size in bytes (used by kBuf only).
// kKm (FC2 form, buffer addressing only): W is K-major, [E, K, N].
// kBwd (FC1 form): the epilogue applies the SiLU-and-mul backward (BwdAct)
// instead of writing act.  kStream (FC2 form): y is stored non-temporally.
// With kKm, a non-null `gather` makes A one row per token, position p
// reading row gather[p] as the FC1 form does.
template <bool kGateUp, bool kBuf, bool kKm = false, bool kBwd = false, bool kStream = false>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bf16_kernel(
    const uint16_t *__restrict__ A, const int32_t *__restrict__ gather,
    const uint16_t *__restrict__ W, const int32_t *__restrict__ offsets, void *__restrict__ Cv,
    int E, int K, int N, int n_tiles, int ksplit, int64_t plane, int a_bytes, BwdAct bw) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[kLds];

    // Block -> tile.  Workgroups are dealt round-robin to the 8 XCDs (block b
    // runs on XCD b % 8), and each XCD has 32 CUs.  Tiles are handed out in
    // chunks of 32 consecutive tile indices per XCD, chunks round-robin over
    // the XCDs: the 32 tiles an XCD runs together are a few weight n-tiles of
    // one expert with all of its m-tiles under each, so they share weight and
    // token tiles in that XCD's L2, and the surplus blocks past the last tile
    // are spread evenly over the XCDs.
    const int bid = blockIdx.x;
    const int slot = bid >> 3;
    int L = ((slot / kXcdChunk) * 8 + (bid & 7)) * kXcdChunk + slot % kXcdChunk;
    // K slices are enumerated slice-major, so the tiles an XCD runs together
    // belong to one slice and still share operands.
    int ks = 0;
    if (ksplit > 1) {
        const int total = count_mtiles(offsets, E) * n_tiles;
        ks = L / total;
        if (ks >= ksplit) return;
        L -= ks * total;
    }
    MTile tile;
    int nt;
    if (!find_tile(offsets, E, L, n_tiles, tile, nt)) return;
    const int kper = K / ksplit;  // a multiple of BK (checked by the host)
    const int kbeg = ks * kper;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // Operand rows this lane loads: row wave * k{Tok,W}RowsPerWave +
    // kRowsPerLoad i + lane / kChunks of each tile; it lands at position
    // lane % kChunks, so it fetches global chunk (lane % kChunks) ^ swz(row)
    // of that row.  The wave index is made scalar so the LDS destinations (M0)
    // need no per-load conversion.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int rr = lane / kChunks;
    const int rows_w = kGateUp ? 2 * N : N;
    const uint16_t *We = W + (int64_t)tile.e * rows_w * K;
    static_assert(!kKm || (kBuf && !kGateUp), "K-major weights: FC2 form, buffer addressing");
    using OpsT = typename std::conditional<kKm, OpsKm, Ops<kBuf>>::type;
    OpsT op;
    if constexpr (kKm) op.ldw = N;
    if constexpr (kBuf) {
        op.a = __builtin_amdgcn_make_buffer_rsrc((void *)A, (short)0, a_bytes, kBufferWord3);
        op.b = __builtin_amdgcn_make_buffer_rsrc((void *)We, (short)0, rows_w * K * 2,
                                                 kBufferWord3);
        op.kb = __builtin_amdgcn_readfirstlane(kbeg);
    }
    op.na = __builtin_amdgcn_readfirstlane(
        min(NLA, max(0, (tile.row_end - tile.row0 - wv * kTokRowsPerWave + kRowsPerLoad - 1) /
                            kRowsPerLoad)));
#pragma unroll
    for (int i = 0; i < NLA; ++i) {
        const int r = wv * kTokRowsPerWave + i * kRowsPerLoad + rr;
        const int c8 = ((lane % kChunks) ^ swz(r)) * 8;
        const int p = min(tile.row0 + r, tile.row_end - 1);
        const int arow = (kGateUp || (kKm && gather != nullptr)) ? gather[p] : p;
        if constexpr (kBuf)
            op.aoff[i] = ((uint32_t)arow * (uint32_t)K + (uint32_t)c8) * 2u;
        else
            op.a[i] = A + (int64_t)arow * K + kbeg + c8;
    }
    if constexpr (kKm) {
#pragma unroll
        for (int i = 0; i < NLB; ++i) {
            // DMA instruction wv NLB + i fills k-rows kk = 2 (wv NLB + i) + lane / 32
            // of the tile, slot lane % 32 of each: chunk (lane % 32) ^ 4 (kk % 4).
            const int kk = 2 * (wv * NLB + i) + (lane >> 5);
            const int c = (lane & 31) ^ (4 * (kk & 3));
            const int n = min(nt * BN + 8 * c, N - 8);
            op.boff[i] = ((uint32_t)kk * (uint32_t)N + (uint32_t)n) * 2u;
        }
    }
#pragma unroll
    for (int i = 0; i < NLB && !kKm; ++i) {
        const int r = wv * kWRowsPerWave + i * kRowsPerLoad + rr;
        const int c8 = ((lane % kChunks) ^ swz(r)) * 8;
        int wrow;
        if (kGateUp) {
            const int n = min(nt * (BN / 2) + (r & (BN / 2 - 1)), N - 1);
            wrow = r < BN / 2 ? n : N + n;
        } else {
            wrow = min(nt * BN + r, N - 1);
        }
        if constexpr (kBuf && !kKm)
            op.boff[i] = ((uint32_t)wrow * (uint32_t)K + (uint32_t)c8) * 2u;
        else if constexpr (!kBuf)
            op.b[i] = We + (int64_t)wrow * K + kbeg + c8;
    }

    const int wn = wave % WN;
    const int wm = wave / WN;
    const int lr = lane & 31;
    const int lk = lane >> 5;
    // LDS byte addresses of this lane's fragment rows at each k-step of stage
    // 0: weight row wn * (rows per wave) + lr (FC1: of the gate half), token
    // row wm * (BM / WM) + lr, 16-byte chunk 2 j + lk swizzled.
    const int sw = swz(lr);
    const int wrow0 = kGateUp ? wn * (BN / 2 / WN) : wn * (BN / WN);
    const int xrow = wm * (BM / WM) + lr;
    using FA = typename std::conditional<kKm, FragAddrKm, FragAddr>::type;
    FA fa;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const uint32_t ch = (uint32_t)(((2 * j + lk) ^ sw) * 16);
        if constexpr (!kKm) fa.w[j] = (uint32_t)((kWOff + (wrow0 + lr) * BK) * 2) + ch;
        fa.x[j] = (uint32_t)(xrow * BK * 2) + ch;
    }
    if constexpr (kKm) {
        // Transposing reads: lane s of 16-lane group g addresses k-row
        // 8 (g / 2) + s / 4 (+ 16 j + 4 h), columns c = column of the fragment's
        // first row + 16 (g % 2) + 4 (s % 4) .. + 3, i.e. the half (s % 2) of
        // chunk c / 8; k-row % 4 = s / 4 for every j and h.
        const int g = lane >> 4, sl = lane & 15;
        const int krow = 8 * (g >> 1) + (sl >> 2);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int chunk = (wrow0 + 32 * f) / 8 + 2 * (g & 1) + ((sl & 3) >> 1);
            fa.w[f] = (uint32_t)(kWOff * 2 + (krow * 32 + (chunk ^ (4 * (sl >> 2)))) * 16 +
                                 8 * (sl & 1));
        }
    }

    // Token fragments of this wave that hold at least one row of the expert
    // (wave-uniform); a wave with none still takes part in loads and barriers.
    const int mvalid = min(MF, max(0, (tile.row_end - tile.row0 - wm * (BM / WM) + 31) / 32));
    const int nk = kper / BK;
    switch (mvalid) {
        case 5:
            if constexpr (MF >= 5)
                run_tile<5, kGateUp, false, kBwd, kStream>(smem, op, nk, wv, fa, tile, nt, wn, wm,
                                                           lr, lk, N, ks, plane, Cv, bw);
            break;
        case 4:
            run_tile<4, kGateUp, false, kBwd, kStream>(smem, op, nk, wv, fa, tile, nt, wn, wm, lr,
                                                       lk, N, ks, plane, Cv, bw);
            break;
        case 3:
            run_tile<3, kGateUp, false, kBwd, kStream>(smem, op, nk, wv, fa, tile, nt, wn, wm, lr,
                                                       lk, N, ks, plane, Cv, bw);
            break;
        case 2:
            run_tile<2, kGateUp, false, kBwd, kStream>(smem, op, nk, wv, fa, tile, nt, wn, wm, lr,
                                                       lk, N, ks, plane, Cv, bw);
            break;
        case 1:
            run_tile<1, kGateUp, false, kBwd, kStream>(smem, op, nk, wv, fa, tile, nt, wn, wm, lr,
                                                       lk, N, ks, plane, Cv, bw);
            break;
        default:
            run_tile<0, kGateUp, false, kBwd, kStream>(smem, op, nk, wv, fa, tile, nt, wn, wm, lr,
                                                       lk, N, ks, plane, Cv, bw);
            break;
    }
}

// Weight gradients on the same machinery: C_e [M, N] float32 (at C + e M N)
// = sum over the k of expert e of A[m, k] B[n, k].  A [M, ld] bf16 has k
// contiguous: the backward's operand transposed to [columns, positions], each
// expert's segment padded to whole k-tiles with zeros, k in [poff[e],
// poff[e+1]).  B is either the same kind of operand ([N, ld], kKmB false) or
// (kKmB) the per-position operand as stored, [positions, N] with N contiguous:
// its k-rows are expert e's positions [offs[e], offs[e+1]), read K-major
// through the transposing fragment reads, the rows past the segment read as
// zeros (OpsKmR).  kTrans stores C_e transposed, as [N, M].  Every expert has
// ceil(M / BM) x ceil(N / BN) tiles, numbered expert by expert in the banded
// order; m rows play the token rows' part, n rows the weight rows'.  An
// expert with no rows runs no k-tile and writes zeros.  A tile's cost is its
// expert's row count, so with `chunked` (experts with at least a chunk of
// tiles for every XCD) tiles go to the XCDs in chunks as in the forward,
// sharing operands in each L2; otherwise block b takes tile b, spreading
// every expert over all XCDs (a chunk would put most of a skewed expert's
// work on one XCD).
template <bool kKmB, bool kTrans>
__global__ __launch_bounds__(kThreads, 1) void grouped_wgrad_bf16_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, int ld,
    const int32_t *__restrict__ poff, const int32_t *__restrict__ offs, int E, int M, int N,
    int m_tiles, int n_tiles, float *__restrict__ C, int a_bytes, int b_bytes, int chunked) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[kLds];
    const int bid = blockIdx.x;
    const int slot = bid >> 3;
    const int L = chunked ? ((slot / kXcdChunk) * 8 + (bid & 7)) * kXcdChunk + slot % kXcdChunk
                          : bid;
    const int per_e = m_tiles * n_tiles;
    if (L >= E * per_e) return;
    const int e = L / per_e;
    int mi, nt;
    band_tile(L - e * per_e, m_tiles, n_tiles, mi, nt);
    MTile tile;
    tile.e = e;
    tile.row0 = mi * BM;
    tile.row_end = min(M, tile.row0 + BM);
    const int kbeg = poff[e];
    const int nk = (poff[e + 1] - kbeg) / BK;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int rr = lane / kChunks;
    using OpsT = typename std::conditional<kKmB, OpsKmR, Ops<true>>::type;
    OpsT op;
    op.a = __builtin_amdgcn_make_buffer_rsrc((void *)A, (short)0, a_bytes, kBufferWord3);
    if constexpr (kKmB) {
        const int r0 = __builtin_amdgcn_readfirstlane(offs[e]);
        op.bp = B + (int64_t)r0 * N;
        op.rows = __builtin_amdgcn_readfirstlane(offs[e + 1] - r0);
        op.ldw = N;
    } else {
        op.b = __builtin_amdgcn_make_buffer_rsrc((void *)B, (short)0, b_bytes, kBufferWord3);
    }
    op.kb = __builtin_amdgcn_readfirstlane(kbeg);
    op.na = __builtin_amdgcn_readfirstlane(
        min(NLA, max(0, (tile.row_end - tile.row0 - wv * kTokRowsPerWave + kRowsPerLoad - 1) /
                            kRowsPerLoad)));
#pragma unroll
    for (int i = 0; i < NLA; ++i) {
        const int r = wv * kTokRowsPerWave + i * kRowsPerLoad + rr;
        const int c8 = ((lane % kChunks) ^ swz(r)) * 8;
        const int m = min(tile.row0 + r, tile.row_end - 1);
        op.aoff[i] = ((uint32_t)m * (uint32_t)ld + (uint32_t)c8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < NLB; ++i) {
        if constexpr (kKmB) {
            // As for OpsKm: DMA instruction wv NLB + i fills k-rows
            // kk = 2 (wv NLB + i) + lane / 32 of the stage, chunk
            // (lane % 32) ^ 4 (kk % 4) of each.
            const int kk = 2 * (wv * NLB + i) + (lane >> 5);
            const int c = (lane & 31) ^ (4 * (kk & 3));
            const int n = min(nt * BN + 8 * c, N - 8);
            op.boff[i] = ((uint32_t)kk * (uint32_t)N + (uint32_t)n) * 2u;
        } else {
            const int r = wv * kWRowsPerWave + i * kRowsPerLoad + rr;
            const int c8 = ((lane % kChunks) ^ swz(r)) * 8;
            const int n = min(nt * BN + r, N - 1);
            op.boff[i] = ((uint32_t)n * (uint32_t)ld + (uint32_t)c8) * 2u;
        }
    }

    const int wn = wave % WN;
    const int wm = wave / WN;
    const int lr = lane & 31;
    const int lk = lane >> 5;
    const int sw = swz(lr);
    const int wrow0 = wn * (BN / WN);
    const int xrow = wm * (BM / WM) + lr;
    using FA = typename std::conditional<kKmB, FragAddrKm, FragAddr>::type;
    FA fa;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const uint32_t ch = (uint32_t)(((2 * j + lk) ^ sw) * 16);
        if constexpr (!kKmB) fa.w[j] = (uint32_t)((kWOff + (wrow0 + lr) * BK) * 2) + ch;
        fa.x[j] = (uint32_t)(xrow * BK * 2) + ch;
    }
    if constexpr (kKmB) {
        // The transposing reads' addresses, as in the forward kernel.
        const int g = lane >> 4, sl = lane & 15;
        const int krow = 8 * (g >> 1) + (sl >> 2);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int chunk = (wrow0 + 32 * f) / 8 + 2 * (g & 1) + ((sl & 3) >> 1);
            fa.w[f] = (uint32_t)(kWOff * 2 + (krow * 32 + (chunk ^ (4 * (sl >> 2)))) * 16 +
                                 8 * (sl & 1));
        }
    }
    float *Ce = C + (int64_t)e * M * N;
    const int mvalid = min(MF, max(0, (tile.row_end - tile.row0 - wm * (BM / WM) + 31) / 32));
    switch (mvalid) {
        case 5:
            if constexpr (MF >= 5)
                run_tile<5, false, kTrans>(smem, op, nk, wv, fa, tile, nt, wn, wm, lr, lk, N, 0, M,
                                           Ce);
            break;
        case 4:
            run_tile<4, false, kTrans>(smem, op, nk, wv, fa, tile, nt, wn, wm, lr, lk, N, 0, M, Ce);
            break;
        case 3:
            run_tile<3, false, kTrans>(smem, op, nk, wv, fa, tile, nt, wn, wm, lr, lk, N, 0, M, Ce);
            break;
        case 2:
            run_tile<2, false, kTrans>(smem, op, nk, wv, fa, tile, nt, wn, wm, lr, lk, N, 0, M, Ce);
            break;
        case 1:
            run_tile<1, false, kTrans>(smem, op, nk, wv, fa, tile, nt, wn, wm, lr, lk, N, 0, M, Ce);
            break;
        default:
            run_tile<0, false, kTrans>(smem, op, nk, wv, fa, tile, nt, wn, wm, lr, lk, N, 0, M, Ce);
            break;
    }
}

int m_slot_bound(int64_t rows, int E) {
    const int64_t nz = rows < E ? rows : E;
    return (int)((rows + BM - 1) / BM + nz);
}

// Blocks for an upper bound of m_slots * n_tiles tiles, rounded up to whole
// rounds of 8 XCDs x kXcdChunk so the block -> tile map is a bijection.
unsigned grid_of(int m_slots, int n_tiles) {
    const int64_t round = 8 * kXcdChunk;
    const int64_t total = (int64_t)m_slots * n_tiles;
    return (unsigned)((total + round - 1) / round * round);
}

}  // namespace

// The buffer-addressed kernels need every operand byte offset to fit in a
// signed 32-bit value.  MOE_GEMM_POINTER_PATH=1 in the environment forces the
// 64-bit pointer path (tests use it to cover that path at small sizes).
bool use_buffer_path(int64_t a_bytes, int64_t w_bytes) {
    const char *v = std::getenv("MOE_GEMM_POINTER_PATH");  // read per launch (host only)
    const bool forced = v != nullptr && v[0] == '1';
    const int64_t lim = (int64_t)1 << 31;
    return !forced && a_bytes < lim && w_bytes < lim;
}

hipError_t launch_gate_up_bf16(const uint16_t *hidden, const uint16_t *w13,
                               const int32_t *offsets, const int32_t *sorted_tok, int64_t T,
                               int H, int I, int E, int k, uint16_t *act, hipStream_t s) {
    const int64_t rows = T * k;
    if (rows == 0) return hipSuccess;
    const int m_slots = m_slot_bound(rows, E);
    const int n_tiles = (I + BN / 2 - 1) / (BN / 2);
    const int64_t a_bytes = T * H * 2, w_bytes = (int64_t)2 * I * H * 2;
    const dim3 grid(grid_of(m_slots, n_tiles));
    if (use_buffer_path(a_bytes, w_bytes))
        hipLaunchKernelGGL((grouped_gemm_bf16_kernel<true, true>), grid, dim3(kThreads), 0, s,
                           hidden, sorted_tok, w13, offsets, act, E, H, I, n_tiles, 1, (int64_t)0,
                           (int)a_bytes, BwdAct{});
    else
        hipLaunchKernelGGL((grouped_gemm_bf16_kernel<true, false>), grid, dim3(kThreads), 0, s,
                           hidden, sorted_tok, w13, offsets, act, E, H, I, n_tiles, 1, (int64_t)0,
                           0, BwdAct{});
    return hipGetLastError();
}

bool gate_up_bwd_ok(int64_t T, int H, int I) {
    return use_buffer_path(T * H * 2, (int64_t)2 * I * H * 2);
}

hipError_t launch_gate_up_bwd_bf16(const uint16_t *hidden, const uint16_t *w13,
                                   const int32_t *offsets, const int32_t *sorted_tok,
                                   const int32_t *sorted_slot, const float *topk_w,
                                   const float *G, int64_t T, int H, int I, int E, int k,
                                   uint16_t *wact, uint16_t *dh13, float *gw_part,
                                   hipStream_t s) {
    const int64_t rows = T * k;
    if (rows == 0) return hipSuccess;
    if (!gate_up_bwd_ok(T, H, I)) return hipErrorInvalidValue;
    const int m_slots = m_slot_bound(rows, E);
    const int n_tiles = gate_up_bwd_tiles(I);
    const dim3 grid(grid_of(m_slots, n_tiles));
    BwdAct bw;
    bw.G = G;
    bw.topk_w = topk_w;
    bw.sorted_slot = sorted_slot;
    bw.wact = wact;
    bw.dh13 = dh13;
    bw.gw_part = gw_part;
    bw.n_tiles = n_tiles;
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<true, true, false, true>), grid, dim3(kThreads),
                       0, s, hidden, sorted_tok, w13, offsets, nullptr, E, H, I, n_tiles, 1,
                       (int64_t)0, (int)(T * H * 2), bw);
    return hipGetLastError();
}

int gate_up_bwd_tiles(int I) { return (I + BN / 2 - 1) / (BN / 2); }

bool down_kmajor_ok(int64_t T, int N, int K, int k) {
    const int64_t a_bytes = T * k * (int64_t)K * 2, w_bytes = (int64_t)K * N * 2;
    return use_buffer_path(a_bytes, w_bytes);
}

hipError_t launch_down_kmajor_bf16(const uint16_t *a, const int32_t *gather, const uint16_t *w,
                                   const int32_t *offsets, int64_t T, int N, int K, int E, int k,
                                   float *y, hipStream_t s) {
    const int64_t rows = T * k;
    if (rows == 0) return hipSuccess;
    if (!down_kmajor_ok(T, N, K, k)) return hipErrorInvalidValue;
    const int m_slots = m_slot_bound(rows, E);
    const int n_tiles = (N + BN - 1) / BN;
    const dim3 grid(grid_of(m_slots, n_tiles));
    const int64_t a_bytes = (gather != nullptr ? T : rows) * K * 2;
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<false, true, true, false, true>), grid,
                       dim3(kThreads), 0, s, a, gather, w, offsets, y, E, K, N, n_tiles, 1,
                       rows * N, (int)a_bytes, BwdAct{});
    return hipGetLastError();
}

bool wgrad_grouped_ok(int M, int N, int64_t ld) {
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)M * ld * 2 < lim && (int64_t)N * ld * 2 < lim && ld % BK == 0;
}

hipError_t launch_wgrad_bf16(const uint16_t *a, const uint16_t *b, int64_t ld,
                             const int32_t *poff, int E, int M, int N, float *c, hipStream_t s) {
    if (!wgrad_grouped_ok(M, N, ld)) return hipErrorInvalidValue;
    const int m_tiles = (M + BM - 1) / BM, n_tiles = (N + BN - 1) / BN;
    const dim3 grid(grid_of(m_tiles * E, n_tiles));
    const int chunked = m_tiles * n_tiles >= 8 * kXcdChunk;
    hipLaunchKernelGGL((grouped_wgrad_bf16_kernel<false, false>), grid, dim3(kThreads), 0, s, a, b,
                       (int)ld, poff, nullptr, E, M, N, m_tiles, n_tiles, c, (int)(M * ld * 2),
                       (int)(N * ld * 2), chunked);
    return hipGetLastError();
}

bool wgrad_km_ok(int M, int N, int64_t ld) {
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)M * ld * 2 < lim && (int64_t)BK * N * 2 < lim && ld % BK == 0 && N % 8 == 0 &&
           M % 4 == 0;
}

hipError_t launch_wgrad_km_bf16(const uint16_t *a, const uint16_t *b, int64_t ld,
                                const int32_t *poff, const int32_t *offs, int E, int M, int N,
                                bool trans, float *c, hipStream_t s) {
    if (!wgrad_km_ok(M, N, ld)) return hipErrorInvalidValue;
    const int m_tiles = (M + BM - 1) / BM, n_tiles = (N + BN - 1) / BN;
    const dim3 grid(grid_of(m_tiles * E, n_tiles));
    const int chunked = m_tiles * n_tiles >= 8 * kXcdChunk;
    if (trans)
        hipLaunchKernelGGL((grouped_wgrad_bf16_kernel<true, true>), grid, dim3(kThreads), 0, s, a,
                           b, (int)ld, poff, offs, E, M, N, m_tiles, n_tiles, c,
                           (int)(M * ld * 2), 0, chunked);
    else
        hipLaunchKernelGGL((grouped_wgrad_bf16_kernel<true, false>), grid, dim3(kThreads), 0, s, a,
                           b, (int)ld, poff, offs, E, M, N, m_tiles, n_tiles, c,
                           (int)(M * ld * 2), 0, chunked);
    return hipGetLastError();
}

int down_splits(int64_t T, int H, int I, int E, int k) {
    // Expected tiles: every full BM rows plus about half a partial m-tile per
    // expert that has rows.  A slice count is worth its extra y plane (written
    // here, read again by the combine: measured at about 8% of the FC2 time
    // each on the Mixtral-shaped layer) when it fills the last round of 256
    // CUs better; slices keep K / ksplit >= 1024 and a multiple of BK.
    const int64_t rows = T * k;
    if (rows == 0) return 1;
    const int64_t nz = rows < E ? rows : E;
    const double tiles = (double)((rows + BM - 1) / BM + nz / 2) * ((H + BN - 1) / BN);
    int best = 1;
    double best_score = 0.0;
    for (int sp = 1; sp <= 4; ++sp) {
        if (sp > 1 && (I % (sp * BK) != 0 || I / sp < 1024)) continue;
        const double rounds = tiles * sp / 256.0;
        const double score = rounds / std::ceil(rounds) - 0.08 * (sp - 1);
        if (score > best_score + 1e-9) {
            best_score = score;
            best = sp;
        }
    }
    return best;
}

hipError_t launch_down_bf16(const uint16_t *act, const uint16_t *w2, const int32_t *offsets,
                            int64_t T, int H, int I, int E, int k, int ksplit, float *y,
                            hipStream_t s) {
    const int64_t rows = T * k;
    if (rows == 0) return hipSuccess;
    const int m_slots = m_slot_bound(rows, E);
    const int n_tiles = (H + BN - 1) / BN;
    const int64_t a_bytes = rows * I * 2, w_bytes = (int64_t)H * I * 2;
    const dim3 grid(grid_of(m_slots * ksplit, n_tiles));
    // y streams past the caches when it is larger than the Infinity Cache.
    const bool stream_y = (int64_t)ksplit * rows * H * 4 > ((int64_t)256 << 20);
    if (!use_buffer_path(a_bytes, w_bytes))
        hipLaunchKernelGGL((grouped_gemm_bf16_kernel<false, false>), grid, dim3(kThreads), 0, s,
                           act, nullptr, w2, offsets, y, E, I, H, n_tiles, ksplit, rows * H, 0,
                           BwdAct{});
    else if (stream_y)
        hipLaunchKernelGGL((grouped_gemm_bf16_kernel<false, true, false, false, true>), grid,
                           dim3(kThreads), 0, s, act, nullptr, w2, offsets, y, E, I, H, n_tiles,
                           ksplit, rows * H, (int)a_bytes, BwdAct{});
    else
        hipLaunchKernelGGL((grouped_gemm_bf16_kernel<false, true>), grid, dim3(kThreads), 0, s,
                           act, nullptr, w2, offsets, y, E, I, H, n_tiles, ksplit, rows * H,
                           (int)a_bytes, BwdAct{});
    return hipGetLastError();
}

}  // namespace moe
