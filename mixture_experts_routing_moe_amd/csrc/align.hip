// Expert alignment: histogram -> exclusive offsets -> stable expert-major order.
//
// Method: mlc-llm moe_misc.py, moe_cumsum / get_indices / get_indptr.  The
// pages form a dense [E, T] mask and take one inclusive prefix sum over all
// E*T entries; position (e, t) of that sum is 1 + the place of token t in
// expert e's contiguous segment.  The same numbers come out of an O(T*k)
// pipeline that never builds the mask:
//
//   1. align_hist:    each block counts the ids of its contiguous chunk of
//                     flat slots into an LDS histogram -> partial[b][e].
//   2. align_scatter: each block sums the partials into per-expert totals,
//                     the exclusive offsets (the indptr) and the first
//                     position it may write for each expert, then walks its
//                     chunk in order, 512 slots at a time; a slot's rank among
//                     earlier slots of the same expert comes from ballots
//                     inside its wave plus the counts of the waves before it,
//                     so positions follow the flat slot order t*k+j --
//                     ascending token inside each expert, exactly the order
//                     of the pages' cumsum.
//
//   With at most 512 slots one scatter block does it all, counting the ids
//   itself, and the histogram kernel is skipped.
//
// Only integer LDS atomics on private counters are used, and no result
// depends on their order, so the output is identical on every run.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

#ifndef MOE_ALIGN_THREADS
#define MOE_ALIGN_THREADS 512
#endif
constexpr int kAlignThreads = MOE_ALIGN_THREADS;
constexpr int kAlignWaves = kAlignThreads / kWave;
#ifndef MOE_ALIGN_BUDGET
#define MOE_ALIGN_BUDGET 16384
#endif
#ifndef MOE_ALIGN_SLOTS
#define MOE_ALIGN_SLOTS 512
#endif
constexpr int kPartialBudget = MOE_ALIGN_BUDGET;  // cap on nb * E partial counts each scatter block sums
constexpr int kSlotsPerBlock = MOE_ALIGN_SLOTS;   // slots per block before the cap
// Partial-count rows a scatter thread loads per batch (all in flight at once).
constexpr int kRowBatch = kPartialBudget / kAlignThreads;

int64_t align_chunk(int64_t n, int nb) {
    int64_t c = (n + nb - 1) / nb;
    return (c + kAlignThreads - 1) / kAlignThreads * kAlignThreads;
}

__global__ __launch_bounds__(kAlignThreads) void align_hist_kernel(
    const int32_t *__restrict__ ids, int64_t n, int E, int64_t chunk,
    int32_t *__restrict__ partial) {
    extern __shared__ int32_t hist[];
    for (int e = threadIdx.x; e < E; e += kAlignThreads) hist[e] = 0;
    __syncthreads();
    const int64_t lo = (int64_t)blockIdx.x * chunk;
    const int64_t hi = lo + chunk < n ? lo + chunk : n;
    for (int64_t s = lo + threadIdx.x; s < hi; s += kAlignThreads) {
        const int e = ids[s];
        if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kAlignThreads)
        partial[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Block-wide exclusive scan of v[0..n) in LDS (n <= 4 * kAlignThreads),
// written to out[0..n); returns the total.  All threads must call it.
__device__ int block_exclusive_scan(const int32_t *v, int32_t *out, int n, int32_t *wsum) {
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    int x[4];
    int tsum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid * 4 + i;
        x[i] = e < n ? v[e] : 0;
        tsum += x[i];
    }
    int incl = tsum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kAlignThreads / kWave; ++w) {
        const int ws = wsum[w];
        if (w < wave) before += ws;
        total += ws;
    }
    int run = before + incl - tsum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid * 4 + i;
        if (e < n) out[e] = run;
        run += x[i];
    }
    __syncthreads();
    return total;
}

// Scan + scatter.  Every block first turns the per-block histograms into the
// expert totals, the exclusive expert offsets and its own first position per
// expert (block 0 also writes counts and offsets); then it walks its chunk
// in order, 512 slots at a time: a slot's rank among earlier slots of the
// same expert comes from ballots inside its wave plus the counts of the
// waves before it, so positions follow the flat slot order.
//
// With one block (n <= 512 slots: decode batches) the block counts the ids
// itself (fused_hist) and the histogram kernel is not launched.
__device__ __forceinline__ void align_scatter_block(
    int b, const int32_t *__restrict__ ids, int n, int k, int E, int chunk, int nbits, int nb,
    int fused_hist, const int32_t *__restrict__ partial, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_tok,
    int32_t *__restrict__ sorted_slot, int32_t *__restrict__ slot_to_sorted, int32_t *sm) {
    // LDS: run[E] | wcnt[W][E] | tot[E] | off[E] | tot_part[P][E] | pre_part[P][E] | wsum[W]
    // (W waves, P parts)
    const int parts = E < kAlignThreads ? kAlignThreads / E : 1;
    int32_t *run = sm;
    int32_t *wcnt = run + E;
    int32_t *tot = wcnt + kAlignWaves * E;
    int32_t *off = tot + E;
    int32_t *tot_part = off + E;
    int32_t *pre_part = tot_part + parts * E;
    int32_t *wsum = pre_part + parts * E;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;

    if (fused_hist) {
        for (int idx = tid; idx < parts * E; idx += kAlignThreads) {
            tot_part[idx] = 0;
            pre_part[idx] = 0;
        }
        __syncthreads();
        for (int s = tid; s < n; s += kAlignThreads) {
            const int e = ids[s];
            if ((unsigned)e < (unsigned)E) atomicAdd(&tot_part[e], 1);
        }
    }
    // The first ids of the chunk, loaded before the partial sums below so
    // that both loads are in flight together.
    const int lo = b * chunk;
    const int hi = lo + chunk < n ? lo + chunk : n;
    int e_first = -1;
    if (lo + tid < hi) e_first = ids[lo + tid];

    // Per (part, expert): sums over the blocks part, part + parts, ... -- all
    // of them and those before b.  Threads of one pass read consecutive
    // experts of one block row (coalesced).  The loads go out in batches of
    // kRowBatch, each issued whole before its first value is used: when E
    // divides 512 a thread sums at most kRowBatch blocks (nb <= 16384 / E
    // over parts = 512 / E threads), so that is one memory round trip.
    for (int idx = tid; idx < (fused_hist ? 0 : parts * E); idx += kAlignThreads) {
        const int e = idx % E, part = idx / E;
        int all = 0, pre = 0;
        for (int r0 = part; r0 < nb; r0 += kRowBatch * parts) {
            int c[kRowBatch];
#pragma unroll
            for (int i = 0; i < kRowBatch; ++i) {
                const int bb = r0 + i * parts;
                c[i] = bb < nb ? partial[(int64_t)bb * E + e] : 0;
            }
#pragma unroll
            for (int i = 0; i < kRowBatch; ++i) {
                all += c[i];
                pre += r0 + i * parts < b ? c[i] : 0;
            }
        }
        tot_part[part * E + e] = all;
        pre_part[part * E + e] = pre;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kAlignThreads) {
        int all = 0, pre = 0;
        for (int part = 0; part < parts; ++part) {
            all += tot_part[part * E + e];
            pre += pre_part[part * E + e];
        }
        tot[e] = all;
        run[e] = pre;
    }
    for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) wcnt[i] = 0;
    __syncthreads();
    const int total = block_exclusive_scan(tot, off, E, wsum);
    for (int e = tid; e < E; e += kAlignThreads) {
        run[e] += off[e];
        if (b == 0) {
            counts[e] = tot[e];
            offsets[e] = off[e];
        }
    }
    if (b == 0 && tid == 0) offsets[E] = total;
    // Positions past the valid slots (ids outside [0, E)) read -1.
    for (int p = total + b * kAlignThreads + tid; p < n; p += nb * kAlignThreads) {
        sorted_tok[p] = -1;
        sorted_slot[p] = -1;
    }
    __syncthreads();

    for (int it = lo; it < hi; it += kAlignThreads) {
        const int s = it + tid;
        int e = e_first;
        if (it != lo) e = s < hi ? ids[s] : -1;
        const bool ok = (unsigned)e < (unsigned)E;
        // Lanes of this wave holding the same expert: filter by each id bit.
        uint64_t peers = __ballot(ok);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool set = (e >> bit) & 1;
            const uint64_t m = __ballot(ok && set);
            peers &= set ? m : ~m;
        }
        const int rank = __popcll(peers & lanemask_lt());
        const int cnt = __popcll(peers);
        if (ok && rank == 0) wcnt[wave * E + e] = cnt;
        __syncthreads();
        if (ok) {
            int pos = run[e] + rank;
            for (int w = 0; w < wave; ++w) pos += wcnt[w * E + e];
            sorted_tok[pos] = s / k;
            sorted_slot[pos] = s;
            slot_to_sorted[s] = pos;
        } else if (s < hi) {
            slot_to_sorted[s] = -1;
        }
        if (it + kAlignThreads >= hi) break;  // the last pass needs no hand-over
        __syncthreads();
        if (ok && rank == 0) {
            atomicAdd(&run[e], cnt);
            wcnt[wave * E + e] = 0;
        }
        __syncthreads();
    }
}

// Blocks nb and up (launched only with inv_w) convert the [T, E] multihot
// maps to indices instead (E <= 256, E % 4 == 0, k <= 16: 16 lanes per row,
// 4 rows per wave, 4, 8 or 16 columns per lane), the work of
// moe_multihot_to_indices, in the same launch as the scatter it does not
// depend on.
__global__ __launch_bounds__(kAlignThreads) void align_scatter_kernel(
    const int32_t *__restrict__ ids, int n, int k, int E, int chunk, int nbits, int nb,
    int fused_hist, const int32_t *__restrict__ partial, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_tok,
    int32_t *__restrict__ sorted_slot, int32_t *__restrict__ slot_to_sorted,
    const float *__restrict__ pim, const int32_t *__restrict__ pos, float *__restrict__ inv_w,
    int32_t *__restrict__ inv_ids) {
    extern __shared__ int32_t sm[];
    if ((int)blockIdx.x >= nb) {
        const int lane = lane_id();
        const int64_t T = n / k;
        const int wave = ((int)blockIdx.x - nb) * kAlignWaves + (int)threadIdx.x / kWave;
        const int nwaves = ((int)gridDim.x - nb) * kAlignWaves;
        for (int64_t t0 = (int64_t)wave * 4; t0 < T; t0 += (int64_t)nwaves * 4) {
            const int64_t t = t0 + (lane >> 4);
            if (E <= 64)
                to_indices_row16<4>(pim, pos, T, t, E, k, inv_w, inv_ids, lane & 15);
            else if (E <= 128)
                to_indices_row16<8>(pim, pos, T, t, E, k, inv_w, inv_ids, lane & 15);
            else
                to_indices_row16<16>(pim, pos, T, t, E, k, inv_w, inv_ids, lane & 15);
        }
        return;
    }
    align_scatter_block(blockIdx.x, ids, n, k, E, chunk, nbits, nb, fused_hist, partial, counts,
                        offsets, sorted_tok, sorted_slot, slot_to_sorted, sm);
}

// Route + align in one block (at most kAlignThreads slots, E <= 64, k <= 16):
// the block's 8 waves route 4 rows each per pass with route16_row (the
// moe_route / moe_route_multihot selection), then the block aligns the ids it
// has just written, counting them itself.
__global__ __launch_bounds__(kAlignThreads) void route_align_small_kernel(
    const float *__restrict__ logits, int T, int E, int k, int norm, int vec4,
    float *__restrict__ topk_w, int32_t *__restrict__ topk_ids, uint8_t *__restrict__ multihot,
    float *__restrict__ pim, int32_t *__restrict__ pos, int chunk, int nbits,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_tok, int32_t *__restrict__ sorted_slot,
    int32_t *__restrict__ slot_to_sorted, float *__restrict__ inv_w,
    int32_t *__restrict__ inv_ids) {
    extern __shared__ int32_t sm[];
    const int lane = lane_id();
    const int g = lane >> 4;
    const int q = lane & 15;
    const int wave = threadIdx.x / kWave;
    for (int t0 = wave * 4; t0 < T; t0 += kAlignWaves * 4)
        route16_row(logits, T, t0 + g, E, k, norm, vec4, topk_w, topk_ids, multihot, pim, pos, g,
                    q);
    __syncthreads();  // every id and map row of the batch is written before the block reads them
    align_scatter_block(0, topk_ids, T * k, k, E, chunk, nbits, 1, 1, nullptr, counts, offsets,
                        sorted_tok, sorted_slot, slot_to_sorted, sm);
    // With inv_w: the multihot maps back to indices (moe_multihot_to_indices),
    // read from the rows written above.
    if (inv_w != nullptr)
        for (int t0 = wave * 4; t0 < T; t0 += kAlignWaves * 4)
            to_indices_row16<4>(pim, pos, T, t0 + g, E, k, inv_w, inv_ids, q);
}

// Route + align in one wave (at most 64 slots, E <= 64, k <= 16: decode
// batches of up to 64 / k tokens).  The wave routes its rows with
// route16_row and keeps the ids in LDS; lane s then takes slot s: its rank
// among the earlier slots of the same expert comes from ceil(log2 E) ballots
// (as in the scatter), the expert leaders record the counts, and lane e
// scans them into the exclusive offsets.  Same outputs as the block path.
__global__ __launch_bounds__(kWave) void route_align_wave_kernel(
    const float *__restrict__ logits, int T, int E, int k, int norm, int vec4,
    float *__restrict__ topk_w, int32_t *__restrict__ topk_ids, uint8_t *__restrict__ multihot,
    float *__restrict__ pim, int32_t *__restrict__ pos, int nbits, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_tok,
    int32_t *__restrict__ sorted_slot, int32_t *__restrict__ slot_to_sorted,
    float *__restrict__ inv_w, int32_t *__restrict__ inv_ids) {
    __shared__ int32_t s_ids[kWave];
    __shared__ int32_t s_cnt[kWave];
    __shared__ int32_t s_off[kWave + 1];
    const int lane = lane_id();
    const int g = lane >> 4;
    const int q = lane & 15;
    const int n = T * k;
    s_ids[lane] = -1;
    s_cnt[lane] = 0;
    __syncthreads();
    for (int t0 = 0; t0 < T; t0 += 4) {
        const int t = t0 + g;
        const uint32_t slot_of = route16_row(logits, T, t, E, k, norm, vec4, topk_w, topk_ids,
                                             multihot, pim, pos, g, q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t r = (slot_of >> (8 * i)) & 0xFFu;
            if (r != 0xFFu) s_ids[t * k + (int)r] = 4 * q + i;
        }
    }
    __syncthreads();
    align_slots_wave(s_ids, n, k, E, nbits, s_cnt, s_off, counts, offsets, sorted_tok,
                     sorted_slot, slot_to_sorted, nullptr);
    // With inv_w: the multihot maps back to indices (moe_multihot_to_indices),
    // read from the rows this wave wrote.
    if (inv_w != nullptr) {
        __threadfence_block();
        for (int t0 = 0; t0 < T; t0 += 4)
            to_indices_row16<4>(pim, pos, T, t0 + g, E, k, inv_w, inv_ids, q);
    }
}

// Route with the alignment's per-block histograms: block b routes the rows of
// alignment chunk b (rows_per_block = chunk / k rows, slots [b chunk,
// (b + 1) chunk)) and counts their ids into partial[b][e], exactly what
// align_hist_kernel would count from the ids, so the scatter kernel follows
// directly.  16 waves of 4 rows: a chunk of at most 64 rows in one pass.
constexpr int kRouteHistThreads = 1024;
constexpr int kRouteHistRows = kRouteHistThreads / kWave * 4;

__global__ __launch_bounds__(kRouteHistThreads) void route_hist_kernel(
    const float *__restrict__ logits, int64_t T, int E, int k, int norm, int vec4,
    int64_t rows_per_block, float *__restrict__ topk_w, int32_t *__restrict__ topk_ids,
    uint8_t *__restrict__ multihot, float *__restrict__ pim, int32_t *__restrict__ pos,
    int32_t *__restrict__ partial) {
    extern __shared__ int32_t hist[];
    for (int e = threadIdx.x; e < E; e += kRouteHistThreads) hist[e] = 0;
    __syncthreads();
    const int lane = lane_id();
    const int g = lane >> 4;
    const int q = lane & 15;
    const int wave = threadIdx.x / kWave;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < T ? r0 + rows_per_block : T;
    // Rows at or past r1 belong to the next block: r1 bounds the rows here.
    for (int64_t t0 = r0 + wave * 4; t0 < r1; t0 += kRouteHistRows) {
        const uint32_t slot_of = route16_row(logits, r1, t0 + g, E, k, norm, vec4, topk_w,
                                             topk_ids, multihot, pim, pos, g, q);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (((slot_of >> (8 * i)) & 0xFFu) != 0xFFu) atomicAdd(&hist[4 * q + i], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kRouteHistThreads)
        partial[(int64_t)blockIdx.x * E + e] = hist[e];
}

// The grouped GEMMs' m-tile list (A3's tile schedule): thread e takes expert
// e (up to 4 per thread), the block scans the tile counts, and each expert
// writes its tiles at its base.  One block of kAlignThreads (E <= 1024).
__global__ __launch_bounds__(kAlignThreads) void tile_schedule_kernel(
    const int32_t *__restrict__ offsets, int E, int64_t max_tiles,
    int32_t *__restrict__ tile_expert, int32_t *__restrict__ tile_row_start,
    int32_t *__restrict__ tile_row_end, int32_t *__restrict__ num_tiles) {
    __shared__ int32_t cnt_tiles[4 * kAlignThreads], base[4 * kAlignThreads], wsum[kAlignWaves];
    for (int e = threadIdx.x; e < E; e += kAlignThreads)
        cnt_tiles[e] = expert_mtiles(offsets[e + 1] - offsets[e]);
    __syncthreads();
    const int total = block_exclusive_scan(cnt_tiles, base, E, wsum);
    for (int e = threadIdx.x; e < E; e += kAlignThreads) {
        const int o0 = offsets[e], cnt = offsets[e + 1] - o0, mt = cnt_tiles[e];
        const int q = mtile_share(cnt, mt);
        for (int i = 0; i < mt; ++i) {
            const int64_t j = (int64_t)base[e] + i;
            if (j >= max_tiles) break;
            tile_expert[j] = e;
            tile_row_start[j] = o0 + min(i * q, cnt);
            tile_row_end[j] = o0 + min((i + 1) * q, cnt);
        }
    }
    if (threadIdx.x == 0) num_tiles[0] = total;
}

}  // namespace

hipError_t launch_tile_schedule(const int32_t *offsets, int E, int64_t max_tiles,
                                int32_t *tile_expert, int32_t *tile_row_start,
                                int32_t *tile_row_end, int32_t *num_tiles, hipStream_t s) {
    hipLaunchKernelGGL(tile_schedule_kernel, dim3(1), dim3(kAlignThreads), 0, s, offsets, E,
                       max_tiles, tile_expert, tile_row_start, tile_row_end, num_tiles);
    return hipGetLastError();
}

size_t scatter_lds_bytes(int E) {
    const int parts = E < kAlignThreads ? kAlignThreads / E : 1;
    return (size_t)((3 + kAlignWaves) * E + 2 * parts * E + kAlignWaves) * sizeof(int32_t);
}

int align_num_blocks(int64_t n, int E) {
    int64_t nb = (n + kSlotsPerBlock - 1) / kSlotsPerBlock;
    int64_t cap = kPartialBudget / E;
    if (cap < 1) cap = 1;
    if (nb > cap) nb = cap;
    if (nb < 1) nb = 1;
    return (int)nb;
}

hipError_t launch_align(const int32_t *ids, int64_t T, int k, int E, int32_t *counts,
                        int32_t *offsets, int32_t *sorted_tok, int32_t *sorted_slot,
                        int32_t *slot_to_sorted, int32_t *ws, hipStream_t s, const float *pim,
                        const int32_t *pos, float *inv_w, int32_t *inv_ids) {
    const int64_t n = T * k;
    const int nb = align_num_blocks(n, E);
    const int64_t chunk = align_chunk(n, nb);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;

    // With no slots the histogram is all zeros and the scatter kernel still
    // writes zero counts and offsets.
    const int fused = nb == 1;
    if (!fused) {
        hipLaunchKernelGGL(align_hist_kernel, dim3(nb), dim3(kAlignThreads), E * sizeof(int32_t),
                           s, ids, n, E, chunk, ws);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    const size_t lds = scatter_lds_bytes(E);
    // With inv_w the launch also carries the inverse conversion's blocks
    // where its 16-lanes-per-row form applies, else the conversion follows.
    const bool inv_in = inv_w != nullptr && E <= 256 && E % 4 == 0 && k <= kKMax16 &&
                        (reinterpret_cast<uintptr_t>(pos) & 15u) == 0;
    const int64_t inv_blocks = inv_in ? std::min<int64_t>((T + 31) / 32, 4096) : 0;
    hipLaunchKernelGGL(align_scatter_kernel, dim3((unsigned)(nb + inv_blocks)),
                       dim3(kAlignThreads), lds, s, ids, (int)n, k, E, (int)chunk, nbits, nb,
                       fused, ws, counts, offsets, sorted_tok, sorted_slot, slot_to_sorted, pim,
                       pos, inv_in ? inv_w : nullptr, inv_ids);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || inv_w == nullptr || inv_in) return err;
    return launch_to_indices(pim, pos, T, E, k, inv_w, inv_ids, s);
}

bool route_align_fused(int64_t T, int E, int k, const uint8_t *mh, const float *pim,
                       const int32_t *pos) {
    if (E > 64 || k > 16) return false;
    if (mh != nullptr && !route_multihot_fused(E, k, mh, pim, pos)) return false;
    const int64_t n = T * k;
    const int nb = align_num_blocks(n, E);
    if (nb == 1) return true;
    // Chunks of whole rows, few enough that one pass of the route kernel's
    // 16 waves covers a chunk (more rows per block measured slower than the
    // separate launches: the route then runs on too few blocks).
    const int64_t chunk = align_chunk(n, nb);
    return chunk % k == 0 && chunk / k <= kRouteHistRows;
}

hipError_t launch_route_align(const float *logits, int64_t T, int E, int k, int norm, float *w,
                              int32_t *ids, uint8_t *mh, float *pim, int32_t *pos,
                              int32_t *counts, int32_t *offsets, int32_t *sorted_tok,
                              int32_t *sorted_slot, int32_t *slot_to_sorted, int32_t *ws,
                              float *inv_w, int32_t *inv_ids, hipStream_t s) {
    if (inv_w != nullptr && mh == nullptr) return hipErrorInvalidValue;
    if (!route_align_fused(T, E, k, mh, pim, pos)) {
        hipError_t err = mh != nullptr
                             ? launch_route_multihot(logits, T, E, k, norm, w, ids, mh, pim, pos, s)
                             : launch_route(logits, T, E, k, norm, w, ids, s);
        if (err != hipSuccess) return err;
        err = launch_align(ids, T, k, E, counts, offsets, sorted_tok, sorted_slot, slot_to_sorted,
                           ws, s);
        if (err != hipSuccess || inv_w == nullptr) return err;
        return launch_to_indices(pim, pos, T, E, k, inv_w, inv_ids, s);
    }
    const int64_t n = T * k;
    const int nb = align_num_blocks(n, E);
    const int64_t chunk = align_chunk(n, nb);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const int vec4 = E == 64 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0;
    if (n <= kWave) {
        hipLaunchKernelGGL(route_align_wave_kernel, dim3(1), dim3(kWave), 0, s, logits, (int)T, E,
                           k, norm, vec4, w, ids, mh, pim, pos, nbits, counts, offsets, sorted_tok,
                           sorted_slot, slot_to_sorted, inv_w, inv_ids);
        return hipGetLastError();
    }
    if (nb == 1) {
        hipLaunchKernelGGL(route_align_small_kernel, dim3(1), dim3(kAlignThreads),
                           scatter_lds_bytes(E), s, logits, (int)T, E, k, norm, vec4, w, ids, mh,
                           pim, pos, (int)chunk, nbits, counts, offsets, sorted_tok, sorted_slot,
                           slot_to_sorted, inv_w, inv_ids);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(route_hist_kernel, dim3(nb), dim3(kRouteHistThreads), E * sizeof(int32_t), s,
                       logits, T, E, k, norm, vec4, chunk / k, w, ids, mh, pim, pos, ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // With inv_w the launch also carries the inverse conversion's blocks
    // (32 rows per block per pass), after the scatter's.
    const int64_t inv_blocks = inv_w == nullptr ? 0 : std::min<int64_t>((T + 31) / 32, 4096);
    hipLaunchKernelGGL(align_scatter_kernel, dim3((unsigned)(nb + inv_blocks)),
                       dim3(kAlignThreads), scatter_lds_bytes(E), s, ids, (int)n, k, E,
                       (int)chunk, nbits, nb, 0, ws, counts, offsets, sorted_tok, sorted_slot,
                       slot_to_sorted, pim, pos, inv_w, inv_ids);
    return hipGetLastError();
}

}  // namespace moe
