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
//   2. align_scan:    one block turns the partials into per-expert totals,
//                     exclusive offsets (the indptr) and, for every (b, e),
//                     the first position block b may write for expert e.
//   3. align_scatter: each block walks its chunk in order, 256 slots at a
//                     time; a slot's rank among earlier slots of the same
//                     expert comes from ballots inside its wave plus the
//                     counts of the waves before it, so positions follow the
//                     flat slot order t*k+j -- ascending token inside each
//                     expert, exactly the order of the pages' cumsum.
//
// Only integer LDS atomics on private counters are used, and no result
// depends on their order, so the output is identical on every run.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kAlignThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kPartialBudget = 12288;  // nb * E partial counts kept in LDS by the scan

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

__global__ __launch_bounds__(kScanThreads) void align_scan_kernel(
    int32_t *__restrict__ partial, int nb, int E, int64_t n, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_tok,
    int32_t *__restrict__ sorted_slot) {
    extern __shared__ int32_t sm[];
    int32_t *P = sm;                 // [nb][E]
    int32_t *base = sm + nb * E;     // [E]
    int32_t *wtot = base + E;        // [kScanThreads / 64]
    int32_t *total = wtot + kScanThreads / kWave;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;

    for (int i = tid; i < nb * E; i += kScanThreads) P[i] = partial[i];
    __syncthreads();
    // Per expert: exclusive prefix over blocks (in place) and the total.
    for (int e = tid; e < E; e += kScanThreads) {
        int run = 0;
        for (int b = 0; b < nb; ++b) {
            const int c = P[b * E + e];
            P[b * E + e] = run;
            run += c;
        }
        base[e] = run;
    }
    __syncthreads();
    // Exclusive prefix over experts (E <= kScanThreads: one per thread).
    const int x = tid < E ? base[tid] : 0;
    int incl = x;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) wtot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int w = lane < kScanThreads / kWave ? wtot[lane] : 0;
        int wi = w;
#pragma unroll
        for (int o = 1; o < kScanThreads / kWave; o <<= 1) {
            const int y = __shfl_up(wi, o, kWave);
            if (lane >= o) wi += y;
        }
        if (lane < kScanThreads / kWave) wtot[lane] = wi - w;  // exclusive wave prefix
    }
    __syncthreads();
    const int excl = incl - x + wtot[wave];
    if (tid < E) {
        counts[tid] = x;
        offsets[tid] = excl;
        base[tid] = excl;
        if (tid == E - 1) {
            offsets[E] = excl + x;
            *total = excl + x;
        }
    }
    __syncthreads();
    for (int i = tid; i < nb * E; i += kScanThreads) partial[i] = base[i % E] + P[i];
    // Positions past the valid slots (ids outside [0, E)) read -1.
    for (int64_t p = *total + tid; p < n; p += kScanThreads) {
        sorted_tok[p] = -1;
        sorted_slot[p] = -1;
    }
}

__global__ __launch_bounds__(kAlignThreads) void align_scatter_kernel(
    const int32_t *__restrict__ ids, int n, int k, int E, int chunk, int nbits,
    const int32_t *__restrict__ start, int32_t *__restrict__ sorted_tok,
    int32_t *__restrict__ sorted_slot, int32_t *__restrict__ slot_to_sorted) {
    extern __shared__ int32_t sm[];
    int32_t *run = sm;        // [E]   next free position per expert for this block
    int32_t *wcnt = sm + E;   // [4][E] per-wave counts of the current 256 slots
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    for (int e = tid; e < E; e += kAlignThreads) run[e] = start[(int64_t)blockIdx.x * E + e];
    for (int i = tid; i < 4 * E; i += kAlignThreads) wcnt[i] = 0;
    __syncthreads();

    const int lo = blockIdx.x * chunk;
    const int hi = lo + chunk < n ? lo + chunk : n;
    for (int it = lo; it < hi; it += kAlignThreads) {
        const int s = it + tid;
        int e = -1;
        if (s < hi) e = ids[s];
        const bool ok = (unsigned)e < (unsigned)E;
        // Lanes of this wave holding the same expert: filter by each id bit.
        uint64_t peers = __ballot(ok);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t m = __ballot(ok && bit);
            peers &= bit ? m : ~m;
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
        __syncthreads();
        if (ok && rank == 0) {
            atomicAdd(&run[e], cnt);
            wcnt[wave * E + e] = 0;
        }
        __syncthreads();
    }
}

}  // namespace

int align_num_blocks(int64_t n, int E) {
    int64_t nb = (n + 1023) / 1024;
    int64_t cap = kPartialBudget / E;
    if (cap < 1) cap = 1;
    if (nb > cap) nb = cap;
    if (nb < 1) nb = 1;
    return (int)nb;
}

hipError_t launch_align(const int32_t *ids, int64_t T, int k, int E, int32_t *counts,
                        int32_t *offsets, int32_t *sorted_tok, int32_t *sorted_slot,
                        int32_t *slot_to_sorted, int32_t *ws, hipStream_t s) {
    const int64_t n = T * k;
    const int nb = align_num_blocks(n, E);
    const int64_t chunk = align_chunk(n, nb);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;

    // With no slots the histogram is all zeros and the scan still writes
    // zero counts and offsets.
    hipLaunchKernelGGL(align_hist_kernel, dim3(nb), dim3(kAlignThreads), E * sizeof(int32_t), s,
                       ids, n, E, chunk, ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t scan_lds = (size_t)(nb * E + E + kScanThreads / kWave + 1) * sizeof(int32_t);
    hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(kScanThreads), scan_lds, s, ws, nb, E, n,
                       counts, offsets, sorted_tok, sorted_slot);
    err = hipGetLastError();
    if (err != hipSuccess || n == 0) return err;
    hipLaunchKernelGGL(align_scatter_kernel, dim3(nb), dim3(kAlignThreads),
                       5 * E * sizeof(int32_t), s, ids, (int)n, k, E, (int)chunk, nbits, ws,
                       sorted_tok, sorted_slot, slot_to_sorted);
    return hipGetLastError();
}

}  // namespace moe
