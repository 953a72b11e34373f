/*
 * moe.h -- C ABI of libmoe, the Mixture-of-Experts layer forward on AMD
 * Instinct MI355X (CDNA4, gfx950).
 *
 * The layer forward is split the way the method is stated:
 *
 *   moe_route                 gating softmax + top-k (optionally renormalised)
 *   moe_route_multihot        moe_route + moe_indices_to_multihot in one pass
 *   moe_route_grouped         group-limited top-k (group_limited_greedy, noaux_tc)
 *   moe_router_route          router GEMM (hidden . w_gate^T) + moe_route, one pass
 *   moe_route_align           moe_route(_multihot) + moe_align in fewer launches
 *   moe_route_align_inverse   moe_route_align + moe_multihot_to_indices on its maps
 *   moe_route_align_gate_up   moe_route_align(_inverse) + moe_ffn_gate_up (one launch
 *                             for the smallest decode batches)
 *   moe_align                 per-expert histogram, exclusive offsets, stable
 *                             expert-major order of the (token, slot) pairs
 *   moe_align_inverse         moe_align + moe_multihot_to_indices on given maps
 *   moe_tile_schedule         the grouped GEMMs' m-tile list from the offsets
 *   moe_indices_to_multihot   [T,k] routing -> [T,E] multihot / probs / position map
 *   moe_multihot_to_indices   the inverse conversion
 *   moe_expert_ffn            grouped w13 GEMM + SiLU-and-mul, grouped w2 GEMM,
 *                             weighted combine (prefill, any T)
 *   moe_expert_ffn_decode     the same for T <= MOE_DECODE_MAX_T, streaming only
 *                             the selected experts' weights
 *   moe_route_backward        gradient of the gating softmax weights w.r.t. the logits
 *   moe_route_grouped_backward gradient of the group-limited weights w.r.t. the scores
 *   moe_router_backward       gradients of the gate's hidden states and weights
 *   moe_expert_ffn_backward   gradients of moe_expert_ffn w.r.t. hidden, w13, w2
 *                             and the routing weights
 *
 * plus the three phases of moe_expert_ffn as separate calls, so a caller can
 * place its own events between them.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor arguments are DEVICE pointers to row-major, contiguous memory
 *   owned by the caller.  The library never allocates or frees device memory,
 *   never synchronises the host and never reads device memory from the host.
 *   Scratch memory is passed in as a workspace whose size comes from the
 *   matching *_workspace_size query.
 * - `stream` is a hipStream_t (NULL = the legacy default stream).  All work is
 *   enqueued on it asynchronously; results are ready when the stream reaches
 *   that point.  Calls that share a workspace on different streams race.
 * - Shapes: T tokens, E experts, k experts per token, H hidden size,
 *   I expert intermediate size.  Ids are int32.  Expert weights are stored
 *   [out, in]: w13 is [E, 2I, H] (rows [0,I) = gate, rows [I,2I) = up) and w2
 *   is [E, H, I]; a linear layer computes y = x . W^T.
 * - An expert id is valid iff 0 <= id < E.  Invalid ids (e.g. -1 for a
 *   dropped slot) are skipped by every call that consumes ids.
 * - Errors are reported by return value only.  Argument checks (null
 *   pointers, sizes, alignment, workspace size) happen on the host BEFORE any
 *   launch; on error nothing is enqueued and outputs are untouched.  Device
 *   preconditions (finite logits, distinct valid ids within a row, offsets
 *   produced by moe_align for the same ids) are documented, not checked.
 *   moe_last_error() returns a message for the last failing call on the
 *   calling thread.
 * - T = 0 is a valid no-op for every call.
 *
 * Method sources (cited per call below):
 *   [mlc] mlc-llm, python/mlc_llm/op/moe_misc.py ("Mixture of Experts operators")
 *   [mgt] Megatron-LM, megatron/core/fusions/fused_indices_converter.py
 *   [p6]  project_6, ex_engine/csrc/moe_expert_gemm.cpp
 */
#ifndef LIBMOE_MOE_H
#define LIBMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_VERSION 6
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 64
#define MOE_DECODE_MAX_T 64
#define MOE_MAX_SPLITS 8
#define MOE_MAX_GROUPS 64

/* moe_route_grouped methods */
#define MOE_GROUP_LIMITED_GREEDY 0
#define MOE_NOAUX_TC 1

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, k > E, misaligned pointer */
    MOE_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels handle */
    MOE_ERR_WORKSPACE = 3,   /* workspace pointer null or too small */
    MOE_ERR_HIP = 4          /* a HIP launch failed; see moe_last_error() */
} moe_status_t;

typedef enum {
    MOE_F32 = 0, /* float32 hidden / weights / activations / output */
    MOE_BF16 = 1 /* bfloat16 hidden / weights / activations / output, fp32 accumulation */
} moe_dtype_t;

/* Library version (MOE_VERSION). */
int moe_version(void);
/* Static text for a status code. */
const char *moe_status_string(moe_status_t s);
/* Detail of the last failing call on this thread ("" if none).  Thread-local,
 * valid until the next failing call on the same thread. */
const char *moe_last_error(void);

/*
 * moe_route -- gating top-k with softmax weights.
 * [mlc] gating_topk, _gating_topk_process_value, gating_softmax_topk.
 *
 * logits    [T, E] float32, finite.
 * topk_w    [T, k] float32 out: the weights of the selected experts.
 * topk_ids  [T, k] int32 out: selected expert ids, per row in descending
 *           logit order; equal logits keep the lower expert id first.
 * norm_topk_prob != 0: weights = softmax over the k selected logits (they sum
 *           to 1).  == 0: weights = full softmax over all E logits, taken at
 *           the selected ids.  Selection is on the logits in both modes.
 * Requires 1 <= k <= min(E, MOE_MAX_TOPK), E <= MOE_MAX_EXPERTS.
 */
moe_status_t moe_route(const float *logits, int64_t T, int32_t E, int32_t k,
                       int32_t norm_topk_prob, float *topk_w, int32_t *topk_ids, void *stream);

/*
 * moe_route_multihot -- moe_route followed by moe_indices_to_multihot of its
 * own output, in one pass where moe_route_multihot_fused(E, k) is true (and
 * probs_in_multihot / position_map are 16-byte aligned, multihot 4-byte
 * aligned); otherwise the same two launches as the separate calls.
 * [mlc] gating_topk, gating_softmax_topk; [mgt] _indices_to_multihot_kernel.
 *
 * Arguments as moe_route, plus the [T, E] outputs of moe_indices_to_multihot
 * (multihot uint8, probs_in_multihot float32, position_map int32).  Every
 * output is bit-identical to moe_route then moe_indices_to_multihot on the
 * same logits.  All pointers non-null when T > 0.
 */
moe_status_t moe_route_multihot(const float *logits, int64_t T, int32_t E, int32_t k,
                                int32_t norm_topk_prob, float *topk_w, int32_t *topk_ids,
                                uint8_t *multihot, float *probs_in_multihot,
                                int32_t *position_map, void *stream);

/*
 * moe_router_route -- the router GEMM that produces the gating logits,
 * followed by moe_route on them, in one pass where E <= 64 and k <= 16
 * (otherwise the GEMM kernel, then moe_route's kernel).
 * The logits are logits = hidden . w_gate^T (a linear layer, W stored
 * [out, in] as in [p6]); the pages take them as given.  Routing as moe_route
 * ([mlc] gating_topk, gating_softmax_topk).
 *
 * dt        MOE_BF16 (other dtypes return MOE_ERR_UNSUPPORTED).
 * hidden    [T, H] bf16, w_gate [E, H] bf16; 16-byte aligned.
 * logits    [T, E] float32 out: fp32 accumulation of the bf16 products (the
 *           summation order is the kernel's, so values can differ from an
 *           exact dot product by rounding).
 * topk_w, topk_ids  [T, k] out: exactly moe_route(logits, ...) on the
 *           logits written.
 * Requires H % 64 == 0 (else MOE_ERR_UNSUPPORTED), 1 <= k <= min(E,
 * MOE_MAX_TOPK), E <= MOE_MAX_EXPERTS.
 */
moe_status_t moe_router_route(moe_dtype_t dt, const void *hidden, const void *w_gate, int64_t T,
                              int32_t H, int32_t E, int32_t k, int32_t norm_topk_prob,
                              float *logits, float *topk_w, int32_t *topk_ids, void *stream);

/*
 * moe_route_grouped -- group-limited top-k expert selection.
 * [mlc] group_limited_greedy_topk (methods "group_limited_greedy", "noaux_tc").
 *
 * scores    [T, E] float32 routing scores (e.g. a softmax or sigmoid of the
 *           gating logits, computed by the caller), finite and greater than
 *           float32's lowest finite value.
 * e_score_correction_bias
 *           [E] float32, read only by MOE_NOAUX_TC (may be NULL for
 *           MOE_GROUP_LIMITED_GREEDY).
 * The E experts form n_group groups of E / n_group consecutive experts.  The
 * choice score of an expert is its score (greedy) or score + bias, added in
 * float32 (noaux_tc).  A group's score is its largest choice score (greedy)
 * or the float32 sum of its two largest (noaux_tc).  The topk_group best
 * groups are kept and the k best experts among them selected; both rankings
 * are value descending, equal values keeping the lower index first.
 * topk_ids  [T, k] int32 out: selected experts in descending choice order.
 * topk_w    [T, k] float32 out: the scores (without the bias) of the selected
 *           experts; renormalize != 0 divides them by their sum.
 * multihot, probs_in_multihot, position_map
 *           [T, E] outputs of moe_indices_to_multihot on (topk_ids, topk_w),
 *           bit for bit: all three given, or all NULL for none.  On the
 *           16-lanes-per-row path (E % 16 == 0, E <= 256, n_group dividing 16,
 *           k <= 16) the same kernel writes them.
 * Requires E % n_group == 0, 1 <= n_group <= MOE_MAX_GROUPS,
 * 1 <= topk_group <= n_group, 1 <= k <= min(MOE_MAX_TOPK,
 * topk_group * E / n_group), E <= MOE_MAX_EXPERTS, and groups of at least
 * two experts for noaux_tc.  Pointers 4-byte aligned.
 */
moe_status_t moe_route_grouped(const float *scores, const float *e_score_correction_bias,
                               int64_t T, int32_t E, int32_t k, int32_t n_group,
                               int32_t topk_group, int32_t method, int32_t renormalize,
                               float *topk_w, int32_t *topk_ids, uint8_t *multihot,
                               float *probs_in_multihot, int32_t *position_map, void *stream);

/* 1 if moe_route_multihot runs as one kernel for this E and k (E <= 64,
 * E % 4 == 0, k <= 16, k <= E), else 0. */
int32_t moe_route_multihot_fused(int32_t E, int32_t k);

/*
 * moe_align -- expert alignment of the T*k (token, slot) pairs.
 * [mlc] moe_cumsum, get_indices, get_indptr (exclusive form).
 *
 * topk_ids         [T, k] int32 in.  Valid ids within a row must be distinct.
 * expert_counts    [E]    int32 out: number of valid slots routed to each expert.
 * expert_offsets   [E+1]  int32 out: exclusive prefix sum of the counts;
 *                  offsets[0] = 0, offsets[E] = number of valid slots.
 * sorted_token_ids [T*k]  int32 out: token of each position p, expert-major,
 *                  ascending token inside each expert's segment
 *                  [offsets[e], offsets[e+1]).
 * sorted_slot_ids  [T*k]  int32 out: flat slot t*k + j of each position p.
 * slot_to_sorted   [T*k]  int32 out: position p of each flat slot (inverse of
 *                  sorted_slot_ids), -1 for slots with an invalid id.
 * Entries of sorted_token_ids / sorted_slot_ids at p >= offsets[E] are -1.
 * workspace        >= moe_align_workspace_size(T, k, E) bytes of device memory,
 *                  any content; clobbered.
 * The result is identical bit for bit on every run (no order-dependent atomics).
 */
size_t moe_align_workspace_size(int64_t T, int32_t k, int32_t E);
moe_status_t moe_align(const int32_t *topk_ids, int64_t T, int32_t k, int32_t E,
                       int32_t *expert_counts, int32_t *expert_offsets,
                       int32_t *sorted_token_ids, int32_t *sorted_slot_ids,
                       int32_t *slot_to_sorted, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * moe_align_inverse -- moe_align, then moe_multihot_to_indices on the given
 * [T, E] maps (the multihot outputs of the routing that produced topk_ids),
 * in one call.  [mlc] moe_cumsum, get_indices, get_indptr; [mgt]
 * _multihot_to_indices_kernel.
 *
 * Arguments as the two calls: probs_in_multihot and position_map [T, E] in;
 * probs_indices [T, k] float32 and ids_from_multihot [T, k] int32 (may be
 * NULL) out.  Every output is bit-identical to the separate calls.  Where the
 * conversion's 16-lanes-per-row form applies (E <= 256, E % 4 == 0,
 * k <= 16, position_map 16-byte aligned) its blocks ride in the alignment
 * scatter's launch, which does not depend on them; otherwise it is a launch
 * of its own.  Same workspace as moe_align.
 */
moe_status_t moe_align_inverse(const int32_t *topk_ids, int64_t T, int32_t k, int32_t E,
                               int32_t *expert_counts, int32_t *expert_offsets,
                               int32_t *sorted_token_ids, int32_t *sorted_slot_ids,
                               int32_t *slot_to_sorted, const float *probs_in_multihot,
                               const int32_t *position_map, float *probs_indices,
                               int32_t *ids_from_multihot, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * moe_tile_schedule -- the m-tile list of the grouped GEMMs (A3's tile
 * schedule) from moe_align's expert_offsets.  [mlc] get_indptr (exclusive
 * form) gives the segments; the tiles are this library's: an expert with
 * c = offsets[e+1] - offsets[e] rows has ceil(c / 320) m-tiles, and its rows
 * are dealt to them in equal shares rounded up to whole 32-row fragments,
 * q = ceil(c / (32 mt)) * 32, so m-tile i covers rows
 * [offsets[e] + min(i q, c), offsets[e] + min((i + 1) q, c)).  The grouped
 * GEMMs derive the same tiles from the offsets on the device; this call
 * writes them out for callers that want the list (a persistent or external
 * GEMM, a dispatch plan).
 *
 * expert_offsets [E+1] int32 in (device).
 * tile_expert, tile_row_start, tile_row_end [max_tiles] int32 out: tile j's
 *                  expert and row range, expert order then m-tile order;
 *                  entries j >= *num_tiles are left as they were.
 * num_tiles        [1] int32 out (device): the number of tiles; if it
 *                  exceeds max_tiles only the first max_tiles are written.
 * max_tiles >= moe_tile_schedule_max(T, k, E) (ceil(T k / 320) + min(E, T k))
 * always holds every tile.  Requires 1 <= E <= MOE_MAX_EXPERTS; the outputs
 * may be NULL when max_tiles = 0.  One single-block launch.
 */
int64_t moe_tile_schedule_max(int64_t T, int32_t k, int32_t E);
moe_status_t moe_tile_schedule(const int32_t *expert_offsets, int32_t E, int64_t max_tiles,
                               int32_t *tile_expert, int32_t *tile_row_start,
                               int32_t *tile_row_end, int32_t *num_tiles, void *stream);

/*
 * moe_route_align -- moe_route (moe_route_multihot when multihot,
 * probs_in_multihot and position_map are all given; all NULL otherwise)
 * followed by moe_align on the ids it produces.
 * [mlc] gating_topk, gating_softmax_topk, moe_cumsum, get_indices, get_indptr;
 * [mgt] _indices_to_multihot_kernel.
 *
 * Arguments as the separate calls; every output is bit-identical to them.
 * Where moe_route_align_fused(T, E, k) is 1 (E <= 64, k <= 16, and for more
 * than 512 slots alignment chunks of at most 64 whole rows) the calls take
 * fewer launches: for at most 512 slots (decode batches) one kernel routes
 * and aligns (one wave for at most 64 slots); beyond that the route kernel also counts each alignment
 * chunk's ids, so the alignment's histogram kernel is not launched.  (With
 * the multihot outputs the fused path also needs what moe_route_multihot's
 * one-kernel path needs.)  workspace: moe_align_workspace_size(T, k, E)
 * bytes.  T = 0 writes zero counts and offsets, as moe_align does.
 */
moe_status_t moe_route_align(const float *logits, int64_t T, int32_t E, int32_t k,
                             int32_t norm_topk_prob, float *topk_w, int32_t *topk_ids,
                             uint8_t *multihot, float *probs_in_multihot, int32_t *position_map,
                             int32_t *expert_counts, int32_t *expert_offsets,
                             int32_t *sorted_token_ids, int32_t *sorted_slot_ids,
                             int32_t *slot_to_sorted, void *workspace, size_t workspace_bytes,
                             void *stream);
/* 1 if moe_route_align takes the fused launches for this T, E and k. */
int32_t moe_route_align_fused(int64_t T, int32_t E, int32_t k);

/*
 * moe_route_align_inverse -- moe_route_align with the multihot outputs
 * (required here), followed by moe_multihot_to_indices on the maps it wrote:
 * probs_indices [T, k] float32 and ids_from_multihot [T, k] int32 (may be
 * NULL) are that call's outputs.  [mgt] _multihot_to_indices_kernel, after
 * the sources of moe_route_align.
 *
 * Every output is bit-identical to the separate calls.  Where
 * moe_route_align_fused(T, E, k) is 1 the conversion runs in moe_route_align's
 * last launch, reading the maps back from memory: in the one-wave or
 * one-block kernel after it has aligned, or (more slots) as extra blocks of
 * the scatter launch, which does not depend on it; otherwise it is a launch
 * of its own.  Same workspace as moe_route_align.
 */
moe_status_t moe_route_align_inverse(const float *logits, int64_t T, int32_t E, int32_t k,
                                     int32_t norm_topk_prob, float *topk_w, int32_t *topk_ids,
                                     uint8_t *multihot, float *probs_in_multihot,
                                     int32_t *position_map, int32_t *expert_counts,
                                     int32_t *expert_offsets, int32_t *sorted_token_ids,
                                     int32_t *sorted_slot_ids, int32_t *slot_to_sorted,
                                     float *probs_indices, int32_t *ids_from_multihot,
                                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_route_align_gate_up -- moe_route_align (moe_route_align_inverse when
 * probs_indices is given; the multihot outputs may then not be NULL, and
 * without probs_indices they are optional as in moe_route_align) followed by
 * moe_ffn_gate_up (dt, decode, hidden [T, H], w13 [E, 2I, H], act [T*k, I]:
 * that call's arguments and conditions) on the alignment it wrote.  [p6]
 * moe_decode_experts (the FC1 of the selected experts), after the sources of
 * moe_route_align.
 *
 * Where moe_route_align_gate_up_fused(T, E, k, dt, decode, H, I) is 1 (bf16
 * decode, T k <= 16, E <= 64, k <= 16, and when the multihot maps are given,
 * 16-byte aligned rows of them) the whole call is one launch: every FC1 block
 * routes and aligns the batch in its own shared memory and reads its tokens
 * from there, and one block also writes every routing output; otherwise it
 * is the separate calls' launches.  (Every block routing the whole batch
 * pays off only while the batch is this small.)  Every output is
 * bit-identical to the separate calls.  Same workspace as moe_route_align.
 */
moe_status_t moe_route_align_gate_up(
    const float *logits, int64_t T, int32_t E, int32_t k, int32_t norm_topk_prob, float *topk_w,
    int32_t *topk_ids, uint8_t *multihot, float *probs_in_multihot, int32_t *position_map,
    int32_t *expert_counts, int32_t *expert_offsets, int32_t *sorted_token_ids,
    int32_t *sorted_slot_ids, int32_t *slot_to_sorted, float *probs_indices,
    int32_t *ids_from_multihot, moe_dtype_t dt, int32_t decode, const void *hidden,
    const void *w13, int32_t H, int32_t I, void *act, void *workspace, size_t workspace_bytes,
    void *stream);
int32_t moe_route_align_gate_up_fused(int64_t T, int32_t E, int32_t k, moe_dtype_t dt,
                                      int32_t decode, int32_t H, int32_t I);

/*
 * moe_route_align_noalloc -- moe_route_align for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops or harnesses that
 * forbid hipMalloc): the same arguments without the workspace, the same
 * launches and bit-identical outputs.  The alignment's scratch (per-block
 * expert counts, moe_align_workspace_size(T, k, E) bytes, at most 64 KiB for
 * any valid T, k, E) lives in a 256 KiB array that the library holds in
 * device memory, one copy per GPU, until the process ends; a shape whose
 * scratch would exceed it returns MOE_ERR_WORKSPACE before any launch.  The
 * device's address of that array is looked up on the first call on each
 * device (make that first call outside graph capture).  Nothing in the array
 * needs to start at zero.  Every call on a GPU shares that GPU's array, so
 * calls that overlap on one GPU (different streams, or several host threads)
 * race: order them on one stream.
 */
moe_status_t moe_route_align_noalloc(const float *logits, int64_t T, int32_t E, int32_t k,
                                     int32_t norm_topk_prob, float *topk_w, int32_t *topk_ids,
                                     uint8_t *multihot, float *probs_in_multihot,
                                     int32_t *position_map, int32_t *expert_counts,
                                     int32_t *expert_offsets, int32_t *sorted_token_ids,
                                     int32_t *sorted_slot_ids, int32_t *slot_to_sorted,
                                     void *stream);

/*
 * moe_indices_to_multihot -- [T,k] routing to [T,E] multihot form.
 * [mgt] _indices_to_multihot_kernel, IndicesToMultihot.forward.
 *
 * ids               [T, k] int32 in; probs [T, k] float32 in.
 * multihot          [T, E] uint8 out: 1 where expert e is a valid id of row t, else 0.
 * probs_in_multihot [T, E] float32 out: probs[t, j] (bit copy) at e = ids[t, j], else 0.
 * position_map      [T, E] int32 out: slot j at e = ids[t, j], else -1.
 */
moe_status_t moe_indices_to_multihot(const int32_t *ids, const float *probs, int64_t T,
                                     int32_t k, int32_t E, uint8_t *multihot,
                                     float *probs_in_multihot, int32_t *position_map,
                                     void *stream);

/*
 * moe_multihot_to_indices -- inverse of moe_indices_to_multihot.
 * [mgt] _multihot_to_indices_kernel, IndicesToMultihot.backward.
 *
 * probs_in_multihot [T, E] float32 in; position_map [T, E] int32 in (-1 = none).
 * probs_indices     [T, k] float32 out: probs_in_multihot[t, e] at slot
 *                   position_map[t, e], 0 for slots no expert names.
 * ids_out           [T, k] int32 out, may be NULL: the expert e that named the
 *                   slot, -1 if none.
 * Positions outside [0, k) are ignored.  If two experts of a row name the same
 * slot (never produced by the forward conversion), the higher expert id wins.
 * With ids_out = NULL this is also the backward of moe_indices_to_multihot
 * ([mgt] IndicesToMultihot.backward): given the gradient of probs_in_multihot
 * (any values, also where position_map is -1) and the forward's position_map,
 * probs_indices is the gradient of the forward's probs.
 */
moe_status_t moe_multihot_to_indices(const float *probs_in_multihot,
                                     const int32_t *position_map, int64_t T, int32_t E,
                                     int32_t k, float *probs_indices, int32_t *ids_out,
                                     void *stream);

/*
 * moe_expert_ffn -- expert FFN over the aligned slots and weighted combine.
 * [p6] moe_prefill_experts (per-expert FC1, SiLU-and-mul, FC2, weighted
 * index_add), [mlc] scatter_output + moe_sum (un-permute and k-sum).
 *
 * For every valid slot (t, j) with expert e = topk_ids[t, j]:
 *   gu  = hidden[t] . w13[e]^T                         (2I values)
 *   act = silu(gu[0:I]) * gu[I:2I]                     (stored in `dt`)
 *   y   = act . w2[e]^T                                (H values, float32)
 * and out[t] = sum over j = 0..k-1 of topk_w[t, j] * y(t, j), accumulated in
 * float32 in slot order and rounded once to `dt`.  A token with no valid slot
 * gets 0.  Accumulation is float32 throughout; for MOE_BF16 the only
 * roundings are act (the second GEMM's input) and out, once each.  The result
 * is deterministic.
 *
 * hidden [T, H], w13 [E, 2I, H], w2 [E, H, I], out [T, H] in `dt`;
 * topk_w [T, k] float32; expert_offsets [E+1], sorted_token_ids [T*k] and
 * slot_to_sorted [T*k] as written by moe_align for the same ids.
 * workspace >= moe_expert_ffn_workspace_size(dt, T, H, I, E, k) bytes.
 * Requires H % 64 == 0, I % 64 == 0; device pointers 16-byte aligned.
 */
size_t moe_expert_ffn_workspace_size(moe_dtype_t dt, int64_t T, int32_t H, int32_t I,
                                     int32_t E, int32_t k);
moe_status_t moe_expert_ffn(moe_dtype_t dt, const void *hidden, const void *w13,
                            const void *w2, const float *topk_w,
                            const int32_t *expert_offsets, const int32_t *sorted_token_ids,
                            const int32_t *slot_to_sorted, int64_t T, int32_t H, int32_t I,
                            int32_t E, int32_t k, void *out, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * moe_expert_ffn_decode -- moe_expert_ffn for T <= MOE_DECODE_MAX_T.
 * [p6] moe_decode_experts.  Same arguments and result.  Each distinct
 * selected expert's w13 / w2 slice is read from memory once and applied to
 * every token routed to it; unselected experts are never read.
 */
moe_status_t moe_expert_ffn_decode(moe_dtype_t dt, const void *hidden, const void *w13,
                                   const void *w2, const float *topk_w,
                                   const int32_t *expert_offsets,
                                   const int32_t *sorted_token_ids,
                                   const int32_t *slot_to_sorted, int64_t T, int32_t H,
                                   int32_t I, int32_t E, int32_t k, void *out,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_route_backward -- backward of moe_route's weights.
 * The chain rule applied to [mlc] gating_softmax_topk (the pages give only
 * the forward); the selection is piecewise constant and passes no gradient.
 *
 * logits      [T, E] float32 in: the forward's logits.
 * topk_ids    [T, k] int32 in, topk_w [T, k] float32 in: the forward's outputs
 *             (ids valid and distinct within a row, as moe_route writes them).
 * grad_topk_w [T, k] float32 in: gradient of the weights.
 * grad_logits [T, E] float32 out.  With dot = sum_j topk_w[j] grad_topk_w[j]:
 *   norm_topk_prob != 0: grad[e_j] = topk_w[j] (grad_topk_w[j] - dot), 0 for
 *                        unselected experts;
 *   norm_topk_prob == 0: grad[e] = p_e (g(e) - dot), p = softmax of the row's
 *                        E logits, g(e) = grad_topk_w[j] if e = e_j, else 0.
 * Requires k <= E.  Pointers 4-byte aligned.
 */
moe_status_t moe_route_backward(const float *logits, const int32_t *topk_ids,
                                const float *topk_w, const float *grad_topk_w, int64_t T,
                                int32_t E, int32_t k, int32_t norm_topk_prob,
                                float *grad_logits, void *stream);

/*
 * moe_route_grouped_backward -- backward of moe_route_grouped's weights.
 * The chain rule applied to [mlc] group_limited_greedy_topk (the pages give
 * only the forward).  The weights are the selected scores, divided by their
 * sum S when renormalize != 0; the correction bias and the group masking
 * only move the selection, which passes no gradient.
 *
 * scores      [T, E] float32 in: the forward's scores.
 * topk_ids    [T, k] int32 in, topk_w [T, k] float32 in: the forward's outputs
 *             (ids valid and distinct within a row).
 * grad_topk_w [T, k] float32 in.
 * grad_scores [T, E] float32 out: grad[e_j] = grad_topk_w[j], or with
 *             renormalize (grad_topk_w[j] - sum_i topk_w[i] grad_topk_w[i]) / S;
 *             0 for unselected experts.
 * Requires k <= E.  Pointers 4-byte aligned.
 */
moe_status_t moe_route_grouped_backward(const float *scores, const int32_t *topk_ids,
                                        const float *topk_w, const float *grad_topk_w, int64_t T,
                                        int32_t E, int32_t k, int32_t renormalize,
                                        float *grad_scores, void *stream);

/*
 * moe_router_backward -- backward of moe_router_route's gate (the linear
 * layer logits = hidden . w_gate^T; the top-k part's backward is
 * moe_route_backward).  The chain rule on the [p6] linear-layer convention:
 *   grad_hidden [T, H] float32 out = grad_logits . w_gate
 *   grad_w_gate [E, H] float32 out = grad_logits^T . hidden
 * hidden [T, H] and w_gate [E, H] bfloat16 (dt must be MOE_BF16);
 * grad_logits [T, E] float32 (e.g. from moe_route_backward).  float32
 * arithmetic, sums over e and over t in ascending order (t in chunks of 256
 * whose partial sums are added in chunk order): deterministic.
 * workspace >= moe_router_backward_workspace_size(T, H, E) bytes
 * (ceil(T / 256) * E * H * 4), 16-byte aligned, clobbered.  Requires
 * H % 64 == 0; hidden, w_gate and the gradients 16-byte aligned.  T = 0
 * enqueues nothing (grad_w_gate is then left as it was).
 */
size_t moe_router_backward_workspace_size(int64_t T, int32_t H, int32_t E);
moe_status_t moe_router_backward(moe_dtype_t dt, const void *hidden, const void *w_gate,
                                 const float *grad_logits, int64_t T, int32_t H, int32_t E,
                                 float *grad_hidden, float *grad_w_gate, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * moe_expert_ffn_backward -- backward of moe_expert_ffn.
 * The chain rule applied to [p6] moe_prefill_experts and [mlc] moe_sum (the
 * pages give only the forward).  For each valid slot (t, j) with expert e and
 * weight w, with gate/up = hidden[t] . w13[e]^T halves, s = sigmoid(gate),
 * act = gate s up, dy = grad_out[t] and G = dy . w2[e]:
 *   grad_topk_w[t, j] = <G, act>                    (= <dy, y(t, j)>)
 *   d_gate = w G up s (1 + gate (1 - s)),  d_up = w G gate s
 *   grad_hidden[t]    = sum over j of [d_gate ; d_up] . w13[e]
 *   grad_w2[e]        = sum over the slots of e of (w dy)^T act
 *   grad_w13[e]       = sum over the slots of e of [d_gate ; d_up]^T hidden[t]
 * Slots with an invalid id get grad_topk_w = 0 and add nothing; an expert no
 * slot names gets zero weight gradients (every element of every output is
 * written).  gate/up are recomputed.  MOE_BF16: five grouped bf16 products
 * on the matrix cores; w act and d_gate/d_up are rounded to bfloat16 as the
 * inputs of those products, everything else accumulates in float32; w13 and
 * w2 are read as stored (a weight past 2 GiB is first transposed per expert
 * into the workspace; weights change between training steps, so nothing is
 * cached).  MOE_F32 (small
 * layers): float32 throughout, one thread per output element.  Results are
 * deterministic.
 *
 * hidden [T, H], w13 [E, 2I, H], w2 [E, H, I], grad_out [T, H] in `dt`;
 * topk_w [T, k] float32; expert_offsets [E+1],
 * sorted_token_ids, sorted_slot_ids and slot_to_sorted [T*k] as written by
 * moe_align for the forward's ids.  Outputs float32: grad_hidden [T, H],
 * grad_w13 [E, 2I, H], grad_w2 [E, H, I], grad_topk_w [T, k].
 * workspace >= moe_expert_ffn_backward_workspace_size(T, H, I, E, k) bytes
 * (the larger of the bfloat16 path's need, about T*k*(10 I + 12 H) +
 * 256 E H, and the float32 path's T*k*(6 I + H)*4), 16-byte aligned,
 * clobbered.
 * Requires H % 64 == 0, I % 64 == 0; hidden, weights, grad_out and the
 * gradients 16-byte aligned.  T = 0 enqueues nothing, as for every call, so
 * the weight gradients are then left as they were.
 */
size_t moe_expert_ffn_backward_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E,
                                              int32_t k);
moe_status_t moe_expert_ffn_backward(moe_dtype_t dt, const void *hidden, const void *w13,
                                     const void *w2, const float *topk_w,
                                     const int32_t *expert_offsets,
                                     const int32_t *sorted_token_ids,
                                     const int32_t *sorted_slot_ids,
                                     const int32_t *slot_to_sorted, const void *grad_out,
                                     int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                     float *grad_hidden, float *grad_w13, float *grad_w2,
                                     float *grad_topk_w, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * The three phases of moe_expert_ffn (same kernels, same arguments).
 *
 * moe_ffn_gate_up: act [T*k, I] in `dt`, row p = position p of the aligned
 *   order: act[p] = silu(gate) * up for token sorted_token_ids[p] and the
 *   expert whose segment holds p.  Rows p >= offsets[E] are not written.
 * moe_ffn_down:   y [splits, T*k, H] float32: the product act[p] . w2[e]^T
 *   of the same rows with its K = I terms cut into `splits` equal slices,
 *   plane s holding the partial sum over slice s (one plane, the whole
 *   product, when splits = 1).  Slices let a product with few output tiles
 *   fill every compute unit; moe_ffn_down_splits gives the count the library
 *   uses for a shape (1 for decode and float32).  splits > 1 needs the
 *   bfloat16 prefill path and I % (64 * splits) == 0, else
 *   MOE_ERR_UNSUPPORTED; splits outside [1, MOE_MAX_SPLITS] is
 *   MOE_ERR_INVALID_ARG.
 * moe_combine:    out [T, H] in `dt` from y (float32, `splits` planes),
 *   topk_w and slot_to_sorted: each expert row is summed over the planes in
 *   plane order, then weighted and summed over j = 0..k-1 in float32.
 * `decode` != 0 selects the decode kernels (T <= MOE_DECODE_MAX_T).
 * moe_expert_ffn runs the three with splits = moe_ffn_down_splits(dt, decode,
 * ...) (the last two through moe_ffn_down_combine, below), and its workspace
 * holds act and the y planes.
 */
int32_t moe_ffn_down_splits(moe_dtype_t dt, int32_t decode, int64_t T, int32_t H, int32_t I,
                            int32_t E, int32_t k);
moe_status_t moe_ffn_gate_up(moe_dtype_t dt, int32_t decode, const void *hidden,
                             const void *w13, const int32_t *expert_offsets,
                             const int32_t *sorted_token_ids, int64_t T, int32_t H, int32_t I,
                             int32_t E, int32_t k, void *act, void *stream);
moe_status_t moe_ffn_down(moe_dtype_t dt, int32_t decode, const void *act, const void *w2,
                          const int32_t *expert_offsets, int64_t T, int32_t H, int32_t I,
                          int32_t E, int32_t k, int32_t splits, float *y, void *stream);
moe_status_t moe_combine(moe_dtype_t dt, const float *y, int32_t splits, const float *topk_w,
                         const int32_t *slot_to_sorted, int64_t T, int32_t H, int32_t k,
                         void *out, void *stream);

/*
 * moe_ffn_down_combine -- moe_ffn_down (with moe_ffn_down_splits' slice
 * count) followed by moe_combine; moe_expert_ffn and moe_expert_ffn_decode
 * run their last two phases through it.  [p6] moe_decode_experts,
 * moe_prefill_experts (the down projection and the weighted sum).
 *
 * Where moe_ffn_down_combine_fused(...) is 1 (bf16 decode with at most 32
 * routing slots and I <= 1536) the two run as one launch: each block owns 8
 * output columns of every token and every selected expert, and the token's
 * slots are summed in slot order from LDS, so y is not written (it may then
 * be NULL) and, for finite activations, out is bit-identical to the two
 * calls.  Otherwise y [splits, T*k, H] float32 is the intermediate.
 */
moe_status_t moe_ffn_down_combine(moe_dtype_t dt, int32_t decode, const void *act,
                                  const void *w2, const float *topk_w,
                                  const int32_t *expert_offsets, const int32_t *slot_to_sorted,
                                  int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                  float *y, void *out, void *stream);
int32_t moe_ffn_down_combine_fused(moe_dtype_t dt, int32_t decode, int64_t T, int32_t H,
                                   int32_t I, int32_t E, int32_t k);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_MOE_H */
