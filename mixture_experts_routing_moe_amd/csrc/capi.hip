// C ABI of libmoe: host-side argument checks and kernel dispatch.
//
// Every entry point validates its arguments before enqueuing anything, then
// launches on the caller's stream and returns without synchronising.  Nothing
// here allocates device memory or reads it back.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "moe_internal.h"

namespace {

thread_local char g_err[512] = "";

moe_status_t fail(moe_status_t s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

moe_status_t hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return MOE_OK;
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

#define CHECK(cond, status, ...)                      \
    do {                                              \
        if (!(cond)) return fail(status, __VA_ARGS__); \
    } while (0)

moe_status_t check_routing_dims(int64_t T, int32_t E, int32_t k, const char *fn) {
    CHECK(T >= 0, MOE_ERR_INVALID_ARG, "%s: T = %lld < 0", fn, (long long)T);
    CHECK(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_ERR_INVALID_ARG,
          "%s: E = %d outside [1, %d]", fn, E, MOE_MAX_EXPERTS);
    CHECK(k >= 1 && k <= MOE_MAX_TOPK, MOE_ERR_INVALID_ARG, "%s: k = %d outside [1, %d]", fn, k,
          MOE_MAX_TOPK);
    CHECK(T * (int64_t)k < (int64_t)1 << 31, MOE_ERR_INVALID_ARG,
          "%s: T*k = %lld does not fit int32", fn, (long long)(T * k));
    return MOE_OK;
}

// act [T*k, I] in the layer dtype, then y [T*k, H] float32.
size_t ffn_act_bytes(moe_dtype_t dt, int64_t T, int32_t I, int32_t k) {
    const size_t es = dt == MOE_BF16 ? 2 : 4;
    return round_up((size_t)T * (size_t)k * (size_t)I * es, 256);
}
// K slices of the FC2 product for a prefill shape (1 for float32).
int32_t prefill_splits(moe_dtype_t dt, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k) {
    if (dt != MOE_BF16 || T <= 0) return 1;
    return moe::down_splits(T, H, I, E, k);
}
size_t ffn_y_bytes(int64_t T, int32_t H, int32_t k, int32_t splits) {
    return round_up((size_t)splits * (size_t)T * (size_t)k * (size_t)H * 4, 256);
}
size_t ffn_scratch_bytes(moe_dtype_t dt, int64_t T, int32_t H, int32_t I, int32_t E,
                         int32_t k, int32_t splits) {
    (void)E;
    return ffn_act_bytes(dt, T, I, k) + ffn_y_bytes(T, H, k, splits);
}

moe_status_t check_ffn_dims(moe_dtype_t dt, int64_t T, int32_t H, int32_t I, int32_t E,
                            int32_t k, const char *fn) {
    moe_status_t st = check_routing_dims(T, E, k, fn);
    if (st != MOE_OK) return st;
    CHECK(dt == MOE_F32 || dt == MOE_BF16, MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn,
          (int)dt);
    CHECK(H >= 1 && I >= 1, MOE_ERR_INVALID_ARG, "%s: H = %d, I = %d must be >= 1", fn, H, I);
    CHECK(H % 64 == 0 && I % 64 == 0, MOE_ERR_UNSUPPORTED,
          "%s: H = %d and I = %d must be multiples of 64", fn, H, I);
    CHECK((int64_t)E * 2 * I * (int64_t)H < (int64_t)1 << 62, MOE_ERR_INVALID_ARG,
          "%s: weights too large", fn);
    if (dt == MOE_F32)
        CHECK(T * k <= 2147483647LL, MOE_ERR_UNSUPPORTED, "%s: float32 path needs T*k < 2^31",
              fn);
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_version(void) { return MOE_VERSION; }

const char *moe_status_string(moe_status_t s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or configuration";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char *moe_last_error(void) { return g_err; }

moe_status_t moe_route(const float *logits, int64_t T, int32_t E, int32_t k,
                       int32_t norm_topk_prob, float *topk_w, int32_t *topk_ids, void *stream) {
    moe_status_t st = check_routing_dims(T, E, k, "moe_route");
    if (st != MOE_OK) return st;
    CHECK(k <= E, MOE_ERR_INVALID_ARG, "moe_route: k = %d > E = %d", k, E);
    if (T == 0) return MOE_OK;
    CHECK(logits && topk_w && topk_ids, MOE_ERR_INVALID_ARG, "moe_route: null pointer");
    return hip_status(moe::launch_route(logits, T, E, k, norm_topk_prob != 0, topk_w, topk_ids,
                                        static_cast<hipStream_t>(stream)),
                      "moe_route");
}

moe_status_t moe_route_multihot(const float *logits, int64_t T, int32_t E, int32_t k,
                                int32_t norm_topk_prob, float *topk_w, int32_t *topk_ids,
                                uint8_t *multihot, float *probs_in_multihot,
                                int32_t *position_map, void *stream) {
    moe_status_t st = check_routing_dims(T, E, k, "moe_route_multihot");
    if (st != MOE_OK) return st;
    CHECK(k <= E, MOE_ERR_INVALID_ARG, "moe_route_multihot: k = %d > E = %d", k, E);
    if (T == 0) return MOE_OK;
    CHECK(logits && topk_w && topk_ids && multihot && probs_in_multihot && position_map,
          MOE_ERR_INVALID_ARG, "moe_route_multihot: null pointer");
    return hip_status(moe::launch_route_multihot(logits, T, E, k, norm_topk_prob != 0, topk_w,
                                                 topk_ids, multihot, probs_in_multihot,
                                                 position_map, static_cast<hipStream_t>(stream)),
                      "moe_route_multihot");
}

moe_status_t moe_router_route(moe_dtype_t dt, const void *hidden, const void *w_gate, int64_t T,
                              int32_t H, int32_t E, int32_t k, int32_t norm_topk_prob,
                              float *logits, float *topk_w, int32_t *topk_ids, void *stream) {
    const char *fn = "moe_router_route";
    moe_status_t st = check_routing_dims(T, E, k, fn);
    if (st != MOE_OK) return st;
    CHECK(k <= E, MOE_ERR_INVALID_ARG, "%s: k = %d > E = %d", fn, k, E);
    CHECK(dt == MOE_F32 || dt == MOE_BF16, MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn,
          (int)dt);
    CHECK(dt == MOE_BF16, MOE_ERR_UNSUPPORTED, "%s: only bf16 hidden / w_gate", fn);
    CHECK(H >= 1, MOE_ERR_INVALID_ARG, "%s: H = %d < 1", fn, H);
    CHECK(H % 64 == 0, MOE_ERR_UNSUPPORTED, "%s: H = %d must be a multiple of 64", fn, H);
    if (T == 0) return MOE_OK;
    CHECK(hidden && w_gate && logits && topk_w && topk_ids, MOE_ERR_INVALID_ARG,
          "%s: null pointer", fn);
    CHECK(aligned16(hidden) && aligned16(w_gate), MOE_ERR_INVALID_ARG,
          "%s: hidden and w_gate must be 16-byte aligned", fn);
    const auto a4 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
    CHECK(a4(logits) && a4(topk_w) && a4(topk_ids), MOE_ERR_INVALID_ARG,
          "%s: outputs must be 4-byte aligned", fn);
    return hip_status(moe::launch_router_route(static_cast<const uint16_t *>(hidden),
                                               static_cast<const uint16_t *>(w_gate), T, H, E, k,
                                               norm_topk_prob != 0, logits, topk_w, topk_ids,
                                               static_cast<hipStream_t>(stream)),
                      fn);
}

size_t moe_router_backward_workspace_size(int64_t T, int32_t H, int32_t E) {
    if (T <= 0 || H < 1 || E < 1) return 0;
    return moe::router_backward_scratch_bytes(T, H, E);
}

moe_status_t moe_router_backward(moe_dtype_t dt, const void *hidden, const void *w_gate,
                                 const float *grad_logits, int64_t T, int32_t H, int32_t E,
                                 float *grad_hidden, float *grad_w_gate, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    const char *fn = "moe_router_backward";
    CHECK(T >= 0, MOE_ERR_INVALID_ARG, "%s: T = %lld < 0", fn, (long long)T);
    CHECK(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_ERR_INVALID_ARG, "%s: E = %d outside [1, %d]", fn,
          E, MOE_MAX_EXPERTS);
    CHECK(dt == MOE_F32 || dt == MOE_BF16, MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn,
          (int)dt);
    CHECK(dt == MOE_BF16, MOE_ERR_UNSUPPORTED, "%s: only bf16 hidden / w_gate", fn);
    CHECK(H >= 1, MOE_ERR_INVALID_ARG, "%s: H = %d < 1", fn, H);
    CHECK(H % 64 == 0, MOE_ERR_UNSUPPORTED, "%s: H = %d must be a multiple of 64", fn, H);
    CHECK(T / 256 < 65535, MOE_ERR_UNSUPPORTED, "%s: T = %lld exceeds the launch grid", fn,
          (long long)T);
    if (T == 0) return MOE_OK;
    CHECK(hidden && w_gate && grad_logits && grad_hidden && grad_w_gate, MOE_ERR_INVALID_ARG,
          "%s: null pointer", fn);
    CHECK(aligned16(hidden) && aligned16(w_gate) && aligned16(grad_hidden) &&
              aligned16(grad_w_gate),
          MOE_ERR_INVALID_ARG, "%s: hidden, w_gate and the gradients must be 16-byte aligned",
          fn);
    const size_t need = moe::router_backward_scratch_bytes(T, H, E);
    CHECK(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, need);
    CHECK(aligned16(workspace), MOE_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned",
          fn);
    return hip_status(moe::launch_router_backward(static_cast<const uint16_t *>(hidden),
                                                  static_cast<const uint16_t *>(w_gate),
                                                  grad_logits, T, H, E, grad_hidden,
                                                  grad_w_gate, workspace,
                                                  static_cast<hipStream_t>(stream)),
                      fn);
}

moe_status_t moe_route_grouped(const float *scores, const float *e_score_correction_bias,
                               int64_t T, int32_t E, int32_t k, int32_t n_group,
                               int32_t topk_group, int32_t method, int32_t renormalize,
                               float *topk_w, int32_t *topk_ids, uint8_t *multihot,
                               float *probs_in_multihot, int32_t *position_map, void *stream) {
    const char *fn = "moe_route_grouped";
    moe_status_t st = check_routing_dims(T, E, k, fn);
    if (st != MOE_OK) return st;
    CHECK(method == MOE_GROUP_LIMITED_GREEDY || method == MOE_NOAUX_TC, MOE_ERR_INVALID_ARG,
          "%s: unknown method %d", fn, method);
    CHECK(n_group >= 1 && n_group <= MOE_MAX_GROUPS, MOE_ERR_INVALID_ARG,
          "%s: n_group = %d outside [1, %d]", fn, n_group, MOE_MAX_GROUPS);
    CHECK(E % n_group == 0, MOE_ERR_INVALID_ARG, "%s: E = %d not a multiple of n_group = %d", fn,
          E, n_group);
    CHECK(topk_group >= 1 && topk_group <= n_group, MOE_ERR_INVALID_ARG,
          "%s: topk_group = %d outside [1, n_group = %d]", fn, topk_group, n_group);
    const int32_t gs = E / n_group;
    CHECK(k <= topk_group * gs, MOE_ERR_INVALID_ARG,
          "%s: k = %d > topk_group * group size = %d", fn, k, topk_group * gs);
    CHECK(method != MOE_NOAUX_TC || gs >= 2, MOE_ERR_INVALID_ARG,
          "%s: noaux_tc needs groups of at least 2 experts (E / n_group = %d)", fn, gs);
    const int n_mh = (multihot != nullptr) + (probs_in_multihot != nullptr) +
                     (position_map != nullptr);
    CHECK(n_mh == 0 || n_mh == 3, MOE_ERR_INVALID_ARG,
          "%s: give all three multihot outputs or none", fn);
    if (T == 0) return MOE_OK;
    CHECK(scores && topk_w && topk_ids, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    CHECK(method != MOE_NOAUX_TC || e_score_correction_bias, MOE_ERR_INVALID_ARG,
          "%s: noaux_tc needs e_score_correction_bias", fn);
    const auto a4 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
    CHECK(a4(scores) && a4(topk_w) && a4(topk_ids) &&
              (method != MOE_NOAUX_TC || a4(e_score_correction_bias)),
          MOE_ERR_INVALID_ARG, "%s: pointers must be 4-byte aligned", fn);
    return hip_status(moe::launch_route_grouped(scores,
                                                method == MOE_NOAUX_TC ? e_score_correction_bias
                                                                       : nullptr,
                                                T, E, k, n_group, topk_group,
                                                method == MOE_NOAUX_TC, renormalize != 0, topk_w,
                                                topk_ids, multihot, probs_in_multihot,
                                                position_map, static_cast<hipStream_t>(stream)),
                      fn);
}

int32_t moe_route_multihot_fused(int32_t E, int32_t k) {
    return E >= 1 && k >= 1 && k <= E && E <= 64 && E % 4 == 0 && k <= 16;
}

size_t moe_align_workspace_size(int64_t T, int32_t k, int32_t E) {
    if (T < 0 || k < 1 || E < 1 || E > MOE_MAX_EXPERTS) return 0;
    const int nb = moe::align_num_blocks(T * k, E);
    return round_up((size_t)nb * (size_t)E * sizeof(int32_t), 256);
}

moe_status_t moe_align(const int32_t *topk_ids, int64_t T, int32_t k, int32_t E,
                       int32_t *expert_counts, int32_t *expert_offsets,
                       int32_t *sorted_token_ids, int32_t *sorted_slot_ids,
                       int32_t *slot_to_sorted, void *workspace, size_t workspace_bytes,
                       void *stream) {
    moe_status_t st = check_routing_dims(T, E, k, "moe_align");
    if (st != MOE_OK) return st;
    CHECK(expert_counts && expert_offsets, MOE_ERR_INVALID_ARG, "moe_align: null pointer");
    CHECK(T == 0 || (topk_ids && sorted_token_ids && sorted_slot_ids && slot_to_sorted),
          MOE_ERR_INVALID_ARG, "moe_align: null pointer");
    const size_t need = moe_align_workspace_size(T, k, E);
    CHECK(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "moe_align: workspace %zu bytes, need %zu", workspace_bytes, need);
    return hip_status(moe::launch_align(topk_ids, T, k, E, expert_counts, expert_offsets,
                                        sorted_token_ids, sorted_slot_ids, slot_to_sorted,
                                        static_cast<int32_t *>(workspace),
                                        static_cast<hipStream_t>(stream)),
                      "moe_align");
}

moe_status_t moe_align_inverse(const int32_t *topk_ids, int64_t T, int32_t k, int32_t E,
                               int32_t *expert_counts, int32_t *expert_offsets,
                               int32_t *sorted_token_ids, int32_t *sorted_slot_ids,
                               int32_t *slot_to_sorted, const float *probs_in_multihot,
                               const int32_t *position_map, float *probs_indices,
                               int32_t *ids_from_multihot, void *workspace,
                               size_t workspace_bytes, void *stream) {
    const char *fn = "moe_align_inverse";
    moe_status_t st = check_routing_dims(T, E, k, fn);
    if (st != MOE_OK) return st;
    CHECK(expert_counts && expert_offsets, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    CHECK(T == 0 || (topk_ids && sorted_token_ids && sorted_slot_ids && slot_to_sorted &&
                     probs_in_multihot && position_map && probs_indices),
          MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    const size_t need = moe_align_workspace_size(T, k, E);
    CHECK(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, need);
    return hip_status(moe::launch_align(topk_ids, T, k, E, expert_counts, expert_offsets,
                                        sorted_token_ids, sorted_slot_ids, slot_to_sorted,
                                        static_cast<int32_t *>(workspace),
                                        static_cast<hipStream_t>(stream), probs_in_multihot,
                                        position_map, T == 0 ? nullptr : probs_indices,
                                        ids_from_multihot),
                      fn);
}

}  // extern "C"

namespace {

// moe_route_align's checks and launches, with the alignment scratch given as
// a device pointer (the caller's workspace, or the library's static array).
moe_status_t route_align_check(const char *fn, const float *logits, int64_t T, int32_t E,
                               int32_t k, float *topk_w, int32_t *topk_ids, uint8_t *multihot,
                               float *probs_in_multihot, int32_t *position_map,
                               int32_t *expert_counts, int32_t *expert_offsets,
                               int32_t *sorted_token_ids, int32_t *sorted_slot_ids,
                               int32_t *slot_to_sorted, void *workspace, size_t workspace_bytes,
                               float *inv_probs, int32_t *inv_ids) {
    moe_status_t st = check_routing_dims(T, E, k, fn);
    if (st != MOE_OK) return st;
    CHECK(k <= E, MOE_ERR_INVALID_ARG, "%s: k = %d > E = %d", fn, k, E);
    const int n_mh = (multihot != nullptr) + (probs_in_multihot != nullptr) +
                     (position_map != nullptr);
    CHECK(n_mh == 0 || n_mh == 3, MOE_ERR_INVALID_ARG,
          "%s: give all three multihot outputs or none", fn);
    CHECK(inv_ids == nullptr || inv_probs != nullptr, MOE_ERR_INVALID_ARG,
          "%s: ids of the inverse conversion without its probs", fn);
    CHECK(inv_probs == nullptr || n_mh == 3, MOE_ERR_INVALID_ARG,
          "%s: the inverse conversion needs the multihot outputs", fn);
    CHECK(expert_counts && expert_offsets, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    CHECK(T == 0 || (logits && topk_w && topk_ids && sorted_token_ids && sorted_slot_ids &&
                     slot_to_sorted),
          MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    const size_t need = moe_align_workspace_size(T, k, E);
    CHECK(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, need);
    return MOE_OK;
}

moe_status_t route_align_impl(const char *fn, const float *logits, int64_t T, int32_t E,
                              int32_t k, int32_t norm_topk_prob, float *topk_w,
                              int32_t *topk_ids, uint8_t *multihot, float *probs_in_multihot,
                              int32_t *position_map, int32_t *expert_counts,
                              int32_t *expert_offsets, int32_t *sorted_token_ids,
                              int32_t *sorted_slot_ids, int32_t *slot_to_sorted,
                              void *workspace, size_t workspace_bytes, void *stream,
                              float *inv_probs = nullptr, int32_t *inv_ids = nullptr) {
    moe_status_t st = route_align_check(fn, logits, T, E, k, topk_w, topk_ids, multihot,
                                        probs_in_multihot, position_map, expert_counts,
                                        expert_offsets, sorted_token_ids, sorted_slot_ids,
                                        slot_to_sorted, workspace, workspace_bytes, inv_probs,
                                        inv_ids);
    if (st != MOE_OK) return st;
    return hip_status(moe::launch_route_align(logits, T, E, k, norm_topk_prob != 0, topk_w,
                                              topk_ids, multihot, probs_in_multihot,
                                              position_map, expert_counts, expert_offsets,
                                              sorted_token_ids, sorted_slot_ids, slot_to_sorted,
                                              static_cast<int32_t *>(workspace), inv_probs,
                                              inv_ids, static_cast<hipStream_t>(stream)),
                      fn);
}

// The allocation-free variant's scratch: a file-scope device array, one copy
// per GPU, zero at load and held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in
// symbol): each device's address is looked up once, with that device
// current, and kept in scratch_ptr.
constexpr size_t kStaticScratchBytes = 256 * 1024;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

moe_status_t static_scratch(const char *fn, void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, fn);
    CHECK(dev >= 0 && dev < kMaxDevices, MOE_ERR_UNSUPPORTED, "%s: device %d >= %d", fn, dev,
          kMaxDevices);
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
            CHECK(p != nullptr, MOE_ERR_HIP, "%s: no device address for the static scratch",
                  fn);
            scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_route_align(const float *logits, int64_t T, int32_t E, int32_t k,
                             int32_t norm_topk_prob, float *topk_w, int32_t *topk_ids,
                             uint8_t *multihot, float *probs_in_multihot, int32_t *position_map,
                             int32_t *expert_counts, int32_t *expert_offsets,
                             int32_t *sorted_token_ids, int32_t *sorted_slot_ids,
                             int32_t *slot_to_sorted, void *workspace, size_t workspace_bytes,
                             void *stream) {
    return route_align_impl("moe_route_align", logits, T, E, k, norm_topk_prob, topk_w, topk_ids,
                            multihot, probs_in_multihot, position_map, expert_counts,
                            expert_offsets, sorted_token_ids, sorted_slot_ids, slot_to_sorted,
                            workspace, workspace_bytes, stream);
}

moe_status_t moe_route_align_inverse(const float *logits, int64_t T, int32_t E, int32_t k,
                                     int32_t norm_topk_prob, float *topk_w, int32_t *topk_ids,
                                     uint8_t *multihot, float *probs_in_multihot,
                                     int32_t *position_map, int32_t *expert_counts,
                                     int32_t *expert_offsets, int32_t *sorted_token_ids,
                                     int32_t *sorted_slot_ids, int32_t *slot_to_sorted,
                                     float *probs_indices, int32_t *ids_from_multihot,
                                     void *workspace, size_t workspace_bytes, void *stream) {
    const char *fn = "moe_route_align_inverse";
    CHECK(T == 0 || (multihot && probs_in_multihot && position_map && probs_indices),
          MOE_ERR_INVALID_ARG, "%s: null pointer (the multihot outputs are required)", fn);
    if (T == 0)  // no rows to convert: moe_route_align's zero counts and offsets
        return route_align_impl(fn, logits, T, E, k, norm_topk_prob, topk_w, topk_ids, nullptr,
                                nullptr, nullptr, expert_counts, expert_offsets,
                                sorted_token_ids, sorted_slot_ids, slot_to_sorted, workspace,
                                workspace_bytes, stream);
    return route_align_impl(fn, logits, T, E, k, norm_topk_prob, topk_w, topk_ids, multihot,
                            probs_in_multihot, position_map, expert_counts, expert_offsets,
                            sorted_token_ids, sorted_slot_ids, slot_to_sorted, workspace,
                            workspace_bytes, stream, probs_indices, ids_from_multihot);
}

int32_t moe_route_align_gate_up_fused(int64_t T, int32_t E, int32_t k, moe_dtype_t dt,
                                      int32_t decode, int32_t H, int32_t I) {
    return dt == MOE_BF16 && decode && H >= 1 && I >= 1 && H % 64 == 0 && I % 64 == 0 &&
           moe::decode_route_gate_up_fused(T, E, k, H, I);
}

moe_status_t moe_route_align_gate_up(
    const float *logits, int64_t T, int32_t E, int32_t k, int32_t norm_topk_prob, float *topk_w,
    int32_t *topk_ids, uint8_t *multihot, float *probs_in_multihot, int32_t *position_map,
    int32_t *expert_counts, int32_t *expert_offsets, int32_t *sorted_token_ids,
    int32_t *sorted_slot_ids, int32_t *slot_to_sorted, float *probs_indices,
    int32_t *ids_from_multihot, moe_dtype_t dt, int32_t decode, const void *hidden,
    const void *w13, int32_t H, int32_t I, void *act, void *workspace, size_t workspace_bytes,
    void *stream) {
    const char *fn = "moe_route_align_gate_up";
    moe_status_t st = route_align_check(fn, logits, T, E, k, topk_w, topk_ids, multihot,
                                        probs_in_multihot, position_map, expert_counts,
                                        expert_offsets, sorted_token_ids, sorted_slot_ids,
                                        slot_to_sorted, workspace, workspace_bytes, probs_indices,
                                        ids_from_multihot);
    if (st != MOE_OK) return st;
    st = check_ffn_dims(dt, T, H, I, E, k, fn);
    if (st != MOE_OK) return st;
    if (decode)
        CHECK(T <= MOE_DECODE_MAX_T, MOE_ERR_UNSUPPORTED, "%s: decode needs T <= %d", fn,
              MOE_DECODE_MAX_T);
    if (T > 0) {
        CHECK(hidden && w13 && act, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
        CHECK(aligned16(hidden) && aligned16(w13) && aligned16(act), MOE_ERR_INVALID_ARG,
              "%s: hidden, w13 and act must be 16-byte aligned", fn);
    }
    const bool fused = T > 0 && moe_route_align_gate_up_fused(T, E, k, dt, decode, H, I) &&
                       (multihot == nullptr ||
                        moe::route_multihot_fused(E, k, multihot, probs_in_multihot,
                                                  position_map));
    if (T == 0)  // no rows: the alignment's zero counts and offsets only
        return route_align_impl(fn, logits, T, E, k, norm_topk_prob, topk_w, topk_ids, nullptr,
                                nullptr, nullptr, expert_counts, expert_offsets,
                                sorted_token_ids, sorted_slot_ids, slot_to_sorted, workspace,
                                workspace_bytes, stream);
    if (!fused) {
        st = route_align_impl(fn, logits, T, E, k, norm_topk_prob, topk_w, topk_ids, multihot,
                              probs_in_multihot, position_map, expert_counts, expert_offsets,
                              sorted_token_ids, sorted_slot_ids, slot_to_sorted, workspace,
                              workspace_bytes, stream, probs_indices, ids_from_multihot);
        if (st != MOE_OK) return st;
        return moe_ffn_gate_up(dt, decode, hidden, w13, expert_offsets, sorted_token_ids, T, H, I,
                               E, k, act, stream);
    }
    return hip_status(moe::launch_decode_route_gate_up_bf16(
                          logits, T, E, k, norm_topk_prob != 0, topk_w, topk_ids, multihot,
                          probs_in_multihot, position_map, expert_counts, expert_offsets,
                          sorted_token_ids, sorted_slot_ids, slot_to_sorted, probs_indices,
                          ids_from_multihot, static_cast<const uint16_t *>(hidden),
                          static_cast<const uint16_t *>(w13), H, I, static_cast<uint16_t *>(act),
                          static_cast<hipStream_t>(stream)),
                      fn);
}

moe_status_t moe_route_align_noalloc(const float *logits, int64_t T, int32_t E, int32_t k,
                                     int32_t norm_topk_prob, float *topk_w, int32_t *topk_ids,
                                     uint8_t *multihot, float *probs_in_multihot,
                                     int32_t *position_map, int32_t *expert_counts,
                                     int32_t *expert_offsets, int32_t *sorted_token_ids,
                                     int32_t *sorted_slot_ids, int32_t *slot_to_sorted,
                                     void *stream) {
    const char *fn = "moe_route_align_noalloc";
    moe_status_t st = check_routing_dims(T, E, k, fn);
    if (st != MOE_OK) return st;
    const size_t need = moe_align_workspace_size(T, k, E);
    CHECK(need <= kStaticScratchBytes, MOE_ERR_WORKSPACE,
          "%s: needs %zu bytes of scratch, the static array holds %zu", fn, need,
          kStaticScratchBytes);
    void *ws = nullptr;
    st = static_scratch(fn, &ws);
    if (st != MOE_OK) return st;
    return route_align_impl(fn, logits, T, E, k, norm_topk_prob, topk_w, topk_ids, multihot,
                            probs_in_multihot, position_map, expert_counts, expert_offsets,
                            sorted_token_ids, sorted_slot_ids, slot_to_sorted, ws,
                            kStaticScratchBytes, stream);
}

int64_t moe_tile_schedule_max(int64_t T, int32_t k, int32_t E) {
    if (T <= 0 || k < 1 || E < 1) return 0;
    const int64_t rows = T * k;
    return (rows + moe::kGemmBM - 1) / moe::kGemmBM + (rows < E ? rows : E);
}

moe_status_t moe_tile_schedule(const int32_t *expert_offsets, int32_t E, int64_t max_tiles,
                               int32_t *tile_expert, int32_t *tile_row_start,
                               int32_t *tile_row_end, int32_t *num_tiles, void *stream) {
    const char *fn = "moe_tile_schedule";
    CHECK(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED, "%s: E = %d outside [1, %d]", fn,
          E, MOE_MAX_EXPERTS);
    CHECK(max_tiles >= 0, MOE_ERR_INVALID_ARG, "%s: max_tiles < 0", fn);
    CHECK(expert_offsets && num_tiles &&
              (max_tiles == 0 || (tile_expert && tile_row_start && tile_row_end)),
          MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    return hip_status(moe::launch_tile_schedule(expert_offsets, E, max_tiles, tile_expert,
                                                tile_row_start, tile_row_end, num_tiles,
                                                static_cast<hipStream_t>(stream)),
                      fn);
}

int32_t moe_route_align_fused(int64_t T, int32_t E, int32_t k) {
    if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK) return 0;
    return moe::route_align_fused(T, E, k, nullptr, nullptr, nullptr);
}

moe_status_t moe_indices_to_multihot(const int32_t *ids, const float *probs, int64_t T,
                                     int32_t k, int32_t E, uint8_t *multihot,
                                     float *probs_in_multihot, int32_t *position_map,
                                     void *stream) {
    moe_status_t st = check_routing_dims(T, E, k, "moe_indices_to_multihot");
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    CHECK(ids && probs && multihot && probs_in_multihot && position_map, MOE_ERR_INVALID_ARG,
          "moe_indices_to_multihot: null pointer");
    return hip_status(moe::launch_to_multihot(ids, probs, T, k, E, multihot, probs_in_multihot,
                                              position_map, static_cast<hipStream_t>(stream)),
                      "moe_indices_to_multihot");
}

moe_status_t moe_multihot_to_indices(const float *probs_in_multihot,
                                     const int32_t *position_map, int64_t T, int32_t E,
                                     int32_t k, float *probs_indices, int32_t *ids_out,
                                     void *stream) {
    moe_status_t st = check_routing_dims(T, E, k, "moe_multihot_to_indices");
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    CHECK(probs_in_multihot && position_map && probs_indices, MOE_ERR_INVALID_ARG,
          "moe_multihot_to_indices: null pointer");
    return hip_status(moe::launch_to_indices(probs_in_multihot, position_map, T, E, k,
                                             probs_indices, ids_out,
                                             static_cast<hipStream_t>(stream)),
                      "moe_multihot_to_indices");
}

size_t moe_expert_ffn_workspace_size(moe_dtype_t dt, int64_t T, int32_t H, int32_t I,
                                     int32_t E, int32_t k) {
    if (T < 0 || H < 1 || I < 1 || k < 1 || E < 1) return 0;
    return ffn_scratch_bytes(dt, T, H, I, E, k, prefill_splits(dt, T, H, I, E, k));
}

int32_t moe_ffn_down_splits(moe_dtype_t dt, int32_t decode, int64_t T, int32_t H, int32_t I,
                            int32_t E, int32_t k) {
    if (decode || T < 0 || H < 1 || I < 1 || k < 1 || E < 1) return 1;
    return prefill_splits(dt, T, H, I, E, k);
}

moe_status_t moe_ffn_gate_up(moe_dtype_t dt, int32_t decode, const void *hidden,
                             const void *w13, const int32_t *expert_offsets,
                             const int32_t *sorted_token_ids, int64_t T, int32_t H, int32_t I,
                             int32_t E, int32_t k, void *act, void *stream) {
    const char *fn = "moe_ffn_gate_up";
    moe_status_t st = check_ffn_dims(dt, T, H, I, E, k, fn);
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    CHECK(hidden && w13 && expert_offsets && sorted_token_ids && act, MOE_ERR_INVALID_ARG,
          "%s: null pointer", fn);
    CHECK(aligned16(hidden) && aligned16(w13) && aligned16(act), MOE_ERR_INVALID_ARG,
          "%s: hidden, w13 and act must be 16-byte aligned", fn);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dt == MOE_F32) {
        e = moe::launch_gate_up_f32(static_cast<const float *>(hidden),
                                    static_cast<const float *>(w13), expert_offsets,
                                    sorted_token_ids, T, H, I, E, k, static_cast<float *>(act), s);
    } else if (decode) {
        CHECK(T <= MOE_DECODE_MAX_T, MOE_ERR_UNSUPPORTED, "%s: decode needs T <= %d", fn,
              MOE_DECODE_MAX_T);
        e = moe::launch_decode_gate_up_bf16(static_cast<const uint16_t *>(hidden),
                                            static_cast<const uint16_t *>(w13), expert_offsets,
                                            sorted_token_ids, T, H, I, E, k,
                                            static_cast<uint16_t *>(act), s);
    } else {
        e = moe::launch_gate_up_bf16(static_cast<const uint16_t *>(hidden),
                                     static_cast<const uint16_t *>(w13), expert_offsets,
                                     sorted_token_ids, T, H, I, E, k,
                                     static_cast<uint16_t *>(act), s);
    }
    return hip_status(e, fn);
}

moe_status_t moe_ffn_down(moe_dtype_t dt, int32_t decode, const void *act, const void *w2,
                          const int32_t *expert_offsets, int64_t T, int32_t H, int32_t I,
                          int32_t E, int32_t k, int32_t splits, float *y, void *stream) {
    const char *fn = "moe_ffn_down";
    moe_status_t st = check_ffn_dims(dt, T, H, I, E, k, fn);
    if (st != MOE_OK) return st;
    CHECK(splits >= 1 && splits <= MOE_MAX_SPLITS, MOE_ERR_INVALID_ARG,
          "%s: splits = %d outside [1, %d]", fn, splits, MOE_MAX_SPLITS);
    CHECK(splits == 1 || (dt == MOE_BF16 && !decode), MOE_ERR_UNSUPPORTED,
          "%s: K slices need the bfloat16 prefill path", fn);
    CHECK(I % (64 * splits) == 0, MOE_ERR_UNSUPPORTED,
          "%s: I = %d is not a multiple of 64 * splits = %d", fn, I, 64 * splits);
    if (T == 0) return MOE_OK;
    CHECK(act && w2 && expert_offsets && y, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    CHECK(aligned16(act) && aligned16(w2) && aligned16(y), MOE_ERR_INVALID_ARG,
          "%s: act, w2 and y must be 16-byte aligned", fn);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dt == MOE_F32) {
        e = moe::launch_down_f32(static_cast<const float *>(act), static_cast<const float *>(w2),
                                 expert_offsets, T, H, I, E, k, y, s);
    } else if (decode) {
        CHECK(T <= MOE_DECODE_MAX_T, MOE_ERR_UNSUPPORTED, "%s: decode needs T <= %d", fn,
              MOE_DECODE_MAX_T);
        e = moe::launch_decode_down_bf16(static_cast<const uint16_t *>(act),
                                         static_cast<const uint16_t *>(w2), expert_offsets, T, H,
                                         I, E, k, y, s);
    } else {
        e = moe::launch_down_bf16(static_cast<const uint16_t *>(act),
                                  static_cast<const uint16_t *>(w2), expert_offsets, T, H, I, E,
                                  k, splits, y, s);
    }
    return hip_status(e, fn);
}

moe_status_t moe_combine(moe_dtype_t dt, const float *y, int32_t splits, const float *topk_w,
                         const int32_t *slot_to_sorted, int64_t T, int32_t H, int32_t k,
                         void *out, void *stream) {
    const char *fn = "moe_combine";
    CHECK(splits >= 1 && splits <= MOE_MAX_SPLITS, MOE_ERR_INVALID_ARG,
          "%s: splits = %d outside [1, %d]", fn, splits, MOE_MAX_SPLITS);
    CHECK(T >= 0 && k >= 1 && k <= MOE_MAX_TOPK && H >= 1, MOE_ERR_INVALID_ARG,
          "%s: bad sizes T = %lld, H = %d, k = %d", fn, (long long)T, H, k);
    CHECK(dt == MOE_F32 || dt == MOE_BF16, MOE_ERR_INVALID_ARG, "%s: unknown dtype", fn);
    CHECK(H % 64 == 0, MOE_ERR_UNSUPPORTED, "%s: H = %d must be a multiple of 64", fn, H);
    if (T == 0) return MOE_OK;
    CHECK(y && topk_w && slot_to_sorted && out, MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    CHECK(aligned16(y) && aligned16(out), MOE_ERR_INVALID_ARG,
          "%s: y and out must be 16-byte aligned", fn);
    return hip_status(moe::launch_combine(dt, y, splits, topk_w, slot_to_sorted, T, H, k, out,
                                          static_cast<hipStream_t>(stream)),
                      fn);
}

moe_status_t moe_ffn_down_combine(moe_dtype_t dt, int32_t decode, const void *act,
                                  const void *w2, const float *topk_w,
                                  const int32_t *expert_offsets, const int32_t *slot_to_sorted,
                                  int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                  float *y, void *out, void *stream) {
    const char *fn = "moe_ffn_down_combine";
    moe_status_t st = check_ffn_dims(dt, T, H, I, E, k, fn);
    if (st != MOE_OK) return st;
    if (decode)
        CHECK(T <= MOE_DECODE_MAX_T, MOE_ERR_UNSUPPORTED, "%s: decode needs T <= %d", fn,
              MOE_DECODE_MAX_T);
    if (T == 0) return MOE_OK;
    const bool fused = dt == MOE_BF16 && decode && moe::decode_down_combine_fused(T, H, I, E, k);
    CHECK(act && w2 && expert_offsets && topk_w && slot_to_sorted && out && (fused || y),
          MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (fused) {
        CHECK(aligned16(act) && aligned16(w2) && aligned16(out), MOE_ERR_INVALID_ARG,
              "%s: act, w2 and out must be 16-byte aligned", fn);
        return hip_status(moe::launch_decode_down_combine_bf16(
                              static_cast<const uint16_t *>(act),
                              static_cast<const uint16_t *>(w2), expert_offsets, topk_w,
                              slot_to_sorted, T, H, I, E, k, static_cast<uint16_t *>(out),
                              static_cast<hipStream_t>(stream)),
                          fn);
    }
    const int32_t splits = decode ? 1 : prefill_splits(dt, T, H, I, E, k);
    st = moe_ffn_down(dt, decode, act, w2, expert_offsets, T, H, I, E, k, splits, y, stream);
    if (st != MOE_OK) return st;
    return moe_combine(dt, y, splits, topk_w, slot_to_sorted, T, H, k, out, stream);
}

int32_t moe_ffn_down_combine_fused(moe_dtype_t dt, int32_t decode, int64_t T, int32_t H,
                                   int32_t I, int32_t E, int32_t k) {
    return dt == MOE_BF16 && decode && T >= 1 && T <= MOE_DECODE_MAX_T && H >= 1 && I >= 1 &&
           k >= 1 && moe::decode_down_combine_fused(T, H, I, E, k);
}

static moe_status_t expert_ffn_impl(int32_t decode, moe_dtype_t dt, const void *hidden,
                                    const void *w13, const void *w2, const float *topk_w,
                                    const int32_t *expert_offsets,
                                    const int32_t *sorted_token_ids,
                                    const int32_t *slot_to_sorted, int64_t T, int32_t H,
                                    int32_t I, int32_t E, int32_t k, void *out, void *workspace,
                                    size_t workspace_bytes, void *stream, const char *fn) {
    moe_status_t st = check_ffn_dims(dt, T, H, I, E, k, fn);
    if (st != MOE_OK) return st;
    if (decode)
        CHECK(T <= MOE_DECODE_MAX_T, MOE_ERR_UNSUPPORTED, "%s: T = %lld > %d", fn, (long long)T,
              MOE_DECODE_MAX_T);
    if (T == 0) return MOE_OK;
    CHECK(hidden && w13 && w2 && topk_w && expert_offsets && sorted_token_ids &&
              slot_to_sorted && out,
          MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    const int32_t splits = decode ? 1 : prefill_splits(dt, T, H, I, E, k);
    const size_t need = ffn_scratch_bytes(dt, T, H, I, E, k, splits);
    CHECK(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, need);
    CHECK(aligned16(workspace), MOE_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned",
          fn);
    char *act = static_cast<char *>(workspace);
    float *y = reinterpret_cast<float *>(act + ffn_act_bytes(dt, T, I, k));
    st = moe_ffn_gate_up(dt, decode, hidden, w13, expert_offsets, sorted_token_ids, T, H, I, E,
                         k, act, stream);
    if (st != MOE_OK) return st;
    return moe_ffn_down_combine(dt, decode, act, w2, topk_w, expert_offsets, slot_to_sorted, T, H,
                                I, E, k, y, out, stream);
}

moe_status_t moe_expert_ffn(moe_dtype_t dt, const void *hidden, const void *w13,
                            const void *w2, const float *topk_w,
                            const int32_t *expert_offsets, const int32_t *sorted_token_ids,
                            const int32_t *slot_to_sorted, int64_t T, int32_t H, int32_t I,
                            int32_t E, int32_t k, void *out, void *workspace,
                            size_t workspace_bytes, void *stream) {
    return expert_ffn_impl(0, dt, hidden, w13, w2, topk_w, expert_offsets, sorted_token_ids,
                           slot_to_sorted, T, H, I, E, k, out, workspace, workspace_bytes, stream,
                           "moe_expert_ffn");
}

moe_status_t moe_expert_ffn_decode(moe_dtype_t dt, const void *hidden, const void *w13,
                                   const void *w2, const float *topk_w,
                                   const int32_t *expert_offsets,
                                   const int32_t *sorted_token_ids,
                                   const int32_t *slot_to_sorted, int64_t T, int32_t H,
                                   int32_t I, int32_t E, int32_t k, void *out, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    return expert_ffn_impl(1, dt, hidden, w13, w2, topk_w, expert_offsets, sorted_token_ids,
                           slot_to_sorted, T, H, I, E, k, out, workspace, workspace_bytes, stream,
                           "moe_expert_ffn_decode");
}

moe_status_t moe_route_backward(const float *logits, const int32_t *topk_ids,
                                const float *topk_w, const float *grad_topk_w, int64_t T,
                                int32_t E, int32_t k, int32_t norm_topk_prob,
                                float *grad_logits, void *stream) {
    const char *fn = "moe_route_backward";
    moe_status_t st = check_routing_dims(T, E, k, fn);
    if (st != MOE_OK) return st;
    CHECK(k <= E, MOE_ERR_INVALID_ARG, "%s: k = %d > E = %d", fn, k, E);
    if (T == 0) return MOE_OK;
    CHECK(logits && topk_ids && topk_w && grad_topk_w && grad_logits, MOE_ERR_INVALID_ARG,
          "%s: null pointer", fn);
    return hip_status(moe::launch_route_backward(logits, topk_ids, topk_w, grad_topk_w, T, E, k,
                                                 norm_topk_prob ? 1 : 0, grad_logits,
                                                 static_cast<hipStream_t>(stream)),
                      fn);
}

moe_status_t moe_route_grouped_backward(const float *scores, const int32_t *topk_ids,
                                        const float *topk_w, const float *grad_topk_w, int64_t T,
                                        int32_t E, int32_t k, int32_t renormalize,
                                        float *grad_scores, void *stream) {
    const char *fn = "moe_route_grouped_backward";
    moe_status_t st = check_routing_dims(T, E, k, fn);
    if (st != MOE_OK) return st;
    CHECK(k <= E, MOE_ERR_INVALID_ARG, "%s: k = %d > E = %d", fn, k, E);
    if (T == 0) return MOE_OK;
    CHECK(scores && topk_ids && topk_w && grad_topk_w && grad_scores, MOE_ERR_INVALID_ARG,
          "%s: null pointer", fn);
    return hip_status(moe::launch_route_grouped_backward(scores, topk_ids, topk_w, grad_topk_w, T,
                                                         E, k, renormalize ? 1 : 0, grad_scores,
                                                         static_cast<hipStream_t>(stream)),
                      fn);
}

size_t moe_expert_ffn_backward_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E,
                                              int32_t k) {
    if (T <= 0 || H < 1 || I < 1 || E < 1 || k < 1) return 0;
    const size_t b16 = moe::ffn_backward_scratch_bytes(T, H, I, E, k);
    const size_t f32 = moe::ffn_backward_f32_scratch_bytes(T, H, I, k);
    return b16 > f32 ? b16 : f32;
}

moe_status_t moe_expert_ffn_backward(moe_dtype_t dt, const void *hidden, const void *w13,
                                     const void *w2, const float *topk_w,
                                     const int32_t *expert_offsets,
                                     const int32_t *sorted_token_ids,
                                     const int32_t *sorted_slot_ids,
                                     const int32_t *slot_to_sorted, const void *grad_out,
                                     int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                                     float *grad_hidden, float *grad_w13, float *grad_w2,
                                     float *grad_topk_w, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    const char *fn = "moe_expert_ffn_backward";
    moe_status_t st = check_ffn_dims(dt, T, H, I, E, k, fn);
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    CHECK(hidden && w13 && w2 && topk_w && expert_offsets && sorted_token_ids &&
              sorted_slot_ids && slot_to_sorted && grad_out && grad_hidden && grad_w13 &&
              grad_w2 && grad_topk_w,
          MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
    CHECK(aligned16(hidden) && aligned16(w13) && aligned16(w2) && aligned16(grad_out) &&
              aligned16(grad_hidden) && aligned16(grad_w13) && aligned16(grad_w2),
          MOE_ERR_INVALID_ARG, "%s: hidden, weights, gradients must be 16-byte aligned", fn);
    const size_t need = dt == MOE_F32 ? moe::ffn_backward_f32_scratch_bytes(T, H, I, k)
                                      : moe::ffn_backward_scratch_bytes(T, H, I, E, k);
    CHECK(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, need);
    CHECK(aligned16(workspace), MOE_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned",
          fn);
    // Launch grids: 64 x 64 transpose tiles (the weight transposes put E times
    // H / 64 or I / 64 block rows in one grid dimension), weight-gradient
    // tiles of 128 x 128, padded positions within int32.
    const int64_t Pp = T * k + 64 * (int64_t)E + 64;
    CHECK(Pp < (int64_t)1 << 31 && (int64_t)E * H / 64 <= 65535 &&
              (int64_t)E * I / 64 <= 65535 &&
              (2 * (int64_t)I / 128 + 1) * ((int64_t)H / 128 + 1) < (int64_t)1 << 31,
          MOE_ERR_UNSUPPORTED, "%s: shape exceeds the launch grids", fn);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dt == MOE_F32) {
        CHECK((int64_t)E * 2 * I < (int64_t)1 << 31 && (int64_t)E * H < (int64_t)1 << 31,
              MOE_ERR_UNSUPPORTED, "%s: shape exceeds the launch grids", fn);
        return hip_status(moe::launch_ffn_backward_f32(
                              static_cast<const float *>(hidden), static_cast<const float *>(w13),
                              static_cast<const float *>(w2), topk_w, expert_offsets,
                              sorted_token_ids, sorted_slot_ids, slot_to_sorted,
                              static_cast<const float *>(grad_out), T, H, I, E, k, grad_hidden,
                              grad_w13, grad_w2, grad_topk_w, workspace, s),
                          fn);
    }
    return hip_status(moe::launch_ffn_backward_bf16(
                          static_cast<const uint16_t *>(hidden), static_cast<const uint16_t *>(w13),
                          static_cast<const uint16_t *>(w2), topk_w, expert_offsets,
                          sorted_token_ids, sorted_slot_ids, slot_to_sorted,
                          static_cast<const uint16_t *>(grad_out), T, H, I, E, k, grad_hidden,
                          grad_w13, grad_w2, grad_topk_w, workspace, s),
                      fn);
}

}  // extern "C"
