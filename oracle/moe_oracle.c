/*
 * moe_oracle.c -- plain, slow CPU oracle of the MoE layer forward and of its
 * backward (the chain rule on the same definitions).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or table with the HIP
 * library.
 *
 * Every floating-point step runs in double precision from inputs converted
 * exactly (float32, or bfloat16 bit patterns).  Loops follow the pages' own
 * formulations, not the GPU's: top-k by in-order insertion, alignment through
 * the dense transposed cumulative sum, converters by init-then-scatter, and
 * the expert FFN one token and one selected expert at a time.
 *
 * Sources (the three pages this method is described on):
 *   [mlc]  mlc-llm, python/mlc_llm/op/moe_misc.py ("Mixture of Experts
 *          operators"): gating_topk, _gating_topk_process_value,
 *          gating_softmax_topk, moe_cumsum, get_indices, get_indptr,
 *          scatter_output, moe_sum.
 *   [mgt]  Megatron-LM, megatron/core/fusions/fused_indices_converter.py:
 *          _indices_to_multihot_kernel, _multihot_to_indices_kernel,
 *          IndicesToMultihot.forward / backward.
 *   [p6]   project_6, ex_engine/csrc/moe_expert_gemm.cpp:
 *          moe_decode_experts, moe_prefill_experts.
 *
 * Readings where the pages are silent or garbled are listed in the design
 * notes; the ones that shape code here are restated at each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

int oracle_version(void) { return 1; }

static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Element h of a float32 (dt=0) or bfloat16-bits (dt=1) array, as double. */
static double load_elem(int dt, const void *base, int64_t i)
{
    if (dt == 0)
        return (double)((const float *)base)[i];
    return bf16_bits_to_double(((const uint16_t *)base)[i]);
}

/*
 * Gating top-k with softmax weights.
 *
 * [mlc] gating_topk / _gating_topk_process_value: scan the experts of a row
 * in ascending order and insert each score into a descending k-list at the
 * first place where it is strictly greater than the held value, shifting the
 * rest down.  Equal scores therefore keep the lower expert index first.  The
 * pages' initialisation of the list is garbled; read here as "empty slots
 * lose to every value", which makes the selection a total order (value
 * descending, then index ascending) and needs k <= E.
 *
 * [mlc] gating_softmax_topk: with norm_topk_prob the weights are the softmax
 * of the k selected logits (max-subtracted, summed in slot order).  Without
 * it they are the full softmax over the E logits, taken at the selected
 * experts.  Selection always runs on the logits: softmax is strictly
 * increasing, so this picks the same experts as selecting on probabilities
 * in exact arithmetic.
 */
int oracle_route(const float *logits, int64_t T, int32_t E, int32_t k,
                 int32_t norm_topk_prob, double *topk_w, int32_t *topk_ids)
{
    if (T < 0 || E < 1 || k < 1 || k > E)
        return ORACLE_EINVAL;
    double *val = (double *)malloc(sizeof(double) * (size_t)k);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    if (!val || !idx) {
        free(val);
        free(idx);
        return ORACLE_ENOMEM;
    }
    for (int64_t t = 0; t < T; ++t) {
        const float *x = logits + t * E;
        int filled = 0;
        for (int32_t e = 0; e < E; ++e) {
            double v = (double)x[e];
            for (int i = 0; i < k; ++i) {
                if (i == filled || v > val[i]) {
                    int last = filled < k ? filled : k - 1;
                    for (int j = last; j > i; --j) {
                        val[j] = val[j - 1];
                        idx[j] = idx[j - 1];
                    }
                    val[i] = v;
                    idx[i] = e;
                    if (filled < k)
                        ++filled;
                    break;
                }
            }
        }
        double m, s = 0.0;
        if (norm_topk_prob) {
            m = val[0];
            for (int i = 1; i < k; ++i)
                m = fmax(m, val[i]);
            for (int i = 0; i < k; ++i)
                s += exp(val[i] - m);
        } else {
            m = (double)x[0];
            for (int32_t e = 1; e < E; ++e)
                m = fmax(m, (double)x[e]);
            for (int32_t e = 0; e < E; ++e)
                s += exp((double)x[e] - m);
        }
        for (int i = 0; i < k; ++i) {
            topk_w[t * k + i] = exp(val[i] - m) / s;
            topk_ids[t * k + i] = idx[i];
        }
    }
    free(val);
    free(idx);
    return ORACLE_OK;
}

/*
 * Router logits, the step before gating: logits[t][e] = sum over h of
 * hidden[t][h] * w_gate[e][h], i.e. a linear layer y = x . W^T with W stored
 * [out, in] ([p6] moe_decode_experts / moe_prefill_experts apply their
 * expert weights the same way).  The pages take the logits as given; this is
 * the plain definition, one dot product per (token, expert), in double from
 * float32 (dt=0) or bfloat16-bits (dt=1) inputs, summed in ascending h.
 */
int oracle_router_logits(int32_t dt, const void *hidden, const void *w_gate, int64_t T,
                         int32_t H, int32_t E, double *logits)
{
    if (T < 0 || H < 1 || E < 1 || (dt != 0 && dt != 1))
        return ORACLE_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int32_t h = 0; h < H; ++h)
                acc += load_elem(dt, hidden, t * H + h) * load_elem(dt, w_gate, (int64_t)e * H + h);
            logits[t * E + e] = acc;
        }
    }
    return ORACLE_OK;
}

/*
 * Insertion top-k over the entries of v[0..n) that have use[e] != 0, taken in
 * ascending e: each entry goes to the first place where the list is unfilled
 * or the entry is strictly greater than the held value, shifting the rest
 * down ([mlc] _gating_topk_process_value; empty places lose to everything).
 * Returns how many places were filled (min(k, number of usable entries)).
 */
static int insert_topk(const float *v, const unsigned char *use, int32_t n, int32_t k,
                       float *val, int32_t *idx)
{
    int filled = 0;
    for (int32_t e = 0; e < n; ++e) {
        if (use && !use[e])
            continue;
        for (int i = 0; i < k; ++i) {
            if (i == filled || v[e] > val[i]) {
                int last = filled < k ? filled : k - 1;
                for (int j = last; j > i; --j) {
                    val[j] = val[j - 1];
                    idx[j] = idx[j - 1];
                }
                val[i] = v[e];
                idx[i] = e;
                if (filled < k)
                    ++filled;
                break;
            }
        }
    }
    return filled;
}

/*
 * Group-limited expert selection, [mlc] group_limited_greedy_topk.
 *
 * The E experts of a row form n_group groups of E / n_group consecutive
 * experts.  The score used for choosing is the float32 score, plus (method 1,
 * "noaux_tc") the float32 per-expert correction bias, added in float32 as
 * the page adds two float32 tensors.  A group's score is its largest choice
 * score (method 0, "group_limited_greedy") or the float32 sum of its two
 * largest (method 1; the page's top-2 then sum).  The topk_group best groups
 * are kept (top-k order: value descending, lower group first on ties), the
 * experts of the other groups are masked out, and the k best remaining
 * experts are selected in the same order.  The page fills masked entries
 * with float32's lowest finite value, which its strict-greater insertion
 * never takes; here they are simply skipped (the two agree whenever at least
 * k experts remain, which is required: k <= topk_group * group size).
 *
 * Weights: method 0 returns the selected choice scores (the scores
 * themselves); method 1 gathers the scores WITHOUT the bias at the selected
 * experts.  renormalize != 0 divides them by their sum (not on the page;
 * the optional renormalisation callers apply to these weights), in double.
 *
 * Every comparison is between float32 values, as on the page, so the
 * selection is exactly the page's; only the renormalisation runs in double.
 */
int oracle_route_grouped(const float *scores, const float *bias, int64_t T, int32_t E,
                         int32_t k, int32_t n_group, int32_t topk_group, int32_t method,
                         int32_t renormalize, double *topk_w, int32_t *topk_ids)
{
    if (T < 0 || E < 1 || k < 1 || n_group < 1 || E % n_group != 0 || topk_group < 1 ||
        topk_group > n_group || (method != 0 && method != 1))
        return ORACLE_EINVAL;
    const int32_t gs = E / n_group;
    if (k > topk_group * gs || (method == 1 && (gs < 2 || bias == NULL)))
        return ORACLE_EINVAL;
    float *choice = (float *)malloc(sizeof(float) * (size_t)E);
    float *gscore = (float *)malloc(sizeof(float) * (size_t)n_group);
    unsigned char *use = (unsigned char *)malloc((size_t)E);
    float *val = (float *)malloc(sizeof(float) * (size_t)(k > topk_group ? k : topk_group));
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k > topk_group ? k : topk_group));
    if (!choice || !gscore || !use || !val || !idx) {
        free(choice);
        free(gscore);
        free(use);
        free(val);
        free(idx);
        return ORACLE_ENOMEM;
    }
    for (int64_t t = 0; t < T; ++t) {
        const float *s = scores + t * E;
        for (int32_t e = 0; e < E; ++e)
            choice[e] = method == 1 ? s[e] + bias[e] : s[e];
        for (int32_t g = 0; g < n_group; ++g) {
            const float *c = choice + (int64_t)g * gs;
            if (method == 1) {
                float top2[2];
                int32_t at[2];
                insert_topk(c, NULL, gs, 2, top2, at);
                gscore[g] = top2[0] + top2[1];
            } else {
                float m = c[0];
                for (int32_t j = 1; j < gs; ++j)
                    if (c[j] > m)
                        m = c[j];
                gscore[g] = m;
            }
        }
        insert_topk(gscore, NULL, n_group, topk_group, val, idx);
        memset(use, 0, (size_t)E);
        for (int32_t i = 0; i < topk_group; ++i)
            memset(use + (int64_t)idx[i] * gs, 1, (size_t)gs);
        insert_topk(choice, use, E, k, val, idx);
        double sum = 0.0;
        for (int32_t i = 0; i < k; ++i)
            sum += (double)s[idx[i]];
        for (int32_t i = 0; i < k; ++i) {
            double w = (double)s[idx[i]];
            topk_w[t * k + i] = renormalize ? w / sum : w;
            topk_ids[t * k + i] = idx[i];
        }
    }
    free(choice);
    free(gscore);
    free(use);
    free(val);
    free(idx);
    return ORACLE_OK;
}

/*
 * [mlc] moe_cumsum: expert_mask[t][e] = 1 when any of row t's k ids equals e;
 * transpose to [E, T], flatten, inclusive int32 prefix sum.  An id outside
 * [0, E) matches no column, so it is dropped.  cs must hold E*T entries.
 */
int oracle_moe_cumsum(const int32_t *ids, int64_t T, int32_t k, int32_t E, int32_t *cs)
{
    if (T < 0 || E < 1 || k < 1)
        return ORACLE_EINVAL;
    int64_t run = 0;
    for (int32_t e = 0; e < E; ++e) {
        for (int64_t t = 0; t < T; ++t) {
            int hit = 0;
            for (int32_t j = 0; j < k; ++j)
                hit |= ids[t * k + j] == e;
            run += hit;
            cs[(int64_t)e * T + t] = (int32_t)run;
        }
    }
    return ORACLE_OK;
}

/*
 * Expert alignment from the cumulative sum.
 *
 * [mlc] get_indptr, exclusive form (the code, not the swapped docstring):
 *   offsets[0] = 0, offsets[i] = cs[i*T - 1] for i in 1..E.
 * [mlc] get_indices: for slot (t, j) with expert e, position
 *   p = cs[e*T + t] - 1; reverse_indices[p] = t*k + j, token_indices[p] = t.
 * The inverse map slot_to_sorted[t*k+j] = p is the same scatter read the
 * other way; slots with an id outside [0, E) get -1 there, and entries of
 * the sorted arrays past offsets[E] stay -1.
 */
int oracle_align(const int32_t *ids, int64_t T, int32_t k, int32_t E,
                 int32_t *counts, int32_t *offsets, int32_t *sorted_token_ids,
                 int32_t *sorted_slot_ids, int32_t *slot_to_sorted)
{
    if (T < 0 || E < 1 || k < 1)
        return ORACLE_EINVAL;
    int64_t n = T * k;
    for (int64_t i = 0; i < n; ++i) {
        sorted_token_ids[i] = -1;
        sorted_slot_ids[i] = -1;
        slot_to_sorted[i] = -1;
    }
    offsets[0] = 0;
    if (T == 0) {
        for (int32_t e = 0; e < E; ++e) {
            offsets[e + 1] = 0;
            counts[e] = 0;
        }
        return ORACLE_OK;
    }
    int32_t *cs = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E * T));
    if (!cs)
        return ORACLE_ENOMEM;
    oracle_moe_cumsum(ids, T, k, E, cs);
    for (int32_t i = 1; i <= E; ++i)
        offsets[i] = cs[(int64_t)i * T - 1];
    for (int32_t e = 0; e < E; ++e)
        counts[e] = offsets[e + 1] - offsets[e];
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = ids[t * k + j];
            if (e < 0 || e >= E)
                continue;
            int32_t p = cs[(int64_t)e * T + t] - 1;
            sorted_slot_ids[p] = (int32_t)(t * k + j);
            sorted_token_ids[p] = (int32_t)t;
            slot_to_sorted[t * k + j] = p;
        }
    }
    free(cs);
    return ORACLE_OK;
}

/*
 * [mgt] _indices_to_multihot_kernel: per row, first initialise
 * multihot = 0, probs_in_multihot = 0, position_map = -1 over all E columns,
 * then for each slot j whose id is valid (not -1, below E; read here as
 * 0 <= id < E) set multihot[id] = 1, probs_in_multihot[id] = probs[j] (bits
 * copied) and position_map[id] = j.
 */
int oracle_indices_to_multihot(const int32_t *ids, const float *probs, int64_t T, int32_t k,
                               int32_t E, uint8_t *multihot, float *probs_in_multihot,
                               int32_t *position_map)
{
    if (T < 0 || E < 1 || k < 1)
        return ORACLE_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t e = 0; e < E; ++e) {
            multihot[t * E + e] = 0;
            probs_in_multihot[t * E + e] = 0.0f;
            position_map[t * E + e] = -1;
        }
        for (int32_t j = 0; j < k; ++j) {
            int32_t id = ids[t * k + j];
            if (id < 0 || id >= E)
                continue;
            multihot[t * E + id] = 1;
            probs_in_multihot[t * E + id] = probs[t * k + j];
            position_map[t * E + id] = j;
        }
    }
    return ORACLE_OK;
}

/*
 * [mgt] _multihot_to_indices_kernel: per row, initialise probs_indices = 0
 * over the k slots, then for every expert e with position_map[e] != -1 write
 * probs_indices[position_map[e]] = probs_in_multihot[e].  The id each slot
 * came from is recovered the same way (ids_out[pos] = e, else -1).  Positions
 * outside [0, k) are ignored.  With two experts naming one slot (not produced
 * by the forward conversion) the later expert wins, as in this loop.
 */
int oracle_multihot_to_indices(const float *probs_in_multihot, const int32_t *position_map,
                               int64_t T, int32_t E, int32_t k, float *probs_indices,
                               int32_t *ids_out)
{
    if (T < 0 || E < 1 || k < 1)
        return ORACLE_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            probs_indices[t * k + j] = 0.0f;
            if (ids_out)
                ids_out[t * k + j] = -1;
        }
        for (int32_t e = 0; e < E; ++e) {
            int32_t p = position_map[t * E + e];
            if (p < 0 || p >= k)
                continue;
            probs_indices[t * k + p] = probs_in_multihot[t * E + e];
            if (ids_out)
                ids_out[t * k + p] = e;
        }
    }
    return ORACLE_OK;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * Expert FFN and weighted combine for a list of tokens.
 *
 * [p6] moe_decode_experts / moe_prefill_experts: for each selected expert of
 * a token, gate_up = x . w13[e]^T (weights are [out, in]), act =
 * silu(gate) * up with rows [0, I) of w13 read as the gate and rows [I, 2I)
 * as the up projection, y = act . w2[e]^T, and out += weight * y.
 * [mlc] moe_sum: the k expert outputs of a token are summed; here in slot
 * order j = 0..k-1.  Slots with an id outside [0, E) contribute nothing.
 *
 * dt: 0 = float32 inputs, 1 = bfloat16 bit patterns.  tokens[0..ntok) lists
 * which rows to evaluate (NULL = all T rows in order); out is [ntok, H]
 * double.  Nothing is rounded on the way.
 */
int oracle_expert_ffn(int32_t dt, const void *hidden, const void *w13, const void *w2,
                      const double *topk_w, const int32_t *topk_ids, int64_t T, int32_t H,
                      int32_t I, int32_t E, int32_t k, const int64_t *tokens, int64_t ntok,
                      double *out, int32_t nthreads)
{
    if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1 || (dt != 0 && dt != 1))
        return ORACLE_EINVAL;
    if (!tokens)
        ntok = T;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t r = 0; r < ntok; ++r) {
        int64_t t = tokens ? tokens[r] : r;
        double *x = (double *)malloc(sizeof(double) * (size_t)H);
        double *act = (double *)malloc(sizeof(double) * (size_t)I);
        if (!x || !act || t < 0 || t >= T) {
            free(x);
            free(act);
#pragma omp atomic write
            fail = 1;
            continue;
        }
        for (int32_t h = 0; h < H; ++h) {
            x[h] = load_elem(dt, hidden, t * H + h);
            out[r * H + h] = 0.0;
        }
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = topk_ids[t * k + j];
            if (e < 0 || e >= E)
                continue;
            double w = topk_w[t * k + j];
            int64_t base13 = (int64_t)e * 2 * I * H;
            for (int32_t i = 0; i < I; ++i) {
                double g = 0.0, u = 0.0;
                for (int32_t h = 0; h < H; ++h) {
                    g += x[h] * load_elem(dt, w13, base13 + (int64_t)i * H + h);
                    u += x[h] * load_elem(dt, w13, base13 + (int64_t)(I + i) * H + h);
                }
                act[i] = silu(g) * u;
            }
            int64_t base2 = (int64_t)e * H * I;
            for (int32_t h = 0; h < H; ++h) {
                double y = 0.0;
                for (int32_t i = 0; i < I; ++i)
                    y += act[i] * load_elem(dt, w2, base2 + (int64_t)h * I + i);
                out[r * H + h] += w * y;
            }
        }
        free(x);
        free(act);
    }
    return fail ? ORACLE_EINVAL : ORACLE_OK;
}

/*
 * Backward of the gating softmax of oracle_route, by the chain rule (the
 * pages give only the forward).  grad_topk_w [T, k] is the gradient of the
 * routing weights; the selection is piecewise constant and passes none.
 * topk_ids are the forward's (valid and distinct within a row).  The weights
 * are recomputed from the logits in double.
 *   norm_topk_prob:  w = softmax of the k selected logits, so
 *                    grad_logits[e_j] = w_j (g_j - sum_i w_i g_i), 0 elsewhere.
 *   otherwise:       w_j = p[e_j] of the softmax p over all E logits, so
 *                    grad_logits[e] = p[e] (g(e) - sum_j w_j g_j), where
 *                    g(e) = g_j if e = e_j, else 0.
 */
int oracle_route_backward(const float *logits, const int32_t *topk_ids, int64_t T, int32_t E,
                          int32_t k, int32_t norm_topk_prob, const double *grad_topk_w,
                          double *grad_logits)
{
    if (T < 0 || E < 1 || k < 1 || k > E)
        return ORACLE_EINVAL;
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    if (!p)
        return ORACLE_ENOMEM;
    int fail = 0;
    for (int64_t t = 0; t < T && !fail; ++t) {
        const float *x = logits + t * E;
        const int32_t *ids = topk_ids + t * k;
        const double *g = grad_topk_w + t * k;
        double *out = grad_logits + t * E;
        for (int32_t j = 0; j < k; ++j)
            if (ids[j] < 0 || ids[j] >= E)
                fail = 1;
        if (fail)
            break;
        /* p[e]: the probability the forward assigns (selected experts only
         * under norm_topk_prob). */
        double m = -INFINITY, s = 0.0;
        if (norm_topk_prob) {
            for (int32_t j = 0; j < k; ++j)
                m = fmax(m, (double)x[ids[j]]);
            for (int32_t j = 0; j < k; ++j)
                s += exp((double)x[ids[j]] - m);
        } else {
            for (int32_t e = 0; e < E; ++e)
                m = fmax(m, (double)x[e]);
            for (int32_t e = 0; e < E; ++e)
                s += exp((double)x[e] - m);
        }
        for (int32_t e = 0; e < E; ++e)
            p[e] = exp((double)x[e] - m) / s;
        double dot = 0.0;
        for (int32_t j = 0; j < k; ++j)
            dot += p[ids[j]] * g[j];
        for (int32_t e = 0; e < E; ++e)
            out[e] = norm_topk_prob ? 0.0 : -p[e] * dot;
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = ids[j];
            if (norm_topk_prob)
                out[e] = p[e] * (g[j] - dot);
            else
                out[e] += p[e] * g[j];
        }
    }
    free(p);
    return fail ? ORACLE_EINVAL : ORACLE_OK;
}

/*
 * Backward of oracle_expert_ffn (same inputs), by the chain rule; the pages
 * print only the forward.  grad_out [T, H] is the gradient of the layer
 * output (dt as the other inputs).  For a token t and a slot j with a valid
 * expert e and weight w, with w1 = rows [0, I) of w13[e], w3 = rows [I, 2I),
 * gate = x . w1^T, up = x . w3^T, s = sigmoid(gate), act = gate s up and
 * y = act . w2[e]^T:
 *   grad_topk_w[t, j] = <grad_out[t], y>
 *   d_act  = w (grad_out[t] . w2[e])                       (I values)
 *   d_gate = d_act up s (1 + gate (1 - s)),   d_up = d_act gate s
 *   grad_hidden[t] = sum over j of d_gate . w1 + d_up . w3
 *   grad_w2[e]  += w grad_out[t]^T act                     ([H, I])
 *   grad_w13[e] += [d_gate ; d_up]^T x                     ([2I, H])
 * Invalid slots give grad_topk_w 0 and add nothing; experts no slot names get
 * zero weight gradients.
 *
 * tokens[0..ntok) lists the rows whose grad_hidden [ntok, H] and grad_topk_w
 * [ntok, k] are wanted (NULL = all T in order).  grad_w13 [E, 2I, H] and
 * grad_w2 [E, H, I] may be NULL; when given, tokens must be NULL and the
 * tokens run one after another in ascending order (so every sum has a fixed
 * order); otherwise tokens are spread over nthreads.  All outputs double.
 */
int oracle_expert_ffn_backward(int32_t dt, const void *hidden, const void *w13, const void *w2,
                               const double *topk_w, const int32_t *topk_ids,
                               const void *grad_out, int64_t T, int32_t H, int32_t I, int32_t E,
                               int32_t k, const int64_t *tokens, int64_t ntok,
                               double *grad_hidden, double *grad_topk_w, double *grad_w13,
                               double *grad_w2, int32_t nthreads)
{
    if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1 || (dt != 0 && dt != 1))
        return ORACLE_EINVAL;
    const int weights = grad_w13 != NULL || grad_w2 != NULL;
    if (weights && (tokens || !grad_w13 || !grad_w2))
        return ORACLE_EINVAL;
    if (!tokens)
        ntok = T;
    if (weights) {
        for (int64_t q = 0; q < (int64_t)E * 2 * I * H; ++q)
            grad_w13[q] = 0.0;
        for (int64_t q = 0; q < (int64_t)E * H * I; ++q)
            grad_w2[q] = 0.0;
    }
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(weights ? 1 : (nthreads > 0 ? nthreads : 1))
    for (int64_t r = 0; r < ntok; ++r) {
        int64_t t = tokens ? tokens[r] : r;
        double *x = (double *)malloc(sizeof(double) * (size_t)H);
        double *dy = (double *)malloc(sizeof(double) * (size_t)H);
        double *v = (double *)malloc(sizeof(double) * (size_t)I * 5);
        if (!x || !dy || !v || t < 0 || t >= T) {
            free(x);
            free(dy);
            free(v);
#pragma omp atomic write
            fail = 1;
            continue;
        }
        double *gate = v, *up = v + I, *act = v + 2 * I, *dgate = v + 3 * I, *dup = v + 4 * I;
        for (int32_t h = 0; h < H; ++h) {
            x[h] = load_elem(dt, hidden, t * H + h);
            dy[h] = load_elem(dt, grad_out, t * H + h);
            grad_hidden[r * H + h] = 0.0;
        }
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = topk_ids[t * k + j];
            grad_topk_w[r * k + j] = 0.0;
            if (e < 0 || e >= E)
                continue;
            double w = topk_w[t * k + j];
            int64_t base13 = (int64_t)e * 2 * I * H;
            int64_t base2 = (int64_t)e * H * I;
            for (int32_t i = 0; i < I; ++i) {
                double g = 0.0, u = 0.0;
                for (int32_t h = 0; h < H; ++h) {
                    g += x[h] * load_elem(dt, w13, base13 + (int64_t)i * H + h);
                    u += x[h] * load_elem(dt, w13, base13 + (int64_t)(I + i) * H + h);
                }
                gate[i] = g;
                up[i] = u;
                act[i] = silu(g) * u;
            }
            /* grad_topk_w = <grad_out, y> with y = act . w2^T */
            double dw = 0.0;
            for (int32_t h = 0; h < H; ++h) {
                double y = 0.0;
                for (int32_t i = 0; i < I; ++i)
                    y += act[i] * load_elem(dt, w2, base2 + (int64_t)h * I + i);
                dw += dy[h] * y;
            }
            grad_topk_w[r * k + j] = dw;
            for (int32_t i = 0; i < I; ++i) {
                double da = 0.0;
                for (int32_t h = 0; h < H; ++h)
                    da += dy[h] * load_elem(dt, w2, base2 + (int64_t)h * I + i);
                da *= w;
                double s = 1.0 / (1.0 + exp(-gate[i]));
                dgate[i] = da * up[i] * s * (1.0 + gate[i] * (1.0 - s));
                dup[i] = da * gate[i] * s;
            }
            for (int32_t h = 0; h < H; ++h) {
                double acc = 0.0;
                for (int32_t i = 0; i < I; ++i)
                    acc += dgate[i] * load_elem(dt, w13, base13 + (int64_t)i * H + h) +
                           dup[i] * load_elem(dt, w13, base13 + (int64_t)(I + i) * H + h);
                grad_hidden[r * H + h] += acc;
            }
            if (weights) {
                for (int32_t h = 0; h < H; ++h)
                    for (int32_t i = 0; i < I; ++i)
                        grad_w2[base2 + (int64_t)h * I + i] += w * dy[h] * act[i];
                for (int32_t i = 0; i < I; ++i)
                    for (int32_t h = 0; h < H; ++h) {
                        grad_w13[base13 + (int64_t)i * H + h] += dgate[i] * x[h];
                        grad_w13[base13 + (int64_t)(I + i) * H + h] += dup[i] * x[h];
                    }
            }
        }
        free(x);
        free(dy);
        free(v);
    }
    return fail ? ORACLE_EINVAL : ORACLE_OK;
}

/*
 * Single rows and columns of the weight gradients of
 * oracle_expert_ffn_backward, each from its definition, for checks at sizes
 * where the whole gradient is too slow on a CPU.  Row c of grad_w13[e] sums
 * d_c x[t] over the slots of e (d_c = d_gate or d_up of unit c mod I), and
 * column i of grad_w2[e] sums w act_i grad_out[t] over them; each needs only
 * gate and up of one unit per slot.  Slots are visited in ascending (t, j).
 * row13 [n13, H] gets row c13[q] of grad_w13[e13[q]]; col2 [n2, H] gets
 * column i2[q] of grad_w2[e2[q]].
 */
int oracle_expert_wgrad_entries(int32_t dt, const void *hidden, const void *w13, const void *w2,
                                const double *topk_w, const int32_t *topk_ids,
                                const void *grad_out, int64_t T, int32_t H, int32_t I,
                                int32_t E, int32_t k, int64_t n13, const int32_t *e13,
                                const int32_t *c13, double *row13, int64_t n2,
                                const int32_t *e2, const int32_t *i2, double *col2,
                                int32_t nthreads)
{
    if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1 || (dt != 0 && dt != 1))
        return ORACLE_EINVAL;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t q = 0; q < n13 + n2; ++q) {
        const int is13 = q < n13;
        const int32_t e = is13 ? e13[q] : e2[q - n13];
        const int32_t c = is13 ? c13[q] : i2[q - n13];
        double *out = is13 ? row13 + q * H : col2 + (q - n13) * H;
        if (e < 0 || e >= E || c < 0 || c >= (is13 ? 2 * I : I)) {
#pragma omp atomic write
            fail = 1;
            continue;
        }
        const int32_t i = is13 ? c % I : c;
        const int64_t base13 = (int64_t)e * 2 * I * H;
        const int64_t base2 = (int64_t)e * H * I;
        for (int32_t h = 0; h < H; ++h)
            out[h] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            for (int32_t j = 0; j < k; ++j) {
                if (topk_ids[t * k + j] != e)
                    continue;
                double w = topk_w[t * k + j];
                double g = 0.0, u = 0.0, da = 0.0;
                for (int32_t h = 0; h < H; ++h) {
                    double xh = load_elem(dt, hidden, t * H + h);
                    g += xh * load_elem(dt, w13, base13 + (int64_t)i * H + h);
                    u += xh * load_elem(dt, w13, base13 + (int64_t)(I + i) * H + h);
                    da += load_elem(dt, grad_out, t * H + h) *
                          load_elem(dt, w2, base2 + (int64_t)h * I + i);
                }
                da *= w;
                double s = 1.0 / (1.0 + exp(-g));
                if (is13) {
                    double d = c < I ? da * u * s * (1.0 + g * (1.0 - s)) : da * g * s;
                    for (int32_t h = 0; h < H; ++h)
                        out[h] += d * load_elem(dt, hidden, t * H + h);
                } else {
                    double a = silu(g) * u;
                    for (int32_t h = 0; h < H; ++h)
                        out[h] += w * load_elem(dt, grad_out, t * H + h) * a;
                }
            }
        }
    }
    return fail ? ORACLE_EINVAL : ORACLE_OK;
}

/*
 * Backward of the weights of oracle_route_grouped, by the chain rule (the
 * pages give only the forward).  The weights are the selected experts'
 * scores (the correction bias moves only the selection, which is piecewise
 * constant and passes no gradient), divided by their sum S when
 * renormalize != 0.  With g = grad_topk_w:
 *   plain:        grad_scores[e_j] = g_j
 *   renormalized: grad_scores[e_j] = (g_j - sum_i w_i g_i) / S
 * and 0 for every unselected expert.  topk_ids are the forward's (valid and
 * distinct within a row).
 */
int oracle_route_grouped_backward(const float *scores, const int32_t *topk_ids, int64_t T,
                                  int32_t E, int32_t k, int32_t renormalize,
                                  const double *grad_topk_w, double *grad_scores)
{
    if (T < 0 || E < 1 || k < 1 || k > E)
        return ORACLE_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        const int32_t *ids = topk_ids + t * k;
        const double *g = grad_topk_w + t * k;
        double *out = grad_scores + t * E;
        for (int32_t e = 0; e < E; ++e)
            out[e] = 0.0;
        double S = 0.0, dot = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            if (ids[j] < 0 || ids[j] >= E)
                return ORACLE_EINVAL;
            S += (double)scores[t * E + ids[j]];
        }
        for (int32_t j = 0; j < k; ++j)
            dot += (double)scores[t * E + ids[j]] / S * g[j];
        for (int32_t j = 0; j < k; ++j)
            out[ids[j]] = renormalize ? (g[j] - dot) / S : g[j];
    }
    return ORACLE_OK;
}

/*
 * Backward of oracle_router_logits (logits = hidden . w_gate^T), by the chain
 * rule: with g = grad_logits [T, E],
 *   grad_hidden[t][h] = sum over e of g[t][e] w_gate[e][h]
 *   grad_w_gate[e][h] = sum over t of g[t][e] hidden[t][h]
 * in double, sums in ascending e and t.  dt as in oracle_router_logits.
 */
int oracle_router_backward(int32_t dt, const void *hidden, const void *w_gate,
                           const double *grad_logits, int64_t T, int32_t H, int32_t E,
                           double *grad_hidden, double *grad_w_gate)
{
    if (T < 0 || H < 1 || E < 1 || (dt != 0 && dt != 1))
        return ORACLE_EINVAL;
    for (int64_t t = 0; t < T; ++t)
        for (int32_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int32_t e = 0; e < E; ++e)
                acc += grad_logits[t * E + e] * load_elem(dt, w_gate, (int64_t)e * H + h);
            grad_hidden[t * H + h] = acc;
        }
    for (int32_t e = 0; e < E; ++e)
        for (int32_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; ++t)
                acc += grad_logits[t * E + e] * load_elem(dt, hidden, t * H + h);
            grad_w_gate[(int64_t)e * H + h] = acc;
        }
    return ORACLE_OK;
}
