/*
 * CPU oracle for the sparse MoE layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the bench's CPU-baseline leg may load
 * this library. It shares no code, header or table with the HIP library; it
 * sees the same inputs because both sides draw them from the seeded
 * generator module.
 *
 * It computes the layer exactly as the pages define it, in float64, one
 * token at a time, with plain loops (no blocking, no fusion, no reordering):
 *
 *   [MoE]     mini-sglang guide, chapter 7 (models, MoE backend, kernel
 *             infrastructure): paragraph on the MoE routing layer (router
 *             linear -> per-expert logits; top-k experts chosen as
 *             torch.topk does; expert outputs weighted by softmax scores and
 *             summed) and paragraph on the fused backend (tokens grouped by
 *             their assigned expert).
 *   [Linear]  handbook page "The op layer: BaseOP and the layers", section
 *             "Linear layers" (a linear layer is F.linear: y = x W^T + b; the
 *             MoE router is the replicated, unsharded one).
 *   [Norm]    handbook page "The op layer: BaseOP and the layers": section
 *             "Ops: reference implementations and dispatch" (rmsnorm computes
 *             in fp32, casts the normalized value back to the input dtype,
 *             then multiplies by the weight; fused_add_rmsnorm adds x into
 *             the residual in place, then normalizes the residual into x) and
 *             section "RMSNorm and the residual" (the fused op returns the
 *             normalized result and the new residual; without a residual, x
 *             is the residual).
 *   [Models]  handbook page "Models and weight loading" (模型与权重加载):
 *             section "ModelConfig" (num_experts, num_experts_per_tok,
 *             moe_intermediate_size, norm_topk_prob), section "Model
 *             structure" (GatedMLP: merged gate_up projection, silu(gate) * up,
 *             down projection, only the silu activation) and section
 *             "Streaming weight loading" (per-expert tensors stacked into one
 *             [E, ...] tensor; gate and up merged in that order).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 * softmax over all E experts, then top-k, then optional renormalisation;
 * ties in the top-k go to the lower expert index and the k slots come out in
 * descending order; silu(z) = z / (1 + exp(-z)); gate rows 0..I-1 and up rows
 * I..2I-1 of the merged weight; within an expert's group tokens appear in
 * ascending flat index t*k+j, each group padded to a multiple of block_m with
 * the sentinel T*k; no residual is added inside the layer.
 *
 * bf16 inputs arrive as raw bit patterns and are widened exactly to float64.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads an OpenMP parallel region of this library will use. */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the later parallel regions use (n >= 1): a thread-count control
 * for timing the oracle, no arithmetic. */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Router linear [MoE], [Linear]: logits[t,e] = sum_h x[t,h] * wr[e,h] + bias[e].
 * x: [T,H] bf16, wr: [E,H] bf16, bias: [E] float or NULL, logits: [T,E]. */
void oracle_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias, int64_t T, int64_t H,
                          int64_t E, double* logits) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            double s = 0.0;
            for (int64_t h = 0; h < H; ++h) s += bf16_value(x[t * H + h]) * bf16_value(wr[e * H + h]);
            if (bias) s += (double)bias[e];
            logits[t * E + e] = s;
        }
    }
}

/* Does expert a come before expert b in torch.topk order (larger value first,
 * equal values -> lower index first)? */
static int ranks_before(const double* row, int32_t a, int32_t b) {
    if (row[a] != row[b]) return row[a] > row[b];
    return a < b;
}

/* Softmax scores, top-k and optional renormalisation [MoE], [Models]:
 * p = softmax(logits[t, :]) over all E experts; ids[t, j] = the j-th ranked
 * expert (full stable sort of the E logits, which orders the softmax scores
 * identically because softmax is increasing in each logit); w[t, j] =
 * p[ids[t, j]], divided by the sum of the k selected scores when
 * norm_topk_prob is set. */
void oracle_select_topk(const double* logits, int64_t T, int64_t E, int64_t k, int norm_topk_prob,
                        int32_t* ids, double* weights) {
#pragma omp parallel
    {
        int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
        double* p = (double*)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const double* row = logits + t * E;
            /* insertion sort of expert indices by rank */
            for (int64_t e = 0; e < E; ++e) {
                int64_t pos = e;
                while (pos > 0 && ranks_before(row, (int32_t)e, order[pos - 1])) {
                    order[pos] = order[pos - 1];
                    --pos;
                }
                order[pos] = (int32_t)e;
            }
            double mx = row[0];
            for (int64_t e = 1; e < E; ++e)
                if (row[e] > mx) mx = row[e];
            double z = 0.0;
            for (int64_t e = 0; e < E; ++e) {
                p[e] = exp(row[e] - mx);
                z += p[e];
            }
            for (int64_t e = 0; e < E; ++e) p[e] /= z;
            double sel = 0.0;
            for (int64_t j = 0; j < k; ++j) sel += p[order[j]];
            for (int64_t j = 0; j < k; ++j) {
                ids[t * k + j] = order[j];
                weights[t * k + j] = norm_topk_prob ? p[order[j]] / sel : p[order[j]];
            }
        }
        free(order);
        free(p);
    }
}

/* Group tokens by assigned expert [MoE], fused-backend paragraph.
 * Flat index i = t*k + j names slot j of token t. counts[e] = number of i
 * with ids[i] == e. Expert e owns rows [off_e, off_e + pad_e) of sorted_ids,
 * pad_e = ceil(counts[e] / block_m) * block_m, off_e = sum of pad_e' for
 * e' < e; its first counts[e] rows hold its flat indices in ascending order
 * and the rest hold the sentinel T*k. Rows from num_padded = off_E up to cap
 * also hold the sentinel. block_expert[b] = owner of rows
 * [b*block_m, (b+1)*block_m), or -1 beyond num_padded. Returns num_padded,
 * or -1 if cap is too small. */
int64_t oracle_align(const int32_t* ids, int64_t T, int64_t k, int64_t E, int64_t block_m, int64_t cap,
                     int32_t* sorted_ids, int32_t* block_expert, int32_t* counts) {
    const int64_t n = T * k;
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t i = 0; i < n; ++i) counts[ids[i]] += 1;
    int64_t total = 0;
    for (int64_t e = 0; e < E; ++e) total += (counts[e] + block_m - 1) / block_m * block_m;
    if (total > cap) return -1;
    for (int64_t r = 0; r < cap; ++r) sorted_ids[r] = (int32_t)n;
    for (int64_t b = 0; b < cap / block_m; ++b) block_expert[b] = -1;
    int64_t off = 0;
    for (int64_t e = 0; e < E; ++e) {
        int64_t fill = off;
        for (int64_t i = 0; i < n; ++i)
            if (ids[i] == e) sorted_ids[fill++] = (int32_t)i;
        int64_t padded = (counts[e] + block_m - 1) / block_m * block_m;
        for (int64_t b = off / block_m; b < (off + padded) / block_m; ++b) block_expert[b] = (int32_t)e;
        off += padded;
    }
    return off;
}

/* First half of one expert's gated MLP [Models], section "Model structure"
 * (gate_up_proj, then silu(gate) * up):
 * g_i = sum_h x_h * w13[i, h], u_i = sum_h x_h * w13[I + i, h],
 * act_i = silu(g_i) * u_i with silu(z) = z / (1 + exp(-z)).
 * x: [H] float64, w13: [2I, H] bf16, act: [I]. */
void oracle_expert_gate_up(const double* x, const uint16_t* w13, int64_t H, int64_t I, double* act) {
    for (int64_t i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            g += x[h] * bf16_value(w13[i * H + h]);
            u += x[h] * bf16_value(w13[(I + i) * H + h]);
        }
        act[i] = g / (1.0 + exp(-g)) * u;
    }
}

/* Second half [Models], "Model structure" (down_proj):
 * y_h = sum_i act_i * w2[h, i]. act: [I] float64, w2: [H, I] bf16, y: [H]. */
void oracle_expert_down(const double* act, const uint16_t* w2, int64_t H, int64_t I, double* y) {
    for (int64_t h = 0; h < H; ++h) {
        double s = 0.0;
        for (int64_t i = 0; i < I; ++i) s += act[i] * bf16_value(w2[h * I + i]);
        y[h] = s;
    }
}

/* One expert's whole gated MLP: gate_up then down. act: [I] scratch. */
void oracle_expert_mlp(const double* x, const uint16_t* w13, const uint16_t* w2, int64_t H, int64_t I,
                       double* act, double* y) {
    oracle_expert_gate_up(x, w13, H, I, act);
    oracle_expert_down(act, w2, H, I, y);
}

/* Weighted sum of one token's k expert outputs [MoE] ("weighted by softmax
 * scores and summed"): out_h = sum_j w_j * y[j, h]. y: [k, H], w: [k]. */
void oracle_combine(const double* y, const double* w, int64_t k, int64_t H, double* out) {
    for (int64_t h = 0; h < H; ++h) out[h] = 0.0;
    for (int64_t j = 0; j < k; ++j)
        for (int64_t h = 0; h < H; ++h) out[h] += w[j] * y[j * H + h];
}

/* The whole layer for the listed tokens, one token at a time [MoE]:
 * logits -> softmax / top-k (/ renorm) -> for each of the k selected experts
 * its gated MLP -> out[t] = sum_j w[t, j] * y_j. No residual.
 * x: [T,H], wr: [E,H], w13: [E,2I,H], w2: [E,H,I] (bf16); bias [E] or NULL.
 * tokens: n_tokens indices into [0, T) (NULL = all T tokens in order).
 * out: [n_tokens, H]; ids_out: [n_tokens, k] and w_out: [n_tokens, k] may be
 * NULL. */
void oracle_moe_layer(const uint16_t* x, const uint16_t* wr, const float* bias, const uint16_t* w13,
                      const uint16_t* w2, int64_t T, int64_t H, int64_t E, int64_t k, int64_t I,
                      int norm_topk_prob, const int64_t* tokens, int64_t n_tokens, double* out,
                      int32_t* ids_out, double* w_out) {
    (void)T;
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* logits = (double*)malloc(sizeof(double) * (size_t)E);
        double* act = (double*)malloc(sizeof(double) * (size_t)I);
        double* y = (double*)malloc(sizeof(double) * (size_t)(k * H));
        int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
        double* w = (double*)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_tokens; ++n) {
            int64_t t = tokens ? tokens[n] : n;
            for (int64_t h = 0; h < H; ++h) xr[h] = bf16_value(x[t * H + h]);
            oracle_router_logits(x + t * H, wr, bias, 1, H, E, logits);
            oracle_select_topk(logits, 1, E, k, norm_topk_prob, ids, w);
            for (int64_t j = 0; j < k; ++j) {
                int64_t e = ids[j];
                oracle_expert_mlp(xr, w13 + e * 2 * I * H, w2 + e * H * I, H, I, act, y + j * H);
            }
            oracle_combine(y, w, k, H, out + n * H);
            if (ids_out)
                for (int64_t j = 0; j < k; ++j) ids_out[n * k + j] = ids[j];
            if (w_out)
                for (int64_t j = 0; j < k; ++j) w_out[n * k + j] = w[j];
        }
        free(xr);
        free(logits);
        free(act);
        free(y);
        free(ids);
        free(w);
    }
}

/* Round a finite double to the nearest bf16 value, ties to even (used where
 * [Norm] casts to the bf16 model dtype). */
static double round_bf16(double v) {
    if (v == 0.0) return v;
    int e;
    double m = frexp(v, &e); /* v = m * 2^e, 0.5 <= |m| < 1 */
    return ldexp(rint(m * 256.0), e - 8);
}

static uint16_t bf16_bits_of(double v) { /* v already representable in bf16 */
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* Fused residual add + RMSNorm [Norm], in place on [T, H] bf16 rows:
 * with a residual, residual <- bf16(fp32(residual) + fp32(x)) (the add of two
 * bf16 tensors); without one (first layer), residual <- x. Then, per row,
 * ms = mean(r^2), n = bf16(r / sqrt(ms + eps)), x <- bf16(w * n) (the
 * product of two bf16 values, exact in fp32, rounded once). The mean and the
 * square root are taken in float64. */
void oracle_fused_add_rmsnorm(uint16_t* x, uint16_t* residual, const uint16_t* weight, int64_t T, int64_t H,
                              double eps, int has_residual) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        uint16_t* xr = x + t * H;
        uint16_t* rr = residual + t * H;
        double ss = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            double r;
            if (has_residual) {
                float sum = (float)bf16_value(rr[h]) + (float)bf16_value(xr[h]);
                r = round_bf16((double)sum);
            } else {
                r = bf16_value(xr[h]);
            }
            rr[h] = bf16_bits_of(r);
            ss += r * r;
        }
        const double inv = 1.0 / sqrt(ss / (double)H + eps);
        for (int64_t h = 0; h < H; ++h) {
            const double n = round_bf16(bf16_value(rr[h]) * inv);
            xr[h] = bf16_bits_of(round_bf16((double)(float)(bf16_value(weight[h]) * n)));
        }
    }
}
