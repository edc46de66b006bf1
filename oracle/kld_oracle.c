/*
 * kld_oracle.c -- plain float64 CPU reference for the quantized-vs-BF16 logit
 * comparison (per-token KL divergence and top-1 agreement).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header, table or
 * helper with the HIP path under quantization_quality_eval_amd/.
 *
 * What it computes, row by row, and the passages it follows:
 *   - "Qwen3.6 27B Quantization Benchmark" (huy.rocks), section "Understand KLD
 *     and Same Top P": KLD measures how far the quantized model's next-token
 *     confidence distribution drifts from the base model's; "Same Top P" is
 *     whether both models put their top score on the same token.
 *   - "Mistral-Small-4-119B-2603 GSQ-RCO IQ3_S GGUF" model card, "How it was
 *     made" step 5 and the "Quality" section: the divergence is
 *     KL(BF16 || quantized) over the full vocabulary, i.e. the base
 *     distribution is P and the quantized one is Q.
 *   - "Unsloth Dynamic 3.0 GGUFs", "The Divergence-300 @32 Metric": top-1
 *     agreement is an argmax on one prediction.
 *
 * Definition used (natural log, temperature 1, every input row counted):
 *   p = softmax(z_base), q = softmax(z_quant)
 *   KL = sum_i p_i * (log p_i - log q_i)
 *   log p_i = z_base[i] - lse_base,  log q_i = z_quant[i] - lse_quant
 *   lse = m + log(sum_i exp(z[i] - m)),  m = max_i z[i]
 *   argmax = the smallest index attaining the maximum (pages silent; lowest
 *            index is the stated reading), match = (argmax_base == argmax_quant)
 * This is the textbook, uncentred formula evaluated in float64 with plain
 * left-to-right sums; no blocking, no online rescaling, no reordering.
 *
 * Inputs: row-major [n_rows, vocab] arrays of float32, bfloat16 (raw 16-bit
 * patterns, widened exactly by placing them in the high half of a float32) or
 * float64. Finite values are a precondition.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KLDO_F32 0
#define KLDO_BF16 1
#define KLDO_F64 2

/* Exact widening of element i of a row to double. */
static double kldo_load(const void* row, int dtype, int64_t i) {
    if (dtype == KLDO_F64) return ((const double*)row)[i];
    if (dtype == KLDO_F32) return (double)((const float*)row)[i];
    uint32_t bits = ((uint32_t)((const uint16_t*)row)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static size_t kldo_elem_size(int dtype) {
    return dtype == KLDO_F64 ? 8 : (dtype == KLDO_F32 ? 4 : 2);
}

/* Max and first index attaining it. */
static void kldo_max_first(const double* z, int64_t V, double* m, int64_t* idx) {
    double best = z[0];
    int64_t at = 0;
    for (int64_t i = 1; i < V; ++i) {
        if (z[i] > best) { best = z[i]; at = i; }
    }
    *m = best;
    *idx = at;
}

/* log of the softmax normaliser: m + log(sum exp(z - m)). */
static double kldo_lse(const double* z, int64_t V, double m) {
    double s = 0.0;
    for (int64_t i = 0; i < V; ++i) s += exp(z[i] - m);
    return m + log(s);
}

/* The per-row definition: KL(P_base || Q_quant), both argmaxes, both lse. */
static void kldo_row_f64(const double* zb, const double* zq, int64_t V,
                         double* kl, int64_t* ib, int64_t* iq,
                         double* lse_b, double* lse_q) {
    double mb, mq;
    kldo_max_first(zb, V, &mb, ib);
    kldo_max_first(zq, V, &mq, iq);
    const double lb = kldo_lse(zb, V, mb);
    const double lq = kldo_lse(zq, V, mq);
    double acc = 0.0;
    for (int64_t i = 0; i < V; ++i) {
        const double log_p = zb[i] - lb;
        const double log_q = zq[i] - lq;
        acc += exp(log_p) * (log_p - log_q);
    }
    *kl = acc;
    *lse_b = lb;
    *lse_q = lq;
}

/*
 * Evaluate n_rows rows. Any output pointer may be NULL. n_threads <= 0 uses
 * the OpenMP default. Returns 0 on success, -1 on bad arguments, -2 when a
 * scratch allocation fails.
 */
int kldo_rows(const void* base, int base_dtype, const void* quant, int quant_dtype,
              int64_t n_rows, int64_t vocab,
              double* kl_out, int64_t* argmax_base_out, int64_t* argmax_quant_out,
              uint8_t* match_out, double* lse_base_out, double* lse_quant_out,
              int n_threads) {
    if (!base || !quant || n_rows < 0 || vocab < 1) return -1;
    if (base_dtype < 0 || base_dtype > 2 || quant_dtype < 0 || quant_dtype > 2) return -1;
    const size_t sb = kldo_elem_size(base_dtype), sq = kldo_elem_size(quant_dtype);
    int status = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel
    {
        double* zb = (double*)malloc((size_t)vocab * sizeof(double));
        double* zq = (double*)malloc((size_t)vocab * sizeof(double));
        if (!zb || !zq) {
#pragma omp atomic write
            status = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!zb || !zq) continue;
            const char* rb = (const char*)base + (size_t)r * (size_t)vocab * sb;
            const char* rq = (const char*)quant + (size_t)r * (size_t)vocab * sq;
            for (int64_t i = 0; i < vocab; ++i) {
                zb[i] = kldo_load(rb, base_dtype, i);
                zq[i] = kldo_load(rq, quant_dtype, i);
            }
            double kl, lb, lq;
            int64_t ib, iq;
            kldo_row_f64(zb, zq, vocab, &kl, &ib, &iq, &lb, &lq);
            if (kl_out) kl_out[r] = kl;
            if (argmax_base_out) argmax_base_out[r] = ib;
            if (argmax_quant_out) argmax_quant_out[r] = iq;
            if (match_out) match_out[r] = (uint8_t)(ib == iq);
            if (lse_base_out) lse_base_out[r] = lb;
            if (lse_quant_out) lse_quant_out[r] = lq;
        }
        free(zb);
        free(zq);
    }
    return status;
}

/* Number of threads an OpenMP parallel region would use (for reporting). */
int kldo_max_threads(int n_threads) {
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
    return omp_get_max_threads();
#else
    (void)n_threads;
    return 1;
#endif
}
