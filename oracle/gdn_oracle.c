/*
 * gdn_oracle.c -- fp64 CPU oracle for the Gated DeltaNet token mixer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark do. It shares no source,
 * header, table or helper with the HIP library.
 *
 * What it computes. The pages name the layer ("Gated DeltaNet", in the
 * layout 16 x (3 x (Gated DeltaNet -> FFN) -> 1 x (Gated Attention -> FFN))
 * of "The Hybrid Attention in Qwen3.8-27B", section "Why 27B parameters can
 * carry 262K tokens") and say that each such layer keeps one fixed-size
 * state whatever the sequence length (same section; and "The economics of
 * hybrid attention", TL;DR). They do not print the recurrence. The oracle
 * takes the published gated delta rule (Yang, Kautz & Hatamizadeh, "Gated
 * Delta Networks", ICLR 2025) as its plainest reading:
 *
 *     S_t = a_t * S_{t-1} * (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *     o_t = scale * S_t q_t                      (the state after the write)
 *
 * with S in R^{dv x dk}. Multiplying out the first line gives the form the
 * token loop below evaluates, three O(dv*dk) passes per token:
 *
 *     w   = S_{t-1} k_t
 *     u   = b_t (v_t - a_t w)
 *     S_t = a_t S_{t-1} + u k_t^T
 *
 * All arithmetic is fp64. bf16 inputs are widened exactly (a bf16 value is
 * the upper half of an IEEE binary32). No chunking, blocking or reordering
 * beyond the definition: one token after the other, in order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2

/* bf16 bit pattern -> fp64, exact: the 16 bits are the high half of a
 * binary32 with the low mantissa bits zero. */
static double oracle_bf16_to_f64(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static void oracle_load_vec(const void *base, int dtype, int64_t offset, int n,
                            double *dst) {
    if (dtype == ORACLE_BF16) {
        const uint16_t *p = (const uint16_t *)base + offset;
        for (int i = 0; i < n; ++i) dst[i] = oracle_bf16_to_f64(p[i]);
    } else if (dtype == ORACLE_F64) {
        const double *p = (const double *)base + offset;
        for (int i = 0; i < n; ++i) dst[i] = p[i];
    } else {
        const float *p = (const float *)base + offset;
        for (int i = 0; i < n; ++i) dst[i] = (double)p[i];
    }
}

/*
 * One (sequence, value head) chain over T tokens.
 *
 *   q, k      : q/k head of this chain at token 0 (dtype elements)
 *   v         : value head of this chain at token 0 (dtype elements)
 *   dtype     : 0 fp32, 1 bf16 bit patterns, 2 fp64
 *   alpha,beta: this value head at token 0 (ab_dtype elements: 0 fp32, 2 fp64)
 *   T         : number of tokens (>= 0)
 *   stride_qk : elements between consecutive tokens of q and k
 *   stride_v  : elements between consecutive tokens of v
 *   stride_ab : elements between consecutive tokens of alpha and beta
 *   dk, dv    : key and value head dimensions (1..256)
 *   scale     : multiplies every output
 *   S         : dv*dk fp64 row-major (S[i*dk + j], i over dv); the initial
 *               state on entry, the final state on return
 *   o         : T*dv fp64 row-major output, or NULL to skip outputs
 *
 * Returns 0, or -1 for arguments it cannot take.
 */
int gdn_oracle_chain(const void *q, const void *k, const void *v, int dtype,
                     const void *alpha, const void *beta, int ab_dtype, int64_t T,
                     int64_t stride_qk, int64_t stride_v, int64_t stride_ab,
                     int dk, int dv, double scale, double *S, double *o) {
    if (dk < 1 || dk > 256 || dv < 1 || dv > 256 || T < 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return -1;
    if (ab_dtype != ORACLE_F32 && ab_dtype != ORACLE_F64) return -1;
    double qt[256], kt[256], vt[256], u[256];

    for (int64_t t = 0; t < T; ++t) {
        double a, b;
        oracle_load_vec(alpha, ab_dtype, t * stride_ab, 1, &a);
        oracle_load_vec(beta, ab_dtype, t * stride_ab, 1, &b);
        oracle_load_vec(q, dtype, t * stride_qk, dk, qt);
        oracle_load_vec(k, dtype, t * stride_qk, dk, kt);
        oracle_load_vec(v, dtype, t * stride_v, dv, vt);

        /* w = S_{t-1} k_t, then u = b (v - a w) */
        for (int i = 0; i < dv; ++i) {
            double w = 0.0;
            for (int j = 0; j < dk; ++j) w += S[(int64_t)i * dk + j] * kt[j];
            u[i] = b * (vt[i] - a * w);
        }
        /* S_t = a S_{t-1} + u k^T */
        for (int i = 0; i < dv; ++i) {
            double *row = S + (int64_t)i * dk;
            for (int j = 0; j < dk; ++j) row[j] = a * row[j] + u[i] * kt[j];
        }
        /* o_t = scale * S_t q_t */
        if (o) {
            for (int i = 0; i < dv; ++i) {
                const double *row = S + (int64_t)i * dk;
                double acc = 0.0;
                for (int j = 0; j < dk; ++j) acc += row[j] * qt[j];
                o[t * dv + i] = scale * acc;
            }
        }
    }
    return 0;
}

int gdn_oracle_version(void) { return 2; }
