/*
 * CPU oracle for the multi-LoRA adapted linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct definition the
 * GPU library is checked against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load it; the library never does, and the two share no code (not even headers).
 *
 * Arithmetic: every bfloat16 input is decoded exactly and all sums run in fp64 (the pages'
 * worked examples are NumPy float64 scripts), in plain ascending loops, compiled with
 * -ffp-contract=off so no fused multiply-add changes the rounding.  Parity is checked against
 * this fp64 build.  Built with -DORACLE_ACC=float, the same loops accumulate in fp32 instead
 * (the plain fp32 CPU loop that serves as the timed CPU baseline; results still returned as
 * double); nothing else changes.
 *
 * What it computes, for token t with adapter slots idx[t][0..K-1] (-1 = none):
 *
 *   y[t][n] = sum_i W[n][i] x[t][i]
 *           + sum_{j : a = idx[t][j] != -1}  sum_rho B[a][n][rho] * u_j[sigma(n)][rho]
 *   u_j[sigma][rho] = c_tj * sum_i A[a][sigma][rho][i] x[t][i],   c_tj = s[t][j] * f(a)
 *   f(a) = alpha_a / r_a, or alpha_a / sqrt(r_a) for rsLoRA adapters
 *
 * Sources:
 *  - "Multi-LoRA Serving Explained" (sevydevy.com): the layer W x + B(A x) scaled by alpha/r,
 *    B is out-by-rank and A is rank-by-in; the six-token batching script (gather by slot id,
 *    -1 = base model only; stable argsort by slot, one group per adapter); the padding script
 *    (an adapter sits zero-padded in a max-rank slot).
 *  - "[RFC]: Per-request activation of multiple LoRA adapters with static scales" (vLLM
 *    issue 51940), Proposed Change: Semantics (base(x) + sum_i s_i (alpha_i/r_i) B_i A_i x) and
 *    staged implementation steps 2-3 (k slots per token, sentinel fill, one shrink/expand per
 *    slot accumulated into the output with the per-adapter scale).
 *  - vLLM learning book, chapter "04. LoRA Serving", section 6 (PunicaWrapper): shrink applies
 *    the scale and produces the rank-wide intermediate, expand adds it times B into y.
 *  - "[vLLM] LoRA" (blog.secrett2633.cloud), section on PEFTHelper: rsLoRA scale alpha/sqrt(r).
 *
 * Merged QKV layers (several output slices, each with its own A block) follow the learning
 * book's section 7 and the [vLLM] LoRA page's layer list: slice sigma owns output rows
 * [slice_start[sigma], slice_start[sigma+1]) and A[a][sigma] is that slice's down matrix.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_ACC
#define ORACLE_ACC double
#endif
typedef ORACLE_ACC acc_t;   /* type of every product and running sum */

static acc_t bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (acc_t)f;
}

/* Scale factor of one adapter: alpha/r, or alpha/sqrt(r) with rsLoRA ("[vLLM] LoRA",
 * PEFTHelper section).  r is the adapter's own rank, not the padded slot width. */
double oracle_lora_factor(double alpha, int32_t r, int32_t use_rslora)
{
    if (use_rslora)
        return alpha / sqrt((double)r);
    return alpha / (double)r;
}

/* Token mapping plan: the flat (token, position) pairs p = t*K + j are sorted by their slot
 * idx[p] in ascending order, ties kept in ascending p (a stable sort, as the six-token script's
 * argsort(kind="stable") does); pairs holding -1 are dropped.  Each maximal run of one slot is
 * a segment (slot, first position in perm, length).  Returns the number of segments and writes
 * the number of kept pairs to *n_pairs, or returns -1 if some index lies outside [-1, S).
 * The double loop is the definition of a stable sort by key written out. */
int32_t oracle_plan(const int32_t *idx, int64_t T, int32_t K, int32_t S, int32_t *perm,
                    int32_t *seg_slot, int32_t *seg_start, int32_t *seg_len, int64_t *n_pairs)
{
    const int64_t P = T * (int64_t)K;
    for (int64_t p = 0; p < P; ++p)
        if (idx[p] < -1 || idx[p] >= S)
            return -1;
    int64_t n = 0;
    int32_t g = 0;
    for (int32_t a = 0; a < S; ++a) {
        const int64_t first = n;
        for (int64_t p = 0; p < P; ++p)
            if (idx[p] == a)
                perm[n++] = (int32_t)p;
        if (n > first) {
            seg_slot[g] = a;
            seg_start[g] = (int32_t)first;
            seg_len[g] = (int32_t)(n - first);
            ++g;
        }
    }
    *n_pairs = n;
    return g;
}

/* Coefficient c_tj = s[t][j] * f(a) of one (token, position) pair.  scale may be NULL (s = 1). */
static double pair_coef(const float *scale, int64_t p, int32_t a, const double *alpha,
                        const int32_t *rank, const uint8_t *rslora)
{
    const double s = scale ? (double)scale[p] : 1.0;
    return s * oracle_lora_factor(alpha[a], rank[a], rslora[a]);
}

/* Shrink for one pair: u[sigma*R + rho] = c * sum_i A[a][sigma][rho][i] * x_t[i]. */
static void shrink_one(const uint16_t *xt, int64_t n_in, const uint16_t *A, int32_t a, int32_t R,
                       int32_t n_slices, acc_t c, acc_t *u)
{
    for (int32_t sg = 0; sg < n_slices; ++sg)
        for (int32_t rho = 0; rho < R; ++rho) {
            const uint16_t *arow = A + (((int64_t)a * n_slices + sg) * R + rho) * n_in;
            acc_t acc = 0;
            for (int64_t i = 0; i < n_in; ++i)
                acc += bf16_value(arow[i]) * bf16_value(xt[i]);
            u[sg * R + rho] = c * acc;
        }
}

static int32_t slice_of(int64_t n, int32_t n_slices, const int32_t *slice_start)
{
    int32_t sg = 0;
    while (sg + 1 < n_slices && n >= slice_start[sg + 1])
        ++sg;
    return sg;
}

/* Expand for one pair: yt[n] += sum_rho B[a][n][rho] * u[sigma(n)*R + rho]. */
static void expand_one(const acc_t *u, int64_t n_out, const uint16_t *B, int32_t a, int32_t R,
                       int32_t n_slices, const int32_t *slice_start, acc_t *yt)
{
    for (int64_t n = 0; n < n_out; ++n) {
        const int32_t sg = slice_of(n, n_slices, slice_start);
        const uint16_t *brow = B + ((int64_t)a * n_out + n) * R;
        acc_t d = 0;
        for (int32_t rho = 0; rho < R; ++rho)
            d += bf16_value(brow[rho]) * u[sg * R + rho];
        yt[n] += d;
    }
}

/* v[j][t][sigma*R + rho] for every pair; pairs holding -1 get zeros.  (Learning book section 6:
 * add_shrink produces the scaled rank-wide intermediate.)  v is [K][T][n_slices*R]. */
void oracle_shrink(const uint16_t *x, int64_t T, int64_t n_in, const uint16_t *A, int32_t S,
                   int32_t R, int32_t n_slices, const double *alpha, const int32_t *rank,
                   const uint8_t *rslora, const int32_t *idx, int32_t K, const float *scale,
                   double *v)
{
    (void)S;
    const int64_t w = (int64_t)n_slices * R;
#pragma omp parallel
    {
        acc_t *u = (acc_t *)malloc((size_t)w * sizeof(acc_t));
#pragma omp for schedule(dynamic)
        for (int64_t t = 0; t < T; ++t) {
            for (int32_t j = 0; j < K; ++j) {
                const int64_t p = t * K + j;
                double *vt = v + ((int64_t)j * T + t) * w;
                const int32_t a = idx[p];
                if (a == -1) {
                    for (int64_t q = 0; q < w; ++q)
                        vt[q] = 0.0;
                    continue;
                }
                shrink_one(x + t * n_in, n_in, A, a, R, n_slices,
                           (acc_t)pair_coef(scale, p, a, alpha, rank, rslora), u);
                for (int64_t q = 0; q < w; ++q)
                    vt[q] = (double)u[q];
            }
        }
        free(u);
    }
}

/* y[t][n] += sum_j [idx[t][j] != -1] sum_rho B[a][n][rho] v[j][t][sigma(n)*R + rho]
 * (learning book section 6: add_expand adds the intermediate times B into y). */
void oracle_expand(const double *v, int64_t T, int64_t n_out, const uint16_t *B, int32_t S,
                   int32_t R, int32_t n_slices, const int32_t *slice_start, const int32_t *idx,
                   int32_t K, double *y)
{
    (void)S;
    const int64_t w = (int64_t)n_slices * R;
#pragma omp parallel
    {
        acc_t *u = (acc_t *)malloc((size_t)w * sizeof(acc_t));
        acc_t *yt = (acc_t *)malloc((size_t)n_out * sizeof(acc_t));
#pragma omp for schedule(dynamic)
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t n = 0; n < n_out; ++n)
                yt[n] = (acc_t)y[t * n_out + n];
            for (int32_t j = 0; j < K; ++j) {
                const int32_t a = idx[t * K + j];
                if (a == -1)
                    continue;
                for (int64_t q = 0; q < w; ++q)
                    u[q] = (acc_t)v[((int64_t)j * T + t) * w + q];
                expand_one(u, n_out, B, a, R, n_slices, slice_start, yt);
            }
            for (int64_t n = 0; n < n_out; ++n)
                y[t * n_out + n] = (double)yt[n];
        }
        free(yt);
        free(u);
    }
}

/* The whole layer for the tokens listed in tokens[0..n_tokens) (all tokens when tokens is
 * NULL, then n_tokens must equal T).  Output row q is token tokens[q]:
 *   y[q][n] = (with_base ? sum_i W[n][i] x[t][i] : 0) + the K slots' deltas, slot by slot,
 * as the RFC's stage-3 reference execution accumulates them. */
void oracle_linear(const uint16_t *x, const uint16_t *W, int64_t T, int64_t n_in, int64_t n_out,
                   const uint16_t *A, const uint16_t *B, int32_t S, int32_t R, int32_t n_slices,
                   const int32_t *slice_start, const double *alpha, const int32_t *rank,
                   const uint8_t *rslora, const int32_t *idx, int32_t K, const float *scale,
                   int32_t with_base, const int64_t *tokens, int64_t n_tokens, double *y)
{
    (void)S;
    (void)T;
    const int64_t w = (int64_t)n_slices * R;
#pragma omp parallel
    {
        acc_t *u = (acc_t *)malloc((size_t)w * sizeof(acc_t));
        acc_t *yt = (acc_t *)malloc((size_t)n_out * sizeof(acc_t));
#pragma omp for schedule(dynamic)
        for (int64_t q = 0; q < n_tokens; ++q) {
            const int64_t t = tokens ? tokens[q] : q;
            const uint16_t *xt = x + t * n_in;
            for (int64_t n = 0; n < n_out; ++n) {
                acc_t acc = 0;
                if (with_base) {
                    const uint16_t *wrow = W + n * n_in;
                    for (int64_t i = 0; i < n_in; ++i)
                        acc += bf16_value(wrow[i]) * bf16_value(xt[i]);
                }
                yt[n] = acc;
            }
            for (int32_t j = 0; j < K; ++j) {
                const int64_t p = t * K + j;
                const int32_t a = idx[p];
                if (a == -1)
                    continue;
                shrink_one(xt, n_in, A, a, R, n_slices,
                           (acc_t)pair_coef(scale, p, a, alpha, rank, rslora), u);
                expand_one(u, n_out, B, a, R, n_slices, slice_start, yt);
            }
            for (int64_t n = 0; n < n_out; ++n)
                y[q * n_out + n] = (double)yt[n];
        }
        free(yt);
        free(u);
    }
}

/* Bytes of one layer's slot buffers: S slots of n_slices*R*n_in (A) plus n_out*R (B) 16-bit
 * numbers ("Multi-LoRA Serving Explained", memory script: rank x (in + out) numbers per adapted
 * layer, sized at max_lora_rank for GPU slots). */
int64_t oracle_slot_bytes(int32_t S, int32_t R, int64_t n_in, int64_t n_out, int32_t n_slices)
{
    return (int64_t)S * ((int64_t)n_slices * R * n_in + n_out * (int64_t)R) * 2;
}
