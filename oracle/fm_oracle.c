/*
 * fm_oracle.c -- plain, slow CPU oracle for the fused GEMM + tensor-parallel
 * data-movement operators (test infrastructure only).
 *
 * This file is the reference the GPU library is checked against.  It is
 * deliberately naive: fp64 accumulation, explicit gather / scatter / reduce
 * loops, OpenMP only over independent output rows.  It shares no code, header,
 * table or constant with the HIP library and must never be linked into it.
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load it.
 *
 * Sources (the pages these operators are defined on):
 *  - "FLUX: Fast Software-based Communication Overlap On GPUs Through Kernel
 *    Fusion" paper review, section 三 (技术架构), "MLP 前向传播": the first GEMM
 *    is Output1 = GEMM(AllGather(X), W1); the second is
 *    Output2 = ReduceScatter(GEMM(Output1, W2)).
 *  - Flux README mirror ("Flux：细粒度计算-通信重叠的 GPU 内核库"), "快速开始": the
 *    five operators gemm_only, ag_gemm, gemm_rs, moe_ag_scatter, moe_gather_rs.
 *  - COMET article, "COMET 的技术原理": MoE tensors are decomposed along the
 *    token dimension; each expert's rows are gathered, multiplied, and the
 *    results are combined back per token.
 *
 * Element encodings: A/B/X/W/H operands are passed as raw 16-bit patterns
 * (IEEE binary16 when dt == 0, bfloat16 when dt == 1) and decoded exactly to
 * double.  Results are returned in double unless stated otherwise.
 *
 * Build:  gcc -O2 -fopenmp -fPIC -shared fm_oracle.c -o libfm_oracle.so -lm
 * A build with -DFM_ORACLE_MUTANT=<n> plants one deliberate mistake (see the
 * MUTANT() sites); the test suite uses those builds to show that its pins catch
 * each kind of mistake.  The default build plants nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef FM_ORACLE_MUTANT
#define FM_ORACLE_MUTANT 0
#endif
#define MUTANT(n) (FM_ORACLE_MUTANT == (n))

/* ------------------------------------------------------------------------- */
/* Exact decoding of the 16-bit formats (IEEE 754 binary16, bfloat16).        */
/* ------------------------------------------------------------------------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double or_f16_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32 (1/8/7). */
double or_bf16_to_double(uint16_t b) {
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133); /* f * 2^-126 * 2^-7 */
    } else if (e == 255) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + f), e - 134); /* (1 + f/128) * 2^(e-127) */
    }
    return sign ? -v : v;
}

static double dec(int dt, uint16_t x) {
    return dt == 0 ? or_f16_to_double(x) : or_bf16_to_double(x);
}

/* Round a double to the nearest bfloat16, ties to even, directly from the
 * double (no intermediate float, so there is no double rounding).  Overflow
 * goes to infinity as IEEE round-to-nearest requires. */
uint16_t or_double_to_bf16(double x) {
    if (isnan(x)) return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);                  /* a = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;                 /* a in [2^e, 2^(e+1)) */
    if (e < -126) e = -126;         /* subnormal range: fixed quantum */
    double q = ldexp(1.0, e - 7);   /* spacing of bf16 values near a */
    double n = a / q;               /* exact: power-of-two scaling */
    double r = nearbyint(n);        /* current rounding mode = to nearest even */
    double v = r * q;
    if (v == 0.0) return sign;                        /* underflows to zero */
    if (v >= ldexp(1.0, 128)) return sign | 0x7f80;  /* rounds past the max */
    /* re-encode v exactly */
    int ev;
    frexp(v, &ev);
    int be = ev - 1 + 127;          /* biased exponent */
    uint16_t bits;
    if (be <= 0) {
        bits = (uint16_t)(v / ldexp(1.0, -133));  /* subnormal fraction */
    } else {
        double frac = v / ldexp(1.0, ev - 1) - 1.0;  /* in [0,1) */
        bits = (uint16_t)((be << 7) | (int)(frac * 128.0));
    }
    return sign | bits;
}

/* Round a double to the nearest binary16, ties to even. */
uint16_t or_double_to_f16(double x) {
    if (isnan(x)) return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);
    int e = ex - 1;
    if (e < -14) e = -14;
    double q = ldexp(1.0, e - 10);
    double r = nearbyint(a / q);
    double v = r * q;
    if (v == 0.0) return sign;              /* underflows to zero */
    if (v >= 65536.0) return sign | 0x7c00; /* 2^16: beyond the largest finite */
    int ev;
    frexp(v, &ev);
    int be = ev - 1 + 15;
    uint16_t bits;
    if (be <= 0) {
        bits = (uint16_t)(v / ldexp(1.0, -24));
    } else {
        double frac = v / ldexp(1.0, ev - 1) - 1.0;
        bits = (uint16_t)((be << 10) | (int)(frac * 1024.0));
    }
    return sign | bits;
}

void or_round_to_bf16(int64_t n, const double* x, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_double_to_bf16(x[i]);
}

void or_round_to_f16(int64_t n, const double* x, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_double_to_f16(x[i]);
}

/* ------------------------------------------------------------------------- */
/* O1  GEMM:  C[i][j] = sum_k A[i][k] * B[k][j]   (row-major, fp64)           */
/* Follows the definition of GEMM used throughout the FLUX review's MLP       */
/* equations; A is [M,K], B is [K,N], both row-major.                         */
/* ------------------------------------------------------------------------- */

void or_gemm(int dt, int64_t M, int64_t N, int64_t K,
             const uint16_t* A, const uint16_t* B, double* C) {
    double* Bd = (double*)malloc((size_t)(K * N) * sizeof(double));
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) Bd[k * N + j] = dec(dt, B[k * N + j]);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        double* c = C + i * N;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = dec(dt, A[i * K + k]);
            if (MUTANT(1) && k == K - 1) continue;   /* dropped term */
            const double* b = Bd + k * N;
            for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
        }
    }
    free(Bd);
}

/* Selected entries of the same product: C_s = sum_k A[rows[s]][k] B[k][cols[s]].
 * Used where only sampled outputs of a full-size product are checked. */
void or_gemm_entries(int dt, int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, const uint16_t* B,
                     int64_t n_samples, const int64_t* rows, const int64_t* cols,
                     double* out) {
    (void)M;
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < n_samples; ++s) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += dec(dt, A[rows[s] * K + k]) * dec(dt, B[k * N + cols[s]]);
        out[s] = acc;
    }
}

/* ------------------------------------------------------------------------- */
/* O2  AllGather-GEMM:  Output1 = GEMM(AllGather(X), W1)                      */
/* (FLUX review, "MLP 前向传播", first GEMM; "AllGather 重叠").                  */
/* The gathered activation is the concatenation of the n_chunks row chunks in */
/* chunk-index order; chunk c occupies rows [c*Mc, (c+1)*Mc).  The chunks are */
/* copied into place in the given arrival order (an explicit gather loop); the */
/* order of arrival must not change the result.                               */
/* ------------------------------------------------------------------------- */

/* The AllGather itself: chunks land in arrival order and each is copied to */
/* its place by chunk index.  Returns a malloc'ed [n_chunks*Mc, K] buffer.    */
static uint16_t* gather_chunks(int64_t n_chunks, int64_t Mc, int64_t K,
                               const uint16_t* const* chunks, const int32_t* arrival) {
    uint16_t* X = (uint16_t*)malloc((size_t)(n_chunks * Mc * K) * sizeof(uint16_t));
    for (int64_t a = 0; a < n_chunks; ++a) {
        int64_t c = arrival ? arrival[a] : a;           /* which chunk lands now */
        int64_t dst_chunk = MUTANT(2) ? a : c;           /* placed by arrival slot */
        memcpy(X + dst_chunk * Mc * K, chunks[c], (size_t)(Mc * K) * sizeof(uint16_t));
    }
    return X;
}

void or_ag_gemm(int dt, int64_t n_chunks, int64_t Mc, int64_t N, int64_t K,
                const uint16_t* const* chunks, const int32_t* arrival,
                const uint16_t* W, double* C) {
    uint16_t* X = gather_chunks(n_chunks, Mc, K, chunks, arrival);
    or_gemm(dt, n_chunks * Mc, N, K, X, W, C);
    free(X);
}

/* ------------------------------------------------------------------------- */
/* O3  GEMM-ReduceScatter:  Output2 = ReduceScatter(GEMM(Output1, W2))        */
/* (FLUX review, "MLP 前向传播", second GEMM; "ReduceScatter 重叠").            */
/* On one rank the local partial P = A * W (A is [M,K_local]) is reduced into */
/* n_ranks row slices: slice r owns rows [r*M/n_ranks, (r+1)*M/n_ranks) and    */
/* already holds the partial sums of the other ranks (seed_r).  The result is */
/* dst_r = seed_r + P[rows of r], with the addition done in fp64.            */
/* ------------------------------------------------------------------------- */

void or_gemm_rs(int dt, int64_t M, int64_t N, int64_t K, int64_t n_ranks,
                const uint16_t* A, const uint16_t* W,
                const float* const* seeds, double* const* dst) {
    int64_t Ms = M / n_ranks;
    double* P = (double*)malloc((size_t)(M * N) * sizeof(double));
    or_gemm(dt, M, N, K, A, W, P);
    for (int64_t r = 0; r < n_ranks; ++r) {               /* explicit reduce */
        int64_t src_r = MUTANT(3) ? (r + 1) % n_ranks : r; /* wrong slice */
        for (int64_t i = 0; i < Ms; ++i)
            for (int64_t j = 0; j < N; ++j)
                dst[r][i * N + j] = (double)seeds[r][i * N + j] +
                                    P[(src_r * Ms + i) * N + j];
    }
    free(P);
}

/* ------------------------------------------------------------------------- */
/* O4  MoE routing index (COMET: token-dimension decomposition of the tensor  */
/* shared between the MoE layers).                                            */
/* Pairs p = t*topk + k carry expert topk_ids[p].  For the local experts      */
/* [e0, e0+n_local): counts by histogram, offsets by exclusive prefix sum, and */
/* sorted_pairs = the pair ids stably sorted by local expert (so rows of one  */
/* expert appear in increasing pair id).  offsets has n_local+1 entries.      */
/* Returns the number of local pairs.                                         */
/* ------------------------------------------------------------------------- */

int64_t or_moe_route(int64_t T, int64_t topk, int64_t e0, int64_t n_local,
                     const int32_t* topk_ids, int32_t* offsets,
                     int32_t* sorted_pairs) {
    int64_t P = T * topk;
    int64_t* counts = (int64_t*)calloc((size_t)n_local, sizeof(int64_t));
    for (int64_t p = 0; p < P; ++p) {                    /* histogram */
        int64_t e = (int64_t)topk_ids[p] - e0;
        if (e >= 0 && e < n_local) counts[e]++;
    }
    offsets[0] = 0;                                      /* exclusive scan */
    for (int64_t e = 0; e < n_local; ++e)
        offsets[e + 1] = offsets[e] + (int32_t)counts[e];
    int64_t* fill = (int64_t*)calloc((size_t)n_local, sizeof(int64_t));
    for (int64_t p = 0; p < P; ++p) {                    /* stable placement */
        int64_t e = (int64_t)topk_ids[p] - e0;
        if (e >= 0 && e < n_local) {
            int64_t slot = MUTANT(5) ? counts[e] - 1 - fill[e] : fill[e]; /* unstable */
            sorted_pairs[offsets[e] + slot] = (int32_t)p;
            fill[e]++;
        }
    }
    int64_t total = offsets[n_local];
    free(counts);
    free(fill);
    return total;
}

/* ------------------------------------------------------------------------- */
/* O5  MoE layer 0 (gather + per-expert GEMM):                                 */
/*   H[offsets[e] + j] = X[t_j] * W1[e]     with t_j = sorted_pairs[..] / topk */
/* X is [T, hidden], W1 is [n_local, hidden, ffn], H is [rows, ffn] (fp64).    */
/* ------------------------------------------------------------------------- */

void or_moe_layer0(int dt, int64_t T, int64_t hidden, int64_t ffn, int64_t topk,
                   int64_t n_local, const uint16_t* X, const uint16_t* W1,
                   const int32_t* sorted_pairs, const int32_t* offsets,
                   double* H) {
    for (int64_t e = 0; e < n_local; ++e) {
        const uint16_t* W = W1 + e * hidden * ffn;
        int64_t r0 = offsets[e], r1 = offsets[e + 1];
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t r = r0; r < r1; ++r) {
            int64_t t = MUTANT(6) ? sorted_pairs[r] % T   /* pair id as token */
                                  : sorted_pairs[r] / topk; /* explicit gather */
            double* h = H + r * ffn;
            for (int64_t j = 0; j < ffn; ++j) h[j] = 0.0;
            for (int64_t k = 0; k < hidden; ++k) {
                double x = dec(dt, X[t * hidden + k]);
                const uint16_t* w = W + k * ffn;
                for (int64_t j = 0; j < ffn; ++j) h[j] += x * dec(dt, w[j]);
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* O5a Activation applied to layer 0's output before it is stored (Flux       */
/* README: MoE MLP layer 0 is the first GEMM of the expert MLP; the FLUX      */
/* review's MLP forward pass feeds GEMM 1's output to GEMM 2 as is, which is  */
/* act = 0).  In place, elementwise, in fp64:                                 */
/*   1 ReLU        max(x, 0)                                                  */
/*   2 GELU, tanh  x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3)))          */
/*   3 SiLU        x * sigmoid(x) = x / (1 + exp(-x))                         */
/* ------------------------------------------------------------------------- */

void or_activation(int act, int64_t n, double* x) {
    const double c = sqrt(2.0 / 3.14159265358979323846);
    for (int64_t i = 0; i < n; ++i) {
        double v = x[i];
        if (act == 1) {
            v = v > 0.0 ? v : 0.0;
        } else if (act == 2) {
            double half = MUTANT(7) ? 1.0 : 0.5;            /* dropped 1/2 */
            v = half * v * (1.0 + tanh(c * (v + 0.044715 * v * v * v)));
        } else if (act == 3) {
            v = MUTANT(8) ? v / (1.0 + exp(v))               /* sigmoid(-x) */
                          : v / (1.0 + exp(-v));
        }
        x[i] = v;
    }
}

/* ------------------------------------------------------------------------- */
/* O5' MoE layer 0 behind a token AllGather (Flux README: all-gather fused    */
/* with the grouped GEMM of MoE MLP layer 0).  The expert-parallel ranks'     */
/* token chunks are gathered (arrival order, placed by chunk index: chunk c   */
/* holds tokens [c*Tc, (c+1)*Tc)), then layer 0 runs on the gathered tokens.  */
/* ------------------------------------------------------------------------- */

void or_moe_ag_layer0(int dt, int64_t n_chunks, int64_t Tc, int64_t hidden, int64_t ffn,
                      int64_t topk, int64_t n_local, const uint16_t* const* chunks,
                      const int32_t* arrival, const uint16_t* W1,
                      const int32_t* sorted_pairs, const int32_t* offsets, double* H) {
    uint16_t* X = gather_chunks(n_chunks, Tc, hidden, chunks, arrival);
    or_moe_layer0(dt, n_chunks * Tc, hidden, ffn, topk, n_local, X, W1, sorted_pairs, offsets, H);
    free(X);
}

/* ------------------------------------------------------------------------- */
/* O6  MoE layer 1 + top-k weighted combine (scatter-reduce), token-major:     */
/*   out[t] = seed[t] + sum_{k : e(t,k) local} w[t,k] * (H[row(t,k)] * W2[e])  */
/* row(t,k) is the position of pair t*topk+k in sorted_pairs.  H is given as  */
/* 16-bit patterns (the layer-0 output as stored), W2 is [n_local, ffn,       */
/* hidden], out / seed are [T, hidden].                                       */
/* ------------------------------------------------------------------------- */

void or_moe_layer1(int dt, int64_t T, int64_t hidden, int64_t ffn, int64_t topk,
                   int64_t e0, int64_t n_local, const uint16_t* H,
                   const uint16_t* W2, const int32_t* topk_ids,
                   const float* topk_weights, const int32_t* sorted_pairs,
                   const int32_t* offsets, const float* seed, double* out) {
    int64_t rows = offsets[n_local];
    int64_t* row_of_pair = (int64_t*)malloc((size_t)(T * topk) * sizeof(int64_t));
    for (int64_t p = 0; p < T * topk; ++p) row_of_pair[p] = -1;
    for (int64_t r = 0; r < rows; ++r) row_of_pair[sorted_pairs[r]] = r;
#pragma omp parallel
    {
        double* y = (double*)malloc((size_t)hidden * sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < T; ++t) {
            double* o = out + t * hidden;
            for (int64_t j = 0; j < hidden; ++j) o[j] = (double)seed[t * hidden + j];
            for (int64_t k = 0; k < topk; ++k) {
                int64_t p = t * topk + k;
                int64_t e = (int64_t)topk_ids[p] - e0;
                if (e < 0 || e >= n_local) continue;     /* expert not local */
                int64_t r = row_of_pair[p];
                const uint16_t* W = W2 + e * ffn * hidden;
                for (int64_t j = 0; j < hidden; ++j) y[j] = 0.0;
                for (int64_t f = 0; f < ffn; ++f) {
                    double h = dec(dt, H[r * ffn + f]);
                    const uint16_t* w = W + f * hidden;
                    for (int64_t j = 0; j < hidden; ++j) y[j] += h * dec(dt, w[j]);
                }
                double wt = (double)topk_weights[p];
                if (MUTANT(4)) wt = 1.0;                 /* dropped gate weight */
                for (int64_t j = 0; j < hidden; ++j) o[j] += wt * y[j];
            }
        }
        free(y);
    }
    free(row_of_pair);
}

/* Sampled rows of O6 for full-size checks: the same token-major combine for
 * the listed tokens only, written to out[s * hidden + j]. */
void or_moe_layer1_tokens(int dt, int64_t T, int64_t hidden, int64_t ffn,
                          int64_t topk, int64_t e0, int64_t n_local,
                          const uint16_t* H, const uint16_t* W2,
                          const int32_t* topk_ids, const float* topk_weights,
                          const int32_t* sorted_pairs, const int32_t* offsets,
                          const float* seed, int64_t n_tok, const int64_t* toks,
                          double* out) {
    int64_t rows = offsets[n_local];
    int64_t* row_of_pair = (int64_t*)malloc((size_t)(T * topk) * sizeof(int64_t));
    for (int64_t p = 0; p < T * topk; ++p) row_of_pair[p] = -1;
    for (int64_t r = 0; r < rows; ++r) row_of_pair[sorted_pairs[r]] = r;
#pragma omp parallel
    {
        double* y = (double*)malloc((size_t)hidden * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t s = 0; s < n_tok; ++s) {
            int64_t t = toks[s];
            double* o = out + s * hidden;
            for (int64_t j = 0; j < hidden; ++j) o[j] = (double)seed[t * hidden + j];
            for (int64_t k = 0; k < topk; ++k) {
                int64_t p = t * topk + k;
                int64_t e = (int64_t)topk_ids[p] - e0;
                if (e < 0 || e >= n_local) continue;
                int64_t r = row_of_pair[p];
                const uint16_t* W = W2 + e * ffn * hidden;
                for (int64_t j = 0; j < hidden; ++j) y[j] = 0.0;
                for (int64_t f = 0; f < ffn; ++f) {
                    double h = dec(dt, H[r * ffn + f]);
                    const uint16_t* w = W + f * hidden;
                    for (int64_t j = 0; j < hidden; ++j) y[j] += h * dec(dt, w[j]);
                }
                double wt = (double)topk_weights[p];
                for (int64_t j = 0; j < hidden; ++j) o[j] += wt * y[j];
            }
        }
        free(y);
    }
    free(row_of_pair);
}

/* Sampled rows of O5: H rows r in `rs` only (written to out[s * ffn + j]). */
void or_moe_layer0_rows(int dt, int64_t hidden, int64_t ffn, int64_t topk,
                        int64_t n_local, const uint16_t* X, const uint16_t* W1,
                        const int32_t* sorted_pairs, const int32_t* offsets,
                        int64_t n_rows, const int64_t* rs, double* out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t s = 0; s < n_rows; ++s) {
        int64_t r = rs[s];
        int64_t e = 0;
        while (e < n_local && offsets[e + 1] <= r) ++e;  /* expert owning row r */
        const uint16_t* W = W1 + e * hidden * ffn;
        int64_t t = sorted_pairs[r] / topk;
        double* h = out + s * ffn;
        for (int64_t j = 0; j < ffn; ++j) h[j] = 0.0;
        for (int64_t k = 0; k < hidden; ++k) {
            double x = dec(dt, X[t * hidden + k]);
            const uint16_t* w = W + k * ffn;
            for (int64_t j = 0; j < ffn; ++j) h[j] += x * dec(dt, w[j]);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Effective communication time (FLUX review, section 三, "核心公式"):          */
/*   ECT = OverallTime - GEMM_non-split                                        */
/* where GEMM_non-split is the best time of the same GEMM without splitting.  */
/* ------------------------------------------------------------------------- */

double or_ect(double overall_time, double gemm_non_split_time) {
    return overall_time - gemm_non_split_time;
}

int or_mutant_id(void) { return FM_ORACLE_MUTANT; }
