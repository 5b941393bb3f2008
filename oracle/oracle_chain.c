/*
 * oracle_chain.c -- plain, slow, obviously-correct CPU oracle for a chain of
 * dependent GEMMs.  TEST INFRASTRUCTURE ONLY: the product path never links,
 * loads or calls this file; only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark do.
 *
 * What it computes (CTA-Pipelining: A Latency-Oriented Spatial Scaling Method
 * for Multi-GPU Systems, arXiv 2607.07862):
 *   - the running example is a two-layer GEMM whose first output is consumed
 *     directly by the second GEMM (§III-B), generalised to one GEMM per layer
 *     for multi-layer chains (§IV-A, Fig. 4) and written Y = X A B for the MLP
 *     (§IV-B);
 *   - GEMM inputs and outputs are stored in BF16 with an FP32 accumulator
 *     (§III-C); this oracle accumulates in fp64 instead, so it is the exact
 *     definition up to fp64 rounding;
 *   - CTA-pipelining changes only *when* a tile runs, never *what* it computes:
 *     the original kernel body is preserved (§III-C, interference paragraph),
 *     so the oracle is the plain chain with no tiling, no scheduling and no
 *     protocol at all;
 *   - the tanh-approximation GeLU between the two products is the variant the
 *     pith.science review of the paper names in "What would settle it".
 *
 * Per layer l = 1..L:   A = H_{l-1} . W_l   (i-k-j triple loop, fp64)
 *                       A = act_l(A)        (identity or tanh-GeLU, fp64)
 *                       H_l = round(A)      (storage dtype, round-to-nearest-even;
 *                                            skipped for l = L, and for all l when
 *                                            round_intermediates == 0)
 * Readings where the pages are silent: row-major X[M,K], W[K,N] with no
 * transpose and no bias; intermediates stored in the GEMM output dtype;
 * round-to-nearest-even; GeLU applied to the accumulator before rounding.
 *
 * Parity pins: tests/test_oracle.py (exact integer brute force, identity and
 * signed-permutation weights, row independence, power-of-two linearity,
 * associativity bound, GeLU odd identity and limits, bf16 rounding table).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_ACT_NONE = 0, ORACLE_ACT_GELU_TANH = 1 };

/* Exact widening of a bf16 bit pattern: bf16 is the top half of an IEEE
 * binary32, so placing the 16 bits in the high half of a float is exact. */
static double bf16_bits_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even (the plain
 * definition: bf16 keeps 8 significant bits and binary32's exponent range,
 * with subnormals spaced 2^-133).  Returns the bit pattern. */
uint16_t oracle_round_bf16(double x) {
    if (isnan(x)) return 0x7FC0;
    if (isinf(x)) return x > 0 ? 0x7F80 : 0xFF80;
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    int e;
    frexp(x, &e);                     /* |x| = m * 2^e, 0.5 <= m < 1 */
    int qexp = e - 8;                 /* spacing of 8-significant-bit numbers */
    if (qexp < -133) qexp = -133;     /* bf16 subnormal spacing */
    double q = ldexp(1.0, qexp);
    double r = nearbyint(x / q) * q;  /* default rounding mode: ties to even */
    const double maxf = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (fabs(r) > maxf) return r > 0 ? 0x7F80 : 0xFF80;
    float f = (float)r;               /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (r == 0.0) u = signbit(x) ? 0x80000000u : 0u;
    return (uint16_t)(u >> 16);
}

/* tanh-approximation GeLU, fp64:
 *   gelu(x) = x/2 * (1 + tanh( sqrt(2/pi) * (x + 0.044715 x^3) )) */
double oracle_gelu_tanh(double x) {
    const double k0 = sqrt(2.0 / M_PI);
    return 0.5 * x * (1.0 + tanh(k0 * (x + 0.044715 * x * x * x)));
}

static double round_storage(double x, int32_t dtype) {
    if (dtype == ORACLE_BF16) return bf16_bits_to_f64(oracle_round_bf16(x));
    return (double)(float)x;          /* binary32, round-to-nearest-even */
}

static double load_elem(const void *p, int64_t idx, int32_t dtype) {
    if (dtype == ORACLE_BF16) return bf16_bits_to_f64(((const uint16_t *)p)[idx]);
    return (double)((const float *)p)[idx];
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * oracle_chain: the whole chain for the rows listed in `rows` (or all M rows
 * when rows == NULL; then n_rows must equal M).  Rows of a GEMM chain are
 * independent, so a row subset is the same computation as the full run.
 *
 *   widths[0..L]     K0, N1, ..., NL
 *   X                M x K0 in `dtype` (bit patterns: float or uint16 bf16)
 *   W[l]             widths[l] x widths[l+1] in `dtype`
 *   acts[l]          activation after layer l+1 (NULL: none)
 *   Y                n_rows x NL fp64, the unrounded last layer
 *   H[l] (optional)  n_rows x widths[l+1] fp64 for l < L-1: the stored
 *                    intermediate after activation and storage rounding
 * Returns 0, or -1 on a bad argument.
 */
int oracle_chain(int64_t M, int32_t L, const int64_t *widths, int32_t dtype,
                 const void *X, const void *const *W, const int32_t *acts,
                 int32_t round_intermediates, const int64_t *rows,
                 int64_t n_rows, double *Y, double *const *H) {
    if (M < 0 || L < 1 || !widths || !X || !W || !Y) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    if (!rows && n_rows != M) return -1;
    int64_t maxw = 0;
    for (int32_t l = 0; l <= L; ++l) {
        if (widths[l] <= 0) return -1;
        if (widths[l] > maxw) maxw = widths[l];
    }
    for (int64_t r = 0; rows && r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;

    int bad = 0;
#pragma omp parallel
    {
        double *cur = (double *)malloc(sizeof(double) * (size_t)maxw);
        double *nxt = (double *)malloc(sizeof(double) * (size_t)maxw);
        if (!cur || !nxt) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!cur || !nxt) continue;
            int64_t i = rows ? rows[r] : r;
            int64_t K = widths[0];
            for (int64_t k = 0; k < K; ++k) cur[k] = load_elem(X, i * K + k, dtype);
            for (int32_t l = 0; l < L; ++l) {
                int64_t N = widths[l + 1];
                const void *Wl = W[l];
                for (int64_t j = 0; j < N; ++j) nxt[j] = 0.0;
                for (int64_t k = 0; k < K; ++k) {          /* i-k-j order */
                    double a = cur[k];
                    for (int64_t j = 0; j < N; ++j)
                        nxt[j] += a * load_elem(Wl, k * N + j, dtype);
                }
                int32_t act = acts ? acts[l] : ORACLE_ACT_NONE;
                if (act == ORACLE_ACT_GELU_TANH)
                    for (int64_t j = 0; j < N; ++j) nxt[j] = oracle_gelu_tanh(nxt[j]);
                if (l + 1 < L) {
                    if (round_intermediates)
                        for (int64_t j = 0; j < N; ++j) nxt[j] = round_storage(nxt[j], dtype);
                    if (H && H[l]) memcpy(H[l] + r * N, nxt, sizeof(double) * (size_t)N);
                } else {
                    memcpy(Y + r * N, nxt, sizeof(double) * (size_t)N);
                }
                double *t = cur; cur = nxt; nxt = t;
                K = N;
            }
        }
        free(cur);
        free(nxt);
    }
    return bad ? -1 : 0;
}

/* Vector helpers so that the tests can pin rounding and GeLU directly. */
void oracle_round_bf16_array(const double *x, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(x[i]);
}

void oracle_gelu_tanh_array(const double *x, double *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_gelu_tanh(x[i]);
}
