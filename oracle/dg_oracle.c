/*
 * CPU oracle for the fine-grained-scaled FP8 GEMM  D = C + A @ B.T  (NT layout) and its two
 * M-grouped MoE forms.  TEST INFRASTRUCTURE ONLY: it is called by the test-suite, by the
 * library's smoke check and by the benchmark's CPU-baseline leg, never by the product path.
 * It shares no code, header, table or constant with the HIP library.
 *
 * What it follows (DeepGEMM pages):
 *  - pt.news.hada.io, "Interface GEMM e restrições de layout": fp8_gemm_nt computes
 *    D = C + A @ B.T; A row-major (K contiguous), B.T column-major, i.e. B is [N, K] with K
 *    contiguous; the LHS scale factor is FP32 and stored transposed (MN-major).
 *  - feifmx.com (Feb 2025 release article): fine-grained scaling from DeepSeek-V3 with a
 *    two-level accumulation: tensor-core partial sums are promoted into FP32 per block.
 *    The granularity is one scale per 1x128 segment of an A row and one per 128x128 block
 *    of B, so the scales change every 128 values of K and each 128-deep block sum is scaled
 *    by sfa[m,kb] * sfb[n/128,kb] before it is added.
 *  - pt.news.hada.io, "GEMM denso e grouped": contiguous layout groups along M only (N, K
 *    fixed), each expert segment aligned to the M block; masked layout computes only the
 *    valid region given by a per-group count.
 *
 * Arithmetic: float64 throughout.  Every e4m3 value is k*2^-9 with |k| <= 448*512 < 2^18, so
 * a product of two is an integer multiple of 2^-18 below 2^36 in magnitude and a 128-term
 * block sum stays below 2^43: the block sums below are exact in float64 in any order.  The
 * scale product of two FP32 numbers (24-bit significands) is exact in float64 as well; the
 * only roundings are the scaled block-sum accumulation and the final + C.
 *
 * Output convention: D is float64 and only the rows the method computes are written; the
 * caller pre-fills D (e.g. with NaN) to see which rows were left untouched.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KBLK 128

/* OCP 8-bit floating point, E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits
 * 2..0; exponent 0 is subnormal (f * 2^-9); S.1111.111 is NaN; there are no infinities. */
static double e4m3_decode(uint8_t bits)
{
    int s = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xF;
    int f = bits & 0x7;
    double mag;
    if (e == 15 && f == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)f, -9);
    else
        mag = ldexp((double)(8 + f), e - 10);
    return s ? -mag : mag;
}

static double g_table[256];
static int g_table_ready = 0;

static void ensure_table(void)
{
    if (g_table_ready)
        return;
    for (int i = 0; i < 256; ++i)
        g_table[i] = e4m3_decode((uint8_t)i);
    g_table_ready = 1;
}

void dgo_e4m3_table(double *out)
{
    ensure_table();
    for (int i = 0; i < 256; ++i)
        out[i] = g_table[i];
}

/* Threads of the OpenMP loops below (the CPU baseline times the oracle on one thread too). */
void dgo_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int dgo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sum over one 128-deep K block of dec(A[m,k]) * dec(B[n,k]); arow/brow point at the block. */
static double block_partial(const uint8_t *arow, const uint8_t *brow)
{
    double s = 0.0;
    for (int t = 0; t < KBLK; ++t)
        s += g_table[arow[t]] * g_table[brow[t]];
    return s;
}

/* Exposes the block partials P[m][n][kb] (before any scale), for the exactness checks. */
void dgo_block_partials(const uint8_t *a, const uint8_t *b, double *p, int64_t m, int64_t n,
                        int64_t k)
{
    ensure_table();
    int64_t kbs = k / KBLK;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            for (int64_t kb = 0; kb < kbs; ++kb)
                p[(i * n + j) * kbs + kb] =
                    block_partial(a + i * k + kb * KBLK, b + j * k + kb * KBLK);
}

/*
 * One output row:  d[j] = c[j] + sum_kb (sfa_m[kb] * sfb[j/128][kb]) * P(m, j, kb),
 * kb ascending; c == NULL means C = 0.  sfa_m[kb] is read at sfa_col[kb * ld_sfa].
 */
static void gemm_row(const uint8_t *arow, const float *sfa_col, int64_t ld_sfa,
                     const uint8_t *b, const float *sfb, const float *crow, double *drow,
                     int64_t n, int64_t k)
{
    int64_t kbs = k / KBLK;
    for (int64_t j = 0; j < n; ++j) {
        const uint8_t *brow = b + j * k;
        const float *sfb_row = sfb + (j / KBLK) * kbs;
        double acc = 0.0;
        for (int64_t kb = 0; kb < kbs; ++kb) {
            double scale = (double)sfa_col[kb * ld_sfa] * (double)sfb_row[kb];
            acc += scale * block_partial(arow + kb * KBLK, brow + kb * KBLK);
        }
        drow[j] = acc + (crow ? (double)crow[j] : 0.0);
    }
}

/*
 * Dense NT GEMM.  a: e4m3 [m, k]; sfa: FP32 MN-major, element (row, kb) at kb*ld_sfa + row;
 * b: e4m3 [n, k]; sfb: FP32 [ceil(n/128)][k/128]; c: FP32 [m, n] or NULL; d: float64 [m, n].
 * Returns 0, or -1 on a shape it does not define (k % 128 != 0, ld_sfa < m).
 */
int dgo_fp8_gemm_nt(const uint8_t *a, const float *sfa, int64_t ld_sfa, const uint8_t *b,
                    const float *sfb, const float *c, double *d, int64_t m, int64_t n,
                    int64_t k)
{
    if (k % KBLK != 0 || ld_sfa < m || m < 0 || n < 0)
        return -1;
    ensure_table();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i)
        gemm_row(a + i * k, sfa + i, ld_sfa, b, sfb, c ? c + i * n : NULL, d + i * n, n, k);
    return 0;
}

/*
 * Contiguous M-grouped form: rows of all groups concatenated, row r belongs to group
 * m_indices[r]; rows whose index is outside [0, num_groups) (padding, -1) are not computed.
 * b: e4m3 [G, n, k]; sfb: [G][ceil(n/128)][k/128]; sfa MN-major with ld_sfa >= m_total.
 */
int dgo_m_grouped_fp8_gemm_nt_contiguous(const uint8_t *a, const float *sfa, int64_t ld_sfa,
                                         const uint8_t *b, const float *sfb, double *d,
                                         const int32_t *m_indices, int64_t m_total, int64_t n,
                                         int64_t k, int64_t num_groups)
{
    if (k % KBLK != 0 || ld_sfa < m_total || m_total < 0 || n < 0 || num_groups < 1)
        return -1;
    ensure_table();
    int64_t nbs = (n + KBLK - 1) / KBLK;
    int64_t kbs = k / KBLK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < m_total; ++r) {
        int64_t g = m_indices[r];
        if (g < 0 || g >= num_groups)
            continue;
        gemm_row(a + r * k, sfa + r, ld_sfa, b + g * n * k, sfb + g * nbs * kbs, NULL,
                 d + r * n, n, k);
    }
    return 0;
}

/*
 * Masked M-grouped form: group g owns rows [0, masked_m[g]) of its fixed [m_max, k] buffer
 * (masked_m clamped to [0, m_max]); other rows are not computed.
 * a: e4m3 [G, m_max, k]; sfa: [G][k/128][ld_sfa >= m_max]; b: [G, n, k];
 * sfb: [G][ceil(n/128)][k/128]; d: float64 [G, m_max, n].
 */
int dgo_m_grouped_fp8_gemm_nt_masked(const uint8_t *a, const float *sfa, int64_t ld_sfa,
                                     const uint8_t *b, const float *sfb, double *d,
                                     const int32_t *masked_m, int64_t num_groups, int64_t m_max,
                                     int64_t n, int64_t k)
{
    if (k % KBLK != 0 || ld_sfa < m_max || m_max < 0 || n < 0 || num_groups < 1)
        return -1;
    ensure_table();
    int64_t nbs = (n + KBLK - 1) / KBLK;
    int64_t kbs = k / KBLK;
    int64_t rows = num_groups * m_max;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t g = r / m_max, i = r % m_max;
        int64_t valid = masked_m[g];
        if (valid < 0)
            valid = 0;
        if (valid > m_max)
            valid = m_max;
        if (i >= valid)
            continue;
        gemm_row(a + (g * m_max + i) * k, sfa + g * kbs * ld_sfa + i, ld_sfa, b + g * n * k,
                 sfb + g * nbs * kbs, NULL, d + (g * m_max + i) * n, n, k);
    }
    return 0;
}
