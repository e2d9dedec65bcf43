/*
 * dg.h — C ABI of the MI355X (gfx950) fine-grained-scaled FP8 GEMM library (libdg.so).
 *
 * The operation (DeepGEMM pages: pt.news.hada.io, "Interface GEMM e restrições de layout"
 * and "GEMM denso e grouped"; feifmx.com release article on fine-grained scaling with
 * two-level accumulation):
 *
 *     D[m, n] = C[m, n] + sum_kb  sfa[m, kb] * sfb[n / 128, kb] * sum_{k in block kb} A[m, k] * B[n, k]
 *
 * in NT layout: A is e4m3 [M, K] row-major (K contiguous), B is e4m3 [N, K] row-major, so
 * B.T is column-major.  One FP32 scale per 1x128 segment of an A row, stored transposed
 * (MN-major): sfa[m, kb] lives at sfa[kb * ld_sfa + m].  One FP32 scale per 128x128 block of
 * B: sfb[nb, kb] at sfb[nb * (K/128) + kb], nb = n / 128 (ceil(N/128) block rows; the last
 * one may cover fewer than 128 rows).  D is bf16 [M, N] row-major, rounded to nearest-even
 * from the FP32 accumulator.  C is an optional FP32 [M, N] row-major accumulator.
 * e4m3 is the OCP E4M3FN encoding (max normal 448, S.1111.111 = NaN).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library never frees or
 *    retains them and never allocates on their behalf.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream) and never
 *    synchronize the host.  Argument checks happen on the host before any HIP call.
 *  - Return value: DG_OK (0) or a negative dg_status.  dg_last_error() then holds a message
 *    (thread-local).  A launch failure reported by the HIP runtime returns DG_ERR_HIP.
 *  - Preconditions: K > 0 and K % 128 == 0; N > 0 and N % 16 == 0; row counts >= 0 (zero
 *    rows is a no-op that returns DG_OK without touching the device); ld_sfa % 4 == 0 and
 *    ld_sfa >= the number of A rows; A, B, D, C and sfa 16-byte aligned; sfb 4-byte aligned.
 *  - Values in device memory cannot be checked without a synchronization, so their
 *    behaviour is defined instead (see each call).
 */
#ifndef DG_H
#define DG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DG_OK = 0,
    DG_ERR_INVALID_ARG = -1, /* null pointer, negative or zero size, ld_sfa too small     */
    DG_ERR_UNSUPPORTED = -2, /* a shape outside the preconditions (K % 128, N % 16, ...)  */
    DG_ERR_MISALIGNED = -3,  /* a pointer or leading dimension breaks the alignment rules */
    DG_ERR_HIP = -4          /* the HIP runtime reported an error (no device, launch...)   */
} dg_status;

/*
 * Dense NT GEMM: D = C + A @ B.T (pt.news.hada.io, "Interface GEMM e restrições de layout":
 * fp8_gemm_nt computes D = C + A @ B.T; NT layout; LHS scale FP32, transposed).
 *   a      e4m3 [m, k]
 *   sfa    FP32 [k/128][ld_sfa], element (row, kb) at kb*ld_sfa + row, ld_sfa >= m
 *   b      e4m3 [n, k]
 *   sfb    FP32 [ceil(n/128)][k/128]
 *   c      FP32 [m, n] or NULL (then C = 0); must not overlap d
 *   d      bf16 [m, n], written in full
 * Skinny shapes may split K across workgroups; the partial sums then go through a
 * library-owned workspace and are reduced in a fixed order, so results are deterministic.
 * There is one workspace per (device, stream): it is allocated by the first such call made on
 * that stream outside graph capture, grown (never freed) when a call needs more, and a graph
 * keeps using the workspace of the stream it was captured on.  So calls on different streams
 * may run concurrently; calls on one stream are ordered by the stream.  A call captured on a
 * stream that has no workspace yet runs a slower tile configuration that needs none.
 */
int dg_fp8_gemm_nt(const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                   const float *sfb, const float *c, void *d, int m, int n, int k,
                   void *stream);

/*
 * dg_fp8_gemm_nt for callers that cannot allocate device memory: code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments, result and errors as
 * dg_fp8_gemm_nt, except that the split-K partial tiles of skinny shapes go to a static device
 * array of the library (16 MiB, one per device, held until the process ends) instead of a
 * workspace, so the call never allocates.  A shape whose partials would need more than that
 * array returns DG_ERR_UNSUPPORTED (shapes that do not split K need none of it).  Every call of
 * this entry point on one device shares the array: calls that overlap in time on one device
 * (on any streams) race and must be ordered by the caller.
 */
int dg_fp8_gemm_nt_noalloc(const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                           const float *sfb, const float *c, void *d, int m, int n, int k,
                           void *stream);

/*
 * M-grouped GEMM, contiguous layout (pt.news.hada.io, "GEMM denso e grouped": experts share
 * N and K; their token rows are concatenated along M; each expert segment is aligned to the
 * M block, whose size dg_get_mk_alignment_for_contiguous_layout() returns).
 *   a          e4m3 [m_total, k], m_total % 128 == 0
 *   sfa        FP32 [k/128][ld_sfa], ld_sfa >= m_total
 *   b          e4m3 [num_groups, n, k]
 *   sfb        FP32 [num_groups][ceil(n/128)][k/128]
 *   d          bf16 [m_total, n]
 *   m_indices  device int32 [m_total]: the group of each row; -1 marks a padding row
 * Row r is computed with B[m_indices[r]] and written to D; rows whose index is outside
 * [0, num_groups) are neither read into any result nor written (D keeps its old contents).
 * Each aligned 128-row block must hold rows of at most one group (padding aside); rows of a
 * block that mixes two groups may be left unwritten.
 */
int dg_m_grouped_fp8_gemm_nt_contiguous(const void *a, const float *sfa, int64_t ld_sfa,
                                        const void *b, const float *sfb, void *d,
                                        const int32_t *m_indices, int m_total, int n, int k,
                                        int num_groups, void *stream);

/*
 * The contiguous M-grouped GEMM with the activation step between an expert's two GEMMs fused
 * into its epilogue (pt.news.hada.io, "Mega MoE": linear 1 -> SwiGLU -> linear 2 of an MoE
 * block in one pass; "Interface GEMM e restrições de layout": the FP8 cast of the next GEMM's
 * input is otherwise left to the caller).  For each computed row r (as in
 * dg_m_grouped_fp8_gemm_nt_contiguous) the FP32 result D1[r, :] = A[r] @ B[g].T (scaled as
 * there, not rounded) is split into gate = D1[r, :n/2] and up = D1[r, n/2:], and
 *     h = gate * up / (1 + exp(-gate));  per 1x128 segment s of h:
 *     scale = max(amax, 1e-4) / 448,  q = e4m3(h / scale) (nearest even, within +-448)
 *   a, sfa, b, sfb, m_indices, m_total, k, num_groups   as in the contiguous call; n = 2I, the
 *             gate rows of each B[g] first, then the up rows; n % 256 == 0
 *   q         e4m3 [m_total, n/2], 16-byte aligned: the codes of h
 *   sfq       FP32 [n/256][ld_sfq], 16-byte aligned, ld_sfq >= m_total, ld_sfq % 4 == 0: the
 *             scales, MN-major (sfq[s * ld_sfq + r]), the layout of the next GEMM's sfa
 * Padding rows are written in neither q nor sfq.  FP32 scales only.  Errors as above.
 */
int dg_m_grouped_fp8_gemm_nt_contiguous_swiglu(const void *a, const float *sfa,
                                               int64_t ld_sfa, const void *b, const float *sfb,
                                               void *q, float *sfq, int64_t ld_sfq,
                                               const int32_t *m_indices, int m_total, int n,
                                               int k, int num_groups, void *stream);

/*
 * M-grouped GEMM, masked layout (pt.news.hada.io, "GEMM denso e grouped": for decoding under
 * graph capture, when the host does not know the per-expert token counts, a mask tensor
 * tells the kernel which region is valid and only that region is computed).
 *   a         e4m3 [num_groups, m_max, k]
 *   sfa       FP32 [num_groups][k/128][ld_sfa], ld_sfa >= m_max
 *   b         e4m3 [num_groups, n, k]
 *   sfb       FP32 [num_groups][ceil(n/128)][k/128]
 *   d         bf16 [num_groups, m_max, n]
 *   masked_m  device int32 [num_groups]: valid rows of each group, read on the device at run
 *             time (clamped to [0, m_max]); rows at or beyond it are not written
 *   expected_m  host hint of the typical valid-row count (<= 0: m_max/2), printed with the
 *             tile choice under DG_PRINT_CONFIGS.  On gfx950 the measured fastest tile does
 *             not depend on it (256-row tiles whenever m_max > 128, at every expected count
 *             from 8 to 128 rows), so the choice is made from m_max, n and k alone.
 * The call performs no allocation, no host synchronization and no host read of device
 * memory, so it can be captured in a hipGraph and replayed after masked_m is rewritten.
 */
int dg_m_grouped_fp8_gemm_nt_masked(const void *a, const float *sfa, int64_t ld_sfa,
                                    const void *b, const float *sfb, void *d,
                                    const int32_t *masked_m, int num_groups, int m_max, int n,
                                    int k, int expected_m, void *stream);

/*
 * The three calls above with packed UE8M0 scales instead of FP32 ones (pt.news.hada.io,
 * "Interface GEMM e restrições de layout": the newer hardware generation takes the scaling
 * factors as UE8M0, four packed into one 32-bit integer).  Same granularity (1x128 A
 * segments, 128x128 B blocks) and layouts, with the K-block axis packed: word q of a row
 * holds the scales of K blocks 4q .. 4q+3 in its bytes 0..3 (least significant first), and a
 * byte e means 2^(e-127) (0xFF: NaN).  So
 *   sfa  int32 [ceil(k/512)][ld_sfa]                      (dense, contiguous)
 *        int32 [num_groups][ceil(k/512)][ld_sfa]          (masked)
 *   sfb  int32 [ceil(n/128)][ceil(k/512)]                 (dense)
 *        int32 [num_groups][ceil(n/128)][ceil(k/512)]     (grouped)
 * Every other argument, precondition and behaviour is that of the FP32 call (including the
 * split-K path of skinny dense shapes and its workspace); the MFMA applies the exponents.
 */
int dg_fp8_gemm_nt_ue8m0(const void *a, const int32_t *sfa, int64_t ld_sfa, const void *b,
                         const int32_t *sfb, const float *c, void *d, int m, int n, int k,
                         void *stream);
int dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const void *a, const int32_t *sfa, int64_t ld_sfa,
                                              const void *b, const int32_t *sfb, void *d,
                                              const int32_t *m_indices, int m_total, int n,
                                              int k, int num_groups, void *stream);
int dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const void *a, const int32_t *sfa, int64_t ld_sfa,
                                          const void *b, const int32_t *sfb, void *d,
                                          const int32_t *masked_m, int num_groups, int m_max,
                                          int n, int k, int expected_m, void *stream);

/*
 * The other dense memory layouts of the same GEMM (pt.news.hada.io, "Interface GEMM e
 * restrições de layout": NT, TN, NN and TT; "GEMM denso e grouped": fp8_gemm_{nt, nn, tn, tt}).
 * The first letter is A's storage, the second B's:
 *   A "n": e4m3 [m][k] (as in dg_fp8_gemm_nt)    A "t": e4m3 [k][m] (M contiguous)
 *   B "t": e4m3 [n][k] (as in dg_fp8_gemm_nt)    B "n": e4m3 [k][n] (N contiguous)
 * The mathematical operation, the scales (sfa MN-major [k/128][ld_sfa], 1x128 segments of A's
 * rows; sfb [ceil(n/128)][k/128], 128x128 blocks of B), C, D and the error behaviour are those
 * of dg_fp8_gemm_nt.  In addition: m % 16 == 0 when A is stored [k][m], and
 * k * max(m, n) < 2^31.  MN-major operands are transposed into a library-owned workspace, one
 * per (device, stream), allocated or grown (at least doubling) by a call made outside graph
 * capture; a replaced workspace is kept until the process ends, since captured graphs may
 * still use it.  A captured call whose stream has no large enough workspace reads the
 * MN-major operands directly instead (a slower kernel that needs none).
 */
int dg_fp8_gemm_nn(const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                   const float *sfb, const float *c, void *d, int m, int n, int k, void *stream);
int dg_fp8_gemm_tn(const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                   const float *sfb, const float *c, void *d, int m, int n, int k, void *stream);
int dg_fp8_gemm_tt(const void *a, const float *sfa, int64_t ld_sfa, const void *b,
                   const float *sfb, const float *c, void *d, int m, int n, int k, void *stream);

/*
 * K-grouped TN GEMM, the MoE weight gradient (pt.news.hada.io, "GEMM denso e grouped": an API
 * grouped on the K axis for the backward pass of MoE weights, M and N fixed;
 * "Interface GEMM e restrições de layout": D = C + A @ B, the TN memory layout).  For each
 * group g and its run of K (consecutive K indices, ks[g] of them):
 *   D[g, m, n] = C[g, m, n] + sum over the group's K blocks kb of
 *                sfa[kb, m] * sfb[kb, n] * sum_{k in kb} A[k, m] * B[k, n]
 *   a    e4m3 [k_total][m]   token-major (M contiguous), 16-byte aligned
 *   sfa  FP32 [k_total/128][m]   one scale per 128-deep K block per column of A
 *   b    e4m3 [k_total][n]   token-major (N contiguous)
 *   sfb  FP32 [k_total/128][n]
 *   c    FP32 [num_groups][m][n] or NULL (zeros); may be d itself (accumulate in place)
 *   d    FP32 [num_groups][m][n], written whole (a group with ks[g] == 0 gets C, or zeros)
 *   ks   HOST int32 [num_groups]: multiples of 128 (0 allowed) summing to k_total; they go
 *        to the kernel as launch arguments, so the call is graph-capturable
 * Preconditions: 1 <= num_groups <= 256; m, n multiples of 16; k_total a multiple of 128;
 * k_total * max(m, n) < 2^31; A, B, C, D, sfa, sfb 16-byte aligned.  Errors as above.
 */
int dg_k_grouped_fp8_gemm_tn_contiguous(const void *a, const float *sfa, const void *b,
                                        const float *sfb, const float *c, float *d,
                                        const int32_t *ks, int num_groups, int m, int n,
                                        int k_total, void *stream);

/*
 * The activation step between an expert's two GEMMs, fused (pt.news.hada.io, "Interface GEMM
 * e restrições de layout": casting to FP8 is left to the caller).  x: bf16 [m][2i], gate
 * columns first, then up (the first GEMM's D).  Writes
 *   q    e4m3 [m][i]      q = e4m3(h / scale), nearest even, within +-448, where
 *                         h = gate * up / (1 + exp(-gate))
 *   sfa  FP32 [i/128][ld_sfa]   scale = max(amax of the 1x128 segment of h, 1e-4) / 448, at
 *                         sfa[seg * ld_sfa + row] (MN-major: the NT GEMM's A scales for q)
 * i % 128 == 0; ld_sfa >= m; x 16-byte, q 8-byte, sfa 4-byte aligned; m == 0 is a no-op.
 * sfa's columns past m are not written.
 */
int dg_swiglu_fp8_quant(const void *x, void *q, float *sfa, int64_t ld_sfa, int m, int i,
                        void *stream);

/* Row alignment of each group segment in the contiguous layout: 128 (the M block size).
 * pt.news.hada.io, "Utilitários e variáveis de ambiente" (get_mk_alignment_for_contiguous_layout)
 * and "GEMM denso e grouped" (each expert segment aligned to the GEMM M block).  No error. */
int dg_get_mk_alignment_for_contiguous_layout(void);

/* Smallest valid ld_sfa for m rows: m rounded up to a multiple of 4, so that each K-block
 * column of the MN-major A scales starts on a 16-byte boundary; 0 for m <= 0.
 * pt.news.hada.io, "Utilitários e variáveis de ambiente" (get_tma_aligned_size: the alignment
 * the transposed LHS scale layout needs) and "Interface GEMM e restrições de layout" (LHS
 * scale transposed and aligned).  No error. */
int64_t dg_get_sf_aligned_m(int64_t m);

/* Cap (n > 0) or reset (n <= 0) the number of compute units the tile heuristic plans for;
 * returns the previous cap (0 = none).  pt.news.hada.io, "Utilitários e variáveis de
 * ambiente" (set_num_sms: the number of SMs the kernels use).  Process-wide, not per device;
 * no error. */
int dg_set_num_cus(int n);

/* Compute units the heuristic plans for on the current device (the cap if set), or
 * DG_ERR_HIP if no device is available.  pt.news.hada.io, "Utilitários e variáveis de
 * ambiente" (get_num_sms). */
int dg_get_num_cus(void);

/* Message for the most recent non-OK return on this thread ("" after an OK return).  The pages
 * define no error convention for a C interface; this one and dg_status are the library's own. */
const char *dg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
