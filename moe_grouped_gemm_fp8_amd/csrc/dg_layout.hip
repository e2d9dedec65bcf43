// The FP8 GEMM for operands stored MN-major (pt.news.hada.io, "Interface GEMM e restrições
// de layout": D = C + A @ B in the NT, TN, NN and TT memory layouts; "GEMM denso e grouped":
// fp8_gemm_{nt, nn, tn, tt} and the K-grouped k_grouped_fp8_gemm_tn_contiguous for the
// backward pass of MoE weights).  One kernel template covers
//  * the dense NN, TN and TT layouts: A stored [M, K] ("n") or [K, M] ("t"), B stored [N, K]
//    ("t") or [K, N] ("n"), the NT scale layouts (1x128 A segments, 128x128 B blocks), bf16 D
//    and an optional FP32 C;
//  * the K-grouped TN form (the MoE weight gradient): A [K_total, M] and B [K_total, N]
//    token-major, group g a run of K, one FP32 scale per 128-deep K block per column for
//    both operands, FP32 D[g] = C[g] + ..., C optional or D itself:
//        D[g, m, n] = C[g, m, n] + sum over its K blocks kb of
//                     sfa[kb, m] * sfb[kb, n] * sum_{k in kb} A[k, m] * B[k, n]
// (the NT layout has its own, more deeply pipelined kernels; the dense NN/TN/TT calls run
// those by default after dg_transpose_u8_kernel below has made their MN-major operands
// K-major, and use this template under graph capture before their workspace exists).
//
// Design:
//  * One workgroup per tile (of one group); eight waves (2 x 4).  Dense tiles are 128 x 128
//    (wave tile 64 x 32); K-grouped tiles 128 x 256 (wave tile 64 x 64: per MFMA, three
//    quarters of the copies and two thirds of the fragment reads of the 128 x 128 tile; the
//    weight gradient of the routed 8-expert shape 1518 us against 1812 us).  Dense tiles go to
//    the XCDs in 8 raster-order chunks (neighbours share A and B panels in an XCD's L2);
//    K-grouped tiles go round-robin, so each XCD gets an equal share of every group whatever
//    the groups' K extents (one range over all groups gave one XCD the largest group's tiles).
//  * Per K block a tile needs 128 x BM bytes of A and 128 x BN bytes of B.  They are staged
//    whole by direct-to-LDS buffer copies (1 KB per wave instruction) into NS slots, NS - 1
//    blocks ahead: block j starts with a wait for block j + 1 and one barrier, after which
//    block j + NS - 1 refills block j - 1's slot (every wave has read it into registers by
//    then).  Four slots where they fit (128 x 128), three for 128 x 256, whose blocks take
//    twice as long.  Block j + 1's A fragments are read into a second register set during
//    block j's MFMAs; so are its B fragments on 128 x 128 tiles, while the wider tile (one B
//    register set, to fit 256 VGPRs) reads them after block j's last MFMAs and promotions.
//  * A K-major operand's LDS rows are its rows (128 bytes of K each), read as two
//    ds_read_b128 per MFMA operand lane, as in the NT kernels.  An MN-major operand's LDS
//    rows are K indices; ds_read_b64_tr_b8 gives a lane 8 consecutive K values of one column
//    (see dg_device.h), so an operand lane is four transposing reads.  Both use 16-byte chunk
//    swizzles that keep the reads free of bank conflicts.
//  * v_mfma_f32_16x16x128_f8f6f4 as in the NT kernels (D^T = B A^T: a lane holds 4
//    consecutive N columns of one M row); each block's partial is promoted into the FP32
//    accumulators with sa[m] * sb (one B scale per tile and block in the dense forms, four
//    per lane in the K-grouped form).
//  * Epilogue: + C, then bf16 (dense) or FP32 non-temporal (K-grouped; C read before D is
//    written, so C may be D) stores of the valid rows and columns.  A group with no K blocks
//    writes C, or zeros.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

namespace {

// chunk swizzle of the LDS row holding K index k (CH chunks of 16 bytes per row).  A
// transposing read's half-wave covers rows k0 + t and k0 + 32 + t (t = 0..7) at one logical
// chunk: with 128-byte rows two rows share a 256-byte bank line, so rows need distinct
// (k & 1, chunk) pairs, which s = k bits 1, 2, 5 gives; with 256-byte rows every row starts
// on the same bank, so s takes k bits 0, 1, 2, 5.
template <int CH>
__device__ __forceinline__ int kswz(int k)
{
    if constexpr (CH == 8)
        return ((k >> 1) & 3) | ((k >> 3) & 4);
    else
        return (k & 7) | ((k >> 2) & 8);
}

// chunk swizzle of a K-major operand's LDS row r (8 chunks of 16 bytes): r3 | r1 << 1 | r2 << 2,
// the one the NT kernels use
__device__ __forceinline__ int hswz(int r) { return ((r >> 3) & 1) | (r & 2) | (((r >> 2) & 1) << 2); }

// One MFMA operand lane's 32 bytes: four transposing reads (MN-major) or two 16-byte reads
// (K-major).  Valid after lds_wait() and tie().
template <bool MN>
struct Frag;
template <>
struct Frag<true> {
    v2i q[4];
    __device__ __forceinline__ v8i op() const
    {
        return v8i{q[0].x, q[0].y, q[1].x, q[1].y, q[2].x, q[2].y, q[3].x, q[3].y};
    }
    __device__ __forceinline__ void tie_all()
    {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            tie(q[r]);
    }
};
template <>
struct Frag<false> {
    v4i h[2];
    __device__ __forceinline__ v8i op() const
    {
        return v8i{h[0].x, h[0].y, h[0].z, h[0].w, h[1].x, h[1].y, h[1].z, h[1].w};
    }
    __device__ __forceinline__ void tie_all()
    {
        tie(h[0]);
        tie(h[1]);
    }
};

// reads the operand lane of sub-tile S (16 rows or columns) from a slot: MN-major from the
// lane's row base `lo` (read r adds K row offset 8 r), K-major from its two chunks `lo`, `hi`
template <bool MN, int R, int S>
__device__ __forceinline__ void read_frag(Frag<MN> &f, uint32_t lo, uint32_t hi)
{
    if constexpr (MN) {
        f.q[0] = lds_read_tr8_at<0 * 8 * R>(lo);
        f.q[1] = lds_read_tr8_at<1 * 8 * R>(lo);
        f.q[2] = lds_read_tr8_at<2 * 8 * R>(lo);
        f.q[3] = lds_read_tr8_at<3 * 8 * R>(lo);
    } else {
        f.h[0] = lds_read16_at<S * 16 * KBLK>(lo);
        f.h[1] = lds_read16_at<S * 16 * KBLK>(hi);
    }
}

}  // namespace

// KG: the K-grouped form; else dense.  A_MN / B_MN: the operand is stored MN-major.
// (the body is a device function: generic lambdas directly in a kernel template keep the host
// pass from emitting its launch stub)
template <int BM, int BN, int WM, int WN, bool A_MN, bool B_MN, bool KG>
__device__ __forceinline__ void layout_tile(const LayoutArgs &p, int tiles_m, int tiles_n)
{
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int SM = TM / 16, SN = TN / 16;
    constexpr int CHA = BM / 16, CHB = BN / 16;
    static_assert(!A_MN || CHA == 8 || CHA == 16, "MN-major A rows of 128 or 256 bytes");
    static_assert(!B_MN || CHB == 8 || CHB == 16, "MN-major B rows of 128 or 256 bytes");
    static_assert(KG || BN == KBLK, "dense tiles span one 128-column B scale block");
    static_assert(SM % 2 == 0, "partials alternate between two register sets");
    constexpr int A_SLOT = KBLK * BM, B_SLOT = KBLK * BN;
    constexpr int S_SLOT = 1024;  // a block's BM (or BN) scales, 16 bytes per lane of one copy
    // slots: block j in use, j + 1 landed, the rest in flight (four where they fit, else three;
    // a three-slot tile is twice as wide, so one block ahead covers as much time)
    constexpr int NS = 4 * (KBLK * (BM + BN) + 2 * 1024) <= 160 * 1024 ? 4 : 3;
    constexpr int B_BASE = NS * A_SLOT;
    constexpr int SA_BASE = B_BASE + NS * B_SLOT;
    constexpr int SB_BASE = SA_BASE + NS * S_SLOT;
    constexpr int LDS_BYTES = SB_BASE + NS * S_SLOT;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    constexpr int IA = A_SLOT / 1024, IB = B_SLOT / 1024;  // 1 KB copies per block
    static_assert(IA % NW == 0 && IB % NW == 0, "copies must split evenly over the waves");
    constexpr int CA = IA / NW, CB = IB / NW, MAXI = CA + CB;
    static_assert((NS - 1) * (MAXI + 2) < 64, "outstanding copies must fit vmcnt");

    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    DG_LDS uint8_t *ldsp = (DG_LDS uint8_t *)lds;
    const uint32_t lds_base = (uint32_t)(uintptr_t)ldsp;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = (wave / WN) * TM, wn = (wave % WN) * TN;
    const int M = p.m, N = p.n, K = p.k;
    const int64_t ld = p.ld_sfa;
    const int KBT = K / KBLK;  // K blocks of the whole K axis (all groups)

    // ---- the tile.  Workgroup ids go round-robin over the 8 XCDs: XCD x runs ids x, x+8, ...
    // Dense: the tiles, in raster order, are cut into 8 consecutive chunks, and XCD x runs
    // chunk x, so the tiles in flight on one XCD are raster neighbours (4 rows of M by 8
    // columns of N) that share A and B panels in its L2; ids past the chunk (when 8 does not
    // divide the tile count) end at once.  K-grouped: tile id = workgroup id, so every XCD runs
    // an eighth of every group whatever the groups' K extents.  (Cutting each group into such
    // chunks fetched 2.7 GB from memory per routed wgrad call instead of 7.6 GB but ran 4%
    // slower: this kernel is bound inside the CU.)
    const int per_g = tiles_m * tiles_n;
    int g, t;
    if constexpr (KG) {
        g = blockIdx.x / per_g;
        t = blockIdx.x - g * per_g;
    } else {
        const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
        const int lo = (int)(((int64_t)x * per_g) >> 3);
        const int len = (int)((((int64_t)x + 1) * per_g) >> 3) - lo;
        if (len == 0)
            return;
        if (i >= len)
            return;
        g = 0;
        t = lo + i;
    }
    int tm, tn;
    raster(t, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kb_first = KG ? p.kb_start[g] : 0;
    const int nkb = KG ? p.kb_start[g + 1] - kb_first : KBT;

    // ---- copies.  Copy ci of a block is wave + c * NW; lane l writes bytes [16 l, 16 l + 16)
    // of its 1 KB.  MN-major: LDS row = K index (R = 1024 / width rows per copy), row
    // R ci + l / CH, physical chunk l % CH holding logical chunk (l % CH) ^ s(row).  K-major:
    // LDS row = operand row (8 per copy), row 8 ci + l / 8, physical chunk l % 8 holding
    // logical chunk (l % 8) ^ h(row).  The lane fetches the logical chunk.
    auto lane_off = [&](auto MN, auto CH, int ci, int pitch) -> uint32_t {
        if constexpr (decltype(MN)::value) {
            constexpr int ch = decltype(CH)::value;
            const int k = (1024 / (16 * ch)) * ci + lane / ch;
            return (uint32_t)(k * pitch + 16 * ((lane % ch) ^ kswz<ch>(k)));
        } else {
            const int r = 8 * ci + (lane >> 3);
            return (uint32_t)(r * pitch + 16 * ((lane & 7) ^ hswz(r)));
        }
    };
    constexpr auto A_MNc = std::integral_constant<bool, A_MN>{};
    constexpr auto B_MNc = std::integral_constant<bool, B_MN>{};
    constexpr auto CHAc = std::integral_constant<int, CHA>{};
    constexpr auto CHBc = std::integral_constant<int, CHB>{};
    uint32_t voa[CA], vob[CB];
#pragma unroll
    for (int c = 0; c < CA; ++c)
        voa[c] = lane_off(A_MNc, CHAc, wave + c * NW, A_MN ? M : K);
#pragma unroll
    for (int c = 0; c < CB; ++c)
        vob[c] = lane_off(B_MNc, CHBc, wave + c * NW, B_MN ? N : K);
    // block j of the tile's K run into slot s; blocks past the last read empty resources
    // (zeros, no memory access), which keeps the count of copies per block constant.  Every
    // resource ends at the last valid byte of its operand (rows past M or N read zeros).
    auto issue_block = [&](int j, int s) {
        const bool in = j < nkb;
        const int kb = kb_first + (in ? j : 0);
        const int64_t ka = (int64_t)kb * KBLK;
        __amdgpu_buffer_rsrc_t ra, rb;
        uint32_t soa = 0, sob = 0;
        if constexpr (A_MN) {
            ra = make_rsrc(p.a + ka * M + m0, in ? ((int64_t)K - ka) * M - m0 : 0);
        } else {
            ra = make_rsrc(p.a + (int64_t)m0 * K, in ? (int64_t)(M - m0) * K : 0);
            soa = (uint32_t)ka;
        }
        if constexpr (B_MN) {
            rb = make_rsrc(p.b + ka * N + n0, in ? ((int64_t)K - ka) * N - n0 : 0);
        } else {
            rb = make_rsrc(p.b + (int64_t)n0 * K, in ? (int64_t)(N - n0) * K : 0);
            sob = (uint32_t)ka;
        }
#pragma unroll
        for (int c = 0; c < CA; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (DG_LDS void *)(ldsp + s * A_SLOT + (wave + c * NW) * 1024), 16, voa[c], soa,
                0, 0);
#pragma unroll
        for (int c = 0; c < CB; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (DG_LDS void *)(ldsp + B_BASE + s * B_SLOT + (wave + c * NW) * 1024), 16,
                vob[c], sob, 0, 0);
        if (wave == 0) {
            // A scales: row kb of the MN-major [K/128][ld] array, the tile's BM columns.  B
            // scales: K-grouped, row kb of [K/128][N]; dense, the tile's 128x128 block
            // [n0/128][kb] (lane 0's word; the others read on along the row)
            const __amdgpu_buffer_rsrc_t rsa = make_rsrc(
                p.sfa + (int64_t)kb * ld + m0, in ? ((int64_t)(KBT - kb) * ld - m0) * 4 : 0);
            __amdgpu_buffer_rsrc_t rsb;
            if constexpr (KG) {
                rsb = make_rsrc(p.sfb + (int64_t)kb * N + n0,
                                in ? ((int64_t)(KBT - kb) * N - n0) * 4 : 0);
            } else {
                const int nb = n0 / KBLK, NB = (N + KBLK - 1) / KBLK;
                rsb = make_rsrc(p.sfb + (int64_t)nb * KBT + kb,
                                in ? ((int64_t)(NB - nb) * KBT - kb) * 4 : 0);
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsa, (DG_LDS void *)(ldsp + SA_BASE + s * S_SLOT), 16, (uint32_t)lane * 16u, 0, 0,
                0);
            if constexpr (KG)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsb, (DG_LDS void *)(ldsp + SB_BASE + s * S_SLOT), 16, (uint32_t)lane * 16u, 0,
                    0, 0);
            else  // (4-byte words: the block's scale need not be 16-byte aligned)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsb, (DG_LDS void *)(ldsp + SB_BASE + s * S_SLOT), 4, (uint32_t)lane * 4u, 0,
                    0, 0);
        }
    };
    // the next block's copies have landed (only those of the block after it may be in flight)
    auto wait_next_block = [&]() {
        if (wave == 0)
            wait_vm<(NS - 3) * (MAXI + 2)>();
        else
            wait_vm<(NS - 3) * MAXI>();
    };
    // (prologue: the first block's, with the next two in flight)
    auto wait_first_block = [&]() {
        if (wave == 0)
            wait_vm<(NS - 2) * (MAXI + 2)>();
        else
            wait_vm<(NS - 2) * MAXI>();
    };

    // ---- fragment offsets.  MN-major: lane (fr, fg), read r, addresses K row
    // 32 fg + 8 r + fr / 2 at byte 8 (fr & 1) of the sub-tile's chunk and receives K rows
    // 32 fg + 8 r .. + 7 of column fr (r adds 8 r: K row bits 3, 4, which s does not use).
    // K-major: row fr of the sub-tile, chunks 2 fg and 2 fg + 1.
    const int fr = lane & 15, fg = lane >> 4;
    auto frag_off = [&](auto MN, auto CH, int w0, int width, bool second) -> uint32_t {
        if constexpr (decltype(MN)::value) {
            constexpr int ch = decltype(CH)::value;
            const int k = 32 * fg + (fr >> 1);
            return (uint32_t)(k * width + (((w0 >> 4) ^ kswz<ch>(k)) << 4) + 8 * (fr & 1));
        } else {
            const int r = w0 + fr;
            return (uint32_t)(r * KBLK + (((2 * fg + (second ? 1 : 0)) ^ hswz(r)) << 4));
        }
    };
    // MN-major: one base per sub-tile (the swizzle mixes the sub-tile index); K-major: one
    // pair for all sub-tiles (the sub-tile adds 16 rows, which h does not see)
    uint32_t fa_lo[A_MN ? SM : 1], fa_hi, fb_lo[B_MN ? SN : 1], fb_hi;
#pragma unroll
    for (int i = 0; i < (A_MN ? SM : 1); ++i)
        fa_lo[i] = lds_base + frag_off(A_MNc, CHAc, wm + 16 * i, BM, false);
    fa_hi = lds_base + frag_off(A_MNc, CHAc, wm, BM, true);
#pragma unroll
    for (int jj = 0; jj < (B_MN ? SN : 1); ++jj)
        fb_lo[jj] = lds_base + B_BASE + frag_off(B_MNc, CHBc, wn + 16 * jj, BN, false);
    fb_hi = lds_base + B_BASE + frag_off(B_MNc, CHBc, wn, BN, true);
    const uint32_t sa_off = lds_base + SA_BASE + (uint32_t)(wm + fr) * 4;
    const uint32_t sb_off = lds_base + SB_BASE + (KG ? (uint32_t)(wn + 4 * fg) * 4 : 0u);

    // Wide tiles (SN >= 4) hold one set of B fragments and scales: the next block's are read
    // after the current block's last MFMA and promotion that use them (registers); narrower
    // ones read the next block's B into a second set during the current block's MFMAs.
    constexpr bool ONE_B = SN >= 4;
    constexpr int NBB = ONE_B ? 1 : 2;
    Frag<A_MN> fa[2][SM];
    Frag<B_MN> fb[NBB][SN];
    float fsa[2][SM];
    v4f fsb[NBB][KG ? SN : 1];  // K-grouped: the lane's four columns
    float fsb1[2];            // dense: the tile's B scale
    // a block's fragments from slot s into register set BUF: the A row sub-tile I (and its
    // scales), or all of B (and its scales)
    auto read_frags_a = [&](auto BUF, int s, auto I) {
        constexpr int bf = decltype(BUF)::value, i = decltype(I)::value;
        const uint32_t ao = (uint32_t)(s * A_SLOT), so = (uint32_t)(s * S_SLOT);
        read_frag<A_MN, BM, i>(fa[bf][i], fa_lo[A_MN ? i : 0] + ao, fa_hi + ao);
        fsa[bf][i] = lds_read4_at<i * 64>(sa_off + so);
    };
    auto read_frags_b = [&](auto BUF, int s) {
        constexpr int bf = ONE_B ? 0 : decltype(BUF)::value;
        const uint32_t bo = (uint32_t)(s * B_SLOT), so = (uint32_t)(s * S_SLOT);
        static_for<SN>([&](auto J) {
            constexpr int jj = decltype(J)::value;
            read_frag<B_MN, BN, jj>(fb[bf][jj], fb_lo[B_MN ? jj : 0] + bo, fb_hi + bo);
            if constexpr (KG)
                fsb[bf][jj] = lds_read16f_at<jj * 64>(sb_off + so);
        });
        if constexpr (!KG)
            fsb1[decltype(BUF)::value] = lds_read4_at<0>(sb_off + so);
    };
    auto read_frags = [&](auto BUF, int s) {
        static_for<SM>([&](auto I) { read_frags_a(BUF, s, I); });
        read_frags_b(BUF, s);
    };
    auto tie_frags = [&](auto BUF) {
        constexpr int bf = decltype(BUF)::value, bb = ONE_B ? 0 : bf;
#pragma unroll
        for (int i = 0; i < SM; ++i) {
            fa[bf][i].tie_all();
            tie(fsa[bf][i]);
        }
#pragma unroll
        for (int jj = 0; jj < SN; ++jj)
            fb[bb][jj].tie_all();
        if constexpr (KG) {
#pragma unroll
            for (int jj = 0; jj < SN; ++jj)
                tie(fsb[bb][jj]);
        } else {
            tie(fsb1[bf]);
        }
    };

    v4f acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int jj = 0; jj < SN; ++jj)
            acc[i][jj] = v4f{0.f, 0.f, 0.f, 0.f};
    // partials of row step i go to set i % 2; step i promotes step i - 1's
    v4f pend[2][SN];
    auto promote = [&](auto BUF, auto I) {
        constexpr int bf = decltype(BUF)::value, i = decltype(I)::value;
        if constexpr (KG) {
#pragma unroll
            for (int jj = 0; jj < SN; ++jj) {
                acc[i][jj] += pend[i % 2][jj] * (fsa[bf][i] * fsb[ONE_B ? 0 : bf][jj]);
                asm volatile("" : "+v"(acc[i][jj]));
            }
        } else {
            const float sc = fsa[bf][i] * fsb1[bf];
#pragma unroll
            for (int jj = 0; jj < SN; ++jj) {
                acc[i][jj] += pend[i % 2][jj] * sc;
                asm volatile("" : "+v"(acc[i][jj]));
            }
        }
    };

    // block j of the tile's K run: its fragments are in register set BUF (read during block
    // j - 1); block j + 1's are read into the other set during this block's MFMAs, so the
    // LDS reads overlap them, which needs block j + 1 landed at this block's start: the
    // copies run three blocks ahead, into four slots
    auto do_block = [&](auto BUF, int j) {
        constexpr int bf = decltype(BUF)::value;
        constexpr auto OTHER = std::integral_constant<int, 1 - bf>{};
        // block j + 1 has landed everywhere, and every wave is done with block j - 1's slot,
        // which takes block j + 3
        wait_next_block();
        bare_barrier();
        issue_block(j + NS - 1, (j + NS - 1) % NS);
        lds_wait();
        tie_frags(BUF);
        const bool more = j + 1 < nkb;
        const int sn = (j + 1) % NS;
        if constexpr (!ONE_B) {
            if (more)
                read_frags_b(OTHER, sn);
        }
        static_for<SM>([&](auto I) {
            constexpr int i = decltype(I)::value;
            const v8i av = fa[bf][i].op();
#pragma unroll
            for (int jj = 0; jj < SN; ++jj)
                pend[i % 2][jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    fb[ONE_B ? 0 : bf][jj].op(), av, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
            if constexpr (i > 0)
                promote(BUF, std::integral_constant<int, i - 1>{});
            if (more)
                read_frags_a(OTHER, sn, I);
        });
        promote(BUF, std::integral_constant<int, SM - 1>{});
        // one B set: the next block's B once this block's last MFMAs and promotions are issued
        if constexpr (ONE_B) {
            if (more)
                read_frags_b(OTHER, sn);
        }
    };

    // ---- prologue and K loop
#pragma unroll
    for (int d = 0; d < NS - 1; ++d)
        issue_block(d, d);
    wait_first_block();
    bare_barrier();
    constexpr auto B0 = std::integral_constant<int, 0>{};
    constexpr auto B1 = std::integral_constant<int, 1>{};
    if (nkb > 0)
        read_frags(B0, 0);
    for (int j = 0; j < nkb; j += 2) {
        do_block(B0, j);
        if (j + 1 < nkb)
            do_block(B1, j + 1);
    }
    // every copy (also those past the last block) has landed before the workgroup ends
    wait_vm<0>();
    lds_wait();

    // ---- epilogue: + C, stores of the valid rows and columns
#pragma unroll
    for (int i = 0; i < SM; ++i) {
        const int m = m0 + wm + 16 * i + fr;
#pragma unroll
        for (int jj = 0; jj < SN; ++jj) {
            const int n = n0 + wn + 16 * jj + 4 * fg;
            if (m < M && n < N) {
                const int64_t o = (int64_t)g * M * N + (int64_t)m * N + n;
                v4f v = acc[i][jj];
                if (p.c)
                    v += *reinterpret_cast<const v4f *>(p.c + o);
                if constexpr (KG)
                    __builtin_nontemporal_store(v, reinterpret_cast<v4f *>((float *)p.d + o));
                else
                    store_bf16x4((uint16_t *)p.d + o, v);
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, bool A_MN, bool B_MN, bool KG>
__global__ __launch_bounds__(64 * WM * WN) void dg_layout_kernel(LayoutArgs p, int tiles_m,
                                                                  int tiles_n)
{
    layout_tile<BM, BN, WM, WN, A_MN, B_MN, KG>(p, tiles_m, tiles_n);
}

namespace {
constexpr int LY_BM = 128, LY_BN = 128, LY_WM = 2, LY_WN = 4;
// K-grouped tiles are 128 x 256 (B in one register set; three slots): 256 columns per tile
// halve the copies and LDS reads per MFMA of the 128 x 128 tile.  DG_KG_TILE_N=128 selects
// the narrower tile (tests).
int kg_tile_n()
{
    const char *e = getenv("DG_KG_TILE_N");
    return (e && atoi(e) == 128) ? 128 : 256;
}
int tile_n(int layout) { return layout == LAYOUT_KGROUPED_TN ? kg_tile_n() : LY_BN; }
}  // namespace

int64_t layout_grid_size(int layout, const LayoutArgs &a)
{
    const int bn = tile_n(layout);
    const int64_t tiles_m = (a.m + LY_BM - 1) / LY_BM, tiles_n = (a.n + bn - 1) / bn;
    const int64_t per_g = tiles_m * tiles_n;
    if (layout == LAYOUT_KGROUPED_TN)
        return per_g * a.num_groups;  // one workgroup per tile of every group
    if (per_g > (int64_t)1 << 27)
        return -1;  // chunk bounds are computed in 32 bits
    return 8 * ((per_g + 7) / 8);     // 8 XCDs x the longest chunk
}

hipError_t launch_layout(int layout, const LayoutArgs &a, hipStream_t stream)
{
    const int bn = tile_n(layout);
    const int tiles_m = (a.m + LY_BM - 1) / LY_BM, tiles_n = (a.n + bn - 1) / bn;
    const int64_t grid = layout_grid_size(layout, a);
    if (grid <= 0 || grid > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const dim3 g((unsigned)grid), b(64 * LY_WM * LY_WN);
#define DG_LAUNCH_LAYOUT(AMN, BMN, KGR)                                                         \
    hipLaunchKernelGGL((dg_layout_kernel<LY_BM, LY_BN, LY_WM, LY_WN, AMN, BMN, KGR>), g, b, 0,   \
                       stream, a, tiles_m, tiles_n)
    switch (layout) {
    case LAYOUT_KGROUPED_TN:
        if (bn == 256)
            hipLaunchKernelGGL((dg_layout_kernel<LY_BM, 256, LY_WM, LY_WN, true, true, true>), g, b,
                               0, stream, a, tiles_m, tiles_n);
        else
            DG_LAUNCH_LAYOUT(true, true, true);
        break;
    case LAYOUT_NN:
        DG_LAUNCH_LAYOUT(false, true, false);
        break;
    case LAYOUT_TN:
        DG_LAUNCH_LAYOUT(true, true, false);
        break;
    case LAYOUT_TT:
        DG_LAUNCH_LAYOUT(true, false, false);
        break;
    case LAYOUT_NT:
        DG_LAUNCH_LAYOUT(false, false, false);
        break;
    default:
        return hipErrorInvalidValue;
    }
#undef DG_LAUNCH_LAYOUT
    return hipGetLastError();
}

// ---- byte transpose y[c][r] = x[r][c] (x: rows x cols, pitch cols; y: cols x rows, pitch
// rows) of e4m3 operands, for the dense NN/TN/TT calls: their MN-major operands become
// K-major, which the NT kernels take.  rows % 128 == 0 and cols % 16 == 0.  A workgroup moves
// one 128 x 128 byte tile: 16-byte loads of whole 128-byte row segments into a padded LDS
// tile (144-byte rows), then ds_read_b64_tr_b8, whose 16-lane groups turn an 8 x 16 byte
// block into 16 lanes of 8 consecutive row bytes; two such reads give a lane 16 bytes of one
// output row.  Wave w writes output rows 32 w .. 32 w + 31, each row's 128 bytes as two
// 64-byte halves in consecutive rounds.  So every 128-byte line of x and of y is read or
// written by one workgroup: workgroups are dealt round-robin over the XCDs, whose L2s are
// separate, and a line split between two workgroups is fetched twice.
// One launch moves up to two operands (A and B of the TN layout): workgroups [0, p0.tiles)
// transpose p0, the rest p1.
struct U8Transpose {
    const uint8_t *x;
    uint8_t *y;
    int rows, cols, tiles_c, tiles;
};

constexpr int TR_T = 128;  // tile side in bytes

__global__ __launch_bounds__(256) void dg_transpose_u8_kernel(U8Transpose p0, U8Transpose p1)
{
    constexpr int PITCH = TR_T + 16;
    __shared__ __attribute__((aligned(16))) uint8_t tile[TR_T * PITCH];
    const bool second = (int)blockIdx.x >= p0.tiles;
    const int bid = (int)blockIdx.x - (second ? p0.tiles : 0);
    const uint8_t *__restrict__ x = second ? p1.x : p0.x;
    uint8_t *__restrict__ y = second ? p1.y : p0.y;
    const int rows = second ? p1.rows : p0.rows, cols = second ? p1.cols : p0.cols;
    const int tiles_c = second ? p1.tiles_c : p0.tiles_c;
    const int tid = threadIdx.x;
    const int r0 = (bid / tiles_c) * TR_T, c0 = (bid % tiles_c) * TR_T;
    uint4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // rows 32 q + tid / 8, 16-byte chunk tid % 8
        const int r = 32 * q + (tid >> 3), c = (tid & 7) * 16;
        v[q] = make_uint4(0, 0, 0, 0);
        if (c0 + c < cols)
            v[q] = *reinterpret_cast<const uint4 *>(x + (int64_t)(r0 + r) * cols + c0 + c);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint4 *>(tile + (32 * q + (tid >> 3)) * PITCH + (tid & 7) * 16) = v[q];
    __syncthreads();
    const uint32_t base = (uint32_t)(uintptr_t)(DG_LDS uint8_t *)tile;
    const int lane = tid & 63, w = tid >> 6, g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        // 16-column block cb of the tile, 16-row chunk rc: lane j holds 16 consecutive bytes of
        // output row c0 + 16 cb + j (the four lane groups: four consecutive chunks)
        const int cb = 2 * w + (q >> 1), rc = 4 * (q & 1) + g;
        const uint32_t addr =
            base + (uint32_t)((16 * rc + (j >> 1)) * PITCH + 16 * cb + 8 * (j & 1));
        v2i lo = lds_read_tr8_at<0>(addr);
        v2i hi = lds_read_tr8_at<8 * PITCH>(addr);
        lds_wait();
        tie(lo);
        tie(hi);
        const int c = c0 + 16 * cb + j;  // output row
        if (c < cols)
            *reinterpret_cast<uint4 *>(y + (int64_t)c * rows + r0 + 16 * rc) =
                make_uint4((uint32_t)lo.x, (uint32_t)lo.y, (uint32_t)hi.x, (uint32_t)hi.y);
    }
}

hipError_t launch_transpose_u8(const void *x0, void *y0, int rows0, int cols0, const void *x1,
                               void *y1, int rows1, int cols1, hipStream_t stream)
{
    U8Transpose p[2] = {{(const uint8_t *)x0, (uint8_t *)y0, rows0, cols0, 1, 0},
                        {(const uint8_t *)x1, (uint8_t *)y1, rows1, cols1, 1, 0}};
    int64_t grid = 0;
    for (U8Transpose &t : p) {
        if (!t.x || t.rows <= 0 || t.cols <= 0)
            continue;  // no job
        if (t.rows % TR_T != 0 || t.cols % 16 != 0)
            return hipErrorInvalidValue;
        t.tiles_c = (t.cols + TR_T - 1) / TR_T;
        const int64_t tiles = (int64_t)(t.rows / TR_T) * t.tiles_c;
        if (tiles > 0x3fffffff)
            return hipErrorInvalidConfiguration;
        t.tiles = (int)tiles;
        grid += tiles;
    }
    if (grid == 0)
        return hipSuccess;
    if (p[0].tiles == 0)
        std::swap(p[0], p[1]);
    hipLaunchKernelGGL(dg_transpose_u8_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p[0],
                       p[1]);
    return hipGetLastError();
}

}  // namespace dg
