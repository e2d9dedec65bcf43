// K-grouped TN form of the fine-grained-scaled FP8 GEMM, the MoE weight gradient
// (pt.news.hada.io, "GEMM denso e grouped": grouping on the K axis for the backward pass of
// MoE weights, M and N fixed; "Interface GEMM e restrições de layout": D = C + A @ B, the TN
// memory layout).  For each group g, over its run of K (the expert's tokens):
//     D[g, m, n] = C[g, m, n] + sum over its K blocks kb of
//                  sfa[kb, m] * sfb[kb, n] * sum_{k in kb} A[k, m] * B[k, n]
// A is stored [K_total, M] and B [K_total, N] (both token-major), D and C are FP32 [G, M, N].
//
// Design:
//  * One workgroup per 128 x 128 tile of one group; eight waves (2 x 4), wave tile 64 x 32.
//    Tiles go round-robin to the XCDs, so each gets an equal share of every group whatever
//    the groups' K extents, rastered within a group.
//  * Per K block the tile needs 128 K rows of BM bytes of A and of BN bytes of B.  They are
//    staged whole by direct-to-LDS buffer copies (1 KB per wave instruction), two blocks
//    ahead, into three slots: block j+2 refills block j-1's slot, which every wave has left
//    once it is past block j-1's end barrier, so one barrier per block suffices.
//  * The LDS rows are K indices.  An MFMA operand lane needs 32 consecutive K values of one
//    column; ds_read_b64_tr_b8 delivers 8 of them per read (see dg_device.h), so a 16-column
//    fragment is four transposing reads.  16-byte chunk c of row k sits at chunk c ^ s(k),
//    with s chosen so that the 16 rows one half-wave reads land on distinct banks.
//  * v_mfma_f32_16x16x128_f8f6f4 as in the NT kernels (D^T = B A^T: a lane holds 4
//    consecutive N columns of one M row); each block's partial is promoted into the FP32
//    accumulators with sa[m] * sb[n] (one A scale per lane, four B scales per lane).
//  * Epilogue: + C (read before D is written, so C may be D itself), FP32 non-temporal
//    stores of the valid rows and columns.  A group with no K blocks writes C (or zeros).
#include <hip/hip_runtime.h>
#include <stdint.h>

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

}  // namespace

// (the body is a device function: generic lambdas directly in a kernel template keep the host
// pass from emitting its launch stub)
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void kgrouped_tile(const KGroupedArgs &p, int tiles_m, int tiles_n)
{
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int SM = TM / 16, SN = TN / 16;
    constexpr int CHA = BM / 16, CHB = BN / 16;
    static_assert((CHA == 8 || CHA == 16) && (CHB == 8 || CHB == 16), "rows of 128 or 256 B");
    static_assert(SM % 2 == 0, "partials alternate between two register sets");
    constexpr int A_SLOT = KBLK * BM, B_SLOT = KBLK * BN;
    constexpr int S_SLOT = 1024;  // a block's BM (or BN) scales, 16 bytes per lane of one copy
    constexpr int NS = 3;
    constexpr int B_BASE = NS * A_SLOT;
    constexpr int SA_BASE = B_BASE + NS * B_SLOT;
    constexpr int SB_BASE = SA_BASE + NS * S_SLOT;
    constexpr int LDS_BYTES = SB_BASE + NS * S_SLOT;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    constexpr int IA = A_SLOT / 1024, IB = B_SLOT / 1024;  // 1 KB copies per block
    static_assert(IA % NW == 0 && IB % NW == 0, "copies must split evenly over the waves");
    constexpr int CA = IA / NW, CB = IB / NW, MAXI = CA + CB;
    constexpr int RA = 1024 / BM, RB = 1024 / BN;  // K rows per copy
    static_assert(2 * (MAXI + 2) < 64, "outstanding copies must fit vmcnt");

    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    DG_LDS uint8_t *ldsp = (DG_LDS uint8_t *)lds;
    const uint32_t lds_base = (uint32_t)(uintptr_t)ldsp;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = (wave / WN) * TM, wn = (wave % WN) * TN;
    const int M = p.m, N = p.n;

    // ---- the tile: workgroup ids go round-robin over the 8 XCDs, so XCD x runs tiles x, x+8,
    // ...: an eighth of every group.  (Contiguous ranges per XCD would keep more panel reuse in
    // each L2, but groups differ in K, and a range would give one XCD the largest group's
    // tiles.)  Within a group the raster keeps the tiles in flight on one XCD on the same
    // rows of M.
    const int t = blockIdx.x;
    const int per_g = tiles_m * tiles_n;
    const int g = t / per_g;
    int tm, tn;
    raster(t - g * per_g, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kb_first = p.kb_start[g];
    const int nkb = p.kb_start[g + 1] - kb_first;
    const int KBT = p.k_total / KBLK;

    // ---- copies.  Copy ci of a block (ci = wave + c * NW) holds K rows [R ci, R ci + R); lane
    // l writes bytes [16 l, 16 l + 16) of it, i.e. row R ci + l / CH, physical chunk l % CH,
    // which must hold logical chunk (l % CH) ^ s(row): the lane fetches that one.
    uint32_t voa[CA], vob[CB];
#pragma unroll
    for (int c = 0; c < CA; ++c) {
        const int k = RA * (wave + c * NW) + lane / CHA;
        voa[c] = (uint32_t)(k * M + 16 * ((lane % CHA) ^ kswz<CHA>(k)));
    }
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        const int k = RB * (wave + c * NW) + lane / CHB;
        vob[c] = (uint32_t)(k * N + 16 * ((lane % CHB) ^ kswz<CHB>(k)));
    }
    // block j of the group into slot s; blocks past the group's last read empty resources
    // (zeros, no memory access), which keeps the count of copies per block constant
    auto issue_block = [&](int j, int s) {
        const bool in = j < nkb;
        const int kb = kb_first + (in ? j : 0);
        const int64_t ka = (int64_t)kb * KBLK;
        const __amdgpu_buffer_rsrc_t ra =
            make_rsrc(p.a + ka * M + m0, in ? ((int64_t)p.k_total - ka) * M - m0 : 0);
        const __amdgpu_buffer_rsrc_t rb =
            make_rsrc(p.b + ka * N + n0, in ? ((int64_t)p.k_total - ka) * N - n0 : 0);
#pragma unroll
        for (int c = 0; c < CA; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (DG_LDS void *)(ldsp + s * A_SLOT + (wave + c * NW) * 1024), 16, voa[c], 0,
                0, 0);
#pragma unroll
        for (int c = 0; c < CB; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (DG_LDS void *)(ldsp + B_BASE + s * B_SLOT + (wave + c * NW) * 1024), 16,
                vob[c], 0, 0, 0);
        if (wave == 0) {
            const __amdgpu_buffer_rsrc_t rsa = make_rsrc(
                p.sfa + (int64_t)kb * M + m0, in ? ((int64_t)(KBT - kb) * M - m0) * 4 : 0);
            const __amdgpu_buffer_rsrc_t rsb = make_rsrc(
                p.sfb + (int64_t)kb * N + n0, in ? ((int64_t)(KBT - kb) * N - n0) * 4 : 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsa, (DG_LDS void *)(ldsp + SA_BASE + s * S_SLOT), 16, (uint32_t)lane * 16u, 0, 0,
                0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsb, (DG_LDS void *)(ldsp + SB_BASE + s * S_SLOT), 16, (uint32_t)lane * 16u, 0, 0,
                0);
        }
    };
    // the next block's copies have landed (only those of the block after it may be in flight)
    auto wait_next_block = [&]() {
        if (wave == 0)
            wait_vm<MAXI + 2>();
        else
            wait_vm<MAXI>();
    };

    // ---- fragments.  Lane (fr, fg) reads, for read r, row 32 fg + 8 r + fr / 2 at byte
    // 8 (fr & 1) of the sub-tile's 16-byte chunk, and receives K rows 32 fg + 8 r .. + 7 of
    // column fr: the four reads give the 32 K values of its MFMA operand lane.
    const int fr = lane & 15, fg = lane >> 4;
    const int k_lane = 32 * fg + (fr >> 1);  // r adds 8 r: bits 3, 4, which s does not use
    uint32_t fa_off[SM], fb_off[SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
        fa_off[i] = lds_base + (uint32_t)(k_lane * BM + ((((wm >> 4) + i) ^ kswz<CHA>(k_lane)) << 4) +
                                          8 * (fr & 1));
#pragma unroll
    for (int jj = 0; jj < SN; ++jj)
        fb_off[jj] = lds_base + B_BASE +
                     (uint32_t)(k_lane * BN + ((((wn >> 4) + jj) ^ kswz<CHB>(k_lane)) << 4) +
                                8 * (fr & 1));
    const uint32_t sa_off = lds_base + SA_BASE + (uint32_t)(wm + fr) * 4;
    const uint32_t sb_off = lds_base + SB_BASE + (uint32_t)(wn + 4 * fg) * 4;

    v2i fa[2][SM][4], fb[2][SN][4];
    float fsa[2][SM];
    v4f fsb[2][SN];
    auto read_frags = [&](auto BUF, int s) {
        constexpr int bf = decltype(BUF)::value;
        const uint32_t ao = (uint32_t)(s * A_SLOT), bo = (uint32_t)(s * B_SLOT);
        const uint32_t so = (uint32_t)(s * S_SLOT);
        static_for<SM>([&](auto I) {
            constexpr int i = decltype(I)::value;
            fa[bf][i][0] = lds_read_tr8_at<0 * 8 * BM>(fa_off[i] + ao);
            fa[bf][i][1] = lds_read_tr8_at<1 * 8 * BM>(fa_off[i] + ao);
            fa[bf][i][2] = lds_read_tr8_at<2 * 8 * BM>(fa_off[i] + ao);
            fa[bf][i][3] = lds_read_tr8_at<3 * 8 * BM>(fa_off[i] + ao);
            fsa[bf][i] = lds_read4_at<i * 64>(sa_off + so);
        });
        static_for<SN>([&](auto J) {
            constexpr int jj = decltype(J)::value;
            fb[bf][jj][0] = lds_read_tr8_at<0 * 8 * BN>(fb_off[jj] + bo);
            fb[bf][jj][1] = lds_read_tr8_at<1 * 8 * BN>(fb_off[jj] + bo);
            fb[bf][jj][2] = lds_read_tr8_at<2 * 8 * BN>(fb_off[jj] + bo);
            fb[bf][jj][3] = lds_read_tr8_at<3 * 8 * BN>(fb_off[jj] + bo);
            fsb[bf][jj] = lds_read16f_at<jj * 64>(sb_off + so);
        });
    };
    auto tie_frags = [&](auto BUF) {
        constexpr int bf = decltype(BUF)::value;
#pragma unroll
        for (int i = 0; i < SM; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                tie(fa[bf][i][r]);
            tie(fsa[bf][i]);
        }
#pragma unroll
        for (int jj = 0; jj < SN; ++jj) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                tie(fb[bf][jj][r]);
            tie(fsb[bf][jj]);
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
#pragma unroll
        for (int jj = 0; jj < SN; ++jj) {
            acc[i][jj] += pend[i % 2][jj] * (fsa[bf][i] * fsb[bf][jj]);
            asm volatile("" : "+v"(acc[i][jj]));
        }
    };

    // block j of the group: its fragments are in register set BUF (read, maybe in flight)
    auto do_block = [&](auto BUF, int j) {
        constexpr int bf = decltype(BUF)::value;
        constexpr auto OTHER = std::integral_constant<int, 1 - bf>{};
        issue_block(j + 2, (j + 2) % NS);
        lds_wait();
        tie_frags(BUF);
        static_for<SM>([&](auto I) {
            constexpr int i = decltype(I)::value;
            const v8i av = v8i{fa[bf][i][0].x, fa[bf][i][0].y, fa[bf][i][1].x, fa[bf][i][1].y,
                               fa[bf][i][2].x, fa[bf][i][2].y, fa[bf][i][3].x, fa[bf][i][3].y};
#pragma unroll
            for (int jj = 0; jj < SN; ++jj) {
                const v8i bv = v8i{fb[bf][jj][0].x, fb[bf][jj][0].y, fb[bf][jj][1].x,
                                   fb[bf][jj][1].y, fb[bf][jj][2].x, fb[bf][jj][2].y,
                                   fb[bf][jj][3].x, fb[bf][jj][3].y};
                pend[i % 2][jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bv, av, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
            }
            if constexpr (i > 0)
                promote(BUF, std::integral_constant<int, i - 1>{});
        });
        // block j + 1 has landed everywhere, and every wave is done reading block j
        wait_next_block();
        bare_barrier();
        if (j + 1 < nkb)
            read_frags(OTHER, (j + 1) % NS);
        promote(BUF, std::integral_constant<int, SM - 1>{});
    };

    // ---- prologue and K loop
    issue_block(0, 0);
    issue_block(1, 1);
    wait_next_block();
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
    // every copy (also those past the group's blocks) has landed before the workgroup ends
    wait_vm<0>();
    lds_wait();

    // ---- epilogue: + C, FP32 stores of the valid rows and columns
    const int64_t gbase = (int64_t)g * M * N;
#pragma unroll
    for (int i = 0; i < SM; ++i) {
        const int m = m0 + wm + 16 * i + fr;
#pragma unroll
        for (int jj = 0; jj < SN; ++jj) {
            const int n = n0 + wn + 16 * jj + 4 * fg;
            if (m < M && n < N) {
                const int64_t o = gbase + (int64_t)m * N + n;
                v4f v = acc[i][jj];
                if (p.c)
                    v += *reinterpret_cast<const v4f *>(p.c + o);
                __builtin_nontemporal_store(v, reinterpret_cast<v4f *>(p.d + o));
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void dg_kgrouped_kernel(KGroupedArgs p, int tiles_m,
                                                                    int tiles_n)
{
    kgrouped_tile<BM, BN, WM, WN>(p, tiles_m, tiles_n);
}

namespace {
constexpr int KG_BM = 128, KG_BN = 128, KG_WM = 2, KG_WN = 4;
}

int64_t kgrouped_grid_size(const KGroupedArgs &a)
{
    const int64_t tiles_m = (a.m + KG_BM - 1) / KG_BM, tiles_n = (a.n + KG_BN - 1) / KG_BN;
    return tiles_m * tiles_n * a.num_groups;
}

hipError_t launch_kgrouped(const KGroupedArgs &a, hipStream_t stream)
{
    const int tiles_m = (a.m + KG_BM - 1) / KG_BM, tiles_n = (a.n + KG_BN - 1) / KG_BN;
    const int64_t grid = kgrouped_grid_size(a);
    if (grid <= 0 || grid > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((dg_kgrouped_kernel<KG_BM, KG_BN, KG_WM, KG_WN>), dim3((unsigned)grid),
                       dim3(64 * KG_WM * KG_WN), 0, stream, a, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace dg
