// Fine-grained-scaled FP8 GEMM kernels for CDNA4 (gfx950):  D = C + A @ B.T  (NT layout)
// with one FP32 scale per 1x128 segment of an A row and one per 128x128 block of B, plus
// the contiguous and masked M-grouped forms (DeepGEMM pages: pt.news.hada.io, "Interface
// GEMM e restrições de layout" and "GEMM denso e grouped"; feifmx.com release article,
// two-level accumulation of fine-grained-scaled FP8 products).
//
// Design, per workgroup tile of BM x BN outputs split over WM x WN waves:
//  * K advances one 128-deep block at a time: one v_mfma_f32_16x16x128_f8f6f4 per 16x16
//    sub-tile, so every MFMA result is exactly one scale block's partial sum.
//  * The MFMA is issued as D^T = B_tile x A_tile^T (B fragment as the first operand).  A lane
//    of the 16x16 result then holds four consecutive columns of ONE output row, so the A
//    row-segment scale is a single per-lane float and promoting a partial into the FP32
//    accumulators costs one multiply (sa * sb) plus four FMAs per MFMA.
//  * Every global read of the main loop (A, B, the A scales and the tile's B scales) is a
//    gfx950 direct-to-LDS copy through a buffer resource: nothing in flight targets
//    registers, so the only waits are explicit ones.  A has two LDS slots and B three, each
//    a whole 128-deep K block, so block j+1's copies are in flight while block j is
//    multiplied, with one barrier per K block.  A wave holds its A fragments for the whole
//    block and reads B fragments two sub-tile steps ahead of the MFMAs that use them.
//    Barriers are bare s_barrier (a release fence would wait for every copy in flight).
//  * Dense with C: during the last K blocks each wave loads C for one half of an accumulator
//    column at a time (16-byte buffer loads into registers, hidden behind the MFMAs) and adds
//    it in, so that most of C's HBM read overlaps the main loop; the epilogue adds the rest.
//  * LDS rows are 128 bytes (one K block of one row); the 16-byte chunk c of row r sits at
//    chunk c ^ h(r), h(r) = r3 | r1 << 1 | r2 << 2 (bits of r).  gfx950 serves a ds_read_b128
//    16 lanes at a time and its bank selection hashes higher address bits, so the plain
//    XOR-by-row swizzles still conflict two ways on a 16-row fragment read; this h was chosen
//    by measuring the fragment-read rate of every h built from single row bits (it runs at
//    the conflict-free rate, at every slot base used here).  A copy writes 1 KB contiguously
//    per wave, so the swizzle is applied by choosing which global chunk each lane fetches.
//    Every LDS slot starts on a 4 KB boundary.  Fragment reads are inline-asm
//    ds_read_b128 with explicit lgkmcnt waits, so the compiler never pairs an LDS read with
//    the in-flight copies and drains them.
//  * Workgroup ids are remapped so that each XCD (ids are dealt round-robin over the 8 XCDs)
//    runs a contiguous range of tiles, rastered in groups of 4 M-tiles, so tiles that run
//    together on one XCD share A rows and B columns in that XCD's L2.
//  * Shapes too small to fill the CUs with these tiles go to the split-K streaming kernel
//    (dg_stream.hip) instead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

const TileInfo kTiles[CFG_COUNT] = {
    {256, 224, 512, "256x224w8"},
    {128, 256, 256, "128x256w4"},
    {128, 128, 256, "128x128w4"},
    {64, 32, 256, "64x32w4"},
    {256, 128, 512, "256x128w8"},
    {64, 64, 256, "stream64"},
    {128, 128, 256, "128x128w4d4"},
    {128, 128, 512, "128x128w8d4"},
    {128, 256, 512, "128x256w8"},
};

// True when 8 consecutive rows `stride` bytes apart start in 8 distinct 32-byte bank groups
// of a 256-byte bank period (the 32 lanes of a half fragment write then hit distinct banks).
constexpr bool rows_on_distinct_banks(int stride)
{
    int seen = 0;
    for (int r = 0; r < 8; ++r) {
        const int off = (r * stride) % 256;
        if (off % 32 != 0 || (seen >> (off / 32)) & 1)
            return false;
        seen |= 1 << (off / 32);
    }
    return true;
}

template <int BM, int BN, int WM, int WN, int DEPTH, int MODE>
__device__ __forceinline__ void gemm_tile(const GemmArgs &p, int tiles_m, int tiles_n)
{
    constexpr int NW = WM * WN;
    constexpr int NT = 64 * NW;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int SM = TM / 16, SN = TN / 16;
    constexpr int NBUF = bbuf_count(SN);
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be 16-aligned");
    static_assert(BM % 8 == 0 && BN % 8 == 0 && BM <= 256, "tile shape");
    // LDS: DEPTH A slots (BM rows of one K block), DEPTH + 1 B slots (BN rows of one K
    // block), and per A slot a 1 KB area for its A scales and a 256-byte area for the B scales
    // of the 128-column blocks the tile touches.  Block j + DEPTH is copied while block j is
    // multiplied.  Rows are 128 bytes; 16-byte chunk c of row r sits at chunk c ^ h(r)
    // (header comment).
    static_assert(DEPTH >= 2, "at least one block of look-ahead beyond the next");
    constexpr int A_SLOT = BM * KBLK;
    constexpr int B_SLOT = BN * KBLK;
    constexpr int B_BASE = DEPTH * A_SLOT;
    constexpr int SA_BASE = B_BASE + (DEPTH + 1) * B_SLOT;
    constexpr int SB_BASE = SA_BASE + DEPTH * 1024;
    constexpr int LDS_BYTES = SB_BASE + DEPTH * 256;
    static_assert(A_SLOT % 4096 == 0 && B_SLOT % 4096 == 0, "slots start on 4 KB boundaries");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    constexpr int IA = BM / 8, IB = BN / 8;       // 1 KB copies (8 rows of 128 bytes)
    static_assert(IA % NW == 0, "A copies must split evenly over the waves");
    constexpr int CA = IA / NW;                   // A copies per wave per block
    constexpr int CB = (IB + NW - 1) / NW;        // B copies per wave per block (padded)
    constexpr int MAXI = CA + CB;                 // + wave 0 copies the block's scales (2)
    static_assert(DEPTH * (MAXI + 2) < 64, "outstanding copies must fit vmcnt");

    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    __shared__ int s_flag;
    __shared__ int s_grp[MODE == MODE_CONTIG ? BM : 1];  // contiguous: the tile's row groups

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = (wave / WN) * TM;  // wave's row offset inside the tile
    const int wn = (wave % WN) * TN;  // wave's column offset inside the tile

    const int K = p.k, N = p.n;
    const int KB = K / KBLK;
    const int NB = (N + KBLK - 1) / KBLK;
    const int64_t ld = p.ld_sfa;

    // ---- which tile, which group, which rows are valid
    int t = xcd_remap(blockIdx.x, gridDim.x);
    int tm, tn, g = 0, row_limit;
    const int kb0 = 0, kb1 = KB;
    const uint8_t *A = p.a;
    const float *SFA = p.sfa;
    uint16_t *D = p.d;
    if constexpr (MODE == MODE_MASKED) {
        int per_g = tiles_m * tiles_n;
        g = t / per_g;
        int rem = t - g * per_g;
        tn = rem / tiles_m;
        tm = rem - tn * tiles_m;
        int valid = p.grp[g];
        valid = valid < 0 ? 0 : (valid > p.m ? p.m : valid);
        if (tm * BM >= valid)
            return;
        row_limit = valid;
        A += (int64_t)g * p.m * K;
        SFA += (int64_t)g * KB * ld;
        D += (int64_t)g * p.m * N;
    } else if constexpr (MODE == MODE_CONTIG) {
        raster(t, tiles_m, tiles_n, tm, tn);
        if (tid == 0)
            s_flag = -1;
        __syncthreads();
        for (int i = tid; i < BM; i += NT) {
            int v = p.grp[tm * BM + i];
            s_grp[i] = v;
            if (v >= 0 && v < p.num_groups)
                atomicMax(&s_flag, v);
        }
        __syncthreads();
        g = s_flag;
        if (g < 0)
            return;  // a block of padding rows only
        row_limit = p.m;
    } else {
        raster(t, tiles_m, tiles_n, tm, tn);
        row_limit = p.m;
    }
    const int m0 = tm * BM, n0 = tn * BN;
    // masked form: the wave's row sub-tiles that hold a valid row (the others are never
    // stored, so their MFMAs and promotions are skipped; copies and barriers are not)
    int sm_act = SM;
    if constexpr (MODE == MODE_MASKED) {
        const int v = (row_limit - m0 - wm + 15) >> 4;
        sm_act = __builtin_amdgcn_readfirstlane(v < 0 ? 0 : (v > SM ? SM : v));
    }
    const uint8_t *B = p.b + (int64_t)g * N * K;
    const float *SFB = p.sfb + (int64_t)g * NB * KB;
    const int nkb = kb1 - kb0;

    // ---- copies.  Wave w's copy c < CA of a block is A rows [8q, 8q+8) with q = w + c*NW;
    // copy CA + c is B rows [8q, 8q+8) with q = min(w + c*NW, IB-1) (a wave past the last B
    // rows repeats it: same bytes to the same place); wave 0 also copies the block's A
    // scales.  Lane l of a row copy fetches row 8q + l/8, logical chunk (l & 7) ^ h(row), so
    // the contiguous 1 KB that the copy writes is the swizzled layout; h(row) = (q & 1) ^
    // 2(l >> 4) because row bits 1, 2 are lane bits 4, 5 and row bit 3 is q's bit 0.  Operands are read through buffer resources that
    // end at the last valid row, so rows past it read as zeros (their outputs are never
    // stored); past the last K block the resources are empty and the copies only write
    // zeros into slots nobody reads, which keeps the per-wave copy count constant.
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (int64_t)m0 * K, (int64_t)(row_limit - m0) * K);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (int64_t)n0 * K, (int64_t)(N - n0) * K);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(SFA, (int64_t)KB * ld * 4);
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(SFB, (int64_t)NB * KB * 4);
    // B scales of the tile's 128-column blocks nb_first + lane (lanes past the last block read
    // zeros, never used): one float per lane, 256 bytes per K block
    const int nb_first = n0 / KBLK;
    const uint32_t lane_sfb = (uint32_t)((nb_first + lane) * KB) * 4u;
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(SFA, 0);
    const uint32_t lane_even = (uint32_t)(lane >> 3) * (uint32_t)K +
                               (uint32_t)((((lane & 7) ^ ((lane >> 4) << 1))) << 4);
    const uint32_t lane_sfa = (uint32_t)(m0 + 4 * lane) * 4u;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(DG_LDS uint8_t *)lds;
    DG_LDS uint8_t *ldsp = (DG_LDS uint8_t *)lds;

    // Per-copy lane offsets, fixed for the tile (the K block goes into the scalar offset):
    // copy c's row group q and its lanes' byte offsets.  Held in registers, so issuing a copy
    // costs no vector arithmetic.
    int cq[MAXI];
    uint32_t voff[MAXI];
#pragma unroll
    for (int c = 0; c < MAXI; ++c) {
        cq[c] = c < CA ? wave + c * NW : min(wave + (c - CA) * NW, IB - 1);
        voff[c] = (lane_even ^ (uint32_t)((cq[c] & 1) << 4)) + (uint32_t)(8 * cq[c]) * (uint32_t)K;
        asm volatile("" : "+v"(voff[c]));  // kept, not recomputed at each copy
    }
    // issue copy c (a constant after unrolling) of K block kb into A slot aslot or B slot bslot
    // (a plain int parameter: a generic lambda here keeps the host pass from emitting the
    // kernel's launch stub)
    auto issue_copy = [&](int c, int kb, int aslot, int bslot, __amdgpu_buffer_rsrc_t rA,
                          __amdgpu_buffer_rsrc_t rB) {
        if (c < CA)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rA, (DG_LDS void *)(ldsp + aslot * A_SLOT + cq[c] * 1024), 16, voff[c],
                (uint32_t)kb * KBLK, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rB, (DG_LDS void *)(ldsp + B_BASE + bslot * B_SLOT + cq[c] * 1024), 16, voff[c],
                (uint32_t)kb * KBLK, 0, 0);
    };
    auto issue_scales = [&](int kb, int aslot, __amdgpu_buffer_rsrc_t rS,
                            __amdgpu_buffer_rsrc_t rSB) {
        if (wave == 0) {
            uint32_t vo = lane_sfa;
            asm volatile("" : "+v"(vo));
            vo += (uint32_t)((int64_t)kb * ld * 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rS, (DG_LDS void *)(ldsp + SA_BASE + aslot * 1024), 16, vo, 0, 0, 0);
            uint32_t vb = lane_sfb;
            asm volatile("" : "+v"(vb));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rSB, (DG_LDS void *)(ldsp + SB_BASE + aslot * 256), 4, vb, (uint32_t)kb * 4u, 0,
                0);
        }
    };
    // wait until the next block's copies have landed (those of the DEPTH - 1 blocks after it
    // may still be in flight)
    auto wait_older_copies = [&]() {
        if (wave == 0)
            wait_vm<(DEPTH - 1) * (MAXI + 2)>();
        else
            wait_vm<(DEPTH - 1) * MAXI>();
    };

    // per-lane fragment offsets inside a slot: lanes 16g..16g+15 hold K bytes [32g, 32g+32) of
    // 16 consecutive rows, i.e. logical chunks 2g and 2g+1
    const int fr = lane & 15;
    const int fg = lane >> 4;
    const int fh = ((fr >> 3) & 1) | (fr & 2) | (((fr >> 2) & 1) << 2);  // h(fr)
    const uint32_t f_lo = (uint32_t)(fr * KBLK + (((2 * fg) ^ fh) << 4));
    const uint32_t f_hi = (uint32_t)(fr * KBLK + (((2 * fg + 1) ^ fh) << 4));
    const uint32_t a_lo = lds_base + (uint32_t)(wm * KBLK) + f_lo;
    const uint32_t a_hi = lds_base + (uint32_t)(wm * KBLK) + f_hi;
    const uint32_t sa_lane = lds_base + SA_BASE + (uint32_t)(wm + fr) * 4;
    const uint32_t b_lo = lds_base + B_BASE + (uint32_t)(wn * KBLK) + f_lo;
    const uint32_t b_hi = lds_base + B_BASE + (uint32_t)(wn * KBLK) + f_hi;

    // B scales.  A wave's columns touch at most two 128-column blocks, nb_lo and nb_lo + 1
    // (TN <= 128); each K block's two scales come from the LDS copy of the block's B scales
    // (read with the block's A fragments, so the main loop issues no global or scalar loads of
    // its own: a scalar load would share the LDS reads' completion counter).
    static_assert(TN <= KBLK, "a wave's columns must span at most two scale blocks");
    const int nb_lo = min(n0 + wn, N - 1) / KBLK;
    const int nb_hi = min(nb_lo + 1, NB - 1);
    bool sb_hi[SN];  // sub-tile jj takes nb_hi's scale
#pragma unroll
    for (int j = 0; j < SN; ++j)
        sb_hi[j] = min(n0 + wn + 16 * j, N - 1) / KBLK != nb_lo;
    const uint32_t sb_lo_addr = lds_base + SB_BASE + (uint32_t)(nb_lo - nb_first) * 4;
    const uint32_t sb_hi_addr = lds_base + SB_BASE + (uint32_t)(nb_hi - nb_first) * 4;
    float vsb_lo, vsb_hi;  // this block's two B scales (all lanes equal)

    // C, streamed into the accumulators (dense form).  Half h of column jj of the wave's
    // sub-tiles (acc[i][jj] for the SM/2 row sub-tiles i of that half) takes its C values at
    // step jj of block c_j0 + 2 jj + h, from registers cb loaded one block earlier (right
    // after the previous half's add; the first half in the prologue).  The C traffic is thus
    // spread over the K loop instead of arriving in one burst in the epilogue, with a block of
    // compute to hide each load, and every add uses a compile-time accumulator index.
    // Columns whose blocks lie past the last K block (short K) take C in the epilogue.
    bool stream_c = false;
    int c_j0 = 0;
    __amdgpu_buffer_rsrc_t rc = rz;
    uint32_t c_lane = 0;
    if constexpr (MODE == MODE_DENSE) {
        stream_c = p.c != nullptr;
        c_j0 = max(0, nkb - 2 * SN);  // all columns streamed when nkb >= 2 SN
        if (stream_c)
            rc = make_rsrc(p.c + (int64_t)m0 * N, (int64_t)(row_limit - m0) * N * 4);
        c_lane = (uint32_t)(((wm + fr) * N + n0 + wn + 4 * fg) * 4);
    }
    static_assert(SM % 2 == 0, "C is streamed in halves of the row sub-tiles");
    constexpr int HM = SM / 2;
    v4f cb[HM];
    auto load_c_half = [&](int jj, int h) {
#pragma unroll
        for (int i = 0; i < HM; ++i)
            cb[i] = __builtin_bit_cast(
                v4f, __builtin_amdgcn_raw_buffer_load_b128(
                         rc, c_lane + (uint32_t)((16 * (h * HM + i) * N + 16 * jj) * 4), 0, 0));
    };
    // both halves of column jj were streamed (the second half's block is the later one)
    auto c_streamed = [&](int jj) { return stream_c && c_j0 + 2 * jj + 1 < nkb; };
    auto read_sfb = [&](int aslot) {
        vsb_lo = lds_read4(sb_lo_addr + (uint32_t)(aslot * 256));
        vsb_hi = lds_read4(sb_hi_addr + (uint32_t)(aslot * 256));
    };

    v4f acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // Fragments.  A (all SM row sub-tiles) and its scales S are held for a whole block; during
    // the block's last step each A[i] / S[i] is replaced by the next block's right after the
    // last MFMA that reads it.  B fragments are read two steps ahead; the next block's B(0)
    // and B(1) are read during the last step.
    v4i Af[SM][2];
    float Sf[SM];
    v4i Bf[NBUF][2];
    // MFMA partials of the previous step, promoted during the next one, and (across a block
    // boundary) the scales of the last step's partials.  Zero before the first step: a no-op.
    v4f pend[SM];
    float psc[SM];
#pragma unroll
    for (int i = 0; i < SM; ++i) {
        pend[i] = v4f{0.f, 0.f, 0.f, 0.f};
        psc[i] = 0.f;
    }
    float sb_cur[SN];
    // When every wave's columns lie in one 128-column scale block (BN a multiple of 128 and
    // TN dividing 128), a row's promotion scale is the same for all of its sub-tiles in a
    // block: scb[i] = sa[i] * sb, formed once per block instead of once per MFMA.
    constexpr bool ONE_NB = (BN % KBLK == 0) && (KBLK % TN == 0);
    float scb[SM];
    auto take_sfb = [&]() {
        tie(vsb_lo);
        tie(vsb_hi);
        const float lo = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(vsb_lo)));
        const float hi = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(vsb_hi)));
#pragma unroll
        for (int jj = 0; jj < SN; ++jj)
            sb_cur[jj] = sb_hi[jj] ? hi : lo;
    };

    // fragment reads from slot bases (a_lo/a_hi/sa of an A slot, b_lo/b_hi of a B slot) with
    // the sub-tile's offset in the instruction
    auto read_a = [&](uint32_t alo, uint32_t ahi, uint32_t sa, auto I) {
        constexpr int i = decltype(I)::value;
        Af[i][0] = lds_read16_at<i * 16 * KBLK>(alo);
        Af[i][1] = lds_read16_at<i * 16 * KBLK>(ahi);
        Sf[i] = lds_read4_at<i * 64>(sa);
    };
    auto read_b = [&](uint32_t blo, uint32_t bhi, auto JJ, v4i (&bf)[2]) {
        constexpr int jj = decltype(JJ)::value;
        bf[0] = lds_read16_at<jj * 16 * KBLK>(blo);
        bf[1] = lds_read16_at<jj * 16 * KBLK>(bhi);
    };

    // One MFMA step: for each row sub-tile i, first promote the previous step's partial of row
    // i (issued SM MFMAs earlier, so it is ready) with scale `scale(i)`, then issue MFMA
    // (i, jj) into the freed partial; `extra(i)` slots in copies and reads after it.
    auto mfma_step = [&](auto JJ, const v4i (&bf)[2], auto scale, auto extra) {
        constexpr int jj = decltype(JJ)::value;
        const v8i bv = v8i{bf[0].x, bf[0].y, bf[0].z, bf[0].w, bf[1].x, bf[1].y, bf[1].z, bf[1].w};
        static_for<SM>([&](auto I) {
            constexpr int i = decltype(I)::value;
            if (MODE != MODE_MASKED || i < sm_act) {
                {
                    v4f &a = acc[i][jj == 0 ? SN - 1 : jj - 1];
                    a += pend[i] * scale(i);
                    // keep the promotion here: left free, the compiler hoists every MFMA of
                    // the block above all promotions and holds SM*SN partials live at once
                    asm volatile("" : "+v"(a));
                }
                const v8i av = v8i{Af[i][0].x, Af[i][0].y, Af[i][0].z, Af[i][0].w,
                                   Af[i][1].x, Af[i][1].y, Af[i][1].z, Af[i][1].w};
                pend[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bv, av, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
            }
            extra(I);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // C of column JJ's half added when block j is that half's block, then the next half loaded
    auto c_step = [&](int j, auto JJ) {
        constexpr int jj = decltype(JJ)::value;
        if constexpr (MODE == MODE_DENSE) {
            // only columns whose two halves both fall inside the K loop; the others take all
            // of their C in the epilogue
            if (c_streamed(jj) && j == c_j0 + 2 * jj) {
#pragma unroll
                for (int i = 0; i < HM; ++i)
                    acc[i][jj] += cb[i];
                load_c_half(jj, 1);
            }
            if (c_streamed(jj) && j == c_j0 + 2 * jj + 1) {
#pragma unroll
                for (int i = 0; i < HM; ++i)
                    acc[HM + i][jj] += cb[i];
                if constexpr (jj + 1 < SN) {
                    if (c_streamed(jj + 1))
                        load_c_half(jj + 1, 0);
                }
            }
        }
    };

    // ---- prologue: blocks 0 .. DEPTH-1 in flight, block 0's fragments read
    if constexpr (MODE == MODE_DENSE) {
        if (c_streamed(0))
            load_c_half(0, 0);  // older than every copy: landed once the first copies have
    }
    // (blocks past the last are copied from empty resources, which keeps the per-wave copy
    // count constant)
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        const bool in = d < nkb;
        issue_scales(in ? kb0 + d : kb0, d, in ? rs : rz, in ? rsb : rz);
#pragma unroll
        for (int c = 0; c < MAXI; ++c)
            issue_copy(c, in ? kb0 + d : kb0, d, d, in ? ra : rz, in ? rb : rz);
    }
    wait_older_copies();
    bare_barrier();
    static_for<SM>([&](auto I) { read_a(a_lo, a_hi, sa_lane, I); });
    read_sfb(0);
    read_b(b_lo, b_hi, std::integral_constant<int, 0>{}, Bf[0]);
    if constexpr (SN > 1)
        read_b(b_lo, b_hi, std::integral_constant<int, 1>{}, Bf[1]);

    int aslot = 0;  // A slot of the current block: j % DEPTH
    int bslot = 0;  // B slot of the current block: j % (DEPTH + 1)
    for (int j = 0; j < nkb; ++j) {
        const bool refill = j + DEPTH < nkb;
        const int kb_fill = refill ? kb0 + j + DEPTH : kb0;
        const __amdgpu_buffer_rsrc_t fa = refill ? ra : rz;
        const __amdgpu_buffer_rsrc_t fb = refill ? rb : rz;
        const __amdgpu_buffer_rsrc_t fs = refill ? rs : rz;
        const int bslot_next = bslot == DEPTH ? 0 : bslot + 1;
        const int bslot_fill = bslot == 0 ? DEPTH : bslot - 1;  // (j + DEPTH) % (DEPTH + 1)
        const int an = aslot == DEPTH - 1 ? 0 : aslot + 1;
        // slot bases of this block's B reads and of the next block's A and B reads
        const uint32_t blo_c = b_lo + (uint32_t)(bslot * B_SLOT);
        const uint32_t bhi_c = b_hi + (uint32_t)(bslot * B_SLOT);
        // this block's A fragments and scales and its B(0), B(1) were read during the last
        // step of the previous block
        lds_wait();
#pragma unroll
        for (int i = 0; i < SM; ++i) {
            tie(Af[i][0]);
            tie(Af[i][1]);
            tie(Sf[i]);
        }
        tie(Bf[0][0]);
        tie(Bf[0][1]);
        if constexpr (SN > 1) {
            tie(Bf[1][0]);
            tie(Bf[1][1]);
        }
        take_sfb();
        if constexpr (ONE_NB) {
#pragma unroll
            for (int i = 0; i < SM; ++i)
                scb[i] = Sf[i] * sb_cur[0];
        }
        // every wave holds this block's A: its A slot may take block j+DEPTH, whose B slot
        // (block j-1's) was released at the previous block's second barrier
        bare_barrier();
        issue_scales(kb_fill, aslot, fs, refill ? rsb : rz);
        if constexpr (SN == 1)
#pragma unroll
            for (int c = 0; c < MAXI; ++c)
                issue_copy(c, kb_fill, aslot, bslot_fill, fa, fb);
        // steps 0 .. SN-2, with this block's refill copies spread over them
        static_for<SN - 1>([&](auto JJ) {
            constexpr int jj = decltype(JJ)::value;
            auto extra = [&](auto I) {
                constexpr int i = decltype(I)::value;
                if constexpr (i == 0 && jj + 2 < SN)
                    read_b(blo_c, bhi_c, std::integral_constant<int, jj + 2>{},
                           Bf[bbuf(jj + 2, SN)]);
                // copies c with c * (SN - 1) / MAXI == jj, after MFMAs 0, 2, ...
#pragma unroll
                for (int c = 0; c < MAXI; ++c) {
                    if ((c * (SN - 1)) / MAXI == jj) {
                        const int first = (jj * MAXI + SN - 2) / (SN > 1 ? SN - 1 : 1);
                        const int pos = c - first;
                        if (i == (SM == 1 ? 0 : (pos * 2) % SM))
                            issue_copy(c, kb_fill, aslot, bslot_fill, fa, fb);
                    }
                }
            };
            if constexpr (jj >= 2) {
                // B(jj) was read two steps ago; only B(jj+1), read one step ago, may be in
                // flight (LDS reads retire in order)
                lds_wait_n<2>();
                tie(Bf[bbuf(jj, SN)][0]);
                tie(Bf[bbuf(jj, SN)][1]);
            }
            c_step(j, JJ);
            if constexpr (jj == 0)
                mfma_step(JJ, Bf[0], [&](int i) { return psc[i]; }, extra);
            else
                mfma_step(JJ, Bf[bbuf(jj, SN)],
                          [&](int i) { return ONE_NB ? scb[i] : Sf[i] * sb_cur[jj - 1]; },
                          extra);
        });
        // last step: the next block's copies have landed everywhere (past the last block the
        // reads below are harmless and unused)
        wait_older_copies();
        bare_barrier();
        lds_wait();
        if constexpr (SN >= 2) {
            tie(Bf[bbuf(SN - 1, SN)][0]);
            tie(Bf[bbuf(SN - 1, SN)][1]);
        }
        const uint32_t alo_n = a_lo + (uint32_t)(an * A_SLOT);
        const uint32_t ahi_n = a_hi + (uint32_t)(an * A_SLOT);
        const uint32_t sa_n = sa_lane + (uint32_t)(an * 1024);
        const uint32_t blo_n = b_lo + (uint32_t)(bslot_next * B_SLOT);
        const uint32_t bhi_n = b_hi + (uint32_t)(bslot_next * B_SLOT);
        c_step(j, std::integral_constant<int, SN - 1>{});
        constexpr auto C0 = std::integral_constant<int, 0>{};
        constexpr auto C1 = std::integral_constant<int, 1>{};
        if constexpr (SN == 1) {
            mfma_step(C0, Bf[0],
                      [&](int i) {
                          const float prev = psc[i];
                          psc[i] = Sf[i] * sb_cur[0];
                          return prev;
                      },
                      [&](auto I) {
                          constexpr int i = decltype(I)::value;
                          read_a(alo_n, ahi_n, sa_n, I);
                          if constexpr (i == 0)
                              read_sfb(an);
                          if constexpr (i == SM - 1)  // after the last MFMA that reads B(0)
                              read_b(blo_n, bhi_n, C0, Bf[0]);
                      });
        } else {
            mfma_step(std::integral_constant<int, SN - 1>{}, Bf[bbuf(SN - 1, SN)],
                      [&](int i) {
                          psc[i] = ONE_NB ? scb[i] : Sf[i] * sb_cur[SN - 1];
                          return ONE_NB ? scb[i] : Sf[i] * sb_cur[SN - 2];
                      },
                      [&](auto I) {
                          constexpr int i = decltype(I)::value;
                          // B(0) (and B(1) when SN > 2) were last read steps ago; with
                          // SN == 2, B(1) is this step's and is replaced after its last MFMA
                          if constexpr (i == 0) {
                              read_b(blo_n, bhi_n, C0, Bf[0]);
                              read_sfb(an);
                          }
                          if constexpr (i == (SN > 2 ? (SM > 1 ? 1 : 0) : SM - 1))
                              read_b(blo_n, bhi_n, C1, Bf[1]);
                          read_a(alo_n, ahi_n, sa_n, I);
                      });
        }
        aslot = an;
        bslot = bslot_next;
    }
    // the last block also read (unused) fragments: they must land before their registers
    // can be reused
    lds_wait();
    tie(vsb_lo);
    tie(vsb_hi);
#pragma unroll
    for (int i = 0; i < SM; ++i) {
        tie(Af[i][0]);
        tie(Af[i][1]);
        tie(Sf[i]);
    }
    tie(Bf[0][0]);
    tie(Bf[0][1]);
    if constexpr (SN > 1) {
        tie(Bf[1][0]);
        tie(Bf[1][1]);
    }
#pragma unroll
    for (int i = 0; i < SM; ++i)
        acc[i][SN - 1] += pend[i] * psc[i];
    wait_vm<0>();  // no copy may still be writing LDS past this point

    // ---- epilogue: + C, round to bf16, store the valid rows.  All of the wave's C values (and
    // row groups) are requested before any is used, so the loads overlap instead of each
    // waiting for the one before; C goes through a buffer resource bounded by the valid rows,
    // which returns zeros past them (only valid rows are stored).
    if constexpr (MODE == MODE_DENSE) {
        if (p.c) {
            const __amdgpu_buffer_rsrc_t rcc =
                make_rsrc(p.c + (int64_t)m0 * N, (int64_t)(row_limit - m0) * N * 4);
            v4f cv[SM][SN];
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j)
                    cv[i][j] = c_streamed(j)
                                   ? v4f{0.f, 0.f, 0.f, 0.f}
                                   : __builtin_bit_cast(
                                         v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rcc, c_lane + (uint32_t)((16 * i * N + 16 * j) * 4),
                                                  0, 0));
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j)
                    acc[i][j] += cv[i][j];
        }
    }
    // The tile goes out through LDS: each wave writes its sub-tiles there as bf16 (8 bytes per
    // lane), then every thread stores whole 16-byte pieces of rows, so a wave's store covers
    // contiguous row segments instead of sixteen 32-byte pieces.  Output rows are OS bytes
    // apart in LDS; OS = 32 (mod 256) puts a fragment write's 16 rows x 32 bytes on distinct
    // banks (two 256-byte halves).
    constexpr int OS = BN * 2 + ((BN * 2) % 256 == 224 ? 0 : 32);
    static_assert(rows_on_distinct_banks(OS), "output row stride");
    static_assert(BM * OS <= LDS_BYTES, "output tile fits the operand slots");
    constexpr int CPR = BN / 8;  // 16-byte pieces per output row
    static_assert((BM * CPR) % NT == 0, "output pieces split evenly over the threads");
    constexpr int PPT = BM * CPR / NT;  // pieces per thread
    bare_barrier();  // every wave is past its last fragment read and copy: LDS is free
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) {
            const uint32_t lo = pack_bf16x2(acc[i][j].x, acc[i][j].y);
            const uint32_t hi = pack_bf16x2(acc[i][j].z, acc[i][j].w);
            lds_write8(lds_base + (uint32_t)((wm + 16 * i + fr) * OS + (wn + 16 * j + 4 * fg) * 2),
                       lo, hi);
        }
    lds_wait();
    bare_barrier();
    v4i piece[PPT];
#pragma unroll
    for (int t = 0; t < PPT; ++t) {
        const int q = tid + t * NT;
        piece[t] = lds_read16(lds_base + (uint32_t)((q / CPR) * OS + (q % CPR) * 16));
    }
    int rowg[PPT];
    if constexpr (MODE == MODE_CONTIG) {
#pragma unroll
        for (int t = 0; t < PPT; ++t)
            rowg[t] = s_grp[(tid + t * NT) / CPR];
    }
    lds_wait();
#pragma unroll
    for (int t = 0; t < PPT; ++t) {
        const int q = tid + t * NT;
        const int row = m0 + q / CPR;
        const int col = n0 + (q % CPR) * 8;
        bool ok = row < row_limit && col < N;
        if constexpr (MODE == MODE_CONTIG)
            ok = ok && rowg[t] == g;
        if (ok)
            *reinterpret_cast<v4i *>(D + (int64_t)row * N + col) = piece[t];
    }
}

template <int BM, int BN, int WM, int WN, int DEPTH, int MODE>
__global__ __launch_bounds__(64 * WM * WN) void dg_gemm_kernel(GemmArgs p, int tiles_m,
                                                               int tiles_n)
{
    gemm_tile<BM, BN, WM, WN, DEPTH, MODE>(p, tiles_m, tiles_n);
}

// ------------------------------------------------------------------------------ host side

static void tiles_for(int mode, int cfg, const GemmArgs &a, int &tiles_m, int &tiles_n)
{
    const TileInfo &ti = kTiles[cfg];
    tiles_n = (a.n + ti.bn - 1) / ti.bn;
    if (mode == MODE_CONTIG)
        tiles_m = a.m / ti.bm;
    else
        tiles_m = (a.m + ti.bm - 1) / ti.bm;
}

int64_t grid_size(int mode, int cfg, const GemmArgs &a)
{
    if (cfg == CFG_STREAM64)
        return mode == MODE_DENSE ? stream_grid_size(a) : -1;
    int tiles_m, tiles_n;
    tiles_for(mode, cfg, a, tiles_m, tiles_n);
    int64_t g = (int64_t)tiles_m * tiles_n;
    if (mode == MODE_MASKED)
        g *= a.num_groups;
    return g;
}

template <int BM, int BN, int WM, int WN, int DEPTH = 2>
static hipError_t launch_cfg(int mode, const GemmArgs &a, hipStream_t stream)
{
    int tiles_m, tiles_n;
    const int cfg_threads = 64 * WM * WN;
    tiles_n = (a.n + BN - 1) / BN;
    tiles_m = mode == MODE_CONTIG ? a.m / BM : (a.m + BM - 1) / BM;
    int64_t grid = (int64_t)tiles_m * tiles_n;
    if (mode == MODE_MASKED)
        grid *= a.num_groups;
    if (grid <= 0 || grid > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    dim3 g((unsigned)grid), b(cfg_threads);
    switch (mode) {
    case MODE_DENSE:
        hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, DEPTH, MODE_DENSE>), g, b, 0, stream, a,
                           tiles_m, tiles_n);
        break;
    case MODE_CONTIG:
        hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, DEPTH, MODE_CONTIG>), g, b, 0, stream, a,
                           tiles_m, tiles_n);
        break;
    default:
        hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, DEPTH, MODE_MASKED>), g, b, 0, stream, a,
                           tiles_m, tiles_n);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm(int mode, int cfg, const GemmArgs &a, hipStream_t stream)
{
    switch (cfg) {
    case CFG_256x224:
        return launch_cfg<256, 224, 4, 2>(mode, a, stream);
    case CFG_128x256:
        return launch_cfg<128, 256, 2, 2>(mode, a, stream);
    case CFG_128x128:
        return launch_cfg<128, 128, 2, 2>(mode, a, stream);
    case CFG_64x32:
        return launch_cfg<64, 32, 2, 2>(mode, a, stream);
    case CFG_256x128:
        return launch_cfg<256, 128, 4, 2>(mode, a, stream);
    case CFG_128x128d4:
        return launch_cfg<128, 128, 2, 2, 4>(mode, a, stream);
    case CFG_128x128w8d4:
        return launch_cfg<128, 128, 2, 4, 4>(mode, a, stream);
    case CFG_128x256w8:
        return launch_cfg<128, 256, 2, 4>(mode, a, stream);
    case CFG_STREAM64:
        return mode == MODE_DENSE ? launch_stream(a, stream) : hipErrorInvalidValue;
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace dg
