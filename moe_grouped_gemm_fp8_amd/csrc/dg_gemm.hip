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
//    accumulators costs four FMAs per MFMA, plus the product sa * sb: once per row and block
//    where a wave's columns lie in one 128-column scale block, else once per MFMA.
//  * Every global read of the main loop (A, B, the A scales and the tile's B scales) is a
//    gfx950 direct-to-LDS copy through a buffer resource, copied two K blocks ahead of its
//    MFMAs; the waits for them are explicit counts.  B has three LDS slots and A two or three
//    (each a whole 128-deep K block): with three, one barrier per K block, with two, a second
//    one at the block's start.  The 256 x 256 tile's operands fill the LDS, so there each
//    wave loads its scales into registers instead, one block ahead, from the L2: two loads
//    per wave (one A scale per lane of its 64 rows, the two B scales), spread to the lanes
//    that use them by the gfx950 32- and 16-lane swaps and readlane.  A wave
//    holds its A fragments for the whole block and reads B fragments two sub-tile steps ahead
//    of the MFMAs that use them.  Barriers are bare s_barrier (a release fence would wait for
//    every copy in flight).
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
//  * Workgroup ids are mapped so that each XCD (ids are dealt round-robin over the 8 XCDs)
//    runs a contiguous range of tiles, rastered in groups of 4 M-tiles, so tiles that run
//    together on one XCD share A rows and B columns in that XCD's L2.  The smaller tile shapes
//    run persistent workgroups (one per CU) that walk their XCD's range; the next tile's
//    first K blocks are copied while the current tile finishes, hiding the per-tile prologue.
//    The 256-row tiles run one workgroup per tile.  The contiguous form's 256 x 256 tiles can
//    leave the tiles of their last-dispatched workgroups (a last partial wave) to workgroups of
//    128 x 128 tiles at the end of the same launch, which spread them over four times as many
//    CUs.
//  * The contiguous form can instead write the 1x128 FP8 cast of SwiGLU(gate, up) of its
//    FP32 result (the activation between an MoE block's two expert GEMMs), its tiles holding
//    the gate and up columns of one 128-column segment of the activation.
//  * Contiguous form: a tile takes the group of its rows from the per-row group indices.  The
//    groups are aligned to 128 rows, so a 256-row tile (one workgroup per tile) can hold the
//    rows of two groups; it then runs twice, once with each group's B, and each pass stores
//    only the rows of its own group.
//  * Shapes too small to fill the CUs with these tiles go to the split-K streaming kernel
//    (dg_stream.hip) instead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "dg_device.h"
#include "dg_internal.h"
#include "dg_tiles.h"

namespace dg {

const TileInfo kTiles[CFG_COUNT] = {
    // the 256x224 tile runs one workgroup per tile: with the loop over tiles its registers
    // spill (it needs nearly all 256 VGPRs for one tile)
    {256, 224, 512, "256x224w8", false},
    {128, 256, 256, "128x256w4", true},
    {128, 128, 256, "128x128w4", true},
    {64, 32, 256, "64x32w4", true},
    {256, 128, 512, "256x128w8", false},
    {64, 64, 256, "stream64", false},
    {128, 128, 256, "128x128w4d4", true},
    {128, 128, 512, "128x128w8d4", true},
    {128, 256, 512, "128x256w8", true},
    {256, 128, 512, "256x128w8p", true},
    // scales in registers (256 x 256 operands fill the LDS): contiguous MoE and masked with
    // N % 256 == 0
    {256, 256, 512, "256x256w8", false},
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

// Largest value over the wave's 64 lanes (a few lane permutes; used once per tile)
__device__ __forceinline__ int wave_max(int v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = max(v, __shfl_xor(v, off));
    return v;
}

// 8-byte global store issued as inline asm: the compiler then does not count it among the
// wave's outstanding vector-memory operations, so its own waits for later register loads (the
// streamed C) stay exact counts instead of draining everything in flight; every explicit wait
// of the kernel counts it (it is older than the copies issued after it).  (Not
// non-temporal: a row's 32-byte pieces from neighbouring stores merge into whole lines in the
// L2 before they are written out.)
__device__ __forceinline__ void store8_async(uint16_t *dst, uint32_t lo, uint32_t hi)
{
    asm volatile("global_store_dwordx2 %0, %1, off" ::"v"(dst), "v"(make_uint2(lo, hi))
                 : "memory");
}

// 4-byte global store issued as inline asm, for the same reason as store8_async
__device__ __forceinline__ void store4_async(void *dst, uint32_t v)
{
    asm volatile("global_store_dword %0, %1, off" ::"v"(dst), "v"(v) : "memory");
}

// The LDS of a kernel that runs one tile shape (one static allocation per instantiation)
template <int BYTES>
__device__ __forceinline__ uint8_t *own_lds()
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[BYTES];
    return lds;
}

// Tiles of workgroup wg of nwg (the kernel's grid, or its share of a grid that also runs another
// tile shape: EXT, the LDS then given by the kernel).
template <int BM, int BN, int WM, int WN, int DEPTH, int MODE, bool PERSIST, int SF,
          bool EXT = false>
__device__ __forceinline__ void gemm_tiles(const GemmArgs &p, int tiles_m, int tiles_n, int wg,
                                           int nwg, uint8_t *ext_lds = nullptr)
{
    // Scale format.  FP32 scales are applied on the vector unit: every MFMA result is one K
    // block's partial, promoted into the FP32 accumulators with sa * sb.  Packed UE8M0 scales
    // (powers of two, four K blocks per int32) are applied by the MFMA itself
    // (v_mfma_scale_f32_16x16x128_f8f6f4 multiplies by 2^(ea-127) * 2^(eb-127)), which then
    // accumulates straight into the accumulators: no partials, no promotion.  Where the vector
    // unit also writes the accumulators inside the K loop (C added there) or MFMAs are skipped
    // under a branch (masked rows), the UE8M0 partial variant keeps the FP32 path's partials
    // and adds them unscaled: a VALU access to an accumulator that an MFMA has just written
    // waits for that MFMA, and a branch around accumulating MFMAs makes the compiler copy the
    // accumulators.
    constexpr bool UE8 = SF != SF_FP32;
    constexpr bool DIRECT = SF == SF_UE8M0;
    // the activation step fused into the epilogue (contiguous form): see the SwiGLU notes below
    constexpr bool SWIGLU = MODE == MODE_CONTIG_SWIGLU;
    constexpr bool CONTIG = MODE == MODE_CONTIG || SWIGLU;
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int SM = TM / 16, SN = TN / 16;
    constexpr int NBUF = bbuf_count(SN);
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be 16-aligned");
    static_assert(BM % 64 == 0 && BN % 8 == 0 && BM <= 256, "tile shape");
    // LDS: DEPTH A slots (BM rows of one K block), DEPTH + 1 B slots (BN rows of one K
    // block), and per A slot a 1 KB area for its A scales and a 256-byte area for the B scales
    // of the 128-column blocks the tile touches.  Block j + DEPTH is copied while block j is
    // multiplied.  Rows are 128 bytes; 16-byte chunk c of row r sits at chunk c ^ h(r)
    // (header comment).
    //
    // With one more A slot where the LDS holds it (NA = DEPTH + 1), block j's refill goes to
    // the slots of block j - 1 (A and B alike), which every wave is done with once it is past
    // the end-of-block barrier of block j - 1: one barrier per block.  Otherwise (NA = DEPTH)
    // the refill takes block j's own A slot, freed only once every wave holds block j's A
    // fragments, which takes a second barrier at the block's start.
    //
    // Where the scale areas do not fit next to DEPTH A and DEPTH + 1 B slots (256 x 256 tiles:
    // 160 KB of operands alone), the scales go to registers instead (SREG): each wave loads
    // its 64 rows' A scales (one per lane) and its two B scales for block j + 1 at block j's
    // start, from the L2, and takes them at block j's end.
    static_assert(DEPTH >= 2, "at least one block of look-ahead beyond the next");
    constexpr int A_SLOT = BM * KBLK;
    constexpr int B_SLOT = BN * KBLK;
    // (the fused activation step adds an area for the row maxima of its segments: BM x WN
    // floats; with one tile per workgroup it reuses the operand slots, free by then)
    constexpr int AMX_BYTES = SWIGLU ? BM * WN * 4 : 0;
    constexpr bool AMX_ALIAS = !PERSIST;
    constexpr int AMX_OWN = AMX_ALIAS ? 0 : AMX_BYTES;
    constexpr int SCL = 1024 + 256;  // an A slot's scale areas (A scales, B scales)
    constexpr bool SREG =
        DEPTH * (A_SLOT + SCL) + (DEPTH + 1) * B_SLOT + AMX_OWN > 160 * 1024;
    static_assert(!SREG || (!PERSIST && DEPTH * A_SLOT + (DEPTH + 1) * B_SLOT <= 160 * 1024),
                  "scales in registers: one tile per workgroup, operands within the LDS");
    static_assert(!SREG || TM == 64, "scales in registers: one A scale per lane of a 64-row band");
    constexpr int SCL_LDS = SREG ? 0 : SCL;
    constexpr bool ONE_BAR =
        (DEPTH + 1) * (A_SLOT + SCL_LDS + B_SLOT) + AMX_OWN <= 160 * 1024;
    constexpr int NA = ONE_BAR ? DEPTH + 1 : DEPTH;  // A slots (and scale areas)
    constexpr int B_BASE = NA * A_SLOT;
    constexpr int SA_BASE = B_BASE + (DEPTH + 1) * B_SLOT;
    constexpr int SB_BASE = SA_BASE + (SREG ? 0 : NA * 1024);
    constexpr int OPS_END = SB_BASE + (SREG ? 0 : NA * 256);
    constexpr int AMX_BASE = AMX_ALIAS ? 0 : OPS_END;
    constexpr int LDS_BYTES = AMX_ALIAS ? (OPS_END > AMX_BYTES ? OPS_END : AMX_BYTES)
                                        : OPS_END + AMX_BYTES;
    static_assert(A_SLOT % 4096 == 0 && B_SLOT % 4096 == 0, "slots start on 4 KB boundaries");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    constexpr int IA = BM / 8, IB = BN / 8;       // 1 KB copies (8 rows of 128 bytes)
    static_assert(IA % NW == 0, "A copies must split evenly over the waves");
    constexpr int CA = IA / NW;                   // A copies per wave per block
    constexpr int CB = (IB + NW - 1) / NW;        // B copies per wave per block (padded)
    constexpr int MAXI = CA + CB;                 // + wave 0 copies the block's scales (2)
    static_assert(DEPTH * (MAXI + 2) < 64, "outstanding copies must fit vmcnt");

    // the staged epilogue (one tile per workgroup) writes the bf16 output tile there, rows OS
    // bytes apart: OS = 32 (mod 256) puts a fragment write's 16 rows x 32 bytes on distinct banks
    constexpr int OS = BN * 2 + ((BN * 2) % 256 == 224 ? 0 : 32);
    constexpr int LDS_ALLOC = (!PERSIST && BM * OS > LDS_BYTES) ? BM * OS : LDS_BYTES;
    static_assert(LDS_ALLOC <= 160 * 1024, "LDS budget (output tile)");
    uint8_t *lds;
    if constexpr (EXT)
        lds = ext_lds;  // (160 KB, shared with the other tile shape of the launch)
    else
        lds = own_lds<LDS_ALLOC>();

    // SwiGLU: one tile covers the gate and up columns of one 128-wide segment of h (BN = 256),
    // each wave TN / 2 of its h columns (TN / 32 gate/up sub-tile pairs), FP32 scales
    static_assert(!SWIGLU || (BN == 256 && SN % 2 == 0 && (WN == 2 || WN == 4) && SF == SF_FP32),
                  "fused activation step: 256-column tiles, two or four waves across");
    // contiguous tiles that may straddle two groups (their last rows may also lie past M)
    constexpr bool TWO_GROUPS = CONTIG && BM > 128;
    static_assert(!TWO_GROUPS || (BM == 256 && !PERSIST), "straddling tiles: 256 rows, one per workgroup");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = (wave / WN) * TM;  // wave's row offset inside the tile
    const int wn = (wave % WN) * TN;  // wave's column offset inside the tile

    // problem sizes; set again (through an opaque copy) at every tile, so that what the
    // compiler derives from them is recomputed per tile instead of being held in scalar
    // registers for the whole kernel
    int M, K, N, KB, NB, nkb, KS;  // KS: scale columns per row (K blocks, or packed words)
    int64_t ld;
    auto set_dims = [&]() {
        M = p.m;
        K = p.k;
        N = p.n;
        asm volatile("" : "+s"(M), "+s"(K), "+s"(N));
        KB = K / KBLK;
        NB = (N + KBLK - 1) / KBLK;
        nkb = KB;
        KS = UE8 ? (KB + 3) / 4 : KB;
        ld = p.ld_sfa;
    };
    set_dims();

    // ---- this workgroup's tiles.  Workgroup ids are dealt round-robin over the 8 XCDs; XCD x
    // owns a contiguous range [s0, s1) of tile ids (in proportion to its workgroups) and its
    // workgroups stride through it together, so the tiles in flight on one XCD are neighbours
    // in the raster and share A rows and B columns in that XCD's L2.  With one workgroup per
    // tile this is the plain XCD-contiguous remap.
    //
    // Contiguous 256-row tiles can hold the rows of two groups (the groups are aligned to 128
    // rows); such a tile needs a second pass with the other group's B.  Run inside the tile's
    // own workgroup it would double that workgroup's time, and in the last wave of workgroups
    // it would lengthen the whole launch by a tile.  So the "listed" straddles get workgroups
    // of their own, ahead of the tiles: tile-row t is listed when the first rows of its two
    // 128-row blocks hold two different valid groups (one per group boundary for groups laid
    // out in order).  Listed straddles are numbered in tile-row order; the first E workgroups
    // serve the first straddle_rows of them, one per N tile, and a tile's own workgroup runs
    // the second pass itself only for a straddle not served so (a straddle the first rows do
    // not show, or one past straddle_rows).  Both sides decide from the same loads.
    //
    // Tail (dg_gemm_contig_tail_kernel, tail_cus > 0): the last workgroups of 256 x 256 tiles
    // are dispatched last, one per XCD in turn, and where they form a last partial wave of
    // whole tiles the launch ends with most CUs idle.  The workgroups of the last tail_tiles()
    // ids (TAIL_MAIN) then leave their tiles to the launch's workgroups of 128 x 128 tiles
    // (TAIL; 128 x 256 for the fused activation step, whose tiles span 256 columns), which run
    // them over four (two) times as many CUs; the straddle workgroups skip them too, since a
    // 128-row tile holds one group.  Both count the same served straddles.
    constexpr bool TAIL_MAIN = EXT && CONTIG && TWO_GROUPS;
    constexpr bool TAIL = EXT && CONTIG && PERSIST && BM == 128 && (BN == 128 || BN == 256);
    constexpr int SUB = (256 / BM) * (256 / BN);  // TAIL: its tiles per 256 x 256 tile
    int total = tiles_m * tiles_n * (MODE == MODE_MASKED ? p.num_groups : 1);
    const int E = TWO_GROUPS ? ((p.straddle_rows * tiles_n + 7) & ~7) : 0;
    const int bid = wg - E;  // < 0: a workgroup serving a listed straddle
    int tile_id, tile_end, tile_step;
    // listed straddles among 256-row tile-rows 64 c + lane (c < 4; the host lists them only
    // while there are at most 256), and the groups of tile-row t's two block-leading rows
    auto leaders = [&](int t, int &la, int &lb) {
        const int r0 = t * 256;
        la = p.grp[r0];
        lb = r0 + 128 < M ? p.grp[r0 + 128] : -1;
        la = (la >= 0 && la < p.num_groups) ? la : -1;
        lb = (lb >= 0 && lb < p.num_groups) ? lb : -1;
    };
    uint64_t listed[4];
    auto scan_listed = [&](int rows256) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int t = 64 * c + lane;
            int la = -1, lb = -1;
            if (t < rows256)
                leaders(t, la, lb);
            listed[c] = __ballot(la >= 0 && lb >= 0 && la != lb);
        }
    };
    // of `tiles` 256 x 256 tiles (tn256 across), those left to the tail: the busy workgroups of
    // their last partial wave over tail_cus CUs (every tile, and one workgroup per N tile for
    // each served straddle) when they are between tail_cus / 8 and tail_cus / 4, else none;
    // tail_force of them if set.  Needs scan_listed first where straddle_rows > 0.
    auto tail_tiles = [&](int tiles, int tn256) {
        if (p.tail_force > 0)
            return min(p.tail_force, tiles - 1);
        int served = 0;
        if (p.straddle_rows > 0) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                served += __builtin_popcountll(listed[c]);
            served = min(served, p.straddle_rows);
        }
        return tail_count((int64_t)tiles + (int64_t)served * tn256, tiles, p.tail_cus);
    };
    int tail_n = 0;  // TAIL: the 256 x 256 tiles these workgroups cover
    if constexpr (TAIL) {
        if (p.tail_cus > 0) {
            if (p.straddle_rows > 0)
                scan_listed(p.tail_tm);
            tail_n = __builtin_amdgcn_readfirstlane(tail_tiles(p.tail_tm * p.tail_tn, p.tail_tn));
            total = SUB * tail_n;
            if (total == 0)
                return;
        }
    }
    if (TAIL_MAIN && p.tail_cus > 0 && bid >= 0) {
        // (only the last workgroups can be left to the tail)
        const int cap = p.tail_force > 0 ? total : p.tail_cus / 4;
        if (bid >= total - cap) {
            if (p.straddle_rows > 0)
                scan_listed(tiles_m);
            if (bid >= total - tail_tiles(total, tiles_n))
                return;
        }
    }
    if (TWO_GROUPS && bid < 0) {
        const int b = wg / tiles_n, tn = wg - b * tiles_n;
        if (b >= p.straddle_rows)
            return;  // (E is rounded up to whole XCD rounds)
        scan_listed(tiles_m);
        int t = -1, left = b;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint64_t mk = listed[c];
            const int cnt = __builtin_popcountll(mk);
            if (t < 0 && left < cnt) {
                for (int i = 0; i < left; ++i)
                    mk &= mk - 1;
                t = 64 * c + __builtin_ctzll(mk);
            }
            left -= t < 0 ? cnt : 0;
        }
        if (t < 0)
            return;  // fewer listed straddles than served slots
        tile_id = raster_index(t, tn, tiles_m, tiles_n);
        if (TAIL_MAIN && p.tail_cus > 0) {
            // a tile left to the tail (its own workgroup is among the last ids)
            const int left = tail_tiles(total, tiles_n);
            if (left > 0 && xcd_tile_owner(total, E, tile_id) - E >= total - left)
                return;
        }
        tile_end = tile_id + 1;
        tile_step = 1;
    } else {
        const TileRange tr = xcd_tile_range(total, nwg, E, wg);
        tile_id = tr.first;
        tile_end = tr.end;
        tile_step = tr.step;
    }
    if (tile_id >= tile_end)
        return;

    // Tile bookkeeping, wave-uniform: coordinates, group, the rows that are computed, and
    // whether it has none (a contiguous block of padding rows, a masked tile past masked_m).
    // Contiguous tiles taller than the 128-row group alignment can hold the rows of two
    // groups: g is the larger, g2 the other one (or -1), computed by a second pass.
    struct Tile {
        int m0, n0, g, g2, row_limit;
        bool empty;
    };
    // raw per-tile data that comes from device memory: masked_m of the tile's group, or the
    // contiguous row groups (lane l: rows m0 + l + 64 r for the group, and the lane's own
    // epilogue rows)
    int raw_cnt = 0;
    int raw_max[BM / 64];
    int raw_row[SM];
    const int fr = lane & 15;
    const int fg = lane >> 4;
    // Masked form, up to 64 groups: the groups' tiles in an order that pairs the group with
    // the most valid rows with the one with the fewest, the second with the second last, and
    // so on.  Consecutive groups go to the same XCD (two per XCD at 16 groups), and a tile's
    // time grows with its group's rows: in group order, the XCD that draws two large groups
    // sets the launch's time.  Lane l holds masked_m of group l (clamped) and that group's
    // rank (descending, ties by index), from one load per launch; the order changes with
    // masked_m on the device, so graph replays follow it.
    constexpr bool MASK_ORDER = MODE == MODE_MASKED;
    int mcnt = 0, mrank = 0;
    const bool ordered = MASK_ORDER && p.num_groups <= 64;
    if constexpr (MASK_ORDER) {
        if (ordered) {
            const int G = p.num_groups;
            int v = lane < G ? p.grp[lane] : -1;
            v = lane < G ? (v < 0 ? 0 : (v > M ? M : v)) : -1;
            int rk = 0;
            for (int k = 0; k < G; ++k) {
                const int vk = __shfl(v, k);
                rk += (vk > v || (vk == v && k < lane)) ? 1 : 0;
            }
            mcnt = v;
            mrank = rk;
        }
    }
    auto coords = [&](int t, int &tm, int &tn, int &g) {
        if constexpr (MODE == MODE_MASKED) {
            const int per_g = tiles_m * tiles_n;
            g = t / per_g;
            const int rem = t - g * per_g;
            tn = rem / tiles_m;
            tm = rem - tn * tiles_m;
            if (ordered) {
                // slot g: ranks 0, G - 1, 1, G - 2, ...
                const int r = (g & 1) ? p.num_groups - 1 - (g >> 1) : g >> 1;
                const uint64_t at = __ballot(lane < p.num_groups && mrank == r);
                g = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(at));
            }
        } else {
            if (TAIL && tail_n > 0) {
                // tile q of the 256 x 256 tile of the 256 x 256 workgroup tiles - tail_n + u
                // (found with that shape's own mapping)
                const int u = t / SUB, q = t - u * SUB;
                const int tiles = p.tail_tm * p.tail_tn;
                const int lead = (p.straddle_rows * p.tail_tn + 7) & ~7;
                const int big =
                    xcd_tile_range(tiles, lead + tiles, lead, lead + tiles - tail_n + u).first;
                int bm, bn;
                raster(big, p.tail_tm, p.tail_tn, bm, bn);
                tm = bm * (256 / BM) + q / (256 / BN);
                tn = bn * (256 / BN) + q % (256 / BN);
            } else {
                raster(t, tiles_m, tiles_n, tm, tn);
            }
            g = 0;
        }
    };
    // a tile's place (its coordinates and group; the integer divisions of the tile mapping
    // run here, outside the K loop), then its data from device memory
    auto place = [&](int t) {
        Tile u;
        int tm, tn, g;
        coords(t, tm, tn, g);
        u.m0 = tm * BM;
        u.n0 = tn * BN;
        u.g = g;
        u.g2 = -1;
        u.row_limit = M;
        u.empty = false;
        return u;
    };
    auto load_meta = [&](const Tile &u) {
        if constexpr (MODE == MODE_MASKED) {
            raw_cnt = ordered ? __builtin_amdgcn_readlane(mcnt, u.g) : p.grp[u.g];
        } else if constexpr (CONTIG) {
            // (rows past M: only a tile taller than the 128-row alignment, or a tail
            // tile in the second half of a 256-row tile that ends past M, reaches them)
            constexpr bool PAST_M = TWO_GROUPS || TAIL;
#pragma unroll
            for (int r = 0; r < BM / 64; ++r) {
                const int row = u.m0 + lane + 64 * r;
                raw_max[r] = (!PAST_M || row < M) ? p.grp[row] : -1;
            }
#pragma unroll
            for (int i = 0; i < SM; ++i) {
                const int row = u.m0 + wm + 16 * i + fr;
                raw_row[i] = (!PAST_M || row < M) ? p.grp[row] : -1;
            }
        }
    };
    int rowg_next[SM];  // contiguous: the epilogue rows' groups of the tile being prepared
    auto finish_meta = [&](Tile u) {
        if constexpr (MODE == MODE_MASKED) {
            const int v = raw_cnt < 0 ? 0 : (raw_cnt > M ? M : raw_cnt);
            u.row_limit = __builtin_amdgcn_readfirstlane(v);
            u.empty = u.m0 >= u.row_limit;
        } else if constexpr (CONTIG) {
            int best = -1;
#pragma unroll
            for (int r = 0; r < BM / 64; ++r) {
                const int v = raw_max[r];
                best = max(best, (v >= 0 && v < p.num_groups) ? v : -1);
            }
            u.g = __builtin_amdgcn_readfirstlane(wave_max(best));
            if constexpr (TWO_GROUPS) {
                int second = -1;
#pragma unroll
                for (int r = 0; r < BM / 64; ++r) {
                    const int v = raw_max[r];
                    second = max(second, (v >= 0 && v < u.g) ? v : -1);
                }
                u.g2 = __builtin_amdgcn_readfirstlane(wave_max(second));
            }
            // (a tail tile in the second half of a ragged last 256-column tile can
            // start past N)
            u.empty = u.g < 0 || (TAIL && u.n0 >= N);
#pragma unroll
            for (int i = 0; i < SM; ++i)
                rowg_next[i] = raw_row[i];
        }
        return u;
    };

    // copy resources of a tile: operands through buffer resources that end at the last valid
    // row (rows past it read as zeros; an empty tile's are empty); the tile's offsets are in
    // the resource bases, so the lane offsets below are the same for every tile.  They are
    // rebuilt from the tile (scalar arithmetic) where used rather than kept for two tiles.
    struct CopySrc {
        __amdgpu_buffer_rsrc_t a, b, sa, sb;
    };
    auto copy_src = [&](const Tile &u) {
        const int64_t ga = MODE == MODE_MASKED ? (int64_t)u.g * M : 0;
        const uint8_t *A = p.a + ga * K;
        const float *SFA = p.sfa + (MODE == MODE_MASKED ? (int64_t)u.g * KS * ld : 0);
        const uint8_t *B = p.b + (int64_t)u.g * N * K;
        const float *SFB = p.sfb + (int64_t)u.g * NB * KS;
        // SwiGLU: the tile's B rows start at its segment's first gate row, n0 / 2 (the up rows
        // follow I = N / 2 rows further on, inside the same range)
        const int bn0 = SWIGLU ? u.n0 / 2 : u.n0;
        const int nbf = bn0 / KBLK;
        CopySrc s;
        s.a = make_rsrc(A + (int64_t)u.m0 * K, u.empty ? 0 : (int64_t)(u.row_limit - u.m0) * K);
        s.b = make_rsrc(B + (int64_t)bn0 * K, u.empty ? 0 : (int64_t)(N - bn0) * K);
        s.sa = make_rsrc(SFA + u.m0, u.empty ? 0 : ((int64_t)KS * ld - u.m0) * 4);
        s.sb = make_rsrc(SFB + (int64_t)nbf * KS, u.empty ? 0 : (int64_t)(NB - nbf) * KS * 4);
        return s;
    };

    // ---- copies.  Wave w's copy c < CA of a block is A rows [8q, 8q+8) with q = w + c*NW;
    // copy CA + c is B rows [8q, 8q+8) with q = min(w + c*NW, IB-1) (a wave past the last B
    // rows repeats it: same bytes to the same place); wave 0 also copies the block's A scales
    // and the B scales of the tile's 128-column blocks.  Lane l of a row copy fetches row
    // 8q + l/8, logical chunk (l & 7) ^ h(row), so the contiguous 1 KB that the copy writes is
    // the swizzled layout; h(row) = (q & 1) ^ 2(l >> 4) because row bits 1, 2 are lane bits
    // 4, 5 and row bit 3 is q's bit 0.  Copies of blocks past a workgroup's last come from
    // empty resources and only write zeros into slots nobody reads, which keeps the per-wave
    // copy count constant.
    const uint32_t lds_base = (uint32_t)(uintptr_t)(DG_LDS uint8_t *)lds;
    DG_LDS uint8_t *ldsp = (DG_LDS uint8_t *)lds;
    // Per-copy lane offsets (the K block goes into the scalar offset): copy c's row group q
    // and its lanes' byte offsets.  Held in registers during a tile's K loop, so issuing a
    // copy costs no vector arithmetic.  These and the fragment addresses below are set again
    // at every tile from an opaque copy of the lane id (set_lane_consts), so that they are
    // dead, not held, through the epilogue, where the accumulators and C need the registers.
    int cq[MAXI];
#pragma unroll
    for (int c = 0; c < MAXI; ++c)
        cq[c] = c < CA ? wave + c * NW : min(wave + (c - CA) * NW, IB - 1);
    uint32_t voff[MAXI];
    uint32_t lane_sfa, lane_sfb;  // 4 A scales per lane; B scale block `lane`
    // issue copy c (a constant after unrolling) of K block kb into A slot aslot or B slot bslot
    // (a plain int parameter: a generic lambda here keeps the host pass from emitting the
    // kernel's launch stub).  Masked tiles read their B panel once (one tile row per group):
    // non-temporal copies, 3.9% faster on the 16-group decode shape.
    auto issue_copy = [&](int c, int kb, int aslot, int bslot, const CopySrc &s) {
        if (c < CA)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                s.a, (DG_LDS void *)(ldsp + aslot * A_SLOT + cq[c] * 1024), 16, voff[c],
                (uint32_t)kb * KBLK, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                s.b, (DG_LDS void *)(ldsp + B_BASE + bslot * B_SLOT + cq[c] * 1024), 16, voff[c],
                (uint32_t)kb * KBLK, 0, MODE == MODE_MASKED ? CP_NT : 0);
    };
    auto issue_scales = [&](int kb, int aslot, const CopySrc &s) {
        if (!SREG && wave == 0) {
            // the K block's row offset goes into the range-checked lane offset: rows past the
            // last scale row read zeros
            uint32_t vo = lane_sfa;
            asm volatile("" : "+v"(vo));
            const int ks = UE8 ? kb >> 2 : kb;  // the scale column holding block kb
            vo += (uint32_t)((int64_t)ks * ld * 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                s.sa, (DG_LDS void *)(ldsp + SA_BASE + aslot * 1024), 16, vo, 0, 0, 0);
            uint32_t vb = lane_sfb;
            asm volatile("" : "+v"(vb));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                s.sb, (DG_LDS void *)(ldsp + SB_BASE + aslot * 256), 4, vb, (uint32_t)ks * 4u, 0,
                0);
        }
    };
    // wait until the next block's copies have landed (those of the DEPTH - 1 blocks after it
    // may still be in flight).  SREG: no scale copies; inside the K loop each block's register
    // loads of the next block's scales, two per wave, precede its copies and may still be in
    // flight too (their own wait comes at the block's last step).
    auto wait_older_copies = [&](bool in_loop) {
        constexpr int LATER = (DEPTH - 1) * MAXI;
        if constexpr (SREG) {
            if (in_loop)
                wait_vm<LATER + (DEPTH - 1) * 2>();
            else
                wait_vm<LATER>();
        } else if (wave == 0) {
            wait_vm<LATER + (DEPTH - 1) * 2>();
        } else {
            wait_vm<LATER>();
        }
    };

    // per-lane fragment offsets inside a slot: lanes 16g..16g+15 hold K bytes [32g, 32g+32) of
    // 16 consecutive rows, i.e. logical chunks 2g and 2g+1
    uint32_t a_lo, a_hi, sa_lane, b_lo, b_hi;
    auto set_lane_consts = [&]() {
        int l = lane;
        asm volatile("" : "+v"(l));
        const int r = l & 15, gq = l >> 4;
        const uint32_t lane_even =
            (uint32_t)(l >> 3) * (uint32_t)K + (uint32_t)((((l & 7) ^ ((l >> 4) << 1))) << 4);
#pragma unroll
        for (int c = 0; c < MAXI; ++c) {
            // SwiGLU: LDS rows of B alternate 16 gate rows and the 16 up rows of the same
            // columns, so sub-tile pair (2p, 2p + 1) of a wave holds gate and up of 16 columns
            uint32_t row = (uint32_t)(8 * cq[c]);
            if (SWIGLU && c >= CA)
                row = (uint32_t)(16 * (cq[c] >> 2) + 8 * (cq[c] & 1)) +
                      (((cq[c] >> 1) & 1) ? (uint32_t)(N >> 1) : 0u);
            voff[c] = (lane_even ^ (uint32_t)((cq[c] & 1) << 4)) + row * (uint32_t)K;
        }
        lane_sfa = (uint32_t)l * 16u;
        // B scales: lane l copies block nbf + l; SwiGLU: lane 0 the gate block, lane 1 the up
        // block I / 128 further on, the rest nothing (outside the range: zeros)
        lane_sfb = SWIGLU ? (l == 0 ? 0u : (l == 1 ? (uint32_t)(N >> 8) * (uint32_t)KS * 4u
                                                    : 0x80000000u))
                          : (uint32_t)l * (uint32_t)KS * 4u;
        const int h = ((r >> 3) & 1) | (r & 2) | (((r >> 2) & 1) << 2);  // h(r)
        const uint32_t f_lo = (uint32_t)(r * KBLK + (((2 * gq) ^ h) << 4));
        const uint32_t f_hi = (uint32_t)(r * KBLK + (((2 * gq + 1) ^ h) << 4));
        a_lo = lds_base + (uint32_t)(wm * KBLK) + f_lo;
        a_hi = lds_base + (uint32_t)(wm * KBLK) + f_hi;
        sa_lane = lds_base + SA_BASE + (uint32_t)(wm + r) * 4;
        b_lo = lds_base + B_BASE + (uint32_t)(wn * KBLK) + f_lo;
        b_hi = lds_base + B_BASE + (uint32_t)(wn * KBLK) + f_hi;
    };

    // B scales.  A wave's columns touch at most two 128-column blocks, nb_lo and nb_lo + 1
    // (TN <= 128); each K block's two scales come from the LDS copy of the block's B scales
    // (read with the block's A fragments, so the main loop issues no global or scalar loads of
    // its own: a scalar load would share the LDS reads' completion counter).  The LDS copy of
    // a tile starts at its first block nb_first = n0 / 128.
    static_assert(TN <= KBLK, "a wave's columns must span at most two scale blocks");
    struct ScaleSel {
        uint32_t lo, hi;   // LDS byte offsets of the wave's two B scales in a block's area
        uint32_t hi_mask;  // bit jj: sub-tile column jj takes the second one
    };
    auto scale_sel = [&](const Tile &u) {
        ScaleSel s;
        if constexpr (SWIGLU) {
            // gate sub-tiles (even jj) take the gate block's scale, up sub-tiles the up block's
            s.lo = 0;
            s.hi = 4;
            s.hi_mask = 0;
#pragma unroll
            for (int j = 0; j < SN; ++j)
                s.hi_mask |= (uint32_t)(j & 1) << j;
            return s;
        }
        const int nbf = u.n0 / KBLK;
        const int nb_lo = min(u.n0 + wn, N - 1) / KBLK;
        const int nb_hi = min(nb_lo + 1, NB - 1);
        s.lo = (uint32_t)(nb_lo - nbf) * 4;
        s.hi = (uint32_t)(nb_hi - nbf) * 4;
        s.hi_mask = 0;
#pragma unroll
        for (int j = 0; j < SN; ++j)
            s.hi_mask |= (min(u.n0 + wn + 16 * j, N - 1) / KBLK != nb_lo ? 1u : 0u) << j;
        return s;
    };
    float vsb_lo, vsb_hi;  // this block's two B scales (all lanes equal)
    // SREG: the next block's scales, loaded into registers at the current block's start, two
    // loads per wave: lane l the A scale of the wave's row wm + l, and the wave's two B scales,
    // lo in the even lanes and hi in the odd ones (the offsets of the LDS form's lanes
    // sel.lo / 4 and sel.hi / 4 in the B-scale copy)
    float Sn, vbn;
    uint32_t sw_b, sw_hold;  // (lane moves of the A scales, during a block's last step)
    auto load_scales = [&](int kb, const CopySrc &s, const ScaleSel &sl) {
        const int ks = UE8 ? kb >> 2 : kb;  // the scale column holding block kb
        Sn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           s.sa, (uint32_t)(((int64_t)ks * ld + wm + lane) * 4), 0, 0));
        const uint32_t blo = SWIGLU ? 0u : sl.lo * (uint32_t)KS;
        const uint32_t bhi = SWIGLU ? (uint32_t)(N >> 8) * (uint32_t)KS * 4u : sl.hi * (uint32_t)KS;
        vbn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            s.sb, ((lane & 1) ? bhi : blo) + (uint32_t)ks * 4u, 0, 0));
    };
    auto read_sfb = [&](int aslot, const ScaleSel &s) {
        if constexpr (SREG) {
            tie(vbn);
            vsb_lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vbn), 0));
            vsb_hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vbn), 1));
        } else {
            vsb_lo = lds_read4(lds_base + SB_BASE + s.lo + (uint32_t)(aslot * 256));
            vsb_hi = lds_read4(lds_base + SB_BASE + s.hi + (uint32_t)(aslot * 256));
        }
    };

    // C, streamed into the accumulators (dense form).  Block c_j0 + 2 jj + h loads half h of
    // column jj of the wave's sub-tiles (acc[h*SM/2 + i][jj], i < SM/2) right after its opening
    // barrier and adds it after its end-of-block wait for the next block's copies, which were
    // issued after the load, so that wait already covers it and the compiler's own wait for the
    // registers (within one iteration, where it can count) stalls nothing.  The C traffic is
    // spread over the K loop instead of arriving in one burst in the epilogue.  Columns whose
    // blocks lie past the last K block (short K) take C in the epilogue.
    const bool stream_c = MODE == MODE_DENSE && p.c != nullptr;
    auto c_first = [&]() { return max(0, nkb - 2 * SN); };  // all columns streamed when nkb >= 2 SN
    const uint32_t c_lane = (uint32_t)(((wm + fr) * N + wn + 4 * fg) * 4);
    auto c_src = [&](const Tile &u) {
        if (!stream_c && MODE == MODE_DENSE && p.c == nullptr)
            return make_rsrc(p.sfa, 0);
        // C rows from m0 on, columns from n0 on; rows past the last valid one read zeros
        return make_rsrc(p.c + (int64_t)u.m0 * N + u.n0,
                         ((int64_t)(u.row_limit - u.m0) * N - u.n0) * 4);
    };
    static_assert(SM % 2 == 0, "C is streamed in halves of the row sub-tiles");
    constexpr int HM = SM / 2;
    v4f cb[HM];
    auto load_c_half = [&](const __amdgpu_buffer_rsrc_t &rc, int jj, int h) {
#pragma unroll
        for (int i = 0; i < HM; ++i)
            cb[i] = __builtin_bit_cast(
                v4f, __builtin_amdgcn_raw_buffer_load_b128(
                         rc, c_lane + (uint32_t)((16 * (h * HM + i) * N + 16 * jj) * 4), 0, 0));
    };
    // both halves of column jj were streamed (the second half's block is the later one)
    auto c_streamed = [&](int jj) { return stream_c && c_first() + 2 * jj + 1 < nkb; };

    v4f acc[SM][SN];
    // Fragments.  A (all SM row sub-tiles) and its scales S are held for a whole block; during
    // the block's last step each A[i] / S[i] is replaced by the next block's right after the
    // last MFMA that reads it.  B fragments are read two steps ahead; the next block's B(0)
    // and B(1) are read during the last step.
    v4i Af[SM][2];
    float Sf[SM];
    v4i Bf[NBUF][2];
    // MFMA partials of the previous step, promoted during the next one, and (across a block
    // boundary) the scales of the last step's partials.  Zero before a tile's first step.
    v4f pend[SM];
    float psc[SM];
    auto clear_tile_state = [&]() {
#pragma unroll
        for (int i = 0; i < SM; ++i) {
#pragma unroll
            for (int j = 0; j < SN; ++j)
                acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
            pend[i] = v4f{0.f, 0.f, 0.f, 0.f};
            psc[i] = 0.f;
        }
    };
    float sb_cur[SN];
    // When every wave's columns lie in one 128-column scale block (BN a multiple of 128 and
    // TN dividing 128), a row's promotion scale is the same for all of its sub-tiles in a
    // block: scb[i] = sa[i] * sb, formed once per block instead of once per MFMA.
    constexpr bool ONE_NB = (BN % KBLK == 0) && (KBLK % TN == 0) && !SWIGLU;
    float scb[SM];
    // SwiGLU: even sub-tile columns take the gate block's scale and odd ones the up block's,
    // so a row has two promotion scales per block, scb[i] and scb2[i]
    constexpr bool TWO_NB = SWIGLU;
    float scb2[SM];
    // UE8M0: the block's exponents, for the MFMA's scale operands: eb[jj] for the B block of
    // sub-tile column jj, ea[i] for this lane's row of sub-tile row i
    int eb[SN], ea[SM];
    auto take_sfb = [&](uint32_t hi_mask, int kb) {
        tie(vsb_lo);
        tie(vsb_hi);
        if constexpr (UE8) {
            const int sh = 8 * (kb & 3);  // byte of the packed word holding block kb
            const int lo = (__builtin_amdgcn_readfirstlane(__float_as_int(vsb_lo)) >> sh) & 0xFF;
            const int hi = (__builtin_amdgcn_readfirstlane(__float_as_int(vsb_hi)) >> sh) & 0xFF;
#pragma unroll
            for (int jj = 0; jj < SN; ++jj)
                eb[jj] = ((hi_mask >> jj) & 1) ? hi : lo;
#pragma unroll
            for (int i = 0; i < SM; ++i)
                ea[i] = (__float_as_int(Sf[i]) >> sh) & 0xFF;
        } else {
            const float lo = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(vsb_lo)));
            const float hi = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(vsb_hi)));
#pragma unroll
            for (int jj = 0; jj < SN; ++jj)
                sb_cur[jj] = ((hi_mask >> jj) & 1) ? hi : lo;
        }
    };

    // fragment reads from slot bases (a_lo/a_hi/sa of an A slot, b_lo/b_hi of a B slot) with
    // the sub-tile's offset in the instruction
    auto read_a = [&](uint32_t alo, uint32_t ahi, uint32_t sa, auto I) {
        constexpr int i = decltype(I)::value;
        Af[i][0] = lds_read16_at<i * 16 * KBLK>(alo);
        Af[i][1] = lds_read16_at<i * 16 * KBLK>(ahi);
        if constexpr (SREG) {
            // loaded at the block's start; the use here makes the compiler's own wait for
            // them fall inside this block (counting this block's copies after them), not at
            // the next block's start, where it cannot count across the loop and waits for all.
            // Row wm + 16 i + fr's scale is in lane 16 i + fr: the 32- and 16-lane swaps give
            // every lane the rows of lane group i (groups 0, 1 from the lower halves, 2, 3 from
            // the upper), a sub-tile's value taken when its MFMAs no longer need the old one.
            if constexpr (i == 0) {
                tie(Sn);
                const uint32_t v = __builtin_bit_cast(uint32_t, Sn);
                const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
                const auto g = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);
                sw_b = h[1];
                Sf[0] = __builtin_bit_cast(float, g[0]);
                sw_hold = g[1];
            } else if constexpr (i == 2) {
                const auto g = __builtin_amdgcn_permlane16_swap(sw_b, sw_b, false, false);
                Sf[2] = __builtin_bit_cast(float, g[0]);
                sw_hold = g[1];
            } else {
                Sf[i] = __builtin_bit_cast(float, sw_hold);
            }
        } else
            Sf[i] = lds_read4_at<i * 64>(sa);
    };
    auto read_b = [&](uint32_t blo, uint32_t bhi, auto JJ, v4i (&bf)[2]) {
        constexpr int jj = decltype(JJ)::value;
        bf[0] = lds_read16_at<jj * 16 * KBLK>(blo);
        bf[1] = lds_read16_at<jj * 16 * KBLK>(bhi);
    };

    // the current tile and what depends on it
    Tile cur = place(tile_id);
    load_meta(cur);
    cur = finish_meta(cur);
    if constexpr (TWO_GROUPS) {
        // a straddle is served ahead of the tiles when it is listed, among the first
        // straddle_rows listed ones, and its groups are those of its block-leading rows
        if (bid < 0 || cur.g2 >= 0) {
            const int t = cur.m0 / BM;
            int la, lb;
            leaders(t, la, lb);
            la = __builtin_amdgcn_readfirstlane(la);
            lb = __builtin_amdgcn_readfirstlane(lb);
            const bool match = cur.g2 >= 0 && la >= 0 && lb >= 0 && max(la, lb) == cur.g &&
                               min(la, lb) == cur.g2;
            if (bid < 0) {
                if (match)
                    cur.g = cur.g2;  // this workgroup: the second group only
                else
                    cur.empty = true;  // the tile's own workgroup runs it
                cur.g2 = -1;
            } else if (match && p.straddle_rows > 0) {
                scan_listed(tiles_m);
                int rank = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int below = t - 64 * c;
                    const uint64_t m = below >= 64 ? ~0ull : (below <= 0 ? 0ull : (1ull << below) - 1);
                    rank += __builtin_popcountll(listed[c] & m);
                }
                if (rank < p.straddle_rows)
                    cur.g2 = -1;  // served ahead
            }
        }
    }
    int rowg[SM];
#pragma unroll
    for (int i = 0; i < SM; ++i)
        rowg[i] = rowg_next[i];
    ScaleSel sel = scale_sel(cur);
    // masked form: the wave's row sub-tiles that hold a valid row (the others are never
    // stored, so their MFMAs and promotions are skipped; copies and barriers are not).  The
    // contiguous form computes every row sub-tile (an all-padding tile, rare, multiplies the
    // zeros its empty copies wrote and stores nothing).
    auto active_rows = [&](const Tile &u) {
        if constexpr (MODE == MODE_MASKED) {
            const int v = (u.row_limit - u.m0 - wm + 15) >> 4;
            return __builtin_amdgcn_readfirstlane(v < 0 ? 0 : (v > SM ? SM : v));
        } else {
            return u.empty ? 0 : SM;
        }
    };
    int sm_act = active_rows(cur);
    // the next tile, placed before the current one's K loop and completed during its first
    // block; its first DEPTH blocks are copied during the current one's last DEPTH blocks
    // when the K loop is long enough to hold them (else its prologue runs after the current
    // tile's epilogue)
    bool has_next = PERSIST && tile_id + tile_step < tile_end;
    const bool overlap = nkb >= DEPTH + 1;
    Tile nxt = cur;
    ScaleSel nsel = sel;

    // One MFMA step: for each row sub-tile i, first promote the previous step's partial of row
    // i (issued SM MFMAs earlier, so it is ready) with scale `scale(i)`, then issue MFMA
    // (i, jj) into the freed partial; `extra(i)` slots in copies and reads after it.
    auto mfma_step = [&](auto JJ, const v4i (&bf)[2], auto scale, auto extra) {
        constexpr int jj = decltype(JJ)::value;
        const v8i bv = v8i{bf[0].x, bf[0].y, bf[0].z, bf[0].w, bf[1].x, bf[1].y, bf[1].z, bf[1].w};
        static_for<SM>([&](auto I) {
            constexpr int i = decltype(I)::value;
            if (MODE != MODE_MASKED || DIRECT || i < sm_act) {
                const v8i av = v8i{Af[i][0].x, Af[i][0].y, Af[i][0].z, Af[i][0].w,
                                   Af[i][1].x, Af[i][1].y, Af[i][1].z, Af[i][1].w};
                if constexpr (DIRECT) {
                    // first operand B (its block's exponent), second A (this lane's row's)
                    acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        bv, av, acc[i][jj], 0, 0, 0, eb[jj], 0, ea[i]);
                } else {
                    {
                        v4f &a = acc[i][jj == 0 ? SN - 1 : jj - 1];
                        if constexpr (UE8)
                            a += pend[i];  // already scaled by the MFMA
                        else
                            a += pend[i] * scale(i);
                        // keep the promotion here: left free, the compiler hoists every MFMA
                        // of the block above all promotions and holds SM*SN partials live
                        asm volatile("" : "+v"(a));
                    }
                    if constexpr (UE8)
                        pend[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bv, av, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, eb[jj], 0, ea[i]);
                    else
                        pend[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bv, av, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                }
            }
            extra(I);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // C half-column q = j - c_j0 of block j: column q / 2, row half q % 2, added at the end of
    // the block whose start loaded it (compile-time accumulator indices behind a uniform
    // switch on the column)
    auto add_c_half = [&](int q) {
        static_for<SN>([&](auto JJ) {
            constexpr int jj = decltype(JJ)::value;
            // each arm ends in an asm statement with its own constant: without it the compiler
            // merges the arms into one add through a runtime accumulator index and moves the
            // accumulators to scratch memory
            if (q == 2 * jj) {
#pragma unroll
                for (int i = 0; i < HM; ++i)
                    acc[i][jj] += cb[i];
                asm volatile("; C half %0" ::"n"(2 * jj));
            }
            if (q == 2 * jj + 1) {
#pragma unroll
                for (int i = 0; i < HM; ++i)
                    acc[HM + i][jj] += cb[i];
                asm volatile("; C half %0" ::"n"(2 * jj + 1));
            }
        });
    };

    // A slot of the current block (block j of the workgroup's stream of blocks, tiles end to
    // end): j % DEPTH; its B slot: j % (DEPTH + 1).  They run on across tiles.
    int aslot = 0;
    int bslot = 0;
    // block 0's fragments of the current tile, from the current slots (landed and past a
    // barrier)
    auto read_first = [&]() {
        const uint32_t ao = (uint32_t)(aslot * A_SLOT), bo = (uint32_t)(bslot * B_SLOT);
        if constexpr (SREG)
            load_scales(0, copy_src(cur), sel);  // (one tile per workgroup)
        static_for<SM>(
            [&](auto I) { read_a(a_lo + ao, a_hi + ao, sa_lane + (uint32_t)(aslot * 1024), I); });
        read_sfb(aslot, sel);
        read_b(b_lo + bo, b_hi + bo, std::integral_constant<int, 0>{}, Bf[0]);
        if constexpr (SN > 1)
            read_b(b_lo + bo, b_hi + bo, std::integral_constant<int, 1>{}, Bf[1]);
    };
    // prologue of a tile: its blocks 0 .. DEPTH-1 in flight (blocks past the last are copied
    // from empty resources), block 0's fragments read
    auto start_tile = [&]() {
        int as = aslot, bs = bslot;
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const bool in = d < nkb;
            Tile u = cur;
            u.empty = u.empty || !in;
            const CopySrc s = copy_src(u);
            issue_scales(in ? d : 0, as, s);
#pragma unroll
            for (int c = 0; c < MAXI; ++c)
                issue_copy(c, in ? d : 0, as, bs, s);
            as = as == NA - 1 ? 0 : as + 1;
            bs = bs == DEPTH ? 0 : bs + 1;
        }
        wait_older_copies(false);
        bare_barrier();
        read_first();
    };

    bool first = true;
    for (;;) {
        set_dims();
        const int c_j0 = c_first();
        // a tile with nothing to compute (a masked group with masked_m past its rows, a
        // contiguous block of padding) is skipped; the tile after it starts the pipeline anew
        if (cur.empty) {
            if (!has_next)
                break;
            tile_id += tile_step;
            cur = place(tile_id);
            load_meta(cur);
            cur = finish_meta(cur);
#pragma unroll
            for (int i = 0; i < SM; ++i)
                rowg[i] = rowg_next[i];
            sel = scale_sel(cur);
            sm_act = active_rows(cur);
            has_next = PERSIST && tile_id + tile_step < tile_end;
            first = true;
            continue;
        }
        set_lane_consts();
        clear_tile_state();
        // a tile's first blocks were copied during the previous tile when it overlapped
        if (first || !overlap)
            start_tile();
        else
            read_first();
        first = false;
        const bool prefetch = has_next && overlap;
        if (has_next)
            nxt = place(tile_id + tile_step);
        const __amdgpu_buffer_rsrc_t rc = c_src(cur);
        // K block j of the tile, whose refill copies (block kb_fill of the tile behind fs) go
        // out during its steps
        // (SREG: the tile's own source fsr for the next block's scales)
        auto block = [&](int j, const CopySrc &fs, int kb_fill, const CopySrc &fsr) {
            const int bslot_next = bslot == DEPTH ? 0 : bslot + 1;
            const int bslot_fill = bslot == 0 ? DEPTH : bslot - 1;  // (j + DEPTH) % (DEPTH + 1)
            const int an = aslot == NA - 1 ? 0 : aslot + 1;
            // the refill's A slot (and scale areas): block j-1's with NA = DEPTH + 1, else
            // block j's own
            const int afill = ONE_BAR ? (aslot == 0 ? NA - 1 : aslot - 1) : aslot;
            // slot bases of this block's B reads and of the next block's A and B reads
            const uint32_t blo_c = b_lo + (uint32_t)(bslot * B_SLOT);
            const uint32_t bhi_c = b_hi + (uint32_t)(bslot * B_SLOT);
            // this block's A fragments and scales and its B(0), B(1) were read during the
            // last step of the previous block (or the tile's prologue)
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
            take_sfb(sel.hi_mask, j);
            if constexpr (ONE_NB && !UE8) {
#pragma unroll
                for (int i = 0; i < SM; ++i)
                    scb[i] = Sf[i] * sb_cur[0];
            }
            if constexpr (TWO_NB) {
#pragma unroll
                for (int i = 0; i < SM; ++i) {
                    scb[i] = Sf[i] * sb_cur[0];
                    scb2[i] = Sf[i] * sb_cur[1];
                }
            }
            // two-barrier form: every wave holds this block's A, so its A slot may take block
            // j+DEPTH, whose B slot (block j-1's) was released at the previous block's end
            if constexpr (!ONE_BAR)
                bare_barrier();
            // this block's half-column of C: loaded now, added after the end-of-block wait
            // for the next block's copies, which it precedes (so that wait covers it); only
            // columns whose two halves both fall inside the loop are streamed
            const int cq = j - c_j0;
            const bool c_now = stream_c && cq >= 0 && c_j0 + 2 * (cq >> 1) + 1 < nkb;
            if constexpr (MODE == MODE_DENSE) {
                if (c_now)
                    load_c_half(rc, cq >> 1, cq & 1);
            }
            // the next tile's data from device memory, loaded at the first block's start and
            // used at its end
            if constexpr (MODE != MODE_DENSE) {
                if (j == 0 && has_next)
                    load_meta(nxt);
            }
            issue_scales(kb_fill, afill, fs);
            if constexpr (SREG)
                load_scales(j + 1, fsr, sel);  // before the copies: the end-of-block wait counts
            if constexpr (SN == 1)
#pragma unroll
                for (int c = 0; c < MAXI; ++c)
                    issue_copy(c, kb_fill, afill, bslot_fill, fs);
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
                                issue_copy(c, kb_fill, afill, bslot_fill, fs);
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
                if constexpr (jj == 0)
                    mfma_step(JJ, Bf[0], [&](int i) { return psc[i]; }, extra);
                else
                    mfma_step(JJ, Bf[bbuf(jj, SN)],
                              [&](int i) {
                                  if constexpr (TWO_NB)
                                      return ((jj - 1) & 1) ? scb2[i] : scb[i];
                                  return ONE_NB ? scb[i] : Sf[i] * sb_cur[jj - 1];
                              },
                              extra);
            });
            // last step: the next block's copies have landed everywhere (past the last block
            // of the workgroup the reads below are harmless and unused); in the one-barrier
            // form every wave has also finished reading this block's slots, which the next
            // block's refill takes
            wait_older_copies(true);
            if constexpr (ONE_BAR)
                lds_wait();
            bare_barrier();
            lds_wait();
            if constexpr (SN >= 2) {
                tie(Bf[bbuf(SN - 1, SN)][0]);
                tie(Bf[bbuf(SN - 1, SN)][1]);
            }
            if constexpr (MODE == MODE_DENSE) {
                if (c_now)
                    add_c_half(cq);
            }
            if (j == 0 && has_next) {
                nxt = finish_meta(nxt);
                nsel = scale_sel(nxt);
            }
            // the next block's fragments; after a tile's last block they are dropped (waited
            // for right after the loop) and the next tile's first block is read again after
            // the epilogue, so that no fragments are live next to the accumulators and the
            // epilogue's C (reading them under a condition instead would keep both the old
            // and the new fragments live across the branch)
            const uint32_t alo_n = a_lo + (uint32_t)(an * A_SLOT);
            const uint32_t ahi_n = a_hi + (uint32_t)(an * A_SLOT);
            const uint32_t sa_n = sa_lane + (uint32_t)(an * 1024);
            const uint32_t blo_n = b_lo + (uint32_t)(bslot_next * B_SLOT);
            const uint32_t bhi_n = b_hi + (uint32_t)(bslot_next * B_SLOT);
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
                                  read_sfb(an, sel);
                              if constexpr (i == SM - 1)  // after the last MFMA reading B(0)
                                  read_b(blo_n, bhi_n, C0, Bf[0]);
                          });
            } else {
                mfma_step(std::integral_constant<int, SN - 1>{}, Bf[bbuf(SN - 1, SN)],
                          [&](int i) {
                              if constexpr (TWO_NB) {
                                  psc[i] = ((SN - 1) & 1) ? scb2[i] : scb[i];
                                  return ((SN - 2) & 1) ? scb2[i] : scb[i];
                              }
                              psc[i] = ONE_NB ? scb[i] : Sf[i] * sb_cur[SN - 1];
                              return ONE_NB ? scb[i] : Sf[i] * sb_cur[SN - 2];
                          },
                          [&](auto I) {
                              constexpr int i = decltype(I)::value;
                              // B(0) (and B(1) when SN > 2) were last read steps ago; with
                              // SN == 2, B(1) is this step's and is replaced after its last MFMA
                              if constexpr (i == 0) {
                                  read_b(blo_n, bhi_n, C0, Bf[0]);
                                  read_sfb(an, sel);
                              }
                              if constexpr (i == (SN > 2 ? (SM > 1 ? 1 : 0) : SM - 1))
                                  read_b(blo_n, bhi_n, C1, Bf[1]);
                              read_a(alo_n, ahi_n, sa_n, I);
                          });
            }
            aslot = an;
            bslot = bslot_next;
        };
        // Blocks whose refills belong to this tile, then the last DEPTH blocks, whose refills
        // are the next tile's first blocks when it is prefetched (else nothing): each phase
        // holds one set of copy resources.
        // (One workgroup per tile: one loop, whose last DEPTH blocks refill from empty
        // resources.)
        if constexpr (PERSIST) {
            const int j_sw = nkb > DEPTH ? nkb - DEPTH : 0;
            {
                const CopySrc s1 = copy_src(cur);
                for (int j = 0; j < j_sw; ++j)
                    block(j, s1, j + DEPTH, s1);
            }
            {
                Tile u = nxt;
                u.empty = u.empty || !prefetch;
                const CopySrc s2 = copy_src(u);
                for (int j = j_sw; j < nkb; ++j)
                    block(j, s2, prefetch ? j + DEPTH - nkb : 0, s2);
            }
        } else {
            const CopySrc s1 = copy_src(cur);
            Tile e = cur;
            e.empty = true;
            const CopySrc s0 = copy_src(e);
            for (int j = 0; j < nkb; ++j) {
                const bool own = j + DEPTH < nkb;
                block(j, own ? s1 : s0, own ? j + DEPTH : 0, s1);
            }
        }
        // the fragments read during the last step land before their registers can be reused
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
        // the tile's last partials
        if constexpr (!DIRECT) {
#pragma unroll
            for (int i = 0; i < SM; ++i)
                if (MODE != MODE_MASKED || i < sm_act)
                    acc[i][SN - 1] += UE8 ? pend[i] : pend[i] * psc[i];
        }

        // ---- epilogue: + C (columns not streamed), round to bf16, store the valid rows from
        // registers (the LDS holds the next tile's first blocks)
        if constexpr (MODE == MODE_DENSE) {
            if (p.c) {
                v4f cv[SM][SN];
#pragma unroll
                for (int i = 0; i < SM; ++i)
#pragma unroll
                    for (int j = 0; j < SN; ++j)
                        cv[i][j] = c_streamed(j)
                                       ? v4f{0.f, 0.f, 0.f, 0.f}
                                       : __builtin_bit_cast(
                                             v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rc, c_lane + (uint32_t)((16 * i * N + 16 * j) * 4),
                                                      0, 0));
#pragma unroll
                for (int i = 0; i < SM; ++i)
#pragma unroll
                    for (int j = 0; j < SN; ++j)
                        acc[i][j] += cv[i][j];
            }
        }
        uint16_t *D = p.d + (MODE == MODE_MASKED ? (int64_t)cur.g * M * N : 0);
        if constexpr (SWIGLU) {
            // The activation step on the tile's FP32 results, with no rounding in between:
            // lane (fr, fg) of sub-tile pair pp holds gate (jj = 2 pp) and up (jj = 2 pp + 1) of
            // h columns c0 + (TN / 2) wave_n + 16 pp + 4 fg .. + 3 of row wm + 16 i + fr.  A
            // row's segment (the tile's 128 h columns) lies on its four lane groups and the WN
            // waves across: its maximum is a two-step butterfly over the lane groups, then a
            // pass through a small LDS area of its own.  Then, as the unfused activation step does,
            // scale = max(amax, 1e-4) / 448 and q = e4m3(h * 448 / max(amax, 1e-4)), stored for
            // the rows of the tile's group only, with the scales MN-major.
            if (!cur.empty) {
                constexpr int SP = SN / 2;
                const int wave_n = wave % WN;
                const int half = N >> 1;
                const int c0 = cur.n0 >> 1;
                // lane coordinates from an opaque copy of the thread id, and the rows' groups
                // loaded again here: nothing of the epilogue's is held through the K loop
                int et = tid;
                asm volatile("" : "+v"(et));
                const int efr = et & 15, efg = (et >> 4) & 3;
                // h replaces the gate values in the accumulators (no registers of its own)
#pragma unroll
                for (int i = 0; i < SM; ++i) {
                    float rmax = 0.f;
#pragma unroll
                    for (int pp = 0; pp < SP; ++pp) {
                        const v4f g = acc[i][2 * pp], u = acc[i][2 * pp + 1];
                        const v4f h = v4f{silu_times(g.x, u.x), silu_times(g.y, u.y),
                                          silu_times(g.z, u.z), silu_times(g.w, u.w)};
                        acc[i][2 * pp] = h;
                        rmax = fmaxf(rmax, fmaxf(fmaxf(fabsf(h.x), fabsf(h.y)),
                                                 fmaxf(fabsf(h.z), fabsf(h.w))));
                    }
                    rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
                    rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
                    if constexpr (AMX_ALIAS) {
                        // the area lies in the operand slots: every copy has landed (the last
                        // blocks' refills write zeros there) and every wave is past its reads
                        if (i == 0) {
                            wait_vm<0>();
                            bare_barrier();
                        }
                    }
                    if (efg == 0)
                        lds_write4(lds_base + AMX_BASE +
                                       (uint32_t)(((wm + 16 * i + efr) * WN + wave_n) * 4),
                                   rmax);
                }
                lds_wait();
                bare_barrier();  // every wave's maxima are in the LDS area
                // the WN maxima of each row: four in one 16-byte read, or two
                v4f am[SM];
#pragma unroll
                for (int i = 0; i < SM; ++i) {
                    const uint32_t at = lds_base + AMX_BASE + (uint32_t)((wm + 16 * i + efr) * WN * 4);
                    if constexpr (WN == 4) {
                        am[i] = lds_read16f_at<0>(at);
                    } else {
                        am[i].x = lds_read4_at<0>(at);
                        am[i].y = lds_read4_at<4>(at);
                    }
                }
                lds_wait();
                uint8_t *Q = p.q + (int64_t)(c0 + (TN / 2) * wave_n + 4 * efg);
#pragma unroll
                for (int i = 0; i < SM; ++i) {
                    tie(am[i]);
                    const float amax = WN == 4 ? fmaxf(fmaxf(am[i].x, am[i].y), fmaxf(am[i].z, am[i].w))
                                               : fmaxf(am[i].x, am[i].y);
                    const float floor_amax = fmaxf(amax, 1e-4f);
                    const float scale = floor_amax / 448.f;
                    const float inv = 448.f / floor_amax;
                    const int row = cur.m0 + wm + 16 * i + efr;
                    const bool ok = row < cur.row_limit && p.grp[row < M ? row : 0] == cur.g;
#pragma unroll
                    for (int pp = 0; pp < SP; ++pp) {
                        const v4f hh = acc[i][2 * pp];
                        const float y0 = fminf(fmaxf(hh.x * inv, -448.f), 448.f);
                        const float y1 = fminf(fmaxf(hh.y * inv, -448.f), 448.f);
                        const float y2 = fminf(fmaxf(hh.z * inv, -448.f), 448.f);
                        const float y3 = fminf(fmaxf(hh.w * inv, -448.f), 448.f);
                        int w = cvt_pk_e4m3<false>(y0, y1, 0);
                        w = cvt_pk_e4m3<true>(y2, y3, w);
                        if (ok)
                            store4_async(Q + (int64_t)row * half + 16 * pp, (uint32_t)w);
                    }
                    if (ok && wave_n == 0 && efg == 0)
                        store4_async(p.sfq + (int64_t)(c0 / KBLK) * p.ld_sfq + row,
                                     __float_as_uint(scale));
                }
            }
        } else if constexpr (PERSIST) {
            // from registers: the LDS holds the next tile's first blocks
            if (!cur.empty) {
#pragma unroll
                for (int i = 0; i < SM; ++i) {
                    const int row = cur.m0 + wm + 16 * i + fr;
                    bool ok = row < cur.row_limit;
                    if constexpr (CONTIG)
                        ok = ok && rowg[i] == cur.g;
#pragma unroll
                    for (int j = 0; j < SN; ++j) {
                        const int col = cur.n0 + wn + 16 * j + 4 * fg;
                        if (ok && col < N)
                            store8_async(D + (int64_t)row * N + col,
                                         pack_bf16x2(acc[i][j].x, acc[i][j].y),
                                         pack_bf16x2(acc[i][j].z, acc[i][j].w));
                    }
                }
            }
        } else {
            // Through LDS, free once every copy has landed (one tile per workgroup): each wave
            // writes its sub-tiles there as bf16 (8 bytes per lane), then every thread stores
            // whole 16-byte pieces of rows, so a wave's store covers contiguous row segments
            // instead of sixteen 32-byte pieces.  D is written once and never read here: the
            // stores are non-temporal, so they do not push A and B out of the L2.  Output rows are OS bytes apart in LDS; OS = 32
            // (mod 256) puts a fragment write's 16 rows x 32 bytes on distinct banks.
            constexpr int NT = 64 * NW;
            static_assert(rows_on_distinct_banks(OS), "output row stride");
            static_assert(BM * OS <= LDS_ALLOC, "output tile fits the LDS");
            constexpr int CPR = BN / 8;  // 16-byte pieces per output row
            static_assert((BM * CPR) % NT == 0, "output pieces split evenly over the threads");
            constexpr int PPT = BM * CPR / NT;  // pieces per thread
            // addresses from an opaque copy of the thread id: where a workgroup runs a tile
            // twice they are then formed here, not held in registers through the K loop
            int et = tid;
            asm volatile("" : "+v"(et));
            const int el = et & 63, ew = et >> 6;
            const int ewm = (ew / WN) * TM, ewn = (ew % WN) * TN;
            wait_vm<0>();
            bare_barrier();  // every wave is past its last fragment read and copy
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j)
                    lds_write8(lds_base + (uint32_t)((ewm + 16 * i + (el & 15)) * OS +
                                                     (ewn + 16 * j + 4 * (el >> 4)) * 2),
                               pack_bf16x2(acc[i][j].x, acc[i][j].y),
                               pack_bf16x2(acc[i][j].z, acc[i][j].w));
            lds_wait();
            bare_barrier();
            v4i piece[PPT];
#pragma unroll
            for (int t = 0; t < PPT; ++t) {
                const int q = et + t * NT;
                piece[t] = lds_read16(lds_base + (uint32_t)((q / CPR) * OS + (q % CPR) * 16));
            }
            int prow[PPT];
            if constexpr (CONTIG) {
#pragma unroll
                for (int t = 0; t < PPT; ++t) {
                    const int row = cur.m0 + (et + t * NT) / CPR;
                    prow[t] = (!TWO_GROUPS || row < M) ? p.grp[row] : -1;
                }
            }
            lds_wait();
            if (!cur.empty) {
#pragma unroll
                for (int t = 0; t < PPT; ++t) {
                    const int q = et + t * NT;
                    const int row = cur.m0 + q / CPR;
                    const int col = cur.n0 + (q % CPR) * 8;
                    bool ok = row < cur.row_limit && col < N;
                    if constexpr (CONTIG)
                        ok = ok && prow[t] == cur.g;
                    if (ok)
                        __builtin_nontemporal_store(
                            piece[t], reinterpret_cast<v4i *>(D + (int64_t)row * N + col));
                }
            }
        }
        if constexpr (TWO_GROUPS) {
            // a tile holding the rows of two groups runs again for the other group (its
            // epilogue writes only the rows of the group it ran for); its prologue copies
            // into the LDS that every wave has read its output pieces from
            if (cur.g2 >= 0) {
                cur.g = cur.g2;
                cur.g2 = -1;
                bare_barrier();
                first = true;
                continue;
            }
        }
        if (!has_next)
            break;
        // ---- on to the next tile
        tile_id += tile_step;
        cur = nxt;
        sel = nsel;
#pragma unroll
        for (int i = 0; i < SM; ++i)
            rowg[i] = rowg_next[i];
        sm_act = active_rows(cur);
        has_next = PERSIST && tile_id + tile_step < tile_end;
    }
    // no copy may still be writing LDS (or store still reading registers) past this point
    wait_vm<0>();
}

template <int BM, int BN, int WM, int WN, int DEPTH, int MODE, bool PERSIST, int SF>
__global__ __launch_bounds__(64 * WM * WN) void dg_gemm_kernel(GemmArgs p, int tiles_m,
                                                               int tiles_n)
{
    gemm_tiles<BM, BN, WM, WN, DEPTH, MODE, PERSIST, SF>(p, tiles_m, tiles_n, (int)blockIdx.x,
                                                         (int)gridDim.x);
}

// The contiguous form's 256 x 256 tiles and their tail in one launch: workgroups below
// main_wgs run the 256 x 256 tiles (straddle workgroups first), those from main_wgs rounded up
// to a whole XCD round the tail's tiles (persistent), in one LDS allocation both fit: 128 x 128
// tiles (eight waves, copies four blocks ahead), or for the fused activation step 128 x 256
// (eight waves, four across).  The tail workgroups come last in the grid, so they are
// dispatched as the 256 x 256 tiles' CUs free up; where they find no tail tiles they exit at
// once.
constexpr int tail_sub_tiles(int mode) { return mode == MODE_CONTIG_SWIGLU ? 2 : 4; }
template <int MODE, int SF>
__global__ __launch_bounds__(512) void dg_gemm_contig_tail_kernel(GemmArgs p, int tiles_m,
                                                                  int tiles_n, int main_wgs)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[160 * 1024];
    const int wg = (int)blockIdx.x;
    const int tail0 = (main_wgs + 7) & ~7;
    if (wg < main_wgs) {
        gemm_tiles<256, 256, 4, 2, 2, MODE, false, SF, true>(p, tiles_m, tiles_n, wg, main_wgs,
                                                             lds);
    } else if (wg >= tail0) {
        if constexpr (MODE == MODE_CONTIG_SWIGLU)
            gemm_tiles<128, 256, 2, 4, 2, MODE, true, SF, true>(
                p, 2 * tiles_m, tiles_n, wg - tail0, (int)gridDim.x - tail0, lds);
        else
            gemm_tiles<128, 128, 2, 4, 4, MODE, true, SF, true>(
                p, 2 * tiles_m, 2 * tiles_n, wg - tail0, (int)gridDim.x - tail0, lds);
    }
}

// ------------------------------------------------------------------------------ host side

static void tiles_for(int cfg, const GemmArgs &a, int &tiles_m, int &tiles_n)
{
    const TileInfo &ti = kTiles[cfg];
    tiles_n = (a.n + ti.bn - 1) / ti.bn;
    tiles_m = (a.m + ti.bm - 1) / ti.bm;
}

// Workgroups for `total` tiles: one per tile, or for a persistent tile configuration at most
// one per CU (each then loops over its share; xcd_tile_range forms the shares in 64 bits)
static int64_t workgroups(int64_t total, bool persistent, const GemmArgs &a)
{
    if (persistent && a.max_wgs > 0 && total > a.max_wgs)
        return a.max_wgs;
    return total;
}

// Workgroups ahead of the tiles that serve listed straddling tile-rows (contiguous form,
// 256-row tiles, one workgroup per tile), rounded up to whole rounds of the 8 XCDs
static int64_t straddle_wgs(int mode, int bm, bool persistent, const GemmArgs &a, int tiles_n)
{
    if ((mode != MODE_CONTIG && mode != MODE_CONTIG_SWIGLU) || bm <= 128 || persistent ||
        a.straddle_rows <= 0)
        return 0;
    return ((int64_t)a.straddle_rows * tiles_n + 7) / 8 * 8;
}

// Tiles a launch sizes its grid for: the tile grid (times the groups, masked).  -1: the tail
// fields set (they go to launch_contig_tail only).
static int64_t launch_tiles(int mode, const GemmArgs &a, int tiles_m, int tiles_n)
{
    if (a.tail_cus > 0)
        return -1;
    int64_t g = (int64_t)tiles_m * tiles_n;
    if (mode == MODE_MASKED)
        g *= a.num_groups;
    return g;
}

int64_t grid_size(int mode, int cfg, const GemmArgs &a)
{
    if (cfg == CFG_STREAM64)
        return mode == MODE_DENSE ? stream_grid_size(a) : -1;
    int tiles_m, tiles_n;
    tiles_for(cfg, a, tiles_m, tiles_n);
    const TileInfo &ti = kTiles[cfg];
    const int64_t g = launch_tiles(mode, a, tiles_m, tiles_n);
    if (g <= 0)
        return -1;
    return workgroups(g, ti.persistent, a) + straddle_wgs(mode, ti.bm, ti.persistent, a, tiles_n);
}

template <int BM, int BN, int WM, int WN, int DEPTH, bool PERSIST, int SF>
static bool launch_modes(int mode, dim3 g, dim3 b, const GemmArgs &a, int tiles_m, int tiles_n,
                         hipStream_t stream)
{
    // (the UE8M0 variants are built for the forms that use them: direct accumulation for
    // dense and contiguous, partials for dense and masked)
    switch (mode) {
    case MODE_DENSE:
        hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, DEPTH, MODE_DENSE, PERSIST, SF>), g, b, 0,
                           stream, a, tiles_m, tiles_n);
        return true;
    case MODE_CONTIG:
        if constexpr (SF != SF_UE8M0_PARTIAL && !(BM > 128 && PERSIST)) {
            hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, DEPTH, MODE_CONTIG, PERSIST, SF>), g,
                               b, 0, stream, a, tiles_m, tiles_n);
            return true;
        }
        return false;
    case MODE_MASKED:
        if constexpr (SF != SF_UE8M0) {
            hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, DEPTH, MODE_MASKED, PERSIST, SF>), g,
                               b, 0, stream, a, tiles_m, tiles_n);
            return true;
        }
        return false;
    case MODE_CONTIG_SWIGLU:
        // (built for the tiles it runs on: 128 x 256 persistent and 256 x 256, eight waves,
        // FP32 scales)
        if constexpr (SF == SF_FP32 && BN == 256 && WM * WN == 8 &&
                      ((PERSIST && BM == 128 && WN == 4) || (!PERSIST && BM == 256 && WN == 2))) {
            hipLaunchKernelGGL(
                (dg_gemm_kernel<BM, BN, WM, WN, DEPTH, MODE_CONTIG_SWIGLU, PERSIST, SF>), g, b, 0,
                stream, a, tiles_m, tiles_n);
            return true;
        }
        return false;
    default:
        return false;
    }
}

template <int BM, int BN, int WM, int WN, int DEPTH = 2, bool PERSIST = true>
static hipError_t launch_cfg(int mode, const GemmArgs &a, hipStream_t stream)
{
    int tiles_m, tiles_n;
    const int cfg_threads = 64 * WM * WN;
    tiles_n = (a.n + BN - 1) / BN;
    // (contiguous: m is a multiple of 128; a 256-row tile past it reads no group indices there)
    tiles_m = (a.m + BM - 1) / BM;
    if (mode == MODE_CONTIG && BM > 128 && PERSIST)
        return hipErrorInvalidConfiguration;  // straddling tiles need one workgroup per tile
    const int64_t total = launch_tiles(mode, a, tiles_m, tiles_n);
    if (total <= 0 || total > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const int64_t grid = workgroups(total, PERSIST, a) + straddle_wgs(mode, BM, PERSIST, a, tiles_n);
    dim3 g((unsigned)grid), b(cfg_threads);
    // UE8M0: MFMAs accumulate directly unless C is added inside the K loop or masked rows
    // skip MFMAs
    bool launched;
    if (a.sf_fmt == SF_UE8M0 && (mode == MODE_CONTIG || (mode == MODE_DENSE && !a.c)))
        launched = launch_modes<BM, BN, WM, WN, DEPTH, PERSIST, SF_UE8M0>(mode, g, b, a, tiles_m,
                                                                          tiles_n, stream);
    else if (a.sf_fmt == SF_UE8M0)
        launched = launch_modes<BM, BN, WM, WN, DEPTH, PERSIST, SF_UE8M0_PARTIAL>(
            mode, g, b, a, tiles_m, tiles_n, stream);
    else
        launched = launch_modes<BM, BN, WM, WN, DEPTH, PERSIST, SF_FP32>(mode, g, b, a, tiles_m,
                                                                         tiles_n, stream);
    if (!launched)
        return hipErrorInvalidConfiguration;  // no kernel of this form for this tile
    return hipGetLastError();
}

int64_t contig_tail_grid(int mode, const GemmArgs &a)
{
    const int tiles_m = (a.m + 255) / 256, tiles_n = (a.n + 255) / 256;
    const int64_t main_wgs =
        (int64_t)tiles_m * tiles_n + straddle_wgs(mode, 256, false, a, tiles_n);
    return (main_wgs + 7) / 8 * 8 + workgroups((int64_t)tail_sub_tiles(mode) * a.tail_max, true, a);
}

hipError_t launch_contig_tail(int mode, const GemmArgs &a, hipStream_t stream)
{
    if (a.tail_cus <= 0 || a.tail_max <= 0 || a.tail_tm <= 0 || a.tail_tn <= 0 ||
        (mode != MODE_CONTIG && mode != MODE_CONTIG_SWIGLU) ||
        (a.sf_fmt != SF_FP32 && (mode != MODE_CONTIG || a.sf_fmt != SF_UE8M0)))
        return hipErrorInvalidConfiguration;
    const int tiles_m = (a.m + 255) / 256, tiles_n = (a.n + 255) / 256;
    const int64_t main_wgs =
        (int64_t)tiles_m * tiles_n + straddle_wgs(mode, 256, false, a, tiles_n);
    const int64_t grid = contig_tail_grid(mode, a);
    if (tiles_m != a.tail_tm || tiles_n != a.tail_tn || grid <= 0 || grid > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const dim3 g((unsigned)grid), b(512);
    if (mode == MODE_CONTIG_SWIGLU)
        hipLaunchKernelGGL((dg_gemm_contig_tail_kernel<MODE_CONTIG_SWIGLU, SF_FP32>), g, b, 0,
                           stream, a, tiles_m, tiles_n, (int)main_wgs);
    else if (a.sf_fmt == SF_UE8M0)
        hipLaunchKernelGGL((dg_gemm_contig_tail_kernel<MODE_CONTIG, SF_UE8M0>), g, b, 0, stream,
                           a, tiles_m, tiles_n, (int)main_wgs);
    else
        hipLaunchKernelGGL((dg_gemm_contig_tail_kernel<MODE_CONTIG, SF_FP32>), g, b, 0, stream, a,
                           tiles_m, tiles_n, (int)main_wgs);
    return hipGetLastError();
}

hipError_t launch_gemm(int mode, int cfg, const GemmArgs &a, hipStream_t stream)
{
    switch (cfg) {
    case CFG_256x224:
        return launch_cfg<256, 224, 4, 2, 2, false>(mode, a, stream);
    case CFG_128x256:
        return launch_cfg<128, 256, 2, 2>(mode, a, stream);
    case CFG_128x128:
        return launch_cfg<128, 128, 2, 2>(mode, a, stream);
    case CFG_64x32:
        return launch_cfg<64, 32, 2, 2>(mode, a, stream);
    case CFG_256x128:
        return launch_cfg<256, 128, 4, 2, 2, false>(mode, a, stream);
    case CFG_256x256:
        return launch_cfg<256, 256, 4, 2, 2, false>(mode, a, stream);
    case CFG_256x128p:
        return launch_cfg<256, 128, 4, 2, 2, true>(mode, a, stream);
    case CFG_128x128d4:
        return launch_cfg<128, 128, 2, 2, 4, true>(mode, a, stream);
    case CFG_128x128w8d4:
        return launch_cfg<128, 128, 2, 4, 4, true>(mode, a, stream);
    case CFG_128x256w8:
        return launch_cfg<128, 256, 2, 4>(mode, a, stream);
    case CFG_STREAM64:
        return mode == MODE_DENSE ? launch_stream(a, stream) : hipErrorInvalidValue;
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace dg
