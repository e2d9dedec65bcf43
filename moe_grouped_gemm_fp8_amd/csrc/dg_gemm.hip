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
//  * Every global read of the main loop (A, B and the A scales) is a gfx950 direct-to-LDS
//    copy (global_load_lds_dwordx4): nothing in flight targets registers, so the only waits
//    are explicit ones.  Copies run through a ring of RING half-block slots (64 K-bytes of
//    the A and B tiles each), giving (RING - 2) halves of look-ahead with one barrier per
//    K block.  Barriers are bare s_barrier (no release fence, which would drain the ring).
//  * LDS rows are 64 bytes; the 16-byte chunk c of row r sits at chunk c ^ ((r >> 2) & 3),
//    so a 16-lane fragment read (16 consecutive rows, one chunk) touches 16 distinct 16-byte
//    bank groups.  A copy writes 1 KB contiguously per wave, so the swizzle is applied by
//    choosing which global chunk each lane fetches.  Fragment reads are inline-asm
//    ds_read_b128 with explicit lgkmcnt waits, so the compiler never pairs an LDS read with
//    the in-flight copies and drains them.
//  * Workgroup ids are remapped so that each XCD (ids are dealt round-robin over the 8 XCDs)
//    runs a contiguous range of tiles, rastered in groups of 4 M-tiles, so tiles that run
//    together on one XCD share A rows and B columns in that XCD's L2.
//  * Skinny dense shapes split K over workgroups: each writes an FP32 partial tile and the
//    last one to arrive (atomic counter) sums the partials in split order and writes D.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
#define DG_LDS __attribute__((address_space(3)))
#define DG_CONST __attribute__((address_space(4)))  // read-only for the kernel: scalar loads

constexpr int KBLK = 128;   // K block = scale granularity = MFMA depth
constexpr int HALF = 64;    // K bytes per ring slot
constexpr int GROUP_M = 4;  // tile raster: M-tiles per group

const TileInfo kTiles[CFG_COUNT] = {
    {256, 224, 512, "256x224w8"},
    {128, 256, 256, "128x256w4"},
    {128, 128, 256, "128x128w4"},
    {64, 32, 256, "64x32w4"},
    {256, 128, 512, "256x128w8"},
};

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)  // NaN: keep it a (quiet) NaN
        return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ void store_bf16x4(uint16_t *dst, v4f v)
{
    uint32_t lo = f32_to_bf16_rne(v.x) | (f32_to_bf16_rne(v.y) << 16);
    uint32_t hi = f32_to_bf16_rne(v.z) | (f32_to_bf16_rne(v.w) << 16);
    *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Same, for a wave-uniform count known only at run time (anything above 31 waits for all).
__device__ __forceinline__ void wait_vm_dyn(int n)
{
    switch (n) {
#define DG_WAIT_CASE(k) \
    case k:             \
        wait_vm<k>();   \
        break;
        DG_WAIT_CASE(1) DG_WAIT_CASE(2) DG_WAIT_CASE(3) DG_WAIT_CASE(4) DG_WAIT_CASE(5)
        DG_WAIT_CASE(6) DG_WAIT_CASE(7) DG_WAIT_CASE(8) DG_WAIT_CASE(9) DG_WAIT_CASE(10)
        DG_WAIT_CASE(11) DG_WAIT_CASE(12) DG_WAIT_CASE(13) DG_WAIT_CASE(14) DG_WAIT_CASE(15)
        DG_WAIT_CASE(16) DG_WAIT_CASE(17) DG_WAIT_CASE(18) DG_WAIT_CASE(19) DG_WAIT_CASE(20)
        DG_WAIT_CASE(21) DG_WAIT_CASE(22) DG_WAIT_CASE(23) DG_WAIT_CASE(24) DG_WAIT_CASE(25)
        DG_WAIT_CASE(26) DG_WAIT_CASE(27) DG_WAIT_CASE(28) DG_WAIT_CASE(29) DG_WAIT_CASE(30)
        DG_WAIT_CASE(31)
#undef DG_WAIT_CASE
    default:
        wait_vm<0>();
        break;
    }
}

__device__ __forceinline__ void bare_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS reads issued as inline asm (see the header comment).  Their results are valid only
// after lds_wait() followed by tie() on each result, which orders every use after the wait.
__device__ __forceinline__ v4i lds_read16(uint32_t addr)
{
    v4i v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

__device__ __forceinline__ float lds_read4(uint32_t addr)
{
    float v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// All but the N most recent LDS reads have landed (LDS reads retire in order; outstanding
// scalar loads only make the condition stricter).
template <int N>
__device__ __forceinline__ void lds_wait_n()
{
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}
// lds_wait_n for a count that is a constant only after loop unrolling
__device__ __forceinline__ void lds_wait_le(int n)
{
    switch (n) {
#define DG_LGKM_CASE(k)    \
    case k:                \
        lds_wait_n<k>();   \
        break;
        DG_LGKM_CASE(1) DG_LGKM_CASE(2) DG_LGKM_CASE(3) DG_LGKM_CASE(4) DG_LGKM_CASE(5)
        DG_LGKM_CASE(6) DG_LGKM_CASE(7) DG_LGKM_CASE(8) DG_LGKM_CASE(9) DG_LGKM_CASE(10)
        DG_LGKM_CASE(11) DG_LGKM_CASE(12) DG_LGKM_CASE(13) DG_LGKM_CASE(14) DG_LGKM_CASE(15)
#undef DG_LGKM_CASE
    default:
        lds_wait_n<0>();
        break;
    }
}
__device__ __forceinline__ void tie(v4i &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void tie(float &v) { asm volatile("" : "+v"(v)); }

// Workgroup id -> tile id such that XCD x (ids x, x+8, x+16, ...) gets one contiguous range.
__device__ __forceinline__ int xcd_remap(int bid, int nblk)
{
    int q = nblk >> 3, r = nblk & 7, xcd = bid & 7, loc = bid >> 3;
    return (xcd < r) ? xcd * (q + 1) + loc : r * (q + 1) + (xcd - r) * q + loc;
}

// Tile id -> (tm, tn) in groups of GROUP_M M-tiles, N fastest within a group column.
__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n, int &tm, int &tn)
{
    int per_group = GROUP_M * tiles_n;
    int grp = t / per_group;
    int first = grp * GROUP_M;
    int gsz = min(tiles_m - first, GROUP_M);
    int rem = t - grp * per_group;
    tm = first + rem % gsz;
    tn = rem / gsz;
}

template <int BM, int BN, int WM, int WN, int RING, int MODE>
__global__ __launch_bounds__(64 * WM * WN) void dg_gemm_kernel(GemmArgs p, int tiles_m,
                                                               int tiles_n)
{
    constexpr int NW = WM * WN;
    constexpr int NT = 64 * NW;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int SM = TM / 16, SN = TN / 16;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be 16-aligned");
    static_assert(BM % 16 == 0 && BN % 16 == 0 && BM <= 256, "tile shape");
    static_assert(RING >= 4 && RING <= 9, "ring depth");
    constexpr int IA = BM / 16;                   // 1 KB copies per slot: A rows (16 per copy)
    constexpr int IB = BN / 16;                   //                         B rows
    constexpr int ICOPY = IA + IB + 1;            // + the block's A scales (64 x 16 bytes)
    constexpr int MAXI = (ICOPY + NW - 1) / NW;   // copies per wave per slot (padded)
    constexpr int SA_OFF = (BM + BN) * HALF;      // A scales inside a slot
    constexpr int HSLOT = SA_OFF + 1024;          // bytes per ring slot
    static_assert(MAXI * (RING - 2) < 64, "outstanding copies must fit vmcnt");

    __shared__ __attribute__((aligned(1024))) uint8_t lds_ring[RING * HSLOT];
    __shared__ int s_flag;

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
    int tm, tn, split = 0, g = 0, row_limit;
    int kb0 = 0, kb1 = KB;
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
            if (v >= 0 && v < p.num_groups)
                atomicMax(&s_flag, v);
        }
        __syncthreads();
        g = s_flag;
        if (g < 0)
            return;  // a block of padding rows only
        row_limit = p.m;
    } else {
        if (p.splits > 1) {
            split = t % p.splits;
            t /= p.splits;
            kb0 = split * KB / p.splits;
            kb1 = (split + 1) * KB / p.splits;
        }
        raster(t, tiles_m, tiles_n, tm, tn);
        row_limit = p.m;
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const uint8_t *B = p.b + (int64_t)g * N * K;
    // B scales are wave-uniform and never written by the kernel: read them through the
    // constant address space so they become scalar loads
    const DG_CONST float *SFB = (const DG_CONST float *)(p.sfb + (int64_t)g * NB * KB);
    const int nkb = kb1 - kb0;
    const int nhalf = 2 * nkb;

    // ---- this wave's copies of one ring slot.  Copy q of a slot is A rows [16q, 16q+16)
    // for q < IA, B rows [16(q-IA), ...) for q < IA+IB, and the block's A scales (64 lanes x
    // 4 rows, rows clamped to the allocation) for q == IA+IB; both halves of a block carry
    // the scales.  Waves with fewer real copies repeat one (same bytes to the same place),
    // so every wave issues MAXI copies per slot and the waits are compile-time constants.
    // Lane l of a row copy fetches row 16q' + l/4, logical chunk (l & 3) ^ ((row >> 2) & 3):
    // the swizzled layout.  Rows past the valid range are clamped to the last valid row so
    // every read stays inside its operand; the rows they feed are never stored.
    // per copy: a wave-uniform base, K-block stride, half offset and LDS destination, and a
    // 32-bit per-lane offset (the only per-lane part)
    const uint8_t *a_tile = A + (int64_t)m0 * K;
    const uint8_t *b_tile = B + (int64_t)n0 * K;
    const uint8_t *cbase[MAXI];
    int64_t cstride[MAXI];  // bytes per K block
    int choff[MAXI];        // bytes per half block
    int cdst[MAXI];         // byte offset inside a slot
    uint32_t coff[MAXI];    // per-lane byte offset from cbase
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const int q = (wave + i * NW) % ICOPY;
        const int sub = lane >> 2, pc = lane & 3;
        if (q < IA) {
            const int r = 16 * q + sub;
            const int gr = min(m0 + r, row_limit - 1);
            cbase[i] = a_tile;
            coff[i] = (uint32_t)(gr - m0) * (uint32_t)K + ((pc ^ ((r >> 2) & 3)) << 4);
            cstride[i] = KBLK;
            choff[i] = HALF;
            cdst[i] = q * 1024;
        } else if (q < IA + IB) {
            const int r = 16 * (q - IA) + sub;
            const int gr = min(n0 + r, N - 1);
            cbase[i] = b_tile;
            coff[i] = (uint32_t)(gr - n0) * (uint32_t)K + ((pc ^ ((r >> 2) & 3)) << 4);
            cstride[i] = KBLK;
            choff[i] = HALF;
            cdst[i] = BM * HALF + (q - IA) * 1024;
        } else {
            const int64_t r4 = min((int64_t)m0 + 4 * lane, ld - 4);
            cbase[i] = (const uint8_t *)SFA;
            coff[i] = (uint32_t)(r4 * 4);
            cstride[i] = ld * 4;
            choff[i] = 0;
            cdst[i] = SA_OFF;
        }
    }
    DG_LDS uint8_t *ring = (DG_LDS uint8_t *)lds_ring;
    auto issue_half = [&](int h, int slot) {
        const int64_t kb = kb0 + (h >> 1);
        const int hb = h & 1;
#pragma unroll
        for (int i = 0; i < MAXI; ++i)
            __builtin_amdgcn_global_load_lds(
                (const void *)(cbase[i] + kb * cstride[i] + hb * choff[i] + coff[i]),
                (DG_LDS void *)(ring + slot * HSLOT + cdst[i]), 16, 0, 0);
    };

    int sb_off[SN];
#pragma unroll
    for (int j = 0; j < SN; ++j)
        sb_off[j] = __builtin_amdgcn_readfirstlane((min(n0 + wn + 16 * j, N - 1) / KBLK) * KB);

    // a wave whose rows are all invalid (masked tail, ragged M) skips the MFMA work but still
    // issues its copies, so the ring is filled the same way for every wave
    const bool wave_active = (m0 + wm) < row_limit;

    // per-lane fragment addresses inside a slot: lanes 16g..16g+15 hold K bytes [32g, 32g+32)
    // of 16 rows: half g/2 of the block, logical chunks 2(g%2) and 2(g%2)+1
    const int fr = lane & 15;
    const int fc = 2 * ((lane >> 4) & 1);
    const int fsw = (fr >> 2) & 3;
    const uint32_t lo_off = (uint32_t)((fc ^ fsw) << 4), hi_off = (uint32_t)(((fc + 1) ^ fsw) << 4);
    const uint32_t a_row_off = (uint32_t)(wm + fr) * HALF;
    const uint32_t b_row_off = (uint32_t)(BM + wn + fr) * HALF;
    const uint32_t sa_off = SA_OFF + (uint32_t)(wm + fr) * 4;
    const uint32_t ring_base = (uint32_t)(uintptr_t)ring;
    const bool upper = (lane >> 5) & 1;  // this lane reads the block's second half

    v4f acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // prologue: halves 0 .. RING-2 into slots 0 .. RING-2
    int issue_slot = 0;
    for (int h = 0; h < RING - 1 && h < nhalf; ++h) {
        issue_half(h, issue_slot);
        issue_slot = issue_slot + 1 == RING ? 0 : issue_slot + 1;
    }
    float sb_cur[SN], sb_nxt[SN];
#pragma unroll
    for (int jj = 0; jj < SN; ++jj)
        sb_cur[jj] = SFB[sb_off[jj] + kb0];

    int read_slot = 0;  // slot of half 2j
    for (int j = 0; j < nkb; ++j) {
        // block j needs halves 2j and 2j+1; everything issued after them may stay in flight
        const int issued_hi = min(j == 0 ? RING - 2 : 2 * j + RING - 3, nhalf - 1);
        const int pending = issued_hi - (2 * j + 1);
        if (pending == RING - 4 && j > 0) {
            wait_vm<MAXI *(RING - 4)>();  // steady state
        } else {
            switch (pending) {
            case 0: wait_vm<0>(); break;
            case 1: wait_vm<MAXI>(); break;
            case 2: wait_vm<MAXI * 2>(); break;
            case 3: wait_vm<MAXI * 3>(); break;
            case 4: wait_vm<(MAXI * 4 < 64 ? MAXI * 4 : 0)>(); break;
            case 5: wait_vm<(MAXI * 5 < 64 ? MAXI * 5 : 0)>(); break;
            case 6: wait_vm<(MAXI * 6 < 64 ? MAXI * 6 : 0)>(); break;
            default: wait_vm<0>(); break;
            }
        }
        bare_barrier();  // all copies of block j have landed; block j-1's slots are free
        // this block refills the ring with half RING-1 (block 0) or halves 2j+RING-2 and
        // 2j+RING-1
        const int h_first = (j == 0) ? RING - 1 : 2 * j + RING - 2;
        const int n_iss = max(0, min((j == 0) ? 1 : 2, nhalf - h_first));
        auto issue_copy = [&](int c) {  // c is a constant after unrolling
            const int e = c / MAXI, i = c % MAXI;
            if (e < n_iss) {
                const int h = h_first + e;
                const int slot = issue_slot + e >= RING ? issue_slot + e - RING : issue_slot + e;
                // the address is formed at the issue point (kept from being hoisted and held
                // in registers across the MFMA steps)
                uint32_t o = coff[i];
                asm volatile("" : "+v"(o));
                __builtin_amdgcn_global_load_lds(
                    (const void *)(cbase[i] + (int64_t)(kb0 + (h >> 1)) * cstride[i] +
                                   (h & 1) * choff[i] + o),
                    (DG_LDS void *)(ring + slot * HSLOT + cdst[i]), 16, 0, 0);
            }
        };
        const int kb = kb0 + j;
        if (j + 1 < nkb) {  // B scales of the next block, one iteration ahead
#pragma unroll
            for (int jj = 0; jj < SN; ++jj)
                sb_nxt[jj] = SFB[sb_off[jj] + kb + 1];
        }
        if (wave_active) {
            const int slot1 = read_slot + 1 == RING ? 0 : read_slot + 1;
            const uint32_t base = ring_base + (upper ? slot1 : read_slot) * HSLOT;
            const uint32_t sa_addr = ring_base + read_slot * HSLOT + sa_off;
            // Reads go out in the order B(0), then (A_i, A-scale_i) per sub-tile, then B(1);
            // the first step waits for each A_i separately (LDS reads retire in order), so
            // the MFMAs start as soon as their own operands land instead of after the whole
            // burst that every wave issues right after the barrier.
            static_assert(3 * (SM - 1) + 4 < 16, "lgkmcnt range");
            v4i blo[SN], bhi[SN];
            blo[0] = lds_read16(base + b_row_off + lo_off);
            bhi[0] = lds_read16(base + b_row_off + hi_off);
            v4i alo[SM], ahi[SM];
            float sav[SM];
#pragma unroll
            for (int i = 0; i < SM; ++i) {
                alo[i] = lds_read16(base + a_row_off + i * 1024 + lo_off);
                ahi[i] = lds_read16(base + a_row_off + i * 1024 + hi_off);
                sav[i] = lds_read4(sa_addr + i * 64);
            }
            if constexpr (SN > 1) {
                blo[1] = lds_read16(base + b_row_off + 1024 + lo_off);
                bhi[1] = lds_read16(base + b_row_off + 1024 + hi_off);
            }
            // ring refill: after the block's first LDS reads so those are not queued behind
            // the copies (each copy holds the wave's in-order issue until accepted)
#pragma unroll
            for (int c = 0; c < 2 * MAXI; ++c)
                issue_copy(c);
            // Step jj issues the SM MFMAs of fragment jj, each followed by the promotion of
            // the partial of fragment jj-1 in the same row (issued SM MFMAs earlier, so its
            // result is ready), with the reads of fragment jj+2 in flight.  The schedule
            // barriers keep that interleave: the compiler would otherwise cluster the MFMAs.
            v4f pend[SM];
            // reads issued after the A reads and before the first step's waits: B(1), B(2)
            constexpr int B1 = (SN > 1 ? 2 : 0) + (SN > 2 ? 2 : 0);
#pragma unroll
            for (int jj = 0; jj < SN; ++jj) {
                const v8i bf = v8i{blo[jj].x, blo[jj].y, blo[jj].z, blo[jj].w,
                                   bhi[jj].x, bhi[jj].y, bhi[jj].z, bhi[jj].w};
                if (jj + 2 < SN) {
                    blo[jj + 2] = lds_read16(base + b_row_off + (jj + 2) * 1024 + lo_off);
                    bhi[jj + 2] = lds_read16(base + b_row_off + (jj + 2) * 1024 + hi_off);
                }
                v4f part[SM];
#pragma unroll
                for (int i = 0; i < SM; ++i) {
                    if (jj == 0) {  // B(0) and A_i have landed once only younger reads remain
                        lds_wait_le(3 * (SM - 1 - i) + B1);
                        if (i == 0) {
                            tie(blo[0]);
                            tie(bhi[0]);
                        }
                        tie(alo[i]);
                        tie(ahi[i]);
                        tie(sav[i]);
                    }
                    const v8i af = v8i{alo[i].x, alo[i].y, alo[i].z, alo[i].w,
                                       ahi[i].x, ahi[i].y, ahi[i].z, ahi[i].w};
                    part[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        bf, af, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                    if (jj > 0)
                        acc[i][jj - 1] += pend[i] * (sav[i] * sb_cur[jj - 1]);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int i = 0; i < SM; ++i)
                    pend[i] = part[i];
                if (jj + 1 < SN) {
                    if (jj + 2 < SN)
                        lds_wait_n<2>();  // B(jj+1) has landed, B(jj+2) may be in flight
                    else
                        lds_wait_n<0>();
                    tie(blo[jj + 1]);
                    tie(bhi[jj + 1]);
                }
            }
#pragma unroll
            for (int i = 0; i < SM; ++i)
                acc[i][SN - 1] += pend[i] * (sav[i] * sb_cur[SN - 1]);
        } else {
#pragma unroll
            for (int c = 0; c < 2 * MAXI; ++c)
                issue_copy(c);
        }
        issue_slot += n_iss;
        if (issue_slot >= RING)
            issue_slot -= RING;
        if (j + 1 < nkb) {
#pragma unroll
            for (int jj = 0; jj < SN; ++jj)
                sb_cur[jj] = sb_nxt[jj];
        }
        read_slot = read_slot + 2 >= RING ? read_slot + 2 - RING : read_slot + 2;
    }
    wait_vm<0>();  // no copy may still be writing LDS past this point

    // ---- split-K: publish the partial tile; the last arriving workgroup reduces in order
    if constexpr (MODE == MODE_DENSE) {
        if (p.splits > 1) {
            const int tile = tm * tiles_n + tn;
            float *ws_tile = p.ws + (int64_t)tile * p.splits * (BM * BN);
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j)
                    *reinterpret_cast<v4f *>(ws_tile + (int64_t)split * BM * BN +
                                             ((i * SN + j) * NT + tid) * 4) = acc[i][j];
            __threadfence();
            __syncthreads();
            if (tid == 0) {
                int prev = atomicAdd(p.counters + tile, 1);
                int last = prev == p.splits - 1;
                if (last)
                    atomicExch(p.counters + tile, 0);  // ready for the next call
                s_flag = last;
            }
            __syncthreads();
            if (!s_flag)
                return;
            __threadfence();
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j) {
                    v4f sum = v4f{0.f, 0.f, 0.f, 0.f};
                    for (int s = 0; s < p.splits; ++s)
                        sum += *reinterpret_cast<const v4f *>(
                            ws_tile + (int64_t)s * BM * BN + ((i * SN + j) * NT + tid) * 4);
                    acc[i][j] = sum;
                }
        }
    }

    // ---- epilogue: + C, round to bf16, store the valid rows
#pragma unroll
    for (int i = 0; i < SM; ++i) {
        const int row = m0 + wm + 16 * i + (lane & 15);
        bool row_ok = row < row_limit;
        if constexpr (MODE == MODE_CONTIG)
            row_ok = p.grp[row] == g;
        if (!row_ok)
            continue;
#pragma unroll
        for (int j = 0; j < SN; ++j) {
            const int col = n0 + wn + 16 * j + 4 * (lane >> 4);
            if (col >= N)
                continue;
            v4f v = acc[i][j];
            if constexpr (MODE == MODE_DENSE) {
                if (p.c)
                    v += *reinterpret_cast<const v4f *>(p.c + (int64_t)row * N + col);
            }
            store_bf16x4(D + (int64_t)row * N + col, v);
        }
    }
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
    int tiles_m, tiles_n;
    tiles_for(mode, cfg, a, tiles_m, tiles_n);
    int64_t g = (int64_t)tiles_m * tiles_n;
    if (mode == MODE_MASKED)
        g *= a.num_groups;
    if (mode == MODE_DENSE)
        g *= a.splits;
    return g;
}

template <int BM, int BN, int WM, int WN, int RING>
static hipError_t launch_cfg(int mode, const GemmArgs &a, hipStream_t stream)
{
    int tiles_m, tiles_n;
    const int cfg_threads = 64 * WM * WN;
    tiles_n = (a.n + BN - 1) / BN;
    tiles_m = mode == MODE_CONTIG ? a.m / BM : (a.m + BM - 1) / BM;
    int64_t grid = (int64_t)tiles_m * tiles_n;
    if (mode == MODE_MASKED)
        grid *= a.num_groups;
    if (mode == MODE_DENSE)
        grid *= a.splits;
    if (grid <= 0 || grid > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    dim3 g((unsigned)grid), b(cfg_threads);
    switch (mode) {
    case MODE_DENSE:
        hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, RING, MODE_DENSE>), g, b, 0, stream, a,
                           tiles_m, tiles_n);
        break;
    case MODE_CONTIG:
        hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, RING, MODE_CONTIG>), g, b, 0, stream, a,
                           tiles_m, tiles_n);
        break;
    default:
        hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, RING, MODE_MASKED>), g, b, 0, stream, a,
                           tiles_m, tiles_n);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm(int mode, int cfg, const GemmArgs &a, hipStream_t stream)
{
    switch (cfg) {
    case CFG_256x224:
        return launch_cfg<256, 224, 4, 2, 5>(mode, a, stream);
    case CFG_128x256:
        return launch_cfg<128, 256, 2, 2, 6>(mode, a, stream);
    case CFG_128x128:
        return launch_cfg<128, 128, 2, 2, 6>(mode, a, stream);
    case CFG_64x32:
        return launch_cfg<64, 32, 2, 2, 8>(mode, a, stream);
    case CFG_256x128:
        return launch_cfg<256, 128, 4, 2, 6>(mode, a, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace dg
