// Split-K streaming form of the fine-grained-scaled FP8 GEMM D = C + A @ B.T (NT layout; one
// FP32 scale per 1x128 segment of an A row and per 128x128 block of B; DeepGEMM pages:
// pt.news.hada.io, "Interface GEMM e restrições de layout"; feifmx.com release article,
// two-level accumulation) for skinny M, where the work is reading B once from HBM.
//
// Design:
//  * A workgroup owns a 64 x 64 output tile and a range of at most 8 K blocks (a split).  Its
//    whole share of A, B and both scale sets is requested up front as direct-to-LDS copies
//    (up to 128 KB in flight per workgroup) and consumed once all have landed.
//  * Eight waves: wave w takes the 16-column slice w & 3 of the tile and the K half w >> 2 of
//    the split, so each wave's chain of MFMAs and promotions covers at most four K blocks; the
//    two halves of a slice are added through LDS.  A wave runs one v_mfma_f32_16x16x128_f8f6f4
//    per (16-row A sub-tile, K block) and promotes the partial with sa * sb into FP32
//    accumulators, exactly as the pipelined kernels do.  With packed UE8M0 scales (four K
//    blocks' exponents per int32) the block-scaled MFMA applies them and accumulates itself.
//  * With several splits, each writes its FP32 partial tile to a workspace and a second
//    kernel sums the partials in split order (deterministic), adds C, rounds to bf16 and
//    stores the valid rows and columns; the kernel boundary makes the partials visible.
//    Measured alternatives with the reduction inside this kernel (the split that arrives last
//    on a per-tile counter sums the tile), on the 64 x 2112 x 7168 shape: an agent-scope
//    release per workgroup (it writes back the XCD's whole L2) took 25 us, and partials
//    written and read past the L2s (system-coherent accesses, no fence) 14.9 us, against
//    13.3 us for the two launches.
//  * LDS rows are 128 bytes with the same chunk swizzle as the pipelined kernels
//    (c ^ h(r), h(r) = r3 | r1 << 1 | r2 << 2), so the 16-row fragment reads are conflict free.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

constexpr int ST_BM = 64;       // tile rows
constexpr int ST_BN = 64;       // tile columns (4 slices x 16)
constexpr int ST_KSB = 8;       // K blocks per split at most
constexpr int ST_WAVES = 8;     // 4 column slices x 2 K halves

// + C, round to bf16, store four consecutive columns of one row when they are inside D
__device__ __forceinline__ void stream_store(const GemmArgs &p, v4f v, int row, int col)
{
    if (row < p.m && col < p.n) {
        if (p.c)
            v += *reinterpret_cast<const v4f *>(p.c + (int64_t)row * p.n + col);
        store_bf16x4(p.d + (int64_t)row * p.n + col, v);
    }
}

template <bool UE8>
__global__ __launch_bounds__(64 * ST_WAVES) void dg_stream_kernel(GemmArgs p, int tiles_m,
                                                                   int tiles_n)
{
    constexpr int A_SLOT = ST_BM * KBLK;             // one K block of the tile's A rows
    constexpr int B_SLOT = ST_BN * KBLK;
    constexpr int B_BASE = ST_KSB * A_SLOT;          // 64 KB
    constexpr int SA_BASE = B_BASE + ST_KSB * B_SLOT;  // 128 KB: 64 A scales per K block
    constexpr int SB_BASE = SA_BASE + ST_KSB * 256;    // B scales, one per K block
    constexpr int LDS_BYTES = SB_BASE + 256;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cs = wave & 3;   // column slice
    const int kh = wave >> 2;  // K half
    const int K = p.k, N = p.n, M = p.m;
    const int KB = K / KBLK;
    const int NB = (N + KBLK - 1) / KBLK;
    const int KS = UE8 ? (KB + 3) / 4 : KB;  // scale words per row (UE8M0: four blocks each)
    const int64_t ld = p.ld_sfa;

    // workgroup id -> (m tile, n tile, split); splits of one tile are adjacent ids, so they
    // land on different XCDs and finish at about the same time
    int t = blockIdx.x;
    const int split = t % p.splits;
    t /= p.splits;
    const int tn = t % tiles_n;
    const int tm = t / tiles_n;
    const int kbs = (KB + p.splits - 1) / p.splits;  // <= ST_KSB (host-checked)
    const int kb0 = split * kbs;
    const int nk = min(kbs, KB - kb0);               // >= 1 (host-checked)
    const int m0 = tm * ST_BM, n0 = tn * ST_BN;

    // ---- the whole split's operands, as direct-to-LDS copies.  Wave w copies A rows
    // [8w, 8w+8) and B rows [8w, 8w+8) of every K block; lane l of a copy fetches row
    // 8w + l/8, logical chunk (l & 7) ^ h(row): the contiguous 1 KB it writes is the swizzled
    // layout.  Rows past M or N read zeros (buffer range), never stored.
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (int64_t)m0 * K, (int64_t)(M - m0) * K);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b + (int64_t)n0 * K, (int64_t)(N - n0) * K);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.sfa, (int64_t)KS * ld * 4);
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(p.sfb, (int64_t)NB * KS * 4);
    // the scale word holding K block kb (UE8M0: its byte kb % 4)
    auto word = [](int kb) { return UE8 ? kb >> 2 : kb; };
    DG_LDS uint8_t *ldsp = (DG_LDS uint8_t *)lds;
    const uint32_t lane_even = (uint32_t)(lane >> 3) * (uint32_t)K +
                               (uint32_t)((((lane & 7) ^ ((lane >> 4) << 1))) << 4);
    // scales first (older than every operand copy): A scales one 4-byte-per-lane copy per K
    // block (lane = tile row); B scales one copy, the tile's 64 columns lying in one 128-column
    // block (n0 % 128 is 0 or 64), lane l < nk taking K block kb0 + l and the other lanes
    // reading outside the resource (zeros)
    for (int kb = wave; kb < nk; kb += ST_WAVES)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (DG_LDS void *)(ldsp + SA_BASE + kb * 256), 4,
            (uint32_t)(((int64_t)word(kb0 + kb) * ld + m0 + lane) * 4), 0, 0, 0);
    if (wave == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsb, (DG_LDS void *)(ldsp + SB_BASE), 4,
            lane < nk ? (uint32_t)(((n0 / KBLK) * KS + word(kb0 + lane)) * 4) : 0x80000000u, 0,
            0, 0);
    {
        const uint32_t vo =
            (lane_even ^ (uint32_t)((wave & 1) << 4)) + (uint32_t)(8 * wave) * (uint32_t)K;
        for (int kb = 0; kb < nk; ++kb) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (DG_LDS void *)(ldsp + kb * A_SLOT + wave * 1024), 16, vo,
                (uint32_t)(kb0 + kb) * KBLK, 0, 0);
            // (B is read once: non-temporal)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (DG_LDS void *)(ldsp + B_BASE + kb * B_SLOT + wave * 1024), 16, vo,
                (uint32_t)(kb0 + kb) * KBLK, 0, CP_NT);
        }
    }

    // ---- MFMAs: wave (cs, kh) owns columns [n0 + 16 cs, n0 + 16 cs + 16), all 64 rows (4
    // sub-tiles), and the K blocks of its half of the split
    const int fr = lane & 15, fg = lane >> 4;
    const int fh = ((fr >> 3) & 1) | (fr & 2) | (((fr >> 2) & 1) << 2);  // h(fr)
    const int f_lo = fr * KBLK + (((2 * fg) ^ fh) << 4);
    const int f_hi = fr * KBLK + (((2 * fg + 1) ^ fh) << 4);
    // LDS reads are inline asm with an explicit wait (plain loads would make the compiler wait
    // for every outstanding copy first)
    const uint32_t base = (uint32_t)(uintptr_t)(DG_LDS uint8_t *)lds;
    v4f acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
    // fragments of one K block: B slice, four A sub-tiles, their scales, the B scale
    v4i b0, b1, a0[4], a1[4];
    float sa[4], sb;
    auto read_block = [&](int kb) {
        const uint32_t as = base + (uint32_t)(kb * A_SLOT);
        const uint32_t bs = base + (uint32_t)(B_BASE + kb * B_SLOT + cs * 16 * KBLK);
        b0 = lds_read16(bs + f_lo);
        b1 = lds_read16(bs + f_hi);
        sb = lds_read4(base + SB_BASE + kb * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a0[i] = lds_read16(as + i * 16 * KBLK + f_lo);
            a1[i] = lds_read16(as + i * 16 * KBLK + f_hi);
            sa[i] = lds_read4(base + SA_BASE + kb * 256 + (i * 16 + fr) * 4);
        }
    };
    const int half = (nk + 1) >> 1;
    const int kb_lo = kh * half, kb_hi = min(nk, kb_lo + half);
    // one wait for all of the split's copies and one barrier (a split's few MFMAs do not pay
    // for a wait and a barrier per block); no fence: it would wait for every copy in flight
    wait_vm<0>();
    bare_barrier();
    if (kb_lo < kb_hi)
        read_block(kb_lo);
    for (int kb = kb_lo; kb < kb_hi; ++kb) {
        lds_wait();
        tie(b0);
        tie(b1);
        tie(sb);
        const v8i bv = v8i{b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        v8i av[4];
        float sc[4];
        int ea[4], eb = 0;
        const int sh = 8 * ((kb0 + kb) & 3);  // UE8M0: the byte of block kb0 + kb
        if constexpr (UE8)
            eb = (__builtin_amdgcn_readfirstlane(__float_as_int(sb)) >> sh) & 0xFF;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            tie(a0[i]);
            tie(a1[i]);
            tie(sa[i]);
            av[i] = v8i{a0[i].x, a0[i].y, a0[i].z, a0[i].w, a1[i].x, a1[i].y, a1[i].z, a1[i].w};
            if constexpr (UE8)
                ea[i] = (__float_as_int(sa[i]) >> sh) & 0xFF;
            else
                sc[i] = sa[i] * sb;
        }
        if (kb + 1 < kb_hi)  // the next block's reads overlap this block's MFMAs
            read_block(kb + 1);
        // the four MFMAs first, then their promotions (each promotion waits for its MFMA)
        v4f part[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (UE8)
                // first operand B (its block's exponent), second A (this lane's row's)
                acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv, av[i], acc[i], 0, 0,
                                                                          0, eb, 0, ea[i]);
            else
                part[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bv, av[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        }
        if constexpr (!UE8) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] += part[i] * sc[i];
        }
    }

    // ---- the two K halves of each column slice: the second adds into the first through LDS
    // (the operand slots are free once every wave has passed this barrier)
    lds_wait();
    bare_barrier();
    const uint32_t red = base + (uint32_t)((cs * 64 + lane) * 16);  // v4f (i, slot) at + i * 4 KB
    if (kh == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<DG_LDS v4f *>((DG_LDS uint8_t *)lds + (red - base) + i * 4096) =
                acc[i];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[i] += *reinterpret_cast<DG_LDS v4f *>((DG_LDS uint8_t *)lds + (red - base) +
                                                      i * 4096);
    }

    // element q = i * 256 + cs * 64 + lane of a tile (i < 4) is row 16 i + fr, columns
    // 16 cs + 4 fg .. + 3
    if (p.splits == 1) {
        if (kh == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                stream_store(p, acc[i], m0 + i * 16 + fr, n0 + cs * 16 + 4 * fg);
        }
        return;
    }

    // ---- several splits: publish this split's partial tile (the reduce kernel finishes it).
    // Partials are written once and read once, by another workgroup on any XCD: non-temporal
    // stores and loads (with both, the 64 x 2112 x 7168 step took 11.3 us against 12.1 us;
    // non-temporal loads alone changed nothing)
    if (kh == 0) {
        float *ws_tile =
            p.ws + ((int64_t)(tm * tiles_n + tn) * p.splits + split) * (ST_BM * ST_BN);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_nontemporal_store(acc[i],
                                        reinterpret_cast<v4f *>(ws_tile + (i * 256 + cs * 64 + lane) * 4));
    }
}

// Sums the splits' partial tiles in split order, then + C, bf16, store.  Workgroup (tile, i)
// finishes the tile's rows i*16 .. i*16+15: each thread one 16-byte slice, with the slices of
// all splits requested before any is added (one round trip instead of one per split).

__global__ __launch_bounds__(256) void dg_stream_reduce_kernel(GemmArgs p, int tiles_n)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tile = blockIdx.x >> 2, i = blockIdx.x & 3;
    const int tn = tile % tiles_n, tm = tile / tiles_n;
    const int fr = lane & 15, fg = lane >> 4;
    const float *src = p.ws + (int64_t)tile * p.splits * (ST_BM * ST_BN) + (i * 256 + tid) * 4;
    v4f part[8];
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < p.splits; s0 += 8) {  // up to 8 splits in flight, added in order
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < p.splits)
                part[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4f *>(src + (int64_t)(s0 + u) * ST_BM * ST_BN));
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < p.splits)
                acc += part[u];
    }
    const int M = p.m, N = p.n;
    const int row = tm * ST_BM + i * 16 + fr;
    const int col = tn * ST_BN + wave * 16 + 4 * fg;
    if (row < M && col < N) {
        if (p.c)
            acc += *reinterpret_cast<const v4f *>(p.c + (int64_t)row * N + col);
        store_bf16x4(p.d + (int64_t)row * N + col, acc);
    }
}

int64_t stream_grid_size(const GemmArgs &a)
{
    const int tiles_m = (a.m + ST_BM - 1) / ST_BM;
    const int tiles_n = (a.n + ST_BN - 1) / ST_BN;
    return (int64_t)tiles_m * tiles_n * a.splits;
}

int stream_max_kblocks() { return ST_KSB; }

int64_t stream_workspace_bytes(int64_t tiles, int splits)
{
    return splits <= 1 ? 0 : tiles * splits * ST_BM * ST_BN * 4;
}

hipError_t launch_stream(const GemmArgs &a, hipStream_t stream)
{
    const int tiles_m = (a.m + ST_BM - 1) / ST_BM;
    const int tiles_n = (a.n + ST_BN - 1) / ST_BN;
    const int kb = a.k / KBLK;
    const int kbs = (kb + a.splits - 1) / a.splits;
    if (a.splits < 1 || kbs > ST_KSB || (int64_t)(a.splits - 1) * kbs >= kb)
        return hipErrorInvalidValue;  // every split must hold 1..ST_KSB K blocks
    if (a.splits > 1 && !a.ws)
        return hipErrorInvalidValue;
    const int64_t grid = stream_grid_size(a);
    if (grid <= 0 || grid > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    if (a.sf_fmt == SF_UE8M0)
        hipLaunchKernelGGL(dg_stream_kernel<true>, dim3((unsigned)grid), dim3(64 * ST_WAVES), 0,
                           stream, a, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL(dg_stream_kernel<false>, dim3((unsigned)grid), dim3(64 * ST_WAVES), 0,
                           stream, a, tiles_m, tiles_n);
    if (a.splits > 1)
        hipLaunchKernelGGL(dg_stream_reduce_kernel, dim3((unsigned)(tiles_m * tiles_n * 4)),
                           dim3(256), 0, stream, a, tiles_n);
    return hipGetLastError();
}

// Split-K scratch of the entry point that allocates nothing (dg_fp8_gemm_nt_noalloc): the
// FP32 partial tiles go to this file-scope array instead of a library-allocated workspace.
// Every device that runs the library holds its own copy of it, at its own address, until the
// process ends.  Host code never uses the array's name as an address (on the host it names a
// stand-in, not device memory): the device address comes from hipGetSymbolAddress, looked up
// once per device with that device current, and only that address is passed to kernels.
// Nothing in it has to start at zero: every split writes its whole partial tile before the
// reduce kernel reads it.  Calls that overlap on one device share the array and race.
constexpr size_t kScratchFloats = size_t(4) << 20;  // 16 MiB
static __device__ __align__(256) float scratch[kScratchFloats];

hipError_t static_scratch(float **out, size_t *floats)
{
    static std::mutex mu;
    static void *addr[64] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= 64)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        addr[dev] = p;
    }
    *out = (float *)addr[dev];
    *floats = kScratchFloats;
    return hipSuccess;
}

}  // namespace dg
