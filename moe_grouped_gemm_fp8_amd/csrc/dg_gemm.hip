// Fine-grained-scaled FP8 GEMM kernels for CDNA4 (gfx950):  D = C + A @ B.T  (NT layout)
// with one FP32 scale per 1x128 segment of an A row and one per 128x128 block of B, plus
// the contiguous and masked M-grouped forms (DeepGEMM pages: pt.news.hada.io, "Interface
// GEMM e restrições de layout" and "GEMM denso e grouped"; feifmx.com release article,
// two-level accumulation of fine-grained-scaled FP8 products).
//
// Design, per workgroup tile of BM x BN outputs:
//  * K advances one 128-deep block at a time: that is one v_mfma_f32_16x16x128_f8f6f4 per
//    16x16 sub-tile, so each MFMA result is exactly one scale block's partial sum.
//  * The MFMA is issued as D^T = B_tile x A_tile^T (B fragment as the first operand).  A lane
//    of the 16x16 result then holds four consecutive columns of ONE output row, so the A
//    row-segment scale is a single per-lane float and the promotion of a partial into the
//    FP32 accumulators costs one multiply (sa * sb) plus four FMAs per MFMA.
//  * Operands are staged global -> registers -> LDS, double buffered (one barrier per K
//    block).  LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at chunk
//    c ^ ((r >> 1) & 7), which makes both the 16-byte-per-lane stores and the fragment reads
//    (16 rows x one chunk per 16-lane group) hit 16 distinct 16-byte bank groups.
//  * Workgroup ids are remapped so that each XCD (ids are dealt round-robin over the 8 XCDs)
//    runs a contiguous range of tiles, and tiles are rastered in groups of 4 M-tiles, so the
//    tiles that run together on one XCD share A rows and B columns in that XCD's L2.
//  * Skinny dense shapes split K over workgroups: each writes an FP32 partial tile, the last
//    one to arrive (atomic counter) sums the partials in split order and writes D.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int KBLK = 128;       // K block = scale granularity = MFMA depth
constexpr int GROUP_M = 4;      // tile raster: M-tiles per group

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

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(64 * WM * WN) void dg_gemm_kernel(GemmArgs p, int tiles_m,
                                                               int tiles_n)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int SM = TM / 16, SN = TN / 16;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be 16-aligned");
    constexpr int A_CH = BM * 8, B_CH = BN * 8;  // 16-byte chunks per K block
    constexpr int A_PT = (A_CH + NT - 1) / NT, B_PT = (B_CH + NT - 1) / NT;
    constexpr int STAGE = (BM + BN) * KBLK;

    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];
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
    const float *SFB = p.sfb + (int64_t)g * NB * KB;

    // ---- per-thread global sources and LDS destinations of the staged chunks: 32-bit
    // offsets from the tile's first A row / B row (rows past the valid range are clamped to
    // the last valid row, so every load stays inside the operand)
    const uint8_t *a_tile = A + (int64_t)m0 * K;
    const uint8_t *b_tile = B + (int64_t)n0 * K;
    uint32_t a_off[A_PT], b_off[B_PT];
    int a_dst[A_PT], b_dst[B_PT];
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
        int q = tid + i * NT;
        int r = q >> 3, c = q & 7;
        int gr = min(m0 + r, row_limit - 1) - m0;
        a_off[i] = (uint32_t)gr * (uint32_t)K + c * 16;
        a_dst[i] = r * KBLK + ((c ^ ((r >> 1) & 7)) << 4);
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
        int q = tid + i * NT;
        int r = q >> 3, c = q & 7;
        int gr = min(n0 + r, N - 1) - n0;
        b_off[i] = (uint32_t)gr * (uint32_t)K + c * 16;
        b_dst[i] = BM * KBLK + r * KBLK + ((c ^ ((r >> 1) & 7)) << 4);
    }

    // per-lane A-scale rows (one per M sub-tile) and per-sub-tile B-scale block rows
    int sa_row[SM];
#pragma unroll
    for (int i = 0; i < SM; ++i)
        sa_row[i] = min(m0 + wm + 16 * i + (lane & 15), row_limit - 1);
    int sb_off[SN];
#pragma unroll
    for (int j = 0; j < SN; ++j)
        sb_off[j] = (min(n0 + wn + 16 * j, N - 1) / KBLK) * KB;

    // a wave whose rows are all invalid (masked tail) skips the MFMA work
    const bool wave_active = (m0 + wm) < row_limit;

    v4f acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    v4i ra[A_PT], rb[B_PT];
    auto load_regs = [&](int kb) {
        const int off = kb * KBLK;
#pragma unroll
        for (int i = 0; i < A_PT; ++i)
            if (A_CH % NT == 0 || tid + i * NT < A_CH)
                ra[i] = *reinterpret_cast<const v4i *>(a_tile + a_off[i] + off);
#pragma unroll
        for (int i = 0; i < B_PT; ++i)
            if (B_CH % NT == 0 || tid + i * NT < B_CH)
                rb[i] = *reinterpret_cast<const v4i *>(b_tile + b_off[i] + off);
    };
    auto store_lds = [&](int st) {
        uint8_t *base = lds + st * STAGE;
#pragma unroll
        for (int i = 0; i < A_PT; ++i)
            if (A_CH % NT == 0 || tid + i * NT < A_CH)
                *reinterpret_cast<v4i *>(base + a_dst[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_PT; ++i)
            if (B_CH % NT == 0 || tid + i * NT < B_CH)
                *reinterpret_cast<v4i *>(base + b_dst[i]) = rb[i];
    };

    float sa_cur[SM], sa_nxt[SM];
    auto load_sa = [&](int kb, float *dst) {
#pragma unroll
        for (int i = 0; i < SM; ++i)
            dst[i] = SFA[(int64_t)kb * ld + sa_row[i]];
    };

    load_regs(kb0);
    load_sa(kb0, sa_cur);
    store_lds(0);
    __syncthreads();

    const int frag_row = lane & 15;
    const int frag_chunk = (lane >> 4) * 2;  // lanes 16g..16g+15 take K bytes [32g, 32g+32)
    for (int kb = kb0; kb < kb1; ++kb) {
        const int st = (kb - kb0) & 1;
        const bool more = kb + 1 < kb1;
        if (more) {
            load_regs(kb + 1);
            load_sa(kb + 1, sa_nxt);
        }
        if (wave_active) {
            const uint8_t *la = lds + st * STAGE;
            const uint8_t *lb = la + BM * KBLK;
            float sb[SN];
#pragma unroll
            for (int j = 0; j < SN; ++j)
                sb[j] = SFB[sb_off[j] + kb];
            // fragment of 16 rows x 128 K bytes: lane reads row (lane & 15), bytes [32g, 32g+32)
            auto frag = [&](const uint8_t *base, int r) {
                const int sw = (r >> 1) & 7;
                const uint8_t *rowp = base + r * KBLK;
                v4i lo = *reinterpret_cast<const v4i *>(rowp + ((frag_chunk ^ sw) << 4));
                v4i hi = *reinterpret_cast<const v4i *>(rowp + (((frag_chunk + 1) ^ sw) << 4));
                return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            };
            // hold the fragments of the dimension with fewer sub-tiles, stream the other
            if constexpr (SM <= SN) {
                v8i af[SM];
#pragma unroll
                for (int i = 0; i < SM; ++i)
                    af[i] = frag(la, wm + 16 * i + frag_row);
#pragma unroll
                for (int j = 0; j < SN; ++j) {
                    const v8i bf = frag(lb, wn + 16 * j + frag_row);
#pragma unroll
                    for (int i = 0; i < SM; ++i) {
                        v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bf, af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                        acc[i][j] += part * (sa_cur[i] * sb[j]);
                    }
                }
            } else {
                v8i bf[SN];
#pragma unroll
                for (int j = 0; j < SN; ++j)
                    bf[j] = frag(lb, wn + 16 * j + frag_row);
#pragma unroll
                for (int i = 0; i < SM; ++i) {
                    const v8i af = frag(la, wm + 16 * i + frag_row);
#pragma unroll
                    for (int j = 0; j < SN; ++j) {
                        v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bf[j], af, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                        acc[i][j] += part * (sa_cur[i] * sb[j]);
                    }
                }
            }
        }
        if (more) {
            store_lds(st ^ 1);
#pragma unroll
            for (int i = 0; i < SM; ++i)
                sa_cur[i] = sa_nxt[i];
        }
        __syncthreads();
    }

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

template <int BM, int BN, int WM, int WN>
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
        hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, MODE_DENSE>), g, b, 0, stream, a,
                           tiles_m, tiles_n);
        break;
    case MODE_CONTIG:
        hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, MODE_CONTIG>), g, b, 0, stream, a,
                           tiles_m, tiles_n);
        break;
    default:
        hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, MODE_MASKED>), g, b, 0, stream, a,
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
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace dg
