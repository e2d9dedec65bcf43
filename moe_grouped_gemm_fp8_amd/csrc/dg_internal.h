// Internal interface between the C ABI layer (dg_api.cpp) and the HIP kernels (dg_gemm.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace dg {

enum Mode : int {
    MODE_DENSE = 0,
    MODE_CONTIG = 1,
    MODE_MASKED = 2,
    // the contiguous form with the activation step fused into its epilogue: B is [G, 2I, K] with
    // the gate rows first, and instead of D the tile writes the 1x128 FP8 cast of
    // h = gate * up / (1 + exp(-gate)) (codes q [M, I], MN-major FP32 scales sfq)
    MODE_CONTIG_SWIGLU = 3
};

// Scale formats: FP32 (1x128 A segments, 128x128 B blocks), or the same granularity as packed
// UE8M0 exponents (four K blocks per 32-bit word, least significant byte first).
enum ScaleFmt : int { SF_FP32 = 0, SF_UE8M0 = 1 };
// Kernel variant of UE8M0 scales that keeps per-block MFMA partials (added to the accumulators
// on the vector unit, as with FP32 scales but without the multiply): for the masked form, which
// skips the MFMAs of row sub-tiles past masked_m, and for dense calls with C, which add C to
// the accumulators inside the K loop.
constexpr int SF_UE8M0_PARTIAL = 2;

// Tile configurations compiled ahead of time.  Each is (BM x BN) output rows x columns per
// workgroup, split over WM x WN waves of 64 lanes; every wave owns a (BM/WM) x (BN/WN) block
// built from 16x16 MFMA sub-tiles.  Copies run two K blocks ahead of the MFMAs unless the
// name says otherwise (d4: four, for shapes bound by HBM latency).
enum TileCfg : int {
    CFG_256x224 = 0,  // 8 waves (4x2), wave tile 64x112: large dense GEMMs, N % 224 friendly
    CFG_128x256 = 1,  // 4 waves (2x2), wave tile 64x128: contiguous MoE (128-row segments)
    CFG_128x128 = 2,  // 4 waves (2x2), wave tile 64x64
    CFG_64x32 = 3,    // 4 waves (2x2), wave tile 32x16: skinny M with split-K
    CFG_256x128 = 4,  // 8 waves (4x2), wave tile 64x64: masked decode, one tile spans m_max
    CFG_STREAM64 = 5, // split-K streaming kernel, 64x64 tiles, <= 8 K blocks per split: skinny M
    CFG_128x128d4 = 6,   // 4 waves (2x2), wave tile 64x64, copies four K blocks ahead
    CFG_128x128w8d4 = 7, // 8 waves (2x4), wave tile 64x32, copies four K blocks ahead
    CFG_128x256w8 = 8,   // 8 waves (2x4), wave tile 64x64: contiguous MoE, two waves per SIMD
    CFG_256x128p = 9,    // CFG_256x128 with workgroups looping over tiles
    CFG_256x256 = 10,    // 8 waves (4x2), wave tile 64x128, scales loaded into registers
    CFG_COUNT
};

struct TileInfo {
    int bm, bn, threads;
    const char *name;
    bool persistent;  // workgroups loop over tiles (at most one per CU), else one per tile
};
extern const TileInfo kTiles[CFG_COUNT];

struct GemmArgs {
    const uint8_t *a;
    const float *sfa;
    int64_t ld_sfa;
    const uint8_t *b;
    const float *sfb;
    const float *c;       // dense only, may be null
    uint16_t *d;
    const int32_t *grp;   // contiguous: m_indices[m_total]; masked: masked_m[num_groups]
    int m;                // dense: M; contiguous: m_total; masked: m_max
    int n, k;
    int num_groups;
    int splits;           // split-K factor of the streaming kernel (1 = none)
    float *ws;            // split-K partial tiles (streaming kernel, splits > 1)
    int max_wgs;          // persistent tiles: workgroups to launch at most (the CU count);
                          // <= 0 launches one workgroup per tile
    int sf_fmt;           // ScaleFmt of sfa / sfb (UE8M0: int32 words behind the pointers)
    int straddle_rows;    // contiguous, 256-row tiles: listed straddling tile-rows whose second
                          // group runs on workgroups ahead of the tiles (0: none)
    // Contiguous tail.  With tail_cus > 0, the workgroups of 256 x 256 tiles leave the tiles
    // of the last-dispatched ones (the busy ones of their last partial wave over tail_cus CUs,
    // when they number between tail_cus / 8 and tail_cus / 4; tail_force of them, if set) to
    // workgroups of 128-row tiles in the same launch, which are given tail_tm x tail_tn, the
    // 256 x 256 tile grid, and at most tail_max of them.
    int tail_cus;
    int tail_force;
    int tail_tm, tail_tn;
    int tail_max;
    uint8_t *q;           // MODE_CONTIG_SWIGLU: e4m3 codes [m, n/2]
    float *sfq;           // MODE_CONTIG_SWIGLU: FP32 scales [n/256][ld_sfq] (MN-major)
    int64_t ld_sfq;
};

// The MN-major-operand kernel (dg_layout.hip): the dense NN, TN and TT layouts (A stored
// [M, K] or [K, M], B [N, K] or [K, N], the NT scale layouts, bf16 D, optional FP32 C) and the
// K-grouped TN form (MoE weight gradient: A [K_total, M], B [K_total, N], one FP32 scale per
// 128-deep K block per column for both, FP32 D[g] = C[g] + ..., group g covering K blocks
// kb_start[g] .. kb_start[g+1]-1).  The group table travels in the kernel arguments, so a
// launch needs no device copy of it (and can be captured in a graph).
enum Layout : int { LAYOUT_NT = 0, LAYOUT_NN = 1, LAYOUT_TN = 2, LAYOUT_TT = 3, LAYOUT_KGROUPED_TN = 4 };
constexpr int KG_MAX_GROUPS = 256;
struct LayoutArgs {
    const uint8_t *a;
    const float *sfa;
    int64_t ld_sfa;  // K-grouped: m
    const uint8_t *b;
    const float *sfb;
    const float *c;  // may be null; K-grouped: may also equal d (accumulate in place)
    void *d;         // bf16 (dense) or FP32 (K-grouped)
    int m, n, k;     // K-grouped: k = K_total
    int num_groups;  // dense: 1
    int kb_start[KG_MAX_GROUPS + 1];
};

int64_t layout_grid_size(int layout, const LayoutArgs &args);
// y[c][r] = x[r][c] for e4m3 bytes (rows % 128 == 0, cols % 16 == 0), for up to two operands
// in one launch (a job with a null x is skipped)
hipError_t launch_transpose_u8(const void *x0, void *y0, int rows0, int cols0, const void *x1,
                               void *y1, int rows1, int cols1, hipStream_t stream);
hipError_t launch_layout(int layout, const LayoutArgs &args, hipStream_t stream);

// The activation step (dg_quant.hip): SwiGLU of bf16 X [m, 2i] and its 1x128 FP8 cast into
// q [m, i] with scales sfa [i/128][ld] (MN-major).
hipError_t launch_swiglu_quant(const void *x, void *q, float *sfa, int64_t ld, int m, int i,
                               hipStream_t stream);

// Grid size in workgroups for a launch (host-side, no HIP call).
int64_t grid_size(int mode, int cfg, const GemmArgs &args);

// Launches the kernel for (mode, cfg) on `stream`; returns the HIP error of the launch.
hipError_t launch_gemm(int mode, int cfg, const GemmArgs &args, hipStream_t stream);

// The contiguous form (MODE_CONTIG, or MODE_CONTIG_SWIGLU) with 256 x 256 tiles and its tail
// of 128-row tiles in one launch (the tail fields of args set): grid size, and the launch.
int64_t contig_tail_grid(int mode, const GemmArgs &args);
hipError_t launch_contig_tail(int mode, const GemmArgs &args, hipStream_t stream);

// The split-K streaming kernel (dense form only): grid size, the most K blocks one split may
// hold, and the launch (rejects a split count that leaves a split empty or too long).
int64_t stream_grid_size(const GemmArgs &args);
int stream_max_kblocks();
// Workspace bytes of a split-K launch (0 without split-K).
int64_t stream_workspace_bytes(int64_t tiles, int splits);
hipError_t launch_stream(const GemmArgs &args, hipStream_t stream);
// Device address (on the current device) and size in floats of the static split-K scratch
// that the no-allocation entry point uses instead of a workspace.
hipError_t static_scratch(float **out, size_t *floats);

}  // namespace dg
