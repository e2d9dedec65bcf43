// The activation step between an expert's two GEMMs, fused: SwiGLU of the first GEMM's bf16
// output and the 1x128 FP8 cast that the second GEMM's A needs (pt.news.hada.io, "Interface
// GEMM e restrições de layout": casting to FP8 is left to the caller; the feifmx.com release
// article's fine-grained scaling fixes the 1x128 granularity).  For X [M, 2I] (gate columns
// first, then up):
//     h = gate * up / (1 + exp(-gate));   per 1x128 segment of a row of h:
//     scale = max(amax, 1e-4) / 448,  q = e4m3(h / scale) (nearest even, within +-448)
// with the scales written MN-major, sfa[seg * ld + row], the layout of the NT GEMM's sfa.
//
// The step is bound by memory (4 bytes read per byte written), so it is laid out for
// coalescing: a wave takes two tasks of 512 consecutive columns of a row, each lane 8 columns
// of each (16-byte loads of gate and up, an 8-byte store of codes), so a 16-lane quarter of
// the wave holds one segment; its amax is a 4-step butterfly across those lanes.  Measured
// on 32768 x 2048: one task per wave with cached loads and stores 61.0 us, two tasks with
// non-temporal ones 56.8-57.0 us (one task, non-temporal: 59.1-59.2 us).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace

// tasks (512 columns of one row) per wave: both tasks' loads go out before either is used
constexpr int QT = 2;

__global__ __launch_bounds__(256) void dg_swiglu_quant_kernel(const uint16_t *__restrict__ x,
                                                               uint8_t *__restrict__ q,
                                                               float *__restrict__ sfa,
                                                               int64_t ld, int m, int i,
                                                               int tasks_per_row)
{
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    typedef unsigned v2u __attribute__((ext_vector_type(2)));
    const int lane = threadIdx.x & 63;
    const int64_t total = (int64_t)m * tasks_per_row;
    const int64_t task0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * QT;
    v4u gw[QT], uw[QT];
    bool live[QT];
    int64_t rows[QT];
    int cols[QT];
    // x and the codes are touched once: non-temporal loads and stores keep them from
    // displacing other lines in the caches
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const int64_t task = task0 + t;
        rows[t] = task / tasks_per_row;
        cols[t] = (int)(task - rows[t] * tasks_per_row) * 512 + lane * 8;
        live[t] = task < total && cols[t] < i;  // a row's last task may hold fewer than 4 segments
        if (live[t]) {
            const uint16_t *xr = x + rows[t] * 2 * (int64_t)i;
            gw[t] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(xr + cols[t]));
            uw[t] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(xr + i + cols[t]));
        }
    }
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        if (task0 + t >= total)
            break;  // (the whole wave)
        float h[8];
        float amax = 0.f;
        if (live[t]) {
            const uint32_t gs[4] = {gw[t].x, gw[t].y, gw[t].z, gw[t].w};
            const uint32_t us[4] = {uw[t].x, uw[t].y, uw[t].z, uw[t].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h[2 * e] = silu_times(bf16_lo(gs[e]), bf16_lo(us[e]));
                h[2 * e + 1] = silu_times(bf16_hi(gs[e]), bf16_hi(us[e]));
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
                amax = fmaxf(amax, fabsf(h[e]));
        }
        // the segment's 16 lanes (lanes 16 s .. 16 s + 15 share one segment)
#pragma unroll
        for (int o = 1; o < 16; o <<= 1)
            amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        if (!live[t])
            continue;
        // h / scale as h * (448 / amax): one division per segment, a product per element
        const float floor_amax = fmaxf(amax, 1e-4f);
        const float scale = floor_amax / 448.f;
        const float inv = 448.f / floor_amax;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            y[e] = fminf(fmaxf(h[e] * inv, -448.f), 448.f);
        int lo = 0, hi = 0;
        lo = cvt_pk_e4m3<false>(y[0], y[1], lo);
        lo = cvt_pk_e4m3<true>(y[2], y[3], lo);
        hi = cvt_pk_e4m3<false>(y[4], y[5], hi);
        hi = cvt_pk_e4m3<true>(y[6], y[7], hi);
        __builtin_nontemporal_store(v2u{(unsigned)lo, (unsigned)hi},
                                    reinterpret_cast<v2u *>(q + rows[t] * (int64_t)i + cols[t]));
        if ((lane & 15) == 0)
            sfa[(int64_t)(cols[t] / 128) * ld + rows[t]] = scale;
    }
}

hipError_t launch_swiglu_quant(const void *x, void *q, float *sfa, int64_t ld, int m, int i,
                               hipStream_t stream)
{
    const int tasks_per_row = (i + 511) / 512;
    const int64_t waves = (int64_t)m * tasks_per_row;
    const int64_t blocks = (waves + 4 * QT - 1) / (4 * QT);
    if (blocks <= 0 || blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(dg_swiglu_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t *)x, (uint8_t *)q, sfa, ld, m, i, tasks_per_row);
    return hipGetLastError();
}

}  // namespace dg
