// Device-side building blocks shared by the FP8 GEMM kernels for gfx950: vector types, the
// bf16 rounding, explicit wait helpers, LDS fragment reads issued as inline asm, buffer
// resources, compile-time loops and the XCD-aware tile mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace dg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
#define DG_LDS __attribute__((address_space(3)))
#define DG_CONST __attribute__((address_space(4)))  // read-only for the kernel: scalar loads

constexpr int KBLK = 128;   // K block = scale granularity = MFMA depth
constexpr int GROUP_M = 4;  // tile raster: M-tiles per group

// Two FP32 values rounded to nearest-even bf16 and packed (low half = a): gfx950's
// v_cvt_pk_bf16_f32, which keeps a NaN a quiet NaN and infinities infinite.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// 8-byte LDS write (two dwords) at a byte address; completion is counted by lgkmcnt
__device__ __forceinline__ void lds_write8(uint32_t addr, uint32_t lo, uint32_t hi)
{
    asm volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(make_uint2(lo, hi)) : "memory");
}

// gate * up / (1 + exp(-gate)) (SwiGLU) with the hardware reciprocal (v_rcp_f32, 1 ulp) in
// place of an IEEE division, whose expansion makes the activation step bound by the vector unit
__device__ __forceinline__ float silu_times(float g, float u)
{
    return g * u * __builtin_amdgcn_rcpf(1.f + __expf(-g));
}

// two FP32 values (already within +-448) to e4m3 (round to nearest even), packed into bytes
// 2 SEL .. 2 SEL + 1 of `old` (gfx950's v_cvt_pk_fp8_f32)
template <bool SEL>
__device__ __forceinline__ int cvt_pk_e4m3(float a, float b, int old)
{
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, SEL);
}

// 4-byte LDS write at a byte address; completion is counted by lgkmcnt
__device__ __forceinline__ void lds_write4(uint32_t addr, float v)
{
    asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

__device__ __forceinline__ void store_bf16x4(uint16_t *dst, v4f v)
{
    uint32_t lo = pack_bf16x2(v.x, v.y);
    uint32_t hi = pack_bf16x2(v.z, v.w);
    *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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

// The same with a compile-time byte offset in the instruction's offset field, so that reads of
// one slot share a single base register and cost no address arithmetic.
template <int OFF>
__device__ __forceinline__ v4i lds_read16_at(uint32_t base)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    v4i v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF) : "memory");
    return v;
}

template <int OFF>
__device__ __forceinline__ float lds_read4_at(uint32_t base)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    float v;
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF) : "memory");
    return v;
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b8), as measured on the MI355X: within each
// group of 16 lanes, lanes 2t and 2t+1 address the two 8-byte halves of a 16-byte "row" t
// (t = 0..7), and lane j receives byte j of rows 0..7 in order: an 8 x 16 byte block turned
// into 16 lanes x 8 bytes.  With one row per K index of an MN-major tile, lane j gets 8
// consecutive K values of column j, the layout of an MFMA operand.
typedef int v2i __attribute__((ext_vector_type(2)));
template <int OFF>
__device__ __forceinline__ v2i lds_read_tr8_at(uint32_t base)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    v2i v;
    asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF) : "memory");
    return v;
}

template <int OFF>
__device__ __forceinline__ v4f lds_read16f_at(uint32_t base)
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    v4f v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF) : "memory");
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
__device__ __forceinline__ void tie(v4i &v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ void tie(float &v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ void tie(v2i &v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ void tie(v4f &v) { asm volatile("" : "+v"(v)); }

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1: loop indices usable as constants.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
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

// (tm, tn) -> tile id, the inverse of raster()
__device__ __forceinline__ int raster_index(int tm, int tn, int tiles_m, int tiles_n)
{
    const int first = tm / GROUP_M * GROUP_M;
    const int gsz = min(tiles_m - first, GROUP_M);
    return first * tiles_n + tn * gsz + (tm - first);
}

// Cache-policy operand of a buffer load (gfx950): non-temporal, for data read once (a B
// panel that only one tile reads, a skinny GEMM's B), so that it does not push reused lines
// out of the caches.
constexpr int CP_NT = 2;

// 128-bit buffer resource for raw (unstrided) loads of `bytes` bytes from `base`: any lane
// whose offset falls outside the range reads zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    // clamp to [0, 2^31 - 1] with 32-bit compares on the two halves (the scalar unit has no
    // 64-bit signed compare, so an int64 compare would move to the vector unit)
    const uint32_t hi = (uint32_t)((uint64_t)bytes >> 32), lo = (uint32_t)bytes;
    const int n = (int)hi < 0 ? 0 : ((hi != 0 || lo > 0x7fffffffu) ? 0x7fffffff : (int)lo);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// Register buffer that holds B fragment jj (of SN per block).  Fragment jj+2 is read while
// jj is in use and jj+1 may be in flight, and the next block's fragments 0 and 1 are read
// while fragment SN-1 is in use, so any three consecutive fragments (across the block
// boundary too) need distinct buffers: jj % 3, except that the last one takes buffer 3 when
// jj % 3 would collide with the next block's 0 or 1.
__host__ __device__ constexpr int bbuf(int jj, int sn)
{
    return (jj == sn - 1 && sn > 2 && (jj % 3) != 2) ? 3 : jj % 3;
}
__host__ __device__ constexpr int bbuf_count(int sn)
{
    return sn <= 3 ? sn : ((sn - 1) % 3 == 2 ? 3 : 4);
}

}  // namespace dg
