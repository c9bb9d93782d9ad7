// fa_device.hpp -- gfx950 device helpers shared by the kernels: vector types,
// MFMA wrappers and small wave-level utilities.
//
// MFMA operand layouts used throughout (wave64):
//   v_mfma_f32_32x32x16_{bf16,f16}: A is 32(M) x 16(K), lane l holds row l%32
//   and 8 K-values of group l/32; B is 16(K) x 32(N), lane l holds column
//   l%32 and the same 8 K-values of group l/32; the 32x32 fp32 result holds,
//   in lane l and register r, element (row 8*(r/4) + 4*(l/32) + r%4,
//   column l%32).
//   v_mfma_f32_16x16x32_{bf16,f16}: A 16x32, lane l holds row l%16 and the 8
//   K-values of group l/16; B likewise by column; the 16x16 result holds, in
//   lane l and register r, element (row 4*(l/16) + r, column l%16).
//   v_mfma_f32_32x32x2f32: A 32x2, lane l holds A[l%32][l/32]; B 2x32, lane
//   l holds B[l/32][l%32]; result as for 32x32x16.
// A contraction only needs A and B to agree on which K index each
// (lane group, element) slot carries, so the kernels choose the slot->K map
// that makes their loads contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// Native vector integers for raw 8/16-byte moves (HIP's uint4 is a union
// struct whose copies can defeat register promotion).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// 16-bit element traits: storage type, 8-wide MFMA operand type and the two
// MFMA shapes used by the kernels.
template <typename T> struct Mma16;

template <> struct Mma16<__bf16> {
    using v8 = bf16x8_t;
    static __device__ __forceinline__ f32x16_t mma32(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t mma16(v8 a, v8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma16<_Float16> {
    using v8 = f16x8_t;
    static __device__ __forceinline__ f32x16_t mma32(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t mma16(v8 a, v8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From &x) {
    static_assert(sizeof(To) == sizeof(From), "bitcast size");
    return __builtin_bit_cast(To, x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Registers loaded once before a loop (e.g. the Q operand): pass them
// through an empty asm that redefines them.  The wait for their loads then
// happens here, once, and the loop body does not have to drain in-flight
// prefetches before each use.
template <typename V, int N>
__device__ __forceinline__ void settle(V (&r)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(r[i]));
}

// Cross-lane steps within a wave of 64 without LDS: DPP row operations
// (quad_perm, row_half_mirror, row_mirror, row_shr, row_bcast) and the
// permlane swaps.  The reduction pairs lane l with l^1 and l^2 (quad_perm),
// then with 7 - l within each 8 (half mirror: the other quad), 15 - l within
// each 16 (mirror: the other half row), l^16 and l^32; each step combines two
// disjoint partial results symmetrically, so every lane ends with the same
// full reduction.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_mov(int x)
{
    return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, true);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm (1,0,3,2)
constexpr int kDppXor2 = 0x4E;        // quad_perm (2,3,0,1)
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within each 16
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

// The two values of a permlane swap of x with itself: {x[l], x[l^16]} or
// {x[l^16], x[l]} (resp. l^32), in the same order in both lanes of a pair.
__device__ __forceinline__ void pair16(int x, int &a, int &b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    a = (int)r[0];
    b = (int)r[1];
}
__device__ __forceinline__ void pair32(int x, int &a, int &b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    a = (int)r[0];
    b = (int)r[1];
}

template <typename Op>
__device__ __forceinline__ float wave_reduce_f32(float x, Op op)
{
    x = op(x, __int_as_float(dpp_mov<kDppXor1>(__float_as_int(x))));
    x = op(x, __int_as_float(dpp_mov<kDppXor2>(__float_as_int(x))));
    x = op(x, __int_as_float(dpp_mov<kDppHalfMirror>(__float_as_int(x))));
    x = op(x, __int_as_float(dpp_mov<kDppMirror>(__float_as_int(x))));
    int a, b;
    pair16(__float_as_int(x), a, b);
    x = op(__int_as_float(a), __int_as_float(b));
    pair32(__float_as_int(x), a, b);
    return op(__int_as_float(a), __int_as_float(b));
}
__device__ __forceinline__ float wave_sum_f32(float x)
{
    return wave_reduce_f32(x, [](float u, float v) { return u + v; });
}
__device__ __forceinline__ float wave_max_f32(float x)
{
    return wave_reduce_f32(x, [](float u, float v) { return fmaxf(u, v); });
}

// Sum over the wave of a 64-bit integer (the halves move separately).
__device__ __forceinline__ long long wave_sum_i64(long long x)
{
    auto step = [](long long v, int lo, int hi) {
        return v + (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
    };
    x = step(x, dpp_mov<kDppXor1>((int)x), dpp_mov<kDppXor1>((int)(x >> 32)));
    x = step(x, dpp_mov<kDppXor2>((int)x), dpp_mov<kDppXor2>((int)(x >> 32)));
    x = step(x, dpp_mov<kDppHalfMirror>((int)x), dpp_mov<kDppHalfMirror>((int)(x >> 32)));
    x = step(x, dpp_mov<kDppMirror>((int)x), dpp_mov<kDppMirror>((int)(x >> 32)));
    int a0, b0, a1, b1;
    pair16((int)x, a0, b0);
    pair16((int)(x >> 32), a1, b1);
    x = (long long)(((unsigned long long)(unsigned)a1 << 32) | (unsigned)a0) +
        (long long)(((unsigned long long)(unsigned)b1 << 32) | (unsigned)b0);
    pair32((int)x, a0, b0);
    pair32((int)(x >> 32), a1, b1);
    return (long long)(((unsigned long long)(unsigned)a1 << 32) | (unsigned)a0) +
           (long long)(((unsigned long long)(unsigned)b1 << 32) | (unsigned)b0);
}

// Inclusive prefix sum over the 64 lanes: scans within 16-lane rows, then
// row 0's total into row 1 and row 2's into row 3, then rows 0-1's total
// into rows 2-3.
__device__ __forceinline__ int wave_scan_i32(int x)
{
    x += dpp_mov<kDppShr1>(x);
    x += dpp_mov<kDppShr2>(x);
    x += dpp_mov<kDppShr4>(x);
    x += dpp_mov<kDppShr8>(x);
    x += dpp_mov<kDppBcast15, 0xA>(x);
    x += dpp_mov<kDppBcast31, 0xC>(x);
    return x;
}

// Max (sum) of x over the lanes l and l^16 (resp. l^32), the same value in
// both lanes.
__device__ __forceinline__ float max_xor16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier that orders LDS traffic only: it waits for this wave's
// LDS operations, not for outstanding global loads (which only fill
// registers), so prefetches stay in flight across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Pack the low (resp. high) 16-bit halves of two dwords: result.lo = a.half,
// result.hi = b.half.
// (v_perm_b32 byte selects: 0-3 pick bytes of the second operand, 4-7 of
// the first.)
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}


constexpr int kBufferFlags = 0x00020000;  // raw buffer, dword data format (gfx9 V# word 3)

// Cache-policy operand of a buffer load: the non-temporal (NT) bit, for a
// stream read once and too large to stay cached between uses (the decode's
// KV cache above a size threshold).
constexpr int kLoadStream = 2;

// Buffer resource over rows [j0, rows) of a row-major slice of D-element
// rows: loads past the end read as zero (the hardware range check on the
// VGPR offset).  All arguments are wave-uniform.
template <typename T, int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const T *base, int rows, int j0)
{
    // A slice may hold up to 2^31 elements (more bytes than an int), and
    // every load lies within a tile or two of the rebased start, so the byte
    // range is clamped to 31 bits.  Done in 32-bit scalar arithmetic on the
    // row count (a 64-bit compare would run on the vector unit).
    constexpr int kRowBytes = D * (int)sizeof(T);
    constexpr int kMaxRows = 0x7fffffff / kRowBytes;  // rows whose bytes fit in 31 bits
    const int left = rows > j0 ? rows - j0 : 0;
    const int bytes = left > kMaxRows ? 0x7fffffff : left * kRowBytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(base + (size_t)j0 * D), (short)0, bytes,
                                             kBufferFlags);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// ds_read_b64_tr_b16: within each 16-lane group, lane s supplies the address
// of row r0 + s/4, columns c0 + 4(s%4)..+3 of a row-major 16-bit tile, and
// lane i receives column c0 + i of rows r0..r0+3 (four 16-bit values).
template <typename T>
__device__ __forceinline__ u32x2_t read_tr(const T *p)
{
    return bitcast<u32x2_t>(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(p)));
}

}  // namespace fa
