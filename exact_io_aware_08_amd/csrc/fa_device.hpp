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
