// Small device helpers shared by the gfx950 kernels of this library: vector
// types, LDS access (plain and transpose reads), the bf16 MFMA step and
// buffer loads. Not part of the ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace gdn2 {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;  // chunk length (tokens)

__device__ __forceinline__ bf16x8 f32x8_to_bf16(f32x8 x) { return __builtin_convertvector(x, bf16x8); }
__device__ __forceinline__ bf16x4 f32x4_to_bf16(f32x4 x) { return __builtin_convertvector(x, bf16x4); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename T>
__device__ __forceinline__ T lds_ld(const char *base, int off) { return *reinterpret_cast<const T *>(base + off); }
template <typename T>
__device__ __forceinline__ void lds_st(char *base, int off, T v) { *reinterpret_cast<T *>(base + off) = v; }

// LDS transpose read (gfx950 ds_read_b64_tr_b16). Within each group of 16
// lanes, lane s supplies the address of 4 consecutive bf16 of row k0 + s/4,
// columns c0 + 4 (s % 4); lane s receives column c0 + s of rows k0 .. k0 + 3.
__device__ __forceinline__ bf16x4 lds_tr(const char *base, int off)
{
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + off));
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }

// c + a b on one 16x16x32 bf16 tile. Operand layouts (lane = 16 q4 + l16):
// a holds A[m = l16][k = 8 q4 .. 8 q4 + 7], b holds B[k = 8 q4 .. 8 q4 + 7][n = l16],
// and the result C[m = 4 q4 + e][n = l16] is element e of the lane's f32x4.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int BUF_DWORD3 = 0x00020000;  // raw (unformatted) buffer, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, BUF_DWORD3);
}
template <typename T>
__device__ __forceinline__ T buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

}  // namespace dev
}  // namespace gdn2
