// Device-side building blocks shared by the fused tile kernel and the large-tile
// GEMM path (gfx950): vector types, global-memory views, MFMA wrappers, the
// transposing LDS operand read and bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace himuon {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

#define GLOBAL_AS __attribute__((address_space(1)))
#define LDS_AS __attribute__((address_space(3)))

// Global-memory views of generic pointers (global_load/store instead of flat).
template <class T>
__device__ __forceinline__ GLOBAL_AS T *gmem(T *p) {
  return (GLOBAL_AS T *)p;
}
template <class T>
__device__ __forceinline__ const GLOBAL_AS T *gmem(const T *p) {
  return (const GLOBAL_AS T *)p;
}

// 32x32 MFMA, fp32 accumulation.  Output layout (both): lane l, register r holds
// row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.  Operand lane l holds row (or
// column) l % 32 and a run of k selected by l / 32 (8 k for bf16 x16, 1 k for f32 x2).
__device__ __forceinline__ f32x16 mma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// MFMA operand from a row-major bf16 LDS matrix read along its columns: lane l
// receives buf[k .. k+7][m + l % 32] (k includes the lane half's k offset; pitch in
// elements).  ds_read_tr16_b64 works on groups of 16 lanes: lane i of a group
// receives element i % 4 of the 8-byte chunks read by lanes i/4, i/4 + 4, i/4 + 8,
// i/4 + 12.  So lane L reads 4 consecutive columns of row k + L/4 and receives column
// L of rows k..k+3.
__device__ __forceinline__ bf16x8 tr_frag(const __bf16 *buf, int pitch, int k, int m, int lane) {
  const int L = lane & 15, g = (lane >> 4) & 1;
  const int col = m + 16 * g + 4 * (L & 3);
  const __bf16 *p0 = buf + (k + (L >> 2)) * pitch + col;
  const __bf16 *p1 = buf + (k + 4 + (L >> 2)) * pitch + col;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(p0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(p1));
  const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ unsigned short to_bf16_bits(float x) {
  return __builtin_bit_cast(unsigned short, (__bf16)x);
}
__device__ __forceinline__ float bf16_bits_to_f32(unsigned short b) {
  return __builtin_bit_cast(float, (unsigned)b << 16);
}
// two floats rounded to bf16 (nearest even), a in the low half (one v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// ---- fp8 (OCP e4m3: 3 mantissa bits, largest finite 448; larger values convert to NaN)
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// four floats divided by d (a power of two) and rounded to e4m3 (nearest even), a in
// the lowest byte: two v_cvt_scalef32_pk_fp8_f32, which compute e4m3(x / d)
typedef short s16x2 __attribute__((ext_vector_type(2)));
// (the first conversion writes the low half and keeps the high one, which the second
// overwrites, so the initial value is immaterial: a's bits, whose register is often
// free by then, rather than a cleared register)
__device__ __forceinline__ unsigned pack_fp8x4(float a, float b, float c, float d, float div) {
  s16x2 w = __builtin_bit_cast(s16x2, a);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, div, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, div, true);
  return __builtin_bit_cast(unsigned, w);
}

// 32x32x64 e4m3 MFMA with block scales, fp32 accumulation: c + 2^(sa-127) 2^(sb-127) A B.
// Operand lane l holds 32 consecutive k (selected by l / 32) of row (column) l % 32 as
// bytes; any k order works as long as both operands use the same one.  Output layout
// as mma_bf16.
__device__ __forceinline__ f32x16 mma_f8s(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// 2^e as a float, for -126 <= e <= 127
__device__ __forceinline__ float pow2i(int e) { return __builtin_bit_cast(float, (unsigned)(127 + e) << 23); }

// LDS-only workgroup barrier: this wave's LDS traffic is complete, then all waves
// meet; global loads in flight are not waited for.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace dev
}  // namespace himuon
