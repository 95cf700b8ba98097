// Device-side helpers shared by the GEMM kernels (gfx950).
#pragma once

#include "common.h"

namespace ql {

typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// two floats -> packed bf16 pair (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// MXFP4: the two E2M1 codes of byte SEL of `codes` (low nibble first) times
// the E8M0 block scale -> a packed bf16 pair.  The hardware conversion reads
// only the exponent field of `scale` as the E8M0 byte (0 stands for 2^-127,
// 255 gives NaN) and is exact: every E2M1 value times a power of two in
// [2^-127, 2^127] is a bf16 number, subnormal results included.
__device__ __forceinline__ float e8m0_as_scale(uint32_t e) { return __uint_as_float((e & 0xFFu) << 23); }
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t codes, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, SEL));
}

// 8 bf16 along a column of an LDS tile: two transposing 64-bit reads, rows r..r+3 and r+4..r+7
__device__ __forceinline__ bf16x8 tr16x8(const uint16_t* p0, const uint16_t* p1) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p0);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p1);
  s16x8 t = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, t);
}

// Buffer resource over [p, p + bytes): reads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7FFFFFFF) bytes = 0x7FFFFFFF;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint32_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t bload1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// Buffer offset that reads as zero (beyond every resource's size).
constexpr uint32_t OOB = 0x80000000u;

// Place between a kernel's last MFMAs and the epilogue that reads their
// results.  The hardware does not interlock VALU reads of an MFMA's result
// registers: the reader must trail the MFMA by enough wait states, which the
// compiler counts along each path, but a branch right after the last MFMA
// (a conditional store, say) has been seen to leave too few on the path
// that skips it, so the read saw an unfinished value.  Thirty-two wait
// states cover every MFMA, whatever the path; the scheduling barriers keep
// instructions from moving across them.
__device__ __forceinline__ void mfma_result_guard() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace ql
