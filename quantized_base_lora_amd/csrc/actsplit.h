// a1: the per-token two-term E4M3 split, shared by the split kernels.
//
// Row scale s = 2^e, e the smallest integer with 448 * 2^e >= max|x|;
// t = x * 2^-e is exact (|t| <= 448), and so are t - hi and the factor 16,
// leaving the two E4M3 roundings (the hardware conversion, nearest even; it
// is never asked to saturate: |t| <= 448 and |16 (t - hi)| <= 256):
// hi = E4M3(t), lo = E4M3(16 (t - hi)).  A zero row has s = 0 and zero codes.
#pragma once

#include "device.h"

namespace ql {

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// e of a row whose maximum magnitude is amax > 0
__device__ __forceinline__ int split_exponent(float amax) {
  const int E = ilogbf(amax);                        // amax = m 2^E, m in [1, 2)
  return ldexpf(amax, -E) <= 1.75f ? E - 8 : E - 7;  // 448 2^(E-8) = 1.75 2^E
}

// max |x| over 8 bf16 values (4 packed pairs), folded into amax
__device__ __forceinline__ float absmax8(float amax, const uint32_t wd[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    amax = fmaxf(amax, fabsf(__uint_as_float(wd[i] << 16)));
    amax = fmaxf(amax, fabsf(__uint_as_float(wd[i] & 0xFFFF0000u)));
  }
  return amax;
}

// the hi and lo codes of 8 bf16 values (4 packed pairs) at exponent e;
// zero codes when the row is zero
__device__ __forceinline__ void split8(const uint32_t wd[4], int e, bool zero_row, uint2& h8, uint2& l8) {
  float v[8], r[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = ldexpf(__uint_as_float(wd[i] << 16), -e);
    v[2 * i + 1] = ldexpf(__uint_as_float(wd[i] & 0xFFFF0000u), -e);
  }
  uint32_t h[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    h[q] = e4m3x4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    const f2 d0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)h[q], false);
    const f2 d1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)h[q], true);
    r[4 * q] = (v[4 * q] - d0.x) * 16.0f;
    r[4 * q + 1] = (v[4 * q + 1] - d0.y) * 16.0f;
    r[4 * q + 2] = (v[4 * q + 2] - d1.x) * 16.0f;
    r[4 * q + 3] = (v[4 * q + 3] - d1.y) * 16.0f;
  }
  const uint32_t l0 = e4m3x4(r[0], r[1], r[2], r[3]), l1 = e4m3x4(r[4], r[5], r[6], r[7]);
  h8 = zero_row ? make_uint2(0u, 0u) : make_uint2(h[0], h[1]);
  l8 = zero_row ? make_uint2(0u, 0u) : make_uint2(l0, l1);
}

}  // namespace ql
