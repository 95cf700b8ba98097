// a0 quant_pack, verification dequant, and a1 activation split for the FP8 base.
//
// Formats (see include/qlora.h): Q4_0-style blocks of 32 with an fp16 scale
// absmax/7 and value (q-8)*d; NF4 blocks of 64 with an fp32 absmax and the
// normal-quantile book (QLoRA paper, "4-bit NormalFloat"); per-tensor FP8
// E4M3 with scale absmax/448 (the Surogate FP8 recipe's format); MXFP4
// blocks of 32 E2M1 codes with an E8M0 power-of-two scale (OCP
// Microscaling, the FP4 base of the Surogate pages' FP4 recipes); Q8_0
// blocks of 32 int8 codes with an fp16 scale absmax/127 (the 8-bit member
// of the legacy GGUF family); NVFP4 blocks of 16 E2M1 codes with an E4M3
// scale and an fp32 tensor scale (the Surogate pages' NVFP4 (E2M1)).  Every
// quantization decision is taken in IEEE fp32 with correctly rounded
// division and ties-to-even rounding (NVFP4's element codes by exact fp64
// comparisons), so codes are reproducible bit for bit.
//
// Codecs are written out here from the format definitions (integer bit
// manipulation): the hardware fp8 conversion does not saturate, and the fp16
// one depends on the rounding mode register, so neither is used for packing.
#include <algorithm>

#include "common.h"
#include "device.h"
#include "actsplit.h"

namespace ql {
namespace {

constexpr int kThreads = 256;

struct Mids { float m[15]; };
struct Levels { float c[16]; };

__device__ __forceinline__ float fdiv_rn(float a, float b) { return __fdiv_rn(a, b); }

// fp32 -> IEEE binary16, nearest even; sets *ovf if the result is not finite.
__device__ __forceinline__ uint16_t f32_to_f16(float f, bool* ovf) {
  uint32_t u = __float_as_uint(f);
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x477FF000u) {            // >= 65520: rounds past 65504 (or Inf/NaN)
    *ovf = true;
    return (uint16_t)(sign | 0x7C00u);
  }
  if (a < 0x38800000u) {             // below 2^-14: subnormal grid of 2^-24
    float m = rintf(__uint_as_float(a) * 16777216.0f);   // exact scaling, RNE
    return (uint16_t)(sign | (uint32_t)m);               // 1024 encodes 2^-14 exactly
  }
  int e = (int)(a >> 23) - 127;                          // -14..15
  uint32_t mant = (a & 0x7FFFFFu) | 0x800000u;           // 24 bits
  uint32_t r = mant >> 13, rem = mant & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) ++r;
  if (r == 0x800u) { r = 0x400u; ++e; }
  if (e > 15) { *ovf = true; return (uint16_t)(sign | 0x7C00u); }
  return (uint16_t)(sign | ((uint32_t)(e + 15) << 10) | (r & 0x3FFu));
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
  float v = (e == 0) ? (float)m * 5.9604644775390625e-08f              // m * 2^-24
                     : __uint_as_float(((e + 112u) << 23) | (m << 13)); // rebias 15 -> 127
  return (h & 0x8000) ? -v : v;
}

// fp32 -> OCP E4M3FN, nearest even, saturating to +-448; NaN -> 0x7F; keeps sign of zero.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;
  float af = __uint_as_float(a);
  if (af >= 448.0f) return sign | 0x7Eu;
  if (af < 0.015625f) {                                   // below 2^-6: grid of 2^-9
    float m = rintf(af * 512.0f);                          // 0..8; 8 is the smallest normal
    return sign | (uint32_t)m;
  }
  int e = (int)(a >> 23) - 127;                            // -6..8
  uint32_t mant = (a & 0x7FFFFFu) | 0x800000u;
  uint32_t r = mant >> 20, rem = mant & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
  if (r == 16u) { r = 8u; ++e; }
  return sign | ((uint32_t)(e + 7) << 3) | (r & 7u);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 0xF, m = c & 7;
  float v = (e == 0) ? (float)m * 0.001953125f                           // m/8 * 2^-6
                     : __uint_as_float(((e + 120u) << 23) | (m << 20));  // rebias 7 -> 127
  if (e == 15 && m == 7) v = __uint_as_float(0x7FC00000u);
  return (c & 0x80) ? -v : v;
}

__device__ __forceinline__ uint16_t bf16_bits(float v) {
  __bf16 h = (__bf16)v;                                    // v_cvt_pk_bf16_f32, nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// E2M1 code of t (a value already divided by its block scale): nearest of
// 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the even mantissa, saturating at 6;
// the sign bit is the source's (a negative value that rounds to zero keeps it).
__device__ __forceinline__ uint32_t e2m1_code(float t, uint32_t sign) {
  const float a = fabsf(t);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) +
               (a > 5.0f);
  return c | (sign << 3);
}

// ------------------------------------------------------------------ block pack
// One thread per 32-element group of a row (16 output bytes; 32 for Q8_0).
// For NF4 two neighbouring threads share a 64-element block and exchange
// their maxima.
template <int FMT>
__global__ __launch_bounds__(kThreads) void pack4_kernel(const float* __restrict__ w, int64_t groups,
                                                         uint8_t* __restrict__ codes,
                                                         void* __restrict__ scales,
                                                         uint32_t* __restrict__ status, Mids mids) {
  int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  bool valid = gid < groups;
  float v[32];
  float amax = 0.0f;
  bool bad = false;
  if (valid) {
    const float4* src = reinterpret_cast<const float4*>(w + gid * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float4 t = src[i];
      v[4 * i + 0] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      bad |= !isfinite(v[i]);
      amax = fmaxf(amax, fabsf(v[i]));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  }
  if (FMT == QL_FMT_NF4) amax = fmaxf(amax, __shfl_xor(amax, 1));
  uint32_t q[32];
  bool ovf = false;
  if (FMT == QL_FMT_Q4_0) {
    uint16_t d16 = f32_to_f16(fdiv_rn(amax, 7.0f), &ovf);
    float d = f16_to_f32(d16);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float t = (d == 0.0f) ? 0.0f : rintf(fdiv_rn(v[i], d));
      t = fminf(fmaxf(t + 8.0f, 0.0f), 15.0f);
      q[i] = (uint32_t)t;
    }
    if (valid) reinterpret_cast<uint16_t*>(scales)[gid] = d16;
  } else if (FMT == QL_FMT_Q8_0) {
    uint16_t d16 = f32_to_f16(fdiv_rn(amax, 127.0f), &ovf);
    float d = f16_to_f32(d16);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float t = (d == 0.0f) ? 0.0f : rintf(fdiv_rn(v[i], d));
      t = fminf(fmaxf(t, -127.0f), 127.0f);
      q[i] = (uint32_t)(int32_t)t & 0xFFu;           // two's complement byte
    }
    if (valid) reinterpret_cast<uint16_t*>(scales)[gid] = d16;
  } else if (FMT == QL_FMT_MXFP4) {
    // block exponent floor(log2 amax) - 2, so the block's largest magnitude
    // lands in [4, 8) (2 is E2M1's largest exponent); clamped to [-127, 127];
    // a zero (or subnormal-only) block takes -127.  Dividing by 2^sh is the
    // exact product with 2^-sh, a normal fp32 number for sh in [-127, 125].
    const uint32_t eb = __float_as_uint(amax) >> 23;
    const int sh = eb == 0 ? -127 : min(127, max(-127, (int)eb - 127 - 2));
    const float inv = __uint_as_float((uint32_t)(127 - min(sh, 126)) << 23);
#pragma unroll
    for (int i = 0; i < 32; ++i) q[i] = e2m1_code(v[i] * inv, __float_as_uint(v[i]) >> 31);
    if (valid) reinterpret_cast<uint8_t*>(scales)[gid] = (uint8_t)(sh + 127);
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      uint32_t c = 7;
      if (amax != 0.0f) {
        float t = fdiv_rn(v[i], amax);
        c = 0;
#pragma unroll
        for (int j = 0; j < 15; ++j) c += (t > mids.m[j]) ? 1u : 0u;
      }
      q[i] = c;
    }
    if (valid && (gid & 1) == 0) reinterpret_cast<float*>(scales)[gid >> 1] = amax;
  }
  if (valid && FMT == QL_FMT_Q8_0) {
    uint32_t word[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) word[i] = q[4 * i] | (q[4 * i + 1] << 8) | (q[4 * i + 2] << 16) | (q[4 * i + 3] << 24);
    uint4* dst = reinterpret_cast<uint4*>(codes + gid * 32);
    dst[0] = make_uint4(word[0], word[1], word[2], word[3]);
    dst[1] = make_uint4(word[4], word[5], word[6], word[7]);
    if (bad) atomicOr(status, 1u);
    if (ovf) atomicOr(status, 2u);
  } else if (valid) {
    uint32_t word[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      word[i] = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        int j = 4 * i + b;
        if (FMT == QL_FMT_MXFP4) word[i] |= (q[2 * j] | (q[2 * j + 1] << 4)) << (8 * b);   // pair-packed
        else word[i] |= (q[j] | (q[j + 16] << 4)) << (8 * b);                             // split halves
      }
    }
    *reinterpret_cast<uint4*>(codes + gid * 16) = make_uint4(word[0], word[1], word[2], word[3]);
    if (bad) atomicOr(status, 1u);
    if (ovf) atomicOr(status, 2u);
  }
}

// ------------------------------------------------------------------ FP8 pack
__global__ __launch_bounds__(kThreads) void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t value) {
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = value;
}

// ------------------------------------------------------------------ NVFP4 pack
// E2M1 code of w against the block decode scale x > 0: the value nearest to
// the exact quotient w / x, ties to the even mantissa, saturating at 6.  Each
// midpoint m x (m = 0.25, 0.75, ..., 5: at most 3 significant bits) is formed
// exactly in fp64 (x has 24), so the comparisons decide as exact arithmetic.
__device__ __forceinline__ uint32_t e2m1_code_exact(float w, float x) {
  const double a = fabs((double)w), d = (double)x;
  const uint32_t c = (a > 0.25 * d) + (a >= 0.75 * d) + (a > 1.25 * d) + (a >= 1.75 * d) + (a > 2.5 * d) +
                     (a >= 3.5 * d) + (a > 5.0 * d);
  return c | ((__float_as_uint(w) >> 31) << 3);
}

// One thread per 32-element group (two blocks of 16).  ws[0] holds the bits
// of the tensor's largest magnitude (absmax_kernel).  g = fl32(amax / 2688);
// block scale byte E4M3(fl32(fl32(amax_b / 6) / g)) (0 when g = 0); block
// decode scale X = fl32(E4M3(sb) g); codes against X (0 when X = 0), stored
// in split-nibble groups; the scale array is g, 12 zero bytes, then two E4M3
// bytes per group.
__global__ __launch_bounds__(kThreads) void pack_nvfp4_kernel(const float* __restrict__ w, int64_t groups,
                                                              const uint32_t* __restrict__ ws,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales,
                                                              uint32_t* __restrict__ status) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const float g = fdiv_rn(__uint_as_float(ws[0]), 2688.0f);
  if (gid == 0) {
    uint32_t* head = reinterpret_cast<uint32_t*>(scales);
    head[0] = __float_as_uint(g);
    head[1] = head[2] = head[3] = 0u;
  }
  if (gid >= groups) return;
  float v[32];
  const float4* src = reinterpret_cast<const float4*>(w + gid * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 t = src[i];
    v[4 * i + 0] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
  }
  bool bad = false;
  uint32_t q[32];
  uint32_t sb[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      bad |= !isfinite(v[16 * b + i]);
      amax = fmaxf(amax, fabsf(v[16 * b + i]));
    }
    sb[b] = g == 0.0f ? 0u : f32_to_e4m3(fdiv_rn(fdiv_rn(amax, 6.0f), g));
    const float x = e4m3_to_f32(sb[b]) * g;
#pragma unroll
    for (int i = 0; i < 16; ++i) q[16 * b + i] = x == 0.0f ? 0u : e2m1_code_exact(v[16 * b + i], x);
  }
  uint32_t word[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    word[i] = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) word[i] |= (q[4 * i + b] | (q[4 * i + b + 16] << 4)) << (8 * b);
  }
  *reinterpret_cast<uint4*>(codes + gid * 16) = make_uint4(word[0], word[1], word[2], word[3]);
  reinterpret_cast<uint16_t*>(scales + 16)[gid] = (uint16_t)(sb[0] | (sb[1] << 8));
  if (bad) atomicOr(status, 1u);
}

// ws[0] = bits of max|w| (non-negative floats order like their bits), ws[1] |= 1 on non-finite.
__global__ __launch_bounds__(kThreads) void absmax_kernel(const float* __restrict__ w, int64_t n4,
                                                          uint32_t* __restrict__ ws) {
  float amax = 0.0f;
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * kThreads) {
    float4 t = reinterpret_cast<const float4*>(w)[i];
    bad |= !(isfinite(t.x) && isfinite(t.y) && isfinite(t.z) && isfinite(t.w));
    amax = fmaxf(fmaxf(amax, fabsf(t.x)), fmaxf(fabsf(t.y), fmaxf(fabsf(t.z), fabsf(t.w))));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  bad = __any(bad);
  if ((threadIdx.x & 63) == 0) {
    atomicMax(&ws[0], __float_as_uint(amax));
    if (bad) atomicOr(&ws[1], 1u);
  }
}

// 16 elements per thread -> 16 code bytes.
__global__ __launch_bounds__(kThreads) void quant_fp8_kernel(const float* __restrict__ w, int64_t n16,
                                                             const uint32_t* __restrict__ ws,
                                                             uint8_t* __restrict__ codes,
                                                             float* __restrict__ scale) {
  float s = fdiv_rn(__uint_as_float(ws[0]), 448.0f);
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i == 0) scale[0] = s;
  if (i >= n16) return;
  const float4* src = reinterpret_cast<const float4*>(w) + i * 4;
  uint32_t word[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float4 t = src[j];
    float e[4] = {t.x, t.y, t.z, t.w};
    uint32_t wd = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      uint32_t c = (s == 0.0f) ? 0u : f32_to_e4m3(fdiv_rn(e[b], s));
      wd |= c << (8 * b);
    }
    word[j] = wd;
  }
  reinterpret_cast<uint4*>(codes)[i] = make_uint4(word[0], word[1], word[2], word[3]);
}

// ------------------------------------------------------------------ dequant (verification)
// One thread per 32 consecutive elements of a row.
template <int FMT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                           const void* __restrict__ scales,
                                                           int64_t groups, int64_t k,
                                                           float* __restrict__ out_f32,
                                                           uint16_t* __restrict__ out_bf16,
                                                           Levels lv) {
  int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= groups) return;
  float v[32];
  if (FMT == QL_FMT_FP8_E4M3) {
    float s = reinterpret_cast<const float*>(scales)[0];
    const uint4* src = reinterpret_cast<const uint4*>(codes + gid * 32);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 t = src[h];
      uint32_t wd[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int i = 0; i < 16; ++i) v[16 * h + i] = e4m3_to_f32((wd[i / 4] >> (8 * (i % 4))) & 0xFF) * s;
    }
  } else if (FMT == QL_FMT_Q8_0) {
    const float d = f16_to_f32(reinterpret_cast<const uint16_t*>(scales)[gid]);
    const uint4* src = reinterpret_cast<const uint4*>(codes + gid * 32);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 t = src[h];
      uint32_t wd[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int i = 0; i < 16; ++i) v[16 * h + i] = (float)(int8_t)((wd[i / 4] >> (8 * (i % 4))) & 0xFF) * d;
    }
  } else if (FMT == QL_FMT_NVFP4) {
    // fl32(E2M1(q) * X), X = fl32(E4M3(sb) * g); elements 0..15 low nibbles, 16..31 high
    uint4 t = *reinterpret_cast<const uint4*>(codes + gid * 16);
    uint32_t wd[4] = {t.x, t.y, t.z, t.w};
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(scales);
    const float g = reinterpret_cast<const float*>(scales)[0];
    const float x[2] = {e4m3_to_f32(sc[16 + 2 * gid]) * g, e4m3_to_f32(sc[16 + 2 * gid + 1]) * g};
    const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      int j = e & 15, hi = e >> 4;
      uint32_t c = (wd[j / 4] >> (8 * (j % 4) + 4 * hi)) & 0xF;
      const float val = (c & 8) ? -mag[c & 7] : mag[c & 7];
      v[e] = val * x[hi];
    }
  } else if (FMT == QL_FMT_MXFP4) {
    // the conversion the GEMMs use; its bf16 results are exact, so fp32 is the same value
    uint4 t = *reinterpret_cast<const uint4*>(codes + gid * 16);
    uint32_t wd[4] = {t.x, t.y, t.z, t.w};
    const float x = e8m0_as_scale(reinterpret_cast<const uint8_t*>(scales)[gid]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t pr[4] = {fp4x2_to_bf16x2<0>(wd[i], x), fp4x2_to_bf16x2<1>(wd[i], x),
                              fp4x2_to_bf16x2<2>(wd[i], x), fp4x2_to_bf16x2<3>(wd[i], x)};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        v[8 * i + 2 * b] = __uint_as_float(pr[b] << 16);
        v[8 * i + 2 * b + 1] = __uint_as_float(pr[b] & 0xFFFF0000u);
      }
    }
  } else {
    uint4 t = *reinterpret_cast<const uint4*>(codes + gid * 16);
    uint32_t wd[4] = {t.x, t.y, t.z, t.w};
    float d;
    if (FMT == QL_FMT_Q4_0) d = f16_to_f32(reinterpret_cast<const uint16_t*>(scales)[gid]);
    else d = reinterpret_cast<const float*>(scales)[gid >> 1];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      int j = e & 15, hi = e >> 4;
      uint32_t q = (wd[j / 4] >> (8 * (j % 4) + 4 * hi)) & 0xF;
      v[e] = (FMT == QL_FMT_Q4_0) ? ((float)q - 8.0f) * d : lv.c[q] * d;
    }
  }
  (void)k;
  if (out_f32) {
    float4* dst = reinterpret_cast<float4*>(out_f32 + gid * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
  if (out_bf16) {
    uint32_t p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = (uint32_t)bf16_bits(v[2 * i]) | ((uint32_t)bf16_bits(v[2 * i + 1]) << 16);
    uint4* dst = reinterpret_cast<uint4*>(out_bf16 + gid * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]);
  }
}

// ------------------------------------------------------------------ a1: activation split
// The two-term E4M3 split of actsplit.h for up to QL_GROUP_MAX activations
// of one token count in one launch; each workgroup finds its activation in a
// table in the kernel arguments.
struct SplitJob {
  const uint16_t* x;
  uint8_t* hi;
  uint8_t* lo;
  float* scale;
  int64_t k;
  int32_t blk0;          // first workgroup of this activation
};
struct SplitJobs {
  SplitJob j[QL_GROUP_MAX];
  int32_t n;
  int64_t m;
};

// One workgroup per row; the second pass re-reads the row from cache.
__global__ __launch_bounds__(kThreads) void act_quant_kernel(SplitJobs a) {
  __shared__ float red[kThreads / 64];
  const int bid = (int)blockIdx.x;
  int ji = 0;
  while (ji + 1 < a.n && bid >= a.j[ji + 1].blk0) ++ji;
  const SplitJob& J = a.j[ji];
  const int64_t k = J.k;
  const int64_t row = bid - J.blk0;
  const uint16_t* xr = J.x + row * k;
  float amax = 0.0f;
  for (int64_t c = (int64_t)threadIdx.x * 8; c < k; c += kThreads * 8) {
    const uint4 t = *reinterpret_cast<const uint4*>(xr + c);
    const uint32_t wd[4] = {t.x, t.y, t.z, t.w};
    amax = absmax8(amax, wd);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = amax > 0.0f ? split_exponent(amax) : 0;
  if (threadIdx.x == 0) J.scale[row] = amax > 0.0f ? ldexpf(1.0f, e) : 0.0f;
  for (int64_t c = (int64_t)threadIdx.x * 8; c < k; c += kThreads * 8) {
    const uint4 t = *reinterpret_cast<const uint4*>(xr + c);
    const uint32_t wd[4] = {t.x, t.y, t.z, t.w};
    uint2 h8, l8;
    split8(wd, e, amax == 0.0f, h8, l8);
    *reinterpret_cast<uint2*>(J.hi + row * k + c) = h8;
    *reinterpret_cast<uint2*>(J.lo + row * k + c) = l8;
  }
}

// The same split with one workgroup of NT threads per row and the row held
// in registers, so x is read from memory once: with an even chunk count CH,
// thread t takes the 16-element pieces at columns 16 (t + NT i), i < CH / 2
// (16-byte stores of each plane), with CH = 1 the 8 elements at 8 t; pieces
// past K read zero and are not stored (K is a multiple of 16).  The row
// maximum is a workgroup reduction.  With one short workgroup per row the
// launch holds several rounds of workgroups per CU, so the loads of later
// rows overlap the stores of earlier ones.
template <int CH, int NT>
__global__ __launch_bounds__(NT) void act_quant_row_kernel(SplitJobs a) {
  static_assert(CH == 1 || CH % 2 == 0, "chunk count");
  constexpr int W = CH == 1 ? 8 : 16;                  // elements per piece
  __shared__ float red[NT / 64];
  const int bid = (int)blockIdx.x;
  int ji = 0;
  while (ji + 1 < a.n && bid >= a.j[ji + 1].blk0) ++ji;
  const SplitJob& J = a.j[ji];
  const int64_t k = J.k;
  const int64_t row = bid - J.blk0;
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rx = rsrc(J.x + row * k, k * 2);
  uint4 t[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c)
    t[c] = bload16(rx, (uint32_t)((W * (tid + NT * (c * 8 / W)) + 8 * (c % (W / 8))) * 2));
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const uint32_t wd[4] = {t[c].x, t[c].y, t[c].z, t[c].w};
    amax = absmax8(amax, wd);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) amax = fmaxf(amax, red[w]);
  const int e = amax > 0.0f ? split_exponent(amax) : 0;
  if (tid == 0) J.scale[row] = amax > 0.0f ? ldexpf(1.0f, e) : 0.0f;
#pragma unroll
  for (int i = 0; i < CH * 8 / W; ++i) {
    const int64_t col = W * (tid + NT * (int64_t)i);
    if (col >= k) continue;
    uint2 h8[W / 8], l8[W / 8];
#pragma unroll
    for (int h = 0; h < W / 8; ++h) {
      const uint4& q = t[i * (W / 8) + h];
      const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
      split8(wd, e, amax == 0.0f, h8[h], l8[h]);
    }
    if constexpr (W == 16) {
      *reinterpret_cast<uint4*>(J.hi + row * k + col) = make_uint4(h8[0].x, h8[0].y, h8[1].x, h8[1].y);
      *reinterpret_cast<uint4*>(J.lo + row * k + col) = make_uint4(l8[0].x, l8[0].y, l8[1].x, l8[1].y);
    } else {
      *reinterpret_cast<uint2*>(J.hi + row * k + col) = h8[0];
      *reinterpret_cast<uint2*>(J.lo + row * k + col) = l8[0];
    }
  }
}

inline unsigned grid_for(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(n)), dim3(kThreads), 0, s, p, n, value);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s) { return launch_fill_u32(p, n, 0u, s); }

hipError_t launch_pack_blocks(int fmt, const float* w, int64_t n, int64_t k, uint8_t* codes,
                              void* scales, uint32_t* status, hipStream_t s) {
  int64_t groups = n * (k / 32);
  Mids mids{};
  const Nf4Table& t = nf4_table();
  for (int i = 0; i < 15; ++i) mids.m[i] = t.mid[i];
  if (fmt == QL_FMT_Q4_0)
    hipLaunchKernelGGL(pack4_kernel<QL_FMT_Q4_0>, dim3(grid_for(groups)), dim3(kThreads), 0, s, w,
                       groups, codes, scales, status, mids);
  else if (fmt == QL_FMT_MXFP4)
    hipLaunchKernelGGL(pack4_kernel<QL_FMT_MXFP4>, dim3(grid_for(groups)), dim3(kThreads), 0, s, w,
                       groups, codes, scales, status, mids);
  else if (fmt == QL_FMT_Q8_0)
    hipLaunchKernelGGL(pack4_kernel<QL_FMT_Q8_0>, dim3(grid_for(groups)), dim3(kThreads), 0, s, w,
                       groups, codes, scales, status, mids);
  else
    hipLaunchKernelGGL(pack4_kernel<QL_FMT_NF4>, dim3(grid_for(groups)), dim3(kThreads), 0, s, w,
                       groups, codes, scales, status, mids);
  return hipGetLastError();
}

hipError_t launch_pack_fp8(const float* w, int64_t n, int64_t k, uint8_t* codes, float* scale,
                           uint32_t* ws, hipStream_t s) {
  int64_t total = n * k;   // multiple of 16 (validated)
  hipError_t e = launch_zero_u32(ws, 2, s);
  if (e != hipSuccess) return e;
  int64_t n4 = total / 4;
  unsigned blocks = (unsigned)std::min<int64_t>(grid_for(n4), 4096);
  hipLaunchKernelGGL(absmax_kernel, dim3(blocks), dim3(kThreads), 0, s, w, n4, ws);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  int64_t n16 = total / 16;
  hipLaunchKernelGGL(quant_fp8_kernel, dim3(grid_for(n16)), dim3(kThreads), 0, s, w, n16, ws, codes,
                     scale);
  return hipGetLastError();
}

hipError_t launch_pack_nvfp4(const float* w, int64_t n, int64_t k, uint8_t* codes, void* scales,
                             uint32_t* ws, hipStream_t s) {
  int64_t total = n * k;   // multiple of 32 (validated)
  hipError_t e = launch_zero_u32(ws, 2, s);
  if (e != hipSuccess) return e;
  int64_t n4 = total / 4;
  unsigned blocks = (unsigned)std::min<int64_t>(grid_for(n4), 4096);
  hipLaunchKernelGGL(absmax_kernel, dim3(blocks), dim3(kThreads), 0, s, w, n4, ws);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t groups = total / 32;
  hipLaunchKernelGGL(pack_nvfp4_kernel, dim3(grid_for(groups)), dim3(kThreads), 0, s, w, groups, ws, codes,
                     reinterpret_cast<uint8_t*>(scales), ws + 1);
  return hipGetLastError();
}

hipError_t launch_dequant(const ql_qweight& w, float* out_f32, uint16_t* out_bf16, hipStream_t s) {
  int64_t groups = w.n_out * (w.k_in / 32);
  Levels lv{};
  const Nf4Table& t = nf4_table();
  for (int i = 0; i < 16; ++i) lv.c[i] = t.level[i];
  switch (w.format) {
    case QL_FMT_Q4_0:
      hipLaunchKernelGGL(dequant_kernel<QL_FMT_Q4_0>, dim3(grid_for(groups)), dim3(kThreads), 0, s,
                         w.codes, w.scales, groups, w.k_in, out_f32, out_bf16, lv);
      break;
    case QL_FMT_NF4:
      hipLaunchKernelGGL(dequant_kernel<QL_FMT_NF4>, dim3(grid_for(groups)), dim3(kThreads), 0, s,
                         w.codes, w.scales, groups, w.k_in, out_f32, out_bf16, lv);
      break;
    case QL_FMT_MXFP4:
      hipLaunchKernelGGL(dequant_kernel<QL_FMT_MXFP4>, dim3(grid_for(groups)), dim3(kThreads), 0, s,
                         w.codes, w.scales, groups, w.k_in, out_f32, out_bf16, lv);
      break;
    case QL_FMT_Q8_0:
      hipLaunchKernelGGL(dequant_kernel<QL_FMT_Q8_0>, dim3(grid_for(groups)), dim3(kThreads), 0, s,
                         w.codes, w.scales, groups, w.k_in, out_f32, out_bf16, lv);
      break;
    case QL_FMT_NVFP4:
      hipLaunchKernelGGL(dequant_kernel<QL_FMT_NVFP4>, dim3(grid_for(groups)), dim3(kThreads), 0, s,
                         w.codes, w.scales, groups, w.k_in, out_f32, out_bf16, lv);
      break;
    default:
      hipLaunchKernelGGL(dequant_kernel<QL_FMT_FP8_E4M3>, dim3(grid_for(groups)), dim3(kThreads), 0,
                         s, w.codes, w.scales, groups, w.k_in, out_f32, out_bf16, lv);
  }
  return hipGetLastError();
}

hipError_t launch_act_quant_group(const ActSplit* sp, int n, int64_t m, hipStream_t s) {
  if (m == 0 || n == 0) return hipSuccess;
  if (n > QL_GROUP_MAX) return hipErrorInvalidValue;
  // rows of at most 16384 elements: one workgroup per row with the row in
  // registers, x read once (128 threads with 1, 2, 4 or 8 chunks of 1024
  // elements up to 8192, above that 256 threads with 6 or 8 chunks of 2048);
  // longer rows take the two-pass kernel.  One launch per kernel instance
  // for the activations it takes.
  auto kind_for = [](int64_t k) {
    return k <= 1024 ? 0 : k <= 2048 ? 1 : k <= 4096 ? 2 : k <= 8192 ? 3 : k <= 12288 ? 4 : k <= 16384 ? 5 : 6;
  };
  for (int kind = 0; kind < 7; ++kind) {
    SplitJobs a{};
    a.m = m;
    int32_t blocks = 0;
    for (int i = 0; i < n; ++i) {
      if (kind_for(sp[i].k) != kind) continue;
      a.j[a.n] = SplitJob{sp[i].x, sp[i].hi, sp[i].lo, sp[i].scale, sp[i].k, blocks};
      ++a.n;
      blocks += (int32_t)m;
    }
    if (a.n == 0) continue;
    const dim3 grid((unsigned)blocks);
    switch (kind) {
      case 0: hipLaunchKernelGGL((act_quant_row_kernel<1, 128>), grid, dim3(128), 0, s, a); break;
      case 1: hipLaunchKernelGGL((act_quant_row_kernel<2, 128>), grid, dim3(128), 0, s, a); break;
      case 2: hipLaunchKernelGGL((act_quant_row_kernel<4, 128>), grid, dim3(128), 0, s, a); break;
      case 3: hipLaunchKernelGGL((act_quant_row_kernel<8, 128>), grid, dim3(128), 0, s, a); break;
      case 4: hipLaunchKernelGGL((act_quant_row_kernel<6, 256>), grid, dim3(256), 0, s, a); break;
      case 5: hipLaunchKernelGGL((act_quant_row_kernel<8, 256>), grid, dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL(act_quant_kernel, grid, dim3(kThreads), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_act_quant(const uint16_t* x, int64_t m, int64_t k, uint8_t* hi, uint8_t* lo,
                            float* scale, hipStream_t s) {
  const ActSplit sp{x, hi, lo, scale, k};
  return launch_act_quant_group(&sp, 1, m, s);
}

}  // namespace ql
