// Internals shared by the bf16-path GEMM kernels (large-M tiles and the
// small-M split path): tile constants, the per-group dequantizer, the kernel
// parameter block and the split plan.  gfx950 only.
#pragma once

#include "common.h"
#include "device.h"

namespace ql {

constexpr int TK = 64;
constexpr int SA = TK + 8;          // act / forward-W tile row stride (bf16): 144 B
constexpr int SL = 48;              // dX: B-adapter tile [TK][SL] (r <= 32; columns >= r stay 0)
constexpr int AD_ELEMS = 32 * SA;   // forward: A-adapter tile [32][SA] (rows >= r stay 0)
constexpr int BL_ELEMS = TK * SL;

struct Book { float c[16]; };

// ------------------------------------------------------------------ dequantization
// One 32-element group of one row of W: codes plus its raw scale word.
// Loads only fill these registers: every use of a loaded value (scale
// extraction, masking) happens where the group is dequantized, so that no
// instruction right after a load has to wait for it.
struct WGroup {
  uint4 c0, c1;      // 4-bit: c0 = 16 bytes; fp8: c0, c1 = 32 bytes
  uint32_t sraw;     // Q4_0, Q8_0 / MXFP4 / NVFP4: the dword holding the fp16 / E8M0 / two E4M3 scales;
                     // NF4: fp32 bits; FP8: unused
  uint32_t ssh;      // Q4_0, Q8_0, NVFP4: bit offset of the entry in sraw (0 or 16); MXFP4: 0, 8, 16 or 24
};


__device__ __forceinline__ float decode_scale_q40(uint32_t h) {
  h &= 0xFFFF;
  const uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
  float v = (e == 0) ? (float)m * 5.9604644775390625e-08f : __uint_as_float(((e + 112u) << 23) | (m << 13));
  return (h & 0x8000) ? -v : v;
}

// NF4 lookup: 4 codes (one per byte, 0..15) -> 2 dwords of bf16 pairs, from
// byte-plane tables tl/th (entry e's low / high byte at byte e%4 of word e/4).
__device__ __forceinline__ void nf4_lookup4(uint32_t q4, const uint32_t* tl, const uint32_t* th,
                                            uint32_t& out01, uint32_t& out23) {
  const uint32_t s3 = q4 & 0x07070707u;
  const uint32_t s8 = ((q4 >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t l = __builtin_amdgcn_perm(__builtin_amdgcn_perm(tl[3], tl[2], s3),
                                           __builtin_amdgcn_perm(tl[1], tl[0], s3), s8);
  const uint32_t h = __builtin_amdgcn_perm(__builtin_amdgcn_perm(th[3], th[2], s3),
                                           __builtin_amdgcn_perm(th[1], th[0], s3), s8);
  out01 = __builtin_amdgcn_perm(h, l, 0x05010400u);
  out23 = __builtin_amdgcn_perm(h, l, 0x07030602u);
}

// Scale entries per row of W and bytes per entry (NVFP4: one entry is the
// two E4M3 bytes of a 32-element group), and the byte offset of the per-row
// scales in the scale array (NVFP4 keeps its tensor scale in front).
template <int FMT> constexpr int64_t scales_per_row(int64_t k) { return FMT == QL_FMT_NF4 ? k / 64 : k / 32; }
template <int FMT> constexpr int64_t scale_bytes() {
  return (FMT == QL_FMT_Q4_0 || FMT == QL_FMT_Q8_0 || FMT == QL_FMT_NVFP4) ? 2 : (FMT == QL_FMT_MXFP4 ? 1 : 4);
}
template <int FMT> constexpr int64_t scale_offset() { return FMT == QL_FMT_NVFP4 ? 16 : 0; }
// formats with one code byte per element (a 32-element group is 32 bytes)
template <int FMT> constexpr bool byte_codes() { return FMT == QL_FMT_FP8_E4M3 || FMT == QL_FMT_Q8_0; }
// formats with an fp16 scale per 32-element group
template <int FMT> constexpr bool fp16_scales() { return FMT == QL_FMT_Q4_0 || FMT == QL_FMT_Q8_0; }
// formats whose scale entry per 32-element group is 2 bytes (fetched as the
// aligned dword that holds it, plus a shift)
template <int FMT> constexpr bool two_byte_scales() { return fp16_scales<FMT>() || FMT == QL_FMT_NVFP4; }
// formats with one fp32 scale for the whole tensor at the start of the scale array
template <int FMT> constexpr bool tensor_scale() { return FMT == QL_FMT_FP8_E4M3 || FMT == QL_FMT_NVFP4; }

// The dequantization scale(s) of a group from its scale entry `raw` (already
// shifted down) and the tensor scale.  NVFP4 has two: s0 for elements 0..15
// (the low nibbles), s1 for 16..31, each fl32(E4M3(byte) * g); the E4M3
// decode is the hardware conversion (OCP E4M3FN on gfx950, exact).
template <int FMT>
__device__ __forceinline__ void group_scales(uint32_t raw, float tscale, float& s0, float& s1) {
  s1 = 0.0f;
  if constexpr (FMT == QL_FMT_FP8_E4M3) {
    s0 = tscale;
  } else if constexpr (FMT == QL_FMT_NVFP4) {
    s0 = __builtin_amdgcn_cvt_f32_fp8((int)raw, 0) * tscale;
    s1 = __builtin_amdgcn_cvt_f32_fp8((int)raw, 1) * tscale;
  } else if constexpr (fp16_scales<FMT>()) {
    s0 = decode_scale_q40(raw);
  } else if constexpr (FMT == QL_FMT_MXFP4) {
    s0 = e8m0_as_scale(raw);
  } else {
    s0 = __uint_as_float(raw);
  }
}

// Dequantizer of one 32-element group, split so its work can be spread over
// the MFMAs of a contraction step: prepare() once per group (scale decode,
// NF4 / NVFP4 tables), then piece(i) yields elements 8i .. 8i+7 as 4 dwords
// of bf16 pairs.  NVFP4 is decoded like NF4 with the E2M1 values as the code
// book and one table per block of 16 (pieces 0-1 and 2-3).  `scale` is already zero for a group outside W; for MXFP4 (whose
// scale cannot express zero) such a group arrives with its codes cleared.
// MXFP4 codes are pair-packed, so elements 8i .. 8i+7 are the 4 bytes of code
// word i, each turned into a bf16 pair by the hardware conversion.
template <int FMT> struct Deq {
  uint32_t wd[8];
  uint32_t tl[4], th[4];   // NF4: byte planes of the 16-entry bf16 table (NVFP4: elements 0..15)
  uint32_t tl2[4], th2[4]; // NVFP4: the table of elements 16..31
  float d, nd8;            // Q4_0: d and -8 d; Q8_0: d and -128 d; FP8: the tensor scale in d

  // per-thread table of bf16_RNE(fl32(c[q] * a)), split into byte planes
  __device__ __forceinline__ static void build_table(const Book& book, float a, uint32_t* lo, uint32_t* hi) {
    uint32_t pr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pr[i] = pack_bf16x2(book.c[2 * i] * a, book.c[2 * i + 1] * a);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      lo[w] = __builtin_amdgcn_perm(pr[2 * w + 1], pr[2 * w], 0x06040200u);
      hi[w] = __builtin_amdgcn_perm(pr[2 * w + 1], pr[2 * w], 0x07050301u);
    }
  }

  // scale2: NVFP4's scale of elements 16..31 (scale is that of 0..15)
  __device__ __forceinline__ void prepare(const WGroup& g, float scale, const Book& book, bool in = true,
                                          float scale2 = 0.0f) {
    wd[0] = g.c0.x; wd[1] = g.c0.y; wd[2] = g.c0.z; wd[3] = g.c0.w;
    wd[4] = g.c1.x; wd[5] = g.c1.y; wd[6] = g.c1.z; wd[7] = g.c1.w;
    if constexpr (FMT == QL_FMT_MXFP4) {
      const uint32_t keep = in ? ~0u : 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) wd[i] &= keep;
    }
    d = scale;
    nd8 = (FMT == QL_FMT_Q8_0 ? -128.0f : -8.0f) * scale;   // (q - 8) d = fma(q, d, -8d), exact
    if constexpr (FMT == QL_FMT_NF4 || FMT == QL_FMT_NVFP4) build_table(book, scale, tl, th);
    if constexpr (FMT == QL_FMT_NVFP4) build_table(book, scale2, tl2, th2);
  }

  __device__ __forceinline__ uint4 piece(int i) const {
    uint32_t o[4];
    if constexpr (FMT == QL_FMT_MXFP4) {
      o[0] = fp4x2_to_bf16x2<0>(wd[i], d);
      o[1] = fp4x2_to_bf16x2<1>(wd[i], d);
      o[2] = fp4x2_to_bf16x2<2>(wd[i], d);
      o[3] = fp4x2_to_bf16x2<3>(wd[i], d);
    } else if constexpr (FMT == QL_FMT_Q8_0) {
      // two's complement bytes biased to u = q + 128; u d - 128 d = q d exactly
      // (an 8-bit integer times an 11-bit significand), rounded once to bf16
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t u = wd[2 * i + h] ^ 0x80808080u;
        float e[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) e[b] = fmaf((float)((u >> (8 * b)) & 0xFF), d, nd8);
        o[2 * h] = pack_bf16x2(e[0], e[1]);
        o[2 * h + 1] = pack_bf16x2(e[2], e[3]);
      }
    } else if constexpr (FMT == QL_FMT_FP8_E4M3) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[2 * i + h], false);
        const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[2 * i + h], true);
        o[2 * h] = pack_bf16x2(a.x * d, a.y * d);
        o[2 * h + 1] = pack_bf16x2(b.x * d, b.y * d);
      }
    } else {
      // elements 8i .. 8i+7: low nibbles (i < 2) or high nibbles (i >= 2) of words 2(i%2), 2(i%2)+1
      const int sh = i < 2 ? 0 : 4;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t q4 = (wd[2 * (i & 1) + h] >> sh) & 0x0F0F0F0Fu;
        if constexpr (FMT == QL_FMT_Q4_0) {
          float e[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) e[b] = fmaf((float)((q4 >> (8 * b)) & 0xFF), d, nd8);
          o[2 * h] = pack_bf16x2(e[0], e[1]);
          o[2 * h + 1] = pack_bf16x2(e[2], e[3]);
        } else if constexpr (FMT == QL_FMT_NVFP4) {
          if (i < 2) nf4_lookup4(q4, tl, th, o[2 * h], o[2 * h + 1]);
          else nf4_lookup4(q4, tl2, th2, o[2 * h], o[2 * h + 1]);
        } else {
          nf4_lookup4(q4, tl, th, o[2 * h], o[2 * h + 1]);
        }
      }
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  }
};

struct Params {
  const uint16_t* act;   // [M, C]
  const uint8_t* codes;
  const void* scales;
  const uint16_t* down;  // forward: A [R, C]; dX: B [C, R]
  const uint16_t* up;    // forward: B [N, R]; dX: A [R, K]
  uint16_t* out;         // [M, O]
  float* save;           // [M, R] or null
  int64_t M, N, K, C, O;
  float s;
  Book book;
  // split-contraction path: split blockIdx.y covers steps [sps * y, sps * (y + 1)) and
  // writes fp32 partial sums instead of the output
  float* part;           // [splits, M, O]
  float* upart;          // [splits, M, R]
  int sps;
};

// ---- the small-M split path (kernels_split.hip)
// At most SMALL_M tokens: 64-row tiles, STN columns wide, the contraction split
// across workgroups so that up to 256 of them (512 for the 16-token forward)
// stream W with at least 4 steps each, then a fixed-order reduction kernel.
constexpr int64_t SMALL_M = 64;
constexpr int STN = 128;
constexpr int MAX_SPLITS = 16;


struct SplitPlan {
  int splits = 0, sps = 0;
  size_t upart_off = 0, total = 0;
};

SplitPlan split_plan(bool trans, int64_t m, int64_t n, int64_t k, int r);

// A group of independent split-path problems of one format, direction, rank
// and token count, run by one split launch and one reduction launch: each
// problem keeps its own tiles, split plan and summation order, so its results
// are bitwise those of a launch of its own.
constexpr int MAX_GROUP = QL_GROUP_MAX;
struct SplitGroup {
  Params p[MAX_GROUP];
  int32_t splits[MAX_GROUP];
  int32_t n;
};
// split kernel plus reduction for every problem of g; with gf (dX only, one
// entry per problem) the reduction also writes dA and dB
hipError_t launch_split_path(int fmt, bool trans, int r, const SplitGroup& g, const GradFuse* gf, hipStream_t s);

}  // namespace ql
