// a2-a4 and a5-a7: the base GEMM over a block-quantized W, dequantized in
// registers and staged as bf16 tiles in LDS, with the rank-r LoRA terms fused.
//
//   forward (trans = false):  y  = x . deq(W)^T + s . U . B^T,   U = x . A^T
//   dX      (trans = true ):  dX = dY . deq(W)  + s . V . A,     V = dY . B
//
// One kernel serves both: the activation operand act [M, C] is contracted over
// C (C = K forward, C = N for dX); W [N, K] is read in its packed row-major
// form and dequantized into an LDS tile laid out [row of W][K-contiguous],
// which is the MFMA B operand as-is for the forward GEMM and is read with
// LDS transpose loads (ds_read_b64_tr_b16) for dX, so no transposed copy of
// the base ever exists.  The rank-r "down" projection (U or V) rides along
// the same contraction loop on 16x16x32 MFMAs, its adapter tile staged in
// LDS next to the activation tile; the "up" product is one more short MFMA
// contraction over 2r bf16 columns (s.U split into a high and a low bf16
// term, so the epilogue keeps ~16 bits of U) before the single bf16
// rounding of the output.  The base is never written.
//
// Dequantized tile values are bf16_RNE(fl32 value): Q4_0 (q - 8) * d is exact
// in fp32; NF4 uses a per-thread 16-entry table of bf16_RNE(fl32(c[q] * a))
// looked up with byte permutes; FP8 decodes with the hardware E4M3 convert
// and multiplies by the tensor scale.
//
// Tiling (gfx950): the workgroup owns a 256 x TN output tile (TN = 256, or
// 128 when 256-wide tiles would leave CUs idle).  With 512 threads (the
// default) there are two waves per SIMD, so one wave's stalls are covered by
// the other's MFMAs; each wave owns a 128 x 64 (TN = 256) or 64 x 64 block.
// A 256-thread form (one wave per SIMD, 128 x TN/2 blocks) is kept for
// comparison.  The contraction advances 64 at a time through double-buffered
// LDS.  Each step runs the MFMAs of the current stage in four 16-deep slices;
// between them it writes the next stage from registers (activation copy,
// dequantization) and reloads each register from global memory as soon as it
// is stored, so every load has a whole step to land.  The workgroup barrier
// comes before the last slice: the first operands of the next stage are read
// from LDS while that slice's MFMAs run.  All global reads are buffer loads
// through resource descriptors, so reads past the end of a tensor return
// zero with no address clamping in the loop.  Operands are swapped in the
// MFMA (B first), so each lane ends up with 4 consecutive output columns per
// row and writes them with one 8-byte store.  Workgroups are remapped so each
// XCD (own L2) works on a contiguous run of tiles.
#include "common.h"

namespace ql {
namespace {

constexpr int TM = 256, TK = 64;
constexpr int SA = TK + 8;          // act / forward-W tile row stride (bf16): 144 B
constexpr int SL = 48;              // dX: B-adapter tile [TK][SL] (r <= 32; columns >= r stay 0)
constexpr int A_ELEMS = TM * SA;
constexpr int AD_ELEMS = 32 * SA;   // forward: A-adapter tile [32][SA] (rows >= r stay 0)
constexpr int BL_ELEMS = TK * SL;

// NTH = 256: four waves, one per SIMD, each owning a 128 x TN/2 block.
// NTH = 512: eight waves, two per SIMD, each owning a 128 x 64 (TN = 256)
// or 64 x 64 (TN = 128) block.
template <int TN, int NTH> struct Shape {
  static constexpr int NW = NTH / 64;
  static constexpr int SBT = TN + 32;                 // dX W tile [TK][TN] stride (576 / 320 B rows)
  static constexpr int BF_ELEMS = TN * SA;
  static constexpr int BT_ELEMS = TK * SBT;
  static constexpr int WAVES_N = (NW == 8 && TN == 256) ? 4 : 2;
  static constexpr int WAVES_M = NW / WAVES_N;
  static constexpr int WM = TM / WAVES_M, WN = TN / WAVES_N;
  static constexpr int MB = WM / 32, NB = WN / 32;    // 32x32 MFMA blocks per wave
  static constexpr int WGT = TN * TK / 32;            // W groups per stage
  static constexpr int WG = WGT >= NTH ? WGT / NTH : 1;   // W groups per thread
  static constexpr bool WPART = WGT < NTH;            // only threads below WGT carry one
  static constexpr int AR = TM * TK / 8 / NTH;        // 16-byte activation pieces per thread
  static constexpr int ARS = NTH / 8;                 // rows between a thread's pieces
  static constexpr int UI = TM / NW / 16;             // 16-row blocks of the rank-r projection per wave
};

struct Book { float c[16]; };

typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

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

// ------------------------------------------------------------------ dequantization
// One 32-element group of one row of W: codes plus its raw scale word.
struct WGroup {
  uint4 c0, c1;      // 4-bit: c0 = 16 bytes; fp8: c0, c1 = 32 bytes
  uint32_t sraw;     // Q4_0: fp16 bits; NF4: fp32 bits; FP8: unused
};

__device__ __forceinline__ float decode_scale_q40(uint32_t h) {
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

// Dequantizer of one 32-element group, split so its work can be spread over
// the MFMAs of a contraction step: prepare() once per group (scale decode,
// NF4 table), then piece(i) yields elements 8i .. 8i+7 as 4 dwords of bf16
// pairs.  `scale` is already zero for a group outside W.
template <int FMT> struct Deq {
  uint32_t wd[8];
  uint32_t tl[4], th[4];   // NF4: byte planes of the 16-entry bf16 table
  float d, nd8;            // Q4_0: d and -8 d; FP8: the tensor scale in d

  __device__ __forceinline__ void prepare(const WGroup& g, float scale, const Book& book) {
    wd[0] = g.c0.x; wd[1] = g.c0.y; wd[2] = g.c0.z; wd[3] = g.c0.w;
    wd[4] = g.c1.x; wd[5] = g.c1.y; wd[6] = g.c1.z; wd[7] = g.c1.w;
    d = scale;
    nd8 = -8.0f * scale;                 // (q - 8) d = fma(q, d, -8d), exact
    if constexpr (FMT == QL_FMT_NF4) {
      // per-thread table of bf16_RNE(fl32(c[q] * a)), split into byte planes
      uint32_t pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pr[i] = pack_bf16x2(book.c[2 * i] * scale, book.c[2 * i + 1] * scale);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        tl[w] = __builtin_amdgcn_perm(pr[2 * w + 1], pr[2 * w], 0x06040200u);
        th[w] = __builtin_amdgcn_perm(pr[2 * w + 1], pr[2 * w], 0x07050301u);
      }
    }
  }

  __device__ __forceinline__ uint4 piece(int i) const {
    uint32_t o[4];
    if constexpr (FMT == QL_FMT_FP8_E4M3) {
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
};

template <int FMT, bool TRANS, int R, int TN, int NTH>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(NTH / 256, NTH / 256)))
void qgemm_kernel(Params p) {
  using S = Shape<TN, NTH>;
  constexpr int NT = NTH;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  constexpr int B_ELEMS = TRANS ? S::BT_ELEMS : S::BF_ELEMS;
  constexpr int D_ELEMS = TRANS ? BL_ELEMS : AD_ELEMS;
  constexpr int STAGE = A_ELEMS + B_ELEMS + D_ELEMS;
  constexpr int RB = (R + 15) / 16;                  // 16-column blocks of the rank-r projection
  constexpr int MB = S::MB, NB = S::NB, WG = S::WG;
  constexpr int GPR = TRANS ? TN / 32 : TK / 32;     // W groups per W-tile row
  constexpr bool FP8 = FMT == QL_FMT_FP8_E4M3;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / S::WAVES_N, wn = wave % S::WAVES_N;

  // ---- tile assignment: contiguous runs of tiles per XCD (workgroups go round-robin over 8 XCDs)
  const int nt = (int)((p.O + TN - 1) / TN);
  const int mt = (int)((p.M + TM - 1) / TM);
  const int tiles = nt * mt;
  int t = blockIdx.x;
  if ((tiles & 7) == 0) t = (t & 7) * (tiles >> 3) + (t >> 3);
  const int64_t o0 = (int64_t)(t % nt) * TN;
  const int64_t m0 = (int64_t)(t / nt) * TM;
  const int KT = (int)((p.C + TK - 1) / TK);

  // ---- buffer resources (bases rebased to this tile, so 32-bit offsets suffice)
  const __amdgpu_buffer_rsrc_t ract = rsrc(p.act + m0 * p.C, (p.M - m0) * p.C * 2);
  const int64_t crow = FP8 ? p.K : p.K / 2;          // code bytes per row of W
  const int64_t wrow0 = TRANS ? 0 : o0;              // first W row this tile reads
  const int64_t wcol0 = TRANS ? (FP8 ? o0 : o0 / 2) : 0;
  const __amdgpu_buffer_rsrc_t rcode = rsrc(p.codes + wrow0 * crow + wcol0, (p.N - wrow0) * crow - wcol0);
  const int64_t srow = FMT == QL_FMT_Q4_0 ? p.K / 32 : p.K / 64;   // scale words per row
  const int64_t ssz = FMT == QL_FMT_Q4_0 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rscale =
      rsrc((const char*)p.scales + wrow0 * srow * ssz, (p.N - wrow0) * srow * ssz);
  const __amdgpu_buffer_rsrc_t rdown = rsrc(p.down, (int64_t)R * p.C * 2);

  float tscale = 0.0f;
  if constexpr (FP8) tscale = reinterpret_cast<const float*>(p.scales)[0];

  // ---- per-thread load coordinates
  const int arow = tid >> 3, acol = (tid & 7) * 8;   // act: rows arow + ARS i, 8 columns
  constexpr int AR = S::AR, ARS = S::ARS;
  const bool wtask = !S::WPART || tid < S::WGT;     // wave-uniform
  int wr[WG], wg[WG];                                // W groups: row of the W tile, group in that row
  bool wg_in[WG];                                    // dX: the group's output columns lie inside K
#pragma unroll
  for (int j = 0; j < WG; ++j) {
    const int g = tid + NT * j;
    wr[j] = g / GPR;
    wg[j] = g % GPR;
    wg_in[j] = !TRANS || (o0 + 32 * (wg[j] + 1) <= p.K);
  }
  // adapter tile pieces (16 bytes): forward A[j][c0 + 8c ..]; dX B[c0 + row][8c ..]
  constexpr int DPR = TRANS ? R / 8 : TK / 8;        // pieces per adapter row
  const bool dload = tid < 8 * R;                    // TK * R / 8 pieces either way
  const int drow = tid / DPR, dcol = (tid % DPR) * 8;

  uint4 areg[AR];
  WGroup wreg[WG];
#pragma unroll
  for (int j = 0; j < WG; ++j) {
    wreg[j].c1 = make_uint4(0, 0, 0, 0);
    wreg[j].sraw = 0;
  }
  uint4 dreg = make_uint4(0, 0, 0, 0);

  // ---- global loads of stage kt, piece by piece (registers are reloaded as soon as stored)
  auto load_act = [&](int kt, int i) {
    const int64_t c0 = (int64_t)kt * TK;
    areg[i] = bload16(ract, (uint32_t)(((arow + ARS * i) * p.C + c0 + acol) * 2));
    if (c0 + TK > p.C && c0 + acol >= p.C) areg[i] = make_uint4(0, 0, 0, 0);
  };
  auto load_w = [&](int kt, int j) {
    const int64_t c0 = (int64_t)kt * TK;
    // forward: row o0 + wr, K columns c0 + 32 wg; dX: row c0 + wr, K columns o0 + 32 wg
    const int64_t wrow = TRANS ? c0 + wr[j] : wr[j];
    const int64_t kgrp = TRANS ? wg[j] : (c0 >> 5) + wg[j];   // group index relative to the tile base
    const uint32_t coff = (uint32_t)(wrow * crow + kgrp * (FP8 ? 32 : 16));
    if (!wtask) return;
    wreg[j].c0 = bload16(rcode, coff);
    if constexpr (FP8) {
      wreg[j].c1 = bload16(rcode, coff + 16);
    } else {
      const int64_t kabs = TRANS ? (o0 >> 5) + wg[j] : kgrp;   // group index along K
      if constexpr (FMT == QL_FMT_Q4_0) {
        const int64_t idx = wrow * srow + kabs;
        wreg[j].sraw = bload4(rscale, (uint32_t)((idx * 2) & ~3LL)) >> ((idx & 1) * 16);
      } else {
        wreg[j].sraw = bload4(rscale, (uint32_t)((wrow * srow + (kabs >> 1)) * 4));
      }
    }
    if (!TRANS && c0 + TK > p.C && c0 + 32 * wg[j] >= p.C) {
      wreg[j].c0 = make_uint4(0, 0, 0, 0);
      wreg[j].c1 = wreg[j].c0;
      wreg[j].sraw = 0;
    }
  };
  auto load_adapter = [&](int kt) {
    const int64_t c0 = (int64_t)kt * TK;
    if (dload) {
      if constexpr (TRANS) {
        dreg = bload16(rdown, (uint32_t)(((c0 + drow) * R + dcol) * 2));
      } else {
        dreg = bload16(rdown, (uint32_t)((drow * p.C + c0 + dcol) * 2));
        if (c0 + TK > p.C && c0 + dcol >= p.C) dreg = make_uint4(0, 0, 0, 0);
      }
    }
  };

  // ---- stage stores
  Deq<FMT> deq;
  auto store_act = [&](uint16_t* st, int i) {
    *reinterpret_cast<uint4*>(st + (arow + ARS * i) * SA + acol) = areg[i];
  };
  auto prepare_w = [&](int j) {
    float scale;
    if constexpr (FP8) scale = tscale;
    else if constexpr (FMT == QL_FMT_Q4_0) scale = decode_scale_q40(wreg[j].sraw & 0xFFFF);
    else scale = __uint_as_float(wreg[j].sraw);
    deq.prepare(wreg[j], wg_in[j] ? scale : 0.0f, p.book);
  };
  auto store_w = [&](uint16_t* st, int j, int i) {   // elements 8i .. 8i+7 of W group j
    if (!wtask) return;
    uint16_t* dst = st + A_ELEMS + (TRANS ? wr[j] * S::SBT : wr[j] * SA) + wg[j] * 32 + 8 * i;
    *reinterpret_cast<uint4*>(dst) = deq.piece(i);
  };
  auto store_adapter = [&](uint16_t* st) {
    if (dload) *reinterpret_cast<uint4*>(st + A_ELEMS + B_ELEMS + drow * (TRANS ? SL : SA) + dcol) = dreg;
  };

  // ---- accumulators
  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  constexpr int UI = S::UI;
  f32x4 uacc[UI][RB];                                // rank-r projection of rows 16 UI wave + 16 i ..
#pragma unroll
  for (int i = 0; i < UI; ++i)
#pragma unroll
    for (int jb = 0; jb < RB; ++jb) uacc[i][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- MFMA operand fragments, double-buffered across 16-deep slices
  bf16x8 fa[2][MB], fb[2][NB];
  auto read_frags = [&](const uint16_t* st, int ks) {
    const uint16_t* As = st;
    const uint16_t* Bs = st + A_ELEMS;
    const int h = ks & 1;
#pragma unroll
    for (int i = 0; i < MB; ++i)
      fa[h][i] = *reinterpret_cast<const bf16x8*>(As + (S::WM * wm + 32 * i + (lane & 31)) * SA + ks * 16 + 8 * (lane >> 5));
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if constexpr (TRANS) {
        const int b = lane >> 4, sl = lane & 15;
        const int col = S::WN * wn + 32 * j + 16 * (b & 1) + 4 * (sl & 3);
        const int row = ks * 16 + 8 * (b >> 1) + (sl >> 2);
        fb[h][j] = tr16x8(Bs + row * S::SBT + col, Bs + (row + 4) * S::SBT + col);
      } else {
        fb[h][j] = *reinterpret_cast<const bf16x8*>(Bs + (S::WN * wn + 32 * j + (lane & 31)) * SA + ks * 16 + 8 * (lane >> 5));
      }
    }
  };
  auto mfma_ks = [&](int ks) {
    const int h = ks & 1;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[h][j], fa[h][i], acc[i][j], 0, 0, 0);
  };
  // rank-r down projection of this wave's 16 UI rows over the whole stage
  auto compute_u = [&](const uint16_t* st) {
    const uint16_t* As = st;
    const uint16_t* Ds = st + A_ELEMS + B_ELEMS;
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      bf16x8 bd[RB];
#pragma unroll
      for (int jb = 0; jb < RB; ++jb) {
        if constexpr (TRANS) {
          const int b = lane >> 4, sl = lane & 15;
          const int row = 32 * kp + 8 * b + (sl >> 2), col = 16 * jb + 4 * (sl & 3);
          bd[jb] = tr16x8(Ds + row * SL + col, Ds + (row + 4) * SL + col);
        } else {
          bd[jb] = *reinterpret_cast<const bf16x8*>(Ds + (16 * jb + (lane & 15)) * SA + 32 * kp + 8 * (lane >> 4));
        }
      }
#pragma unroll
      for (int i = 0; i < UI; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(As + (16 * UI * wave + 16 * i + (lane & 15)) * SA + 32 * kp + 8 * (lane >> 4));
#pragma unroll
        for (int jb = 0; jb < RB; ++jb) {
          if constexpr (NT == 256) {
            // accumulated with VALU adds: the accumulation registers all hold the 128 x 128 block
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bd[jb], z, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) uacc[i][jb][e] += d[e];
          } else {
            uacc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bd[jb], uacc[i][jb], 0, 0, 0);
          }
        }
      }
    }
  };

  // adapter tiles: the rows / columns past r stay zero in both stages
  for (int i = tid; i < D_ELEMS; i += NT) {
    smem[A_ELEMS + B_ELEMS + i] = 0;
    smem[STAGE + A_ELEMS + B_ELEMS + i] = 0;
  }
  lds_barrier();

  // ---- prologue: stage 0 stored, stage 1 in flight, first fragments read
#pragma unroll
  for (int i = 0; i < AR; ++i) load_act(0, i);
#pragma unroll
  for (int j = 0; j < WG; ++j) load_w(0, j);
  load_adapter(0);
#pragma unroll
  for (int i = 0; i < AR; ++i) store_act(smem, i);
#pragma unroll
  for (int j = 0; j < WG; ++j) {
    prepare_w(j);
#pragma unroll
    for (int i = 0; i < 4; ++i) store_w(smem, j, i);
  }
  store_adapter(smem);
  {
    const int k1 = KT > 1 ? 1 : 0;
#pragma unroll
    for (int i = 0; i < AR; ++i) load_act(k1, i);
#pragma unroll
    for (int j = 0; j < WG; ++j) load_w(k1, j);
    load_adapter(k1);
  }
  lds_barrier();
  read_frags(smem, 0);

  // ---- steady state.  Step kt runs the MFMAs of stage kt (buffer cs) while it
  // writes stage kt+1 (loaded one step earlier) into the other buffer ns,
  // which every wave finished reading before the previous barrier.  The
  // stores are spread over the first three 16-deep slices, each register
  // being reloaded for stage kt+2 as soon as it is stored, so every load has
  // a full step to land.  The barrier sits before the last slice: by then
  // this wave's reads of cs and writes of ns are complete, and the first
  // fragments of ns are read while the last slice's MFMAs run.
  for (int kt = 0; kt + 1 < KT; ++kt) {
    const uint16_t* cs = smem + (kt & 1) * STAGE;
    uint16_t* ns = smem + ((kt & 1) ^ 1) * STAGE;
    const int kl = kt + 2 < KT ? kt + 2 : KT - 1;
    // slice 0: activation tile
    read_frags(cs, 1);
    mfma_ks(0);
#pragma unroll
    for (int i = 0; i < AR; ++i) {
      store_act(ns, i);
      load_act(kl, i);
    }
    // slice 1: W group 0 (and the adapter piece)
    read_frags(cs, 2);
    mfma_ks(1);
    prepare_w(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) store_w(ns, 0, i);
    load_w(kl, 0);
    store_adapter(ns);
    load_adapter(kl);
    // slice 2: W group 1, rank-r projection
    read_frags(cs, 3);
    mfma_ks(2);
    if constexpr (WG > 1) {
      prepare_w(1);
#pragma unroll
      for (int i = 0; i < 4; ++i) store_w(ns, 1, i);
      load_w(kl, 1);
    }
    compute_u(cs);
    lds_barrier();
    // slice 3
    read_frags(ns, 0);
    mfma_ks(3);
  }
  {
    const uint16_t* cs = smem + ((KT - 1) & 1) * STAGE;
    read_frags(cs, 1);
    mfma_ks(0);
    read_frags(cs, 2);
    mfma_ks(1);
    read_frags(cs, 3);
    mfma_ks(2);
    compute_u(cs);
    mfma_ks(3);
  }
  lds_barrier();

  // ---------------------------------------------------------------- epilogue
  // Ax [TM][2R+8]: high and low bf16 parts of s.U; Bx [TN][2R+8]: the up matrix twice.
  constexpr int SX = 2 * R + 8;
  uint16_t* Ax = smem;
  uint16_t* Bx = smem + TM * SX;
#pragma unroll
  for (int i = 0; i < UI; ++i)
#pragma unroll
    for (int jb = 0; jb < RB; ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * UI * wave + 16 * i + 4 * (lane >> 4) + e;
        const int j = 16 * jb + (lane & 15);
        if (j < R) {
          const float u = uacc[i][jb][e];
          if (p.save && (o0 == 0) && m0 + row < p.M) p.save[(m0 + row) * R + j] = u;
          const float su = p.s * u;
          const __bf16 h = (__bf16)su;
          const __bf16 l = (__bf16)(su - (float)h);
          Ax[row * SX + j] = __builtin_bit_cast(uint16_t, h);
          Ax[row * SX + R + j] = __builtin_bit_cast(uint16_t, l);
        }
      }
  for (int idx = tid; idx < TN * R; idx += NT) {
    const int col = idx / R, j = idx % R;
    uint16_t v = 0;
    if (o0 + col < p.O) v = TRANS ? p.up[(int64_t)j * p.K + o0 + col] : p.up[(o0 + col) * R + j];
    Bx[col * SX + j] = v;
    Bx[col * SX + R + j] = v;
  }
  lds_barrier();
#pragma unroll
  for (int ks = 0; ks < (2 * R) / 16; ++ks) {
    bf16x8 af[MB], bfr[NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(Ax + (S::WM * wm + 32 * i + (lane & 31)) * SX + ks * 16 + 8 * (lane >> 5));
#pragma unroll
    for (int j = 0; j < NB; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(Bx + (S::WN * wn + 32 * j + (lane & 31)) * SX + ks * 16 + 8 * (lane >> 5));
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
  }
  // ---- store bf16: lane holds row (lane & 31) and, per 4 accumulators, 4 consecutive columns
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int64_t row = m0 + S::WM * wm + 32 * i + (lane & 31);
    if (row < p.M) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const int64_t col = o0 + S::WN * wn + 32 * j + 8 * k4 + 4 * (lane >> 5);
          if (col < p.O) {
            const uint32_t lo = pack_bf16x2(acc[i][j][4 * k4 + 0], acc[i][j][4 * k4 + 1]);
            const uint32_t hi = pack_bf16x2(acc[i][j][4 * k4 + 2], acc[i][j][4 * k4 + 3]);
            *reinterpret_cast<uint2*>(p.out + row * p.O + col) = make_uint2(lo, hi);
          }
        }
    }
  }
}

template <int FMT, bool TRANS, int R, int TN, int NTH>
hipError_t launch_t(const Params& p, hipStream_t s) {
  using S = Shape<TN, NTH>;
  constexpr int B_ELEMS = TRANS ? S::BT_ELEMS : S::BF_ELEMS;
  constexpr int D_ELEMS = TRANS ? BL_ELEMS : AD_ELEMS;
  constexpr size_t smem = 2 * (size_t)(A_ELEMS + B_ELEMS + D_ELEMS) * sizeof(uint16_t);
  static_assert(smem <= 160 * 1024, "LDS budget");
  static_assert((size_t)(TM + TN) * (2 * R + 8) * sizeof(uint16_t) <= smem, "epilogue LDS");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)qgemm_kernel<FMT, TRANS, R, TN, NTH>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t tiles = ((p.O + TN - 1) / TN) * ((p.M + TM - 1) / TM);
  hipLaunchKernelGGL((qgemm_kernel<FMT, TRANS, R, TN, NTH>), dim3((unsigned)tiles), dim3(NTH), smem, s, p);
  return hipGetLastError();
}

// Output tile width: 256 when that still gives at least one tile per CU, else 128.
template <int FMT, bool TRANS, int R>
hipError_t launch_w(const Params& p, hipStream_t s) {
  const int64_t tiles256 = ((p.O + 255) / 256) * ((p.M + TM - 1) / TM);
#ifndef QL_GEMM_THREADS
#define QL_GEMM_THREADS 512
#endif
  if (tiles256 >= 256) return launch_t<FMT, TRANS, R, 256, QL_GEMM_THREADS>(p, s);
  return launch_t<FMT, TRANS, R, 128, QL_GEMM_THREADS>(p, s);
}

template <int FMT, bool TRANS>
hipError_t launch_r(const Params& p, int r, hipStream_t s) {
  switch (r) {
    case 8: return launch_w<FMT, TRANS, 8>(p, s);
    case 16: return launch_w<FMT, TRANS, 16>(p, s);
    default: return launch_w<FMT, TRANS, 32>(p, s);
  }
}

template <int FMT>
hipError_t launch_f(const Params& p, bool trans, int r, hipStream_t s) {
  return trans ? launch_r<FMT, true>(p, r, s) : launch_r<FMT, false>(p, r, s);
}

}  // namespace

hipError_t launch_qgemm(const GemmCall& c, hipStream_t s) {
  Params p{};
  p.act = c.act;
  p.codes = c.w->codes;
  p.scales = c.w->scales;
  p.down = c.down;
  p.up = c.up;
  p.out = c.out;
  p.save = c.save;
  p.M = c.m;
  p.N = c.w->n_out;
  p.K = c.w->k_in;
  p.C = c.trans ? p.N : p.K;
  p.O = c.trans ? p.K : p.N;
  p.s = c.s;
  const Nf4Table& t = nf4_table();
  for (int i = 0; i < 16; ++i) p.book.c[i] = t.level[i];
  switch (c.w->format) {
    case QL_FMT_Q4_0: return launch_f<QL_FMT_Q4_0>(p, c.trans, c.r, s);
    case QL_FMT_NF4: return launch_f<QL_FMT_NF4>(p, c.trans, c.r, s);
    default: return launch_f<QL_FMT_FP8_E4M3>(p, c.trans, c.r, s);
  }
}

}  // namespace ql
