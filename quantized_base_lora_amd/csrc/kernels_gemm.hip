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
// Tiling (gfx950): one 512-thread workgroup per CU, i.e. two waves per SIMD,
// so one wave's stalls (LDS latency, dependencies, the barrier) are covered
// by the other's MFMAs.  The workgroup owns a 256 x TN output tile (TN = 256:
// waves 2 x 4 of 128 x 64; TN = 128: waves 4 x 2 of 64 x 64).  The
// contraction advances 64 at a time through double-buffered LDS: at the
// start of each step the waves store the next stage from registers
// (activation copy, dequantization) and immediately reissue the global loads
// of the stage after, which then have a whole step of MFMAs to land.  All
// global reads are buffer loads through resource descriptors, so reads past
// the end of a tensor return zero with no address clamping in the loop.
// Operands are swapped in the MFMA (B first), so each lane ends up with 4
// consecutive output columns per row and writes them with one 8-byte store.
// Workgroups are remapped so each XCD (own L2) works on a contiguous run of
// tiles.
#include "common.h"

namespace ql {
namespace {

constexpr int TM = 256, TK = 64;
constexpr int NTHREADS = 512;
constexpr int SA = TK + 8;          // act / forward-W tile row stride (bf16): 144 B
constexpr int SL = 48;              // dX: B-adapter tile [TK][SL] (r <= 32; columns >= r stay 0)
constexpr int A_ELEMS = TM * SA;
constexpr int AD_ELEMS = 32 * SA;   // forward: A-adapter tile [32][SA] (rows >= r stay 0)
constexpr int BL_ELEMS = TK * SL;

template <int TN> struct Shape {
  static constexpr int SBT = TN + 32;                 // dX W tile [TK][TN] stride (576 / 320 B rows)
  static constexpr int BF_ELEMS = TN * SA;
  static constexpr int BT_ELEMS = TK * SBT;
  static constexpr int WAVES_N = TN == 256 ? 4 : 2;   // waves along N
  static constexpr int WAVES_M = 8 / WAVES_N;
  static constexpr int WM = TM / WAVES_M;             // wave tile rows (128 / 64)
  static constexpr int WN = TN / WAVES_N;             // wave tile columns (64)
  static constexpr int MB = WM / 32, NB = WN / 32;    // 32x32 MFMA blocks per wave
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

// Dequantize one 32-element group into 16 dwords (bf16 pairs in element order);
// `scale` is already zero for a group outside W.
template <int FMT>
__device__ __forceinline__ void dequant_group(const WGroup& g, float scale, const Book& book, uint32_t* out) {
  if constexpr (FMT == QL_FMT_FP8_E4M3) {
    const uint32_t wd[8] = {g.c0.x, g.c0.y, g.c0.z, g.c0.w, g.c1.x, g.c1.y, g.c1.z, g.c1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], false);
      const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], true);
      out[2 * i] = pack_bf16x2(a.x * scale, a.y * scale);
      out[2 * i + 1] = pack_bf16x2(b.x * scale, b.y * scale);
    }
  } else {
    const uint32_t wd[4] = {g.c0.x, g.c0.y, g.c0.z, g.c0.w};
    if constexpr (FMT == QL_FMT_Q4_0) {
      const float d = scale, nd8 = -8.0f * scale;        // (q - 8) d = fma(q, d, -8d), exact
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = wd[i] & 0x0F0F0F0Fu, hi = (wd[i] >> 4) & 0x0F0F0F0Fu;
        float e[8];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          e[b] = fmaf((float)((lo >> (8 * b)) & 0xFF), d, nd8);
          e[4 + b] = fmaf((float)((hi >> (8 * b)) & 0xFF), d, nd8);
        }
        out[2 * i] = pack_bf16x2(e[0], e[1]);
        out[2 * i + 1] = pack_bf16x2(e[2], e[3]);
        out[8 + 2 * i] = pack_bf16x2(e[4], e[5]);
        out[8 + 2 * i + 1] = pack_bf16x2(e[6], e[7]);
      }
    } else {
      // per-thread table of bf16_RNE(fl32(c[q] * a)), split into byte planes
      uint32_t pr[8], tl[4], th[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) pr[i] = pack_bf16x2(book.c[2 * i] * scale, book.c[2 * i + 1] * scale);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        tl[w] = __builtin_amdgcn_perm(pr[2 * w + 1], pr[2 * w], 0x06040200u);
        th[w] = __builtin_amdgcn_perm(pr[2 * w + 1], pr[2 * w], 0x07050301u);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = wd[i] & 0x0F0F0F0Fu, hi = (wd[i] >> 4) & 0x0F0F0F0Fu;
        nf4_lookup4(lo, tl, th, out[2 * i], out[2 * i + 1]);
        nf4_lookup4(hi, tl, th, out[8 + 2 * i], out[8 + 2 * i + 1]);
      }
    }
  }
}

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

template <int FMT, bool TRANS, int R, int TN>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qgemm_kernel(Params p) {
  using S = Shape<TN>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  constexpr int B_ELEMS = TRANS ? S::BT_ELEMS : S::BF_ELEMS;
  constexpr int D_ELEMS = TRANS ? BL_ELEMS : AD_ELEMS;
  constexpr int STAGE = A_ELEMS + B_ELEMS + D_ELEMS;
  constexpr int RB = (R + 15) / 16;                  // 16-column blocks of the rank-r projection
  constexpr int MB = S::MB, NB = S::NB;
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
  const int arow = tid >> 3, acol = (tid & 7) * 8;   // act: rows arow + 64 i, 8 columns
  constexpr int W_TASKS = (TRANS ? TK * TN : TN * TK) / 32;   // W groups per stage: 512 or 256
  const bool wtask = W_TASKS == NTHREADS || tid < W_TASKS;    // wave-uniform (waves 0..3 when 256)
  const int wr = tid / GPR, wg = tid % GPR;          // W group: row of the W tile, group in that row
  // dX: output columns of this thread's W group lying outside K read as zero
  const bool wg_in = !TRANS || (o0 + 32 * (wg + 1) <= p.K);
  // adapter tile pieces (16 bytes): forward A[j][c0 + 8c ..]; dX B[c0 + row][8c ..]
  constexpr int DPR = TRANS ? R / 8 : TK / 8;        // pieces per adapter row
  constexpr int DTASKS = TRANS ? TK * DPR : R * DPR;
  const bool dload = tid < DTASKS;
  const int drow = tid / DPR, dcol = (tid % DPR) * 8;

  uint4 areg[4];
  WGroup wreg;
  wreg.c1 = make_uint4(0, 0, 0, 0);
  wreg.sraw = 0;
  uint4 dreg = make_uint4(0, 0, 0, 0);

  auto issue_loads = [&](int kt) {
    const int64_t c0 = (int64_t)kt * TK;
    const bool ragged = c0 + TK > p.C;               // uniform: only the last step of a ragged C
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      areg[i] = bload16(ract, (uint32_t)(((arow + 64 * i) * p.C + c0 + acol) * 2));
      if (ragged && c0 + acol >= p.C) areg[i] = make_uint4(0, 0, 0, 0);
    }
    // W group: forward row o0 + wr, K columns c0 + 32 wg; dX row c0 + wr, K columns o0 + 32 wg
    const int64_t wrow = TRANS ? c0 + wr : wr;
    const int64_t kgrp = TRANS ? wg : (c0 >> 5) + wg;   // group index relative to the tile base
    const uint32_t coff = (uint32_t)(wrow * crow + kgrp * (FP8 ? 32 : 16));
    if (wtask) {
    wreg.c0 = bload16(rcode, coff);
    if constexpr (FP8) {
      wreg.c1 = bload16(rcode, coff + 16);
    } else {
      const int64_t kabs = TRANS ? (o0 >> 5) + wg : kgrp;   // group index along K
      if constexpr (FMT == QL_FMT_Q4_0) {
        const int64_t idx = wrow * srow + kabs;
        wreg.sraw = bload4(rscale, (uint32_t)((idx * 2) & ~3LL)) >> ((idx & 1) * 16);
      } else {
        wreg.sraw = bload4(rscale, (uint32_t)((wrow * srow + (kabs >> 1)) * 4));
      }
    }
    }
    if (ragged && !TRANS && c0 + 32 * wg >= p.C) {
      wreg.c0 = make_uint4(0, 0, 0, 0);
      wreg.c1 = wreg.c0;
      wreg.sraw = 0;
    }
    if (dload) {
      if constexpr (TRANS) {
        dreg = bload16(rdown, (uint32_t)(((c0 + drow) * R + dcol) * 2));
      } else {
        dreg = bload16(rdown, (uint32_t)((drow * p.C + c0 + dcol) * 2));
        if (ragged && c0 + dcol >= p.C) dreg = make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto store_stage = [&](uint16_t* st) {
    uint16_t* As = st;
    uint16_t* Bs = st + A_ELEMS;
    uint16_t* Ds = st + A_ELEMS + B_ELEMS;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(As + (arow + 64 * i) * SA + acol) = areg[i];
    float scale;
    if constexpr (FP8) scale = tscale;
    else if constexpr (FMT == QL_FMT_Q4_0) scale = decode_scale_q40(wreg.sraw & 0xFFFF);
    else scale = __uint_as_float(wreg.sraw);
    scale = wg_in ? scale : 0.0f;
    if (wtask) {
      uint32_t v[16];
      dequant_group<FMT>(wreg, scale, p.book, v);
      uint16_t* dst = TRANS ? (Bs + wr * S::SBT + wg * 32) : (Bs + wr * SA + wg * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(dst + 8 * i) = make_uint4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    }
    if (dload) *reinterpret_cast<uint4*>(Ds + drow * (TRANS ? SL : SA) + dcol) = dreg;
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  f32x4 uacc[2][RB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jb = 0; jb < RB; ++jb) uacc[i][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // adapter tiles: the rows / columns past r stay zero in both stages
  for (int i = tid; i < D_ELEMS; i += NTHREADS) {
    smem[A_ELEMS + B_ELEMS + i] = 0;
    smem[STAGE + A_ELEMS + B_ELEMS + i] = 0;
  }
  lds_barrier();

  // ---- prologue: stage 0 stored, stage 1 in flight
  issue_loads(0);
  store_stage(smem);
  issue_loads(KT > 1 ? 1 : 0);
  lds_barrier();

  auto compute = [&](const uint16_t* st) {
    const uint16_t* As = st;
    const uint16_t* Bs = st + A_ELEMS;
    const uint16_t* Ds = st + A_ELEMS + B_ELEMS;
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      bf16x8 af[MB], bfr[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (S::WM * wm + 32 * i + (lane & 31)) * SA + ks * 16 + 8 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if constexpr (TRANS) {
          const int b = lane >> 4, sl = lane & 15;
          const int col = S::WN * wn + 32 * j + 16 * (b & 1) + 4 * (sl & 3);
          const int row = ks * 16 + 8 * (b >> 1) + (sl >> 2);
          bfr[j] = tr16x8(Bs + row * S::SBT + col, Bs + (row + 4) * S::SBT + col);
        } else {
          bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + (S::WN * wn + 32 * j + (lane & 31)) * SA + ks * 16 + 8 * (lane >> 5));
        }
      }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    // rank-r down projection on this wave's 32 rows
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
      for (int i = 0; i < 2; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(As + (32 * wave + 16 * i + (lane & 15)) * SA + 32 * kp + 8 * (lane >> 4));
#pragma unroll
        for (int jb = 0; jb < RB; ++jb)
          uacc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bd[jb], uacc[i][jb], 0, 0, 0);
      }
    }
  };

  // ---- steady state: store stage kt+1 (loaded one step earlier), reissue the
  // loads of stage kt+2 at once, then the MFMAs of stage kt
  for (int kt = 0; kt + 1 < KT; ++kt) {
    const int cur = kt & 1;
    store_stage(smem + (cur ^ 1) * STAGE);
    issue_loads(kt + 2 < KT ? kt + 2 : KT - 1);
    compute(smem + cur * STAGE);
    lds_barrier();
  }
  compute(smem + ((KT - 1) & 1) * STAGE);
  lds_barrier();

  // ---------------------------------------------------------------- epilogue
  // Ax [TM][2R+8]: high and low bf16 parts of s.U; Bx [TN][2R+8]: the up matrix twice.
  constexpr int SX = 2 * R + 8;
  uint16_t* Ax = smem;
  uint16_t* Bx = smem + TM * SX;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jb = 0; jb < RB; ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 32 * wave + 16 * i + 4 * (lane >> 4) + e;
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
  for (int idx = tid; idx < TN * R; idx += NTHREADS) {
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

template <int FMT, bool TRANS, int R, int TN>
hipError_t launch_t(const Params& p, hipStream_t s) {
  using S = Shape<TN>;
  constexpr int B_ELEMS = TRANS ? S::BT_ELEMS : S::BF_ELEMS;
  constexpr int D_ELEMS = TRANS ? BL_ELEMS : AD_ELEMS;
  constexpr size_t smem = 2 * (size_t)(A_ELEMS + B_ELEMS + D_ELEMS) * sizeof(uint16_t);
  static_assert(smem <= 160 * 1024, "LDS budget");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)qgemm_kernel<FMT, TRANS, R, TN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t tiles = ((p.O + TN - 1) / TN) * ((p.M + TM - 1) / TM);
  hipLaunchKernelGGL((qgemm_kernel<FMT, TRANS, R, TN>), dim3((unsigned)tiles), dim3(NTHREADS), smem, s, p);
  return hipGetLastError();
}

// Output tile width: 256 when that still gives at least one tile per CU, else 128.
template <int FMT, bool TRANS, int R>
hipError_t launch_w(const Params& p, hipStream_t s) {
  const int64_t tiles256 = ((p.O + 255) / 256) * ((p.M + TM - 1) / TM);
  if (tiles256 >= 256) return launch_t<FMT, TRANS, R, 256>(p, s);
  return launch_t<FMT, TRANS, R, 128>(p, s);
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
