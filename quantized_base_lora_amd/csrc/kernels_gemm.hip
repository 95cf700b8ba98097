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
// the same contraction loop on 16x16x32 MFMAs (for dX its B operand is also
// read through transpose loads); the "up" product is one more short MFMA
// contraction over 2r bf16 columns (s.U split into a high and a low bf16
// term, so the epilogue keeps ~16 bits of U) before the single bf16 rounding
// of the output.  The base is never written.
//
// Dequantized tile values are bf16_RNE(fl32 value): Q4_0 (q - 8) * d is exact
// in fp32; NF4 uses a per-thread 16-entry table of bf16_RNE(fl32(c[q] * a))
// looked up with byte permutes; FP8 decodes with the hardware E4M3 convert
// and multiplies by the tensor scale.
//
// Tiling (gfx950, wave64, one 256-thread workgroup per CU): the workgroup
// owns a 256 x TN output tile (TN = 256, or 128 for narrow outputs), each of
// its four waves 128 x TN/2 as 32x32x16 MFMA blocks.  The contraction moves
// 64 at a time through double-buffered LDS: while the MFMAs consume stage
// t, the same waves store stage t+1 (activation copy, dequantization) and
// have the global loads of stage t+2 in flight.  The loop body is free of
// branches (clamped addresses, select-to-zero) so the compiler can
// interleave the VALU dequantization with the MFMAs.  Operands are swapped
// in the MFMA (B first), so each lane ends up with 4 consecutive output
// columns per row and writes them with one 8-byte store.  Workgroups are
// remapped so each XCD (own L2) works on a contiguous run of tiles.
#include "common.h"

namespace ql {
namespace {

constexpr int TM = 256, TK = 64;
constexpr int NTHREADS = 256;
constexpr int SA = TK + 8;          // act tile row stride (bf16): 144 B, conflict-free b128 reads
constexpr int SBF = TK + 8;         // forward W tile [TN][TK] stride
constexpr int SL = 48;              // dX: B-adapter tile [TK][SL] (r <= 32, columns >= r stay 0)
constexpr int A_ELEMS = TM * SA;

template <int TN> struct Shape {
  static constexpr int SBT = TN + 32;                 // dX W tile [TK][TN] stride (576 / 320 B rows)
  static constexpr int BF_ELEMS = TN * SBF;
  static constexpr int BT_ELEMS = TK * SBT;
  static constexpr int BL_ELEMS = TK * SL;
};

struct Book { float c[16]; };

typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

__device__ __forceinline__ uint4 sel4(bool keep, uint4 v) {
  return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}

__device__ __forceinline__ bf16x8 tr16x8(const uint16_t* p0, const uint16_t* p1) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p0);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p1);
  s16x8 t = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, t);
}

// ------------------------------------------------------------------ W group registers
// One 32-element group of one row of W: codes plus its (already decoded) scale.
// An out-of-range group gets scale 0 (its codes come from a clamped, valid
// address), which zeroes every dequantized value without a branch.
struct WGroup {
  uint4 c0, c1;      // 4-bit: c0 = 16 bytes; fp8: c0, c1 = 32 bytes
  float scale;
};

template <int FMT>
__device__ __forceinline__ void load_group(WGroup& g, const uint8_t* __restrict__ codes,
                                           const void* __restrict__ scales, int64_t n, int64_t kg,
                                           int64_t N, int64_t K, float tscale) {
  const bool valid = (n < N) && (kg * 32 < K);
  n = n < N ? n : N - 1;
  kg = kg * 32 < K ? kg : K / 32 - 1;
  if constexpr (FMT == QL_FMT_FP8_E4M3) {
    const uint4* p = reinterpret_cast<const uint4*>(codes + n * K + kg * 32);
    g.c0 = p[0];
    g.c1 = p[1];
    g.scale = valid ? tscale : 0.0f;
  } else {
    g.c0 = *reinterpret_cast<const uint4*>(codes + n * (K / 2) + kg * 16);
    float v;
    if constexpr (FMT == QL_FMT_Q4_0) {
      const uint32_t h = reinterpret_cast<const uint16_t*>(scales)[n * (K / 32) + kg];
      const uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
      v = (e == 0) ? (float)m * 5.9604644775390625e-08f : __uint_as_float(((e + 112u) << 23) | (m << 13));
      v = (h & 0x8000) ? -v : v;
    } else {
      v = reinterpret_cast<const float*>(scales)[n * (K / 64) + (kg >> 1)];
    }
    g.scale = valid ? v : 0.0f;
  }
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

// Dequantize one 32-element group into 16 dwords (bf16 pairs in element order).
template <int FMT>
__device__ __forceinline__ void dequant_group(const WGroup& g, const Book& book, uint32_t* out) {
  if constexpr (FMT == QL_FMT_FP8_E4M3) {
    const uint32_t wd[8] = {g.c0.x, g.c0.y, g.c0.z, g.c0.w, g.c1.x, g.c1.y, g.c1.z, g.c1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], false);
      const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], true);
      out[2 * i] = pack_bf16x2(a.x * g.scale, a.y * g.scale);
      out[2 * i + 1] = pack_bf16x2(b.x * g.scale, b.y * g.scale);
    }
  } else {
    const uint32_t wd[4] = {g.c0.x, g.c0.y, g.c0.z, g.c0.w};
    if constexpr (FMT == QL_FMT_Q4_0) {
      const float d = g.scale, nd8 = -8.0f * g.scale;    // (q - 8) d = fma(q, d, -8d), exact
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
      for (int i = 0; i < 8; ++i) pr[i] = pack_bf16x2(book.c[2 * i] * g.scale, book.c[2 * i + 1] * g.scale);
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
  uint32_t* zero_ptr;    // if set, zeroed by workgroup 0 (counters of a later kernel)
  int32_t zero_n;
  int64_t M, N, K, C, O;
  float s;
  Book book;
};

template <int FMT, bool TRANS, int R, int TN>
__global__ __launch_bounds__(NTHREADS) void qgemm_kernel(Params p) {
  using S = Shape<TN>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  constexpr int B_ELEMS = TRANS ? S::BT_ELEMS : S::BF_ELEMS;
  constexpr int STAGE = A_ELEMS + B_ELEMS + (TRANS ? S::BL_ELEMS : 0);
  constexpr int RB = (R + 15) / 16;                  // 16-column blocks of the rank-r projection
  constexpr int WN = TN / 2;                         // wave tile columns
  constexpr int NB = WN / 32;                        // 32-column MFMA blocks per wave
  constexpr int GPT = TN / 128;                      // W groups per thread per stage
  constexpr int GPR = TRANS ? TN / 32 : TK / 32;     // W groups per W-tile row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile assignment: contiguous runs of tiles per XCD (workgroups go round-robin over 8 XCDs)
  const int nt = (int)((p.O + TN - 1) / TN);
  const int mt = (int)((p.M + TM - 1) / TM);
  const int tiles = nt * mt;
  int t = blockIdx.x;
  if ((tiles & 7) == 0) t = (t & 7) * (tiles >> 3) + (t >> 3);
  const int64_t o0 = (int64_t)(t % nt) * TN;
  const int64_t m0 = (int64_t)(t / nt) * TM;
  const int64_t KT = (p.C + TK - 1) / TK;

  float tscale = 0.0f;
  if constexpr (FMT == QL_FMT_FP8_E4M3) tscale = reinterpret_cast<const float*>(p.scales)[0];
  if (p.zero_ptr && blockIdx.x == 0)
    for (int i = tid; i < p.zero_n; i += NTHREADS) p.zero_ptr[i] = 0u;

  // ---- per-thread load coordinates
  const int arow = tid >> 3, acol = (tid & 7) * 8;   // act: rows arow + 32 i, 8 columns
  int wrow[GPT], wgrp[GPT];
#pragma unroll
  for (int g = 0; g < GPT; ++g) {
    const int task = tid + NTHREADS * g;
    wrow[g] = task / GPR;
    wgrp[g] = task % GPR;
  }
  constexpr int LPT = R / 4;                         // dX: B-adapter elements per thread per stage
  const int lrow = tid >> 2, lcol = (tid & 3) * LPT;

  uint4 areg[8];
  WGroup wreg[GPT];
  uint4 dreg[2][RB];                                 // forward: A fragments; dX: raw B tile piece
  (void)lrow; (void)lcol;

  auto issue_loads = [&](int64_t kt) {
    const int64_t c0 = kt * TK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int64_t row = m0 + 32 * i + arow, col = c0 + acol;
      const bool ok = row < p.M && col < p.C;
      row = row < p.M ? row : p.M - 1;
      col = col < p.C ? col : p.C - 8;
      areg[i] = sel4(ok, *reinterpret_cast<const uint4*>(p.act + row * p.C + col));
    }
#pragma unroll
    for (int g = 0; g < GPT; ++g) {
      if constexpr (TRANS)
        load_group<FMT>(wreg[g], p.codes, p.scales, c0 + wrow[g], (o0 >> 5) + wgrp[g], p.N, p.K, tscale);
      else
        load_group<FMT>(wreg[g], p.codes, p.scales, o0 + wrow[g], (c0 >> 5) + wgrp[g], p.N, p.K, tscale);
    }
    if constexpr (TRANS) {
      // B rows c0 .. c0+63, R columns: LPT consecutive bf16 per thread
      int64_t row = c0 + lrow;
      const bool ok = row < p.C;
      row = row < p.C ? row : p.C - 1;
      const uint16_t* src = p.down + row * R + lcol;
      if constexpr (LPT == 8) dreg[0][0] = sel4(ok, *reinterpret_cast<const uint4*>(src));
      else if constexpr (LPT == 4) { uint2 v = *reinterpret_cast<const uint2*>(src); dreg[0][0] = sel4(ok, make_uint4(v.x, v.y, 0, 0)); }
      else { uint32_t v = *reinterpret_cast<const uint32_t*>(src); dreg[0][0] = sel4(ok, make_uint4(v, 0, 0, 0)); }
    } else {
#pragma unroll
      for (int kp = 0; kp < 2; ++kp)
#pragma unroll
        for (int jb = 0; jb < RB; ++jb) {
          const int j = 16 * jb + (lane & 15);
          int64_t c = c0 + 32 * kp + 8 * (lane >> 4);
          const bool ok = j < R && c < p.C;
          c = c < p.C ? c : p.C - 8;
          const int jj = j < R ? j : R - 1;
          dreg[kp][jb] = sel4(ok, *reinterpret_cast<const uint4*>(p.down + (int64_t)jj * p.C + c));
        }
    }
  };

  auto store_act = [&](uint16_t* As) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(As + (32 * i + arow) * SA + acol) = areg[i];
  };
  auto store_w = [&](uint16_t* Bs, int g) {
    uint32_t v[16];
    dequant_group<FMT>(wreg[g], p.book, v);
    uint16_t* dst = TRANS ? (Bs + wrow[g] * S::SBT + wgrp[g] * 32) : (Bs + wrow[g] * SBF + wgrp[g] * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(dst + 8 * i) = make_uint4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  };
  auto store_down = [&](uint16_t* Bl) {
    if constexpr (TRANS) {
      uint16_t* dst = Bl + lrow * SL + lcol;
      if constexpr (LPT == 8) *reinterpret_cast<uint4*>(dst) = dreg[0][0];
      else if constexpr (LPT == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(dreg[0][0].x, dreg[0][0].y);
      else *reinterpret_cast<uint32_t*>(dst) = dreg[0][0].x;
    }
  };

  f32x16 acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  f32x4 uacc[4][RB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jb = 0; jb < RB; ++jb) uacc[i][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 dcur[2][RB], dnext[2][RB];

  if constexpr (TRANS) {
    // columns R..SL-1 of both B-adapter tiles stay zero
    for (int i = tid; i < TK * SL; i += NTHREADS) {
      smem[A_ELEMS + B_ELEMS + i] = 0;
      smem[STAGE + A_ELEMS + B_ELEMS + i] = 0;
    }
    lds_barrier();
  }

  // ---- prologue: stage 0 stored, stage 1 in flight
  issue_loads(0);
  store_act(smem);
#pragma unroll
  for (int g = 0; g < GPT; ++g) store_w(smem + A_ELEMS, g);
  store_down(smem + A_ELEMS + B_ELEMS);
#pragma unroll
  for (int kp = 0; kp < 2; ++kp)
#pragma unroll
    for (int jb = 0; jb < RB; ++jb) dcur[kp][jb] = dreg[kp][jb];
  issue_loads(KT > 1 ? 1 : 0);
  lds_barrier();

  auto compute = [&](const uint16_t* As, const uint16_t* Bs, const uint16_t* Bl, auto&& side_work) {
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      bf16x8 af[4], bfr[NB];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (128 * wm + 32 * i + (lane & 31)) * SA + ks * 16 + 8 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if constexpr (TRANS) {
          const int b = lane >> 4, sl = lane & 15;
          const int col = WN * wn + 32 * j + 16 * (b & 1) + 4 * (sl & 3);
          const int row = ks * 16 + 8 * (b >> 1) + (sl >> 2);
          bfr[j] = tr16x8(Bs + row * S::SBT + col, Bs + (row + 4) * S::SBT + col);
        } else {
          bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + (WN * wn + 32 * j + (lane & 31)) * SBF + ks * 16 + 8 * (lane >> 5));
        }
      }
      side_work(ks);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    // rank-r down projection on this wave's 64 rows
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      bf16x8 bd[RB];
#pragma unroll
      for (int jb = 0; jb < RB; ++jb) {
        if constexpr (TRANS) {
          const int b = lane >> 4, sl = lane & 15;
          const int row = 32 * kp + 8 * b + (sl >> 2), col = 16 * jb + 4 * (sl & 3);
          bd[jb] = tr16x8(Bl + row * SL + col, Bl + (row + 4) * SL + col);
        } else {
          bd[jb] = __builtin_bit_cast(bf16x8, dcur[kp][jb]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(As + (64 * wave + 16 * i + (lane & 15)) * SA + 32 * kp + 8 * (lane >> 4));
#pragma unroll
        for (int jb = 0; jb < RB; ++jb)
          uacc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bd[jb], uacc[i][jb], 0, 0, 0);
      }
    }
  };

  // ---- steady state: compute stage kt; at its start, store stage kt+1 from the
  // registers (loaded one iteration earlier) and at once reissue the loads of
  // stage kt+2 into them, so the loads have a whole iteration of MFMAs to land
  for (int64_t kt = 0; kt + 1 < KT; ++kt) {
    const int cur = (int)(kt & 1);
    const uint16_t* As = smem + cur * STAGE;
    uint16_t* An = smem + (cur ^ 1) * STAGE;
    compute(As, As + A_ELEMS, As + A_ELEMS + B_ELEMS, [&](int ks) {
      if (ks == 0) {
        store_act(An);
#pragma unroll
        for (int g = 0; g < GPT; ++g) store_w(An + A_ELEMS, g);
        store_down(An + A_ELEMS + B_ELEMS);
        // forward: the A fragments of stage kt+1 stay in registers (dcur) until its compute
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
#pragma unroll
          for (int jb = 0; jb < RB; ++jb) dnext[kp][jb] = dreg[kp][jb];
        issue_loads(kt + 2 < KT ? kt + 2 : KT - 1);
      }
    });
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int jb = 0; jb < RB; ++jb) dcur[kp][jb] = dnext[kp][jb];
    lds_barrier();
  }
  {
    const uint16_t* As = smem + (int)((KT - 1) & 1) * STAGE;
    compute(As, As + A_ELEMS, As + A_ELEMS + B_ELEMS, [](int) {});
  }
  lds_barrier();

  // ---------------------------------------------------------------- epilogue
  // Ax [TM][2R+8]: high and low bf16 parts of s.U; Bx [TN][2R+8]: the up matrix twice.
  constexpr int SX = 2 * R + 8;
  uint16_t* Ax = smem;
  uint16_t* Bx = smem + TM * SX;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jb = 0; jb < RB; ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 64 * wave + 16 * i + 4 * (lane >> 4) + e;
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
    bf16x8 af[4], bfr[NB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(Ax + (128 * wm + 32 * i + (lane & 31)) * SX + ks * 16 + 8 * (lane >> 5));
#pragma unroll
    for (int j = 0; j < NB; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(Bx + (WN * wn + 32 * j + (lane & 31)) * SX + ks * 16 + 8 * (lane >> 5));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
  }
  // ---- store bf16: lane holds row (lane & 31) and, per 4 accumulators, 4 consecutive columns
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + 128 * wm + 32 * i + (lane & 31);
    if (row < p.M) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const int64_t col = o0 + WN * wn + 32 * j + 8 * k4 + 4 * (lane >> 5);
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
  constexpr size_t smem = 2 * (size_t)(A_ELEMS + B_ELEMS + (TRANS ? S::BL_ELEMS : 0)) * sizeof(uint16_t);
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
  p.zero_ptr = c.zero_ptr;
  p.zero_n = c.zero_n;
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
