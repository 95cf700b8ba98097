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
#include <algorithm>

#include "common.h"
#include "device.h"

namespace ql {
namespace {

constexpr int TK = 64;
constexpr int SA = TK + 8;          // act / forward-W tile row stride (bf16): 144 B
constexpr int SL = 48;              // dX: B-adapter tile [TK][SL] (r <= 32; columns >= r stay 0)
constexpr int AD_ELEMS = 32 * SA;   // forward: A-adapter tile [32][SA] (rows >= r stay 0)
constexpr int BL_ELEMS = TK * SL;

// TM = 256 (the large-M tiles): NTH = 256 gives four waves, one per SIMD,
// each owning a 128 x TN/2 block; NTH = 512 gives eight waves, two per SIMD,
// each owning a 128 x 64 (TN = 256) or 64 x 64 (TN = 128) block.
// TM = 64 (the split-contraction path for at most 64 tokens): four waves side
// by side along the output columns, 64 x TN/4 each.
template <int TM_, int TN, int NTH> struct Shape {
  static constexpr int TM = TM_;
  static constexpr int NW = NTH / 64;
  static constexpr int A_ELEMS = TM * SA;
  static constexpr int SBT = TN + 32;                 // dX W tile [TK][TN] stride (576 / 320 B rows)
  static constexpr int BF_ELEMS = TN * SA;
  static constexpr int BT_ELEMS = TK * SBT;
  static constexpr int WAVES_N = TM == 64 ? NW : ((NW == 8 && TN == 256) ? 4 : 2);   // TN = 192: 64 x 96 blocks
  static constexpr int WAVES_M = NW / WAVES_N;
  static constexpr int WM = TM / WAVES_M, WN = TN / WAVES_N;
  static constexpr int MB = WM / 32, NB = WN / 32;    // 32x32 MFMA blocks per wave
  static constexpr int WGT = TN * TK / 32;            // W groups per stage
  static constexpr int WG = WGT >= NTH ? WGT / NTH : 1;   // W groups per thread
  static constexpr bool WPART = WGT < NTH;            // only threads below WGT carry one
  static constexpr int AR = TM * TK / 8 / NTH;        // 16-byte activation pieces per thread
  static constexpr int ARS = NTH / 8;                 // rows between a thread's pieces
  static constexpr int UI = TM / NW / 16;             // 16-row blocks of the rank-r projection per wave
  static_assert(MB >= 1 && NB >= 1 && AR >= 1 && UI >= 1, "tile shape");
};

struct Book { float c[16]; };

// ------------------------------------------------------------------ dequantization
// One 32-element group of one row of W: codes plus its raw scale word.
// Loads only fill these registers: every use of a loaded value (scale
// extraction, masking) happens where the group is dequantized, so that no
// instruction right after a load has to wait for it.
struct WGroup {
  uint4 c0, c1;      // 4-bit: c0 = 16 bytes; fp8: c0, c1 = 32 bytes
  uint32_t sraw;     // Q4_0: the dword holding the fp16 scale; NF4: fp32 bits; FP8: unused
  uint32_t ssh;      // Q4_0: bit offset of the fp16 scale in sraw (0 or 16)
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
  // split-contraction path: split blockIdx.y covers steps [sps * y, sps * (y + 1)) and
  // writes fp32 partial sums instead of the output
  float* part;           // [splits, M, O]
  float* upart;          // [splits, M, R]
  int sps;
};

template <int FMT, bool TRANS, int R, int TM_, int TN, int NTH, bool PART>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(TM_ == 64 ? 2 : NTH / 256, TM_ == 64 ? 2 : NTH / 256)))
void qgemm_kernel(Params p) {
  using S = Shape<TM_, TN, NTH>;
  constexpr int NT = NTH;
  constexpr int TM = S::TM;
  constexpr int A_ELEMS = S::A_ELEMS;
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
  // contraction steps of this workgroup: [kbeg, kend), NKT of them (at least one)
  const int kbeg = PART ? (int)blockIdx.y * p.sps : 0;
  const int kend = PART ? min(KT, kbeg + p.sps) : KT;
  const int NKT = kend - kbeg;

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
    wreg[j].c0 = wreg[j].c1 = make_uint4(0, 0, 0, 0);
    wreg[j].sraw = wreg[j].ssh = 0;
  }
  uint4 dreg = make_uint4(0, 0, 0, 0);

  // ---- global loads of stage kt, piece by piece (registers are reloaded as soon as stored)
  auto load_act = [&](int kt, int i) {
    const int64_t c0 = (int64_t)kt * TK;
    const uint32_t off = (uint32_t)(((arow + ARS * i) * p.C + c0 + acol) * 2);
    areg[i] = bload16(ract, c0 + acol < p.C ? off : OOB);
  };
  auto load_w = [&](int kt, int j) {
    const int64_t c0 = (int64_t)kt * TK;
    // forward: row o0 + wr, K columns c0 + 32 wg; dX: row c0 + wr, K columns o0 + 32 wg
    const int64_t wrow = TRANS ? c0 + wr[j] : wr[j];
    const int64_t kgrp = TRANS ? wg[j] : (c0 >> 5) + wg[j];   // group index relative to the tile base
    // forward: a group past the end of the contraction reads as zero
    const bool live = TRANS || c0 + 32 * wg[j] < p.C;
    const uint32_t coff = live ? (uint32_t)(wrow * crow + kgrp * (FP8 ? 32 : 16)) : OOB;
    if (!wtask) return;
    wreg[j].c0 = bload16(rcode, coff);
    if constexpr (FP8) {
      wreg[j].c1 = bload16(rcode, live ? coff + 16 : OOB);
    } else {
      const int64_t kabs = TRANS ? (o0 >> 5) + wg[j] : kgrp;   // group index along K
      if constexpr (FMT == QL_FMT_Q4_0) {
        const int64_t idx = wrow * srow + kabs;
        wreg[j].sraw = bload4(rscale, live ? (uint32_t)((idx * 2) & ~3LL) : OOB);
        wreg[j].ssh = (uint32_t)(idx & 1) * 16;
      } else {
        wreg[j].sraw = bload4(rscale, live ? (uint32_t)((wrow * srow + (kabs >> 1)) * 4) : OOB);
      }
    }
  };
  auto load_adapter = [&](int kt) {
    const int64_t c0 = (int64_t)kt * TK;
    uint32_t off;
    if constexpr (TRANS) off = (uint32_t)(((c0 + drow) * R + dcol) * 2);
    else off = c0 + dcol < p.C ? (uint32_t)((drow * p.C + c0 + dcol) * 2) : OOB;
    dreg = bload16(rdown, dload ? off : OOB);
  };

  // ---- stage stores
  Deq<FMT> deq;
  auto store_act = [&](uint16_t* st, int i) {
    *reinterpret_cast<uint4*>(st + (arow + ARS * i) * SA + acol) = areg[i];
  };
  auto prepare_w = [&](int j) {
    float scale;
    if constexpr (FP8) scale = tscale;
    else if constexpr (FMT == QL_FMT_Q4_0) scale = decode_scale_q40(wreg[j].sraw >> wreg[j].ssh);
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
  for (int i = 0; i < AR; ++i) load_act(kbeg, i);
#pragma unroll
  for (int j = 0; j < WG; ++j) load_w(kbeg, j);
  load_adapter(kbeg);
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
    const int k1 = NKT > 1 ? kbeg + 1 : kbeg;
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
  for (int it = 0; it + 1 < NKT; ++it) {
    const uint16_t* cs = smem + (it & 1) * STAGE;
    uint16_t* ns = smem + ((it & 1) ^ 1) * STAGE;
    const int kl = it + 2 < NKT ? kbeg + it + 2 : kend - 1;
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
    const uint16_t* cs = smem + ((NKT - 1) & 1) * STAGE;
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

  if constexpr (PART) {
    // fp32 partial sums of this split (each lane: one row, 4 consecutive columns per block),
    // and the partial rank-r projection from the tiles of output column 0
    float* pp = p.part + (int64_t)blockIdx.y * p.M * p.O;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int64_t row = m0 + S::WM * wm + 32 * i + (lane & 31);
      if (row < p.M) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) {
            const int64_t col = o0 + S::WN * wn + 32 * j + 8 * k4 + 4 * (lane >> 5);
            if (col < p.O)
              *reinterpret_cast<float4*>(pp + row * p.O + col) =
                  make_float4(acc[i][j][4 * k4], acc[i][j][4 * k4 + 1], acc[i][j][4 * k4 + 2], acc[i][j][4 * k4 + 3]);
          }
      }
    }
    if (o0 == 0) {
      float* up = p.upart + (int64_t)blockIdx.y * p.M * R;
#pragma unroll
      for (int i = 0; i < UI; ++i)
#pragma unroll
        for (int jb = 0; jb < RB; ++jb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = 16 * UI * wave + 16 * i + 4 * (lane >> 4) + e;
            const int j = 16 * jb + (lane & 15);
            if (j < R && m0 + row < p.M) up[(m0 + row) * R + j] = uacc[i][jb][e];
          }
    }
    return;
  }

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

template <int FMT, bool TRANS, int R, int TM, int TN, int NTH, bool PART>
hipError_t launch_t(const Params& p, int splits, hipStream_t s) {
  using S = Shape<TM, TN, NTH>;
  constexpr int B_ELEMS = TRANS ? S::BT_ELEMS : S::BF_ELEMS;
  constexpr int D_ELEMS = TRANS ? BL_ELEMS : AD_ELEMS;
  constexpr size_t smem = 2 * (size_t)(S::A_ELEMS + B_ELEMS + D_ELEMS) * sizeof(uint16_t);
  static_assert(smem <= 160 * 1024, "LDS budget");
  static_assert(PART || (size_t)(TM + TN) * (2 * R + 8) * sizeof(uint16_t) <= smem, "epilogue LDS");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)qgemm_kernel<FMT, TRANS, R, TM, TN, NTH, PART>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t tiles = ((p.O + TN - 1) / TN) * ((p.M + TM - 1) / TM);
  hipLaunchKernelGGL((qgemm_kernel<FMT, TRANS, R, TM, TN, NTH, PART>), dim3((unsigned)tiles, (unsigned)splits),
                     dim3(NTH), smem, s, p);
  return hipGetLastError();
}

// ------------------------------------------------------------------ small-M path
// At most 64 tokens the base GEMM is bound by streaming W, and each
// workgroup sees only a few contraction steps, so every step's loads must be
// in flight long before they are needed: a ring of D register stages keeps
// the loads of steps it+1 .. it+D outstanding while step it computes.  Tile:
// 64 rows (all tokens) x 128 output columns, four waves side by side (64 x 32
// each), the contraction split over blockIdx.y; fp32 partial sums out.
template <int FMT, bool TRANS, int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qsplit_kernel(Params p) {
  constexpr int TM = 64, TN = 128, NT = 256, D = 4;
  static_assert(D % 2 == 0, "buffer parity of a step is its position in the chunk");
  constexpr int SBT = TN + 32;
  constexpr int A_EL = TM * SA;
  constexpr int B_EL = TRANS ? TK * SBT : TN * SA;
  constexpr int D_EL = TRANS ? BL_ELEMS : AD_ELEMS;
  constexpr int STAGE = A_EL + B_EL + D_EL;
  constexpr int RB = (R + 15) / 16;
  constexpr int GPR = TRANS ? TN / 32 : TK / 32;
  constexpr bool FP8 = FMT == QL_FMT_FP8_E4M3;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // units (column tile, split) are handed to the 8 XCDs (round robin over the
  // linear workgroup id) in contiguous runs, so adjacent column tiles of one
  // split share their XCD's L2: a dX step reads 64 of the 128 bytes of each
  // W-row line, and the neighbouring tile reads the other half
  const int nunits = (int)(gridDim.x * gridDim.y);
  int unit = (int)(blockIdx.y * gridDim.x + blockIdx.x);
  if ((nunits & 7) == 0) unit = (unit & 7) * (nunits >> 3) + (unit >> 3);
  const int ntile = unit % (int)gridDim.x, split = unit / (int)gridDim.x;
  const int64_t o0 = (int64_t)ntile * TN;
  const int KT = (int)((p.C + TK - 1) / TK);
  const int kbeg = split * p.sps;
  const int kend = min(KT, kbeg + p.sps);
  const int NKT = kend - kbeg;

  const __amdgpu_buffer_rsrc_t ract = rsrc(p.act, p.M * p.C * 2);
  const int64_t crow = FP8 ? p.K : p.K / 2;
  const int64_t wrow0 = TRANS ? 0 : o0;
  const int64_t wcol0 = TRANS ? (FP8 ? o0 : o0 / 2) : 0;
  const __amdgpu_buffer_rsrc_t rcode = rsrc(p.codes + wrow0 * crow + wcol0, (p.N - wrow0) * crow - wcol0);
  const int64_t srow = FMT == QL_FMT_Q4_0 ? p.K / 32 : p.K / 64;
  const int64_t ssz = FMT == QL_FMT_Q4_0 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rscale =
      rsrc((const char*)p.scales + wrow0 * srow * ssz, (p.N - wrow0) * srow * ssz);
  const __amdgpu_buffer_rsrc_t rdown = rsrc(p.down, (int64_t)R * p.C * 2);
  float tscale = 0.0f;
  if constexpr (FP8) tscale = reinterpret_cast<const float*>(p.scales)[0];

  const int arow = tid >> 3, acol = (tid & 7) * 8;   // act rows arow, arow + 32
  const int wr = tid / GPR, wg = tid % GPR;          // one W group per thread per step
  const bool wg_in = !TRANS || (o0 + 32 * (wg + 1) <= p.K);
  constexpr int DPR = TRANS ? R / 8 : TK / 8;
  const bool dload = tid < 8 * R;
  const int drow = tid / DPR, dcol = (tid % DPR) * 8;

  struct Slot {
    uint4 a0, a1, d;
    WGroup w;
  };
  Slot ring[D];
  // loads of step kt; a step past the split's end reads zeros (no memory traffic)
  auto issue = [&](Slot& sl, int kt) {
    const bool sv = kt < kend;
    const int64_t c0 = (int64_t)kt * TK;
    const bool alive = sv && c0 + acol < p.C;
    sl.a0 = bload16(ract, alive ? (uint32_t)((arow * p.C + c0 + acol) * 2) : OOB);
    sl.a1 = bload16(ract, alive ? (uint32_t)(((arow + 32) * p.C + c0 + acol) * 2) : OOB);
    const int64_t wrow = TRANS ? c0 + wr : wr;
    const int64_t kgrp = TRANS ? wg : (c0 >> 5) + wg;
    const bool wlive = sv && (TRANS || c0 + 32 * wg < p.C);
    const uint32_t coff = wlive ? (uint32_t)(wrow * crow + kgrp * (FP8 ? 32 : 16)) : OOB;
    sl.w.c0 = bload16(rcode, coff);
    sl.w.ssh = 0;
    if constexpr (FP8) {
      sl.w.c1 = bload16(rcode, wlive ? coff + 16 : OOB);
      sl.w.sraw = 0;
    } else {
      sl.w.c1 = make_uint4(0, 0, 0, 0);
      const int64_t kabs = TRANS ? (o0 >> 5) + wg : kgrp;
      if constexpr (FMT == QL_FMT_Q4_0) {
        const int64_t idx = wrow * srow + kabs;
        sl.w.sraw = bload4(rscale, wlive ? (uint32_t)((idx * 2) & ~3LL) : OOB);
        sl.w.ssh = (uint32_t)(idx & 1) * 16;
      } else {
        sl.w.sraw = bload4(rscale, wlive ? (uint32_t)((wrow * srow + (kabs >> 1)) * 4) : OOB);
      }
    }
    uint32_t doff;
    if constexpr (TRANS) doff = (uint32_t)(((c0 + drow) * R + dcol) * 2);
    else doff = c0 + dcol < p.C ? (uint32_t)((drow * p.C + c0 + dcol) * 2) : OOB;
    sl.d = bload16(rdown, dload && sv ? doff : OOB);
  };
  auto store = [&](const Slot& sl, uint16_t* st) {
    *reinterpret_cast<uint4*>(st + arow * SA + acol) = sl.a0;
    *reinterpret_cast<uint4*>(st + (arow + 32) * SA + acol) = sl.a1;
    float scale;
    if constexpr (FP8) scale = tscale;
    else if constexpr (FMT == QL_FMT_Q4_0) scale = decode_scale_q40(sl.w.sraw >> sl.w.ssh);
    else scale = __uint_as_float(sl.w.sraw);
    Deq<FMT> dq;
    dq.prepare(sl.w, wg_in ? scale : 0.0f, p.book);
    uint16_t* dst = st + A_EL + (TRANS ? wr * SBT : wr * SA) + wg * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(dst + 8 * i) = dq.piece(i);
    if (dload) *reinterpret_cast<uint4*>(st + A_EL + B_EL + drow * (TRANS ? SL : SA) + dcol) = sl.d;
  };
  // every slot starts defined (the prologue may leave some unused)
#pragma unroll
  for (int u = 0; u < D; ++u) {
    ring[u].a0 = ring[u].a1 = ring[u].d = ring[u].w.c0 = ring[u].w.c1 = make_uint4(0, 0, 0, 0);
    ring[u].w.sraw = ring[u].w.ssh = 0;
  }

  f32x16 acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
  f32x4 uacc[RB];
#pragma unroll
  for (int jb = 0; jb < RB; ++jb) uacc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint16_t* st) {
    const uint16_t* As = st;
    const uint16_t* Bs = st + A_EL;
    const uint16_t* Ds = st + A_EL + B_EL;
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      bf16x8 af[2], bf;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (32 * i + (lane & 31)) * SA + ks * 16 + 8 * (lane >> 5));
      if constexpr (TRANS) {
        const int b = lane >> 4, sl = lane & 15;
        const int col = 32 * wave + 16 * (b & 1) + 4 * (sl & 3);
        const int row = ks * 16 + 8 * (b >> 1) + (sl >> 2);
        bf = tr16x8(Bs + row * SBT + col, Bs + (row + 4) * SBT + col);
      } else {
        bf = *reinterpret_cast<const bf16x8*>(Bs + (32 * wave + (lane & 31)) * SA + ks * 16 + 8 * (lane >> 5));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af[i], acc[i], 0, 0, 0);
    }
    // rank-r projection of rows 16 wave .. 16 wave + 15 over this stage
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(As + (16 * wave + (lane & 15)) * SA + 32 * kp + 8 * (lane >> 4));
#pragma unroll
      for (int jb = 0; jb < RB; ++jb) {
        bf16x8 bd;
        if constexpr (TRANS) {
          const int b = lane >> 4, sl = lane & 15;
          const int row = 32 * kp + 8 * b + (sl >> 2), col = 16 * jb + 4 * (sl & 3);
          bd = tr16x8(Ds + row * SL + col, Ds + (row + 4) * SL + col);
        } else {
          bd = *reinterpret_cast<const bf16x8*>(Ds + (16 * jb + (lane & 15)) * SA + 32 * kp + 8 * (lane >> 4));
        }
        uacc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bd, uacc[jb], 0, 0, 0);
      }
    }
  };

  for (int i = tid; i < D_EL; i += NT) {
    smem[A_EL + B_EL + i] = 0;
    smem[STAGE + A_EL + B_EL + i] = 0;
  }
  // prologue: D stages in flight, the first stored and its slot refilled
#pragma unroll
  for (int u = 0; u < D; ++u) issue(ring[u], kbeg + u);
  lds_barrier();
  store(ring[0], smem);
  issue(ring[0], kbeg + D);
  lds_barrier();

  // step it: store stage it+1 from its ring slot and refill the slot with
  // stage it+1+D, then compute stage it.  Whole chunks of D steps run
  // branch-free (slot indices and buffer parities static, D even), so the
  // waits for each slot count only the loads issued after it.
  int it = 0;
  for (; it + D < NKT; it += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      store(ring[(u + 1) % D], smem + ((u + 1) & 1) * STAGE);
      issue(ring[(u + 1) % D], kbeg + it + u + 1 + D);
      compute(smem + (u & 1) * STAGE);
      lds_barrier();
    }
  }
  // the last (at most D) steps: everything they need is already in flight
#pragma unroll
  for (int u = 0; u < D; ++u) {
    if (it + u < NKT) {
      if (it + u + 1 < NKT) store(ring[(u + 1) % D], smem + ((u + 1) & 1) * STAGE);
      compute(smem + (u & 1) * STAGE);
      lds_barrier();
    }
  }

  // fp32 partials: lane holds row (lane & 31) of block i and 4 consecutive columns per 8
  float* pp = p.part + (int64_t)split * p.M * p.O;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t row = 32 * i + (lane & 31);
    if (row < p.M) {
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int64_t col = o0 + 32 * wave + 8 * k4 + 4 * (lane >> 5);
        if (col < p.O)
          *reinterpret_cast<float4*>(pp + row * p.O + col) =
              make_float4(acc[i][4 * k4], acc[i][4 * k4 + 1], acc[i][4 * k4 + 2], acc[i][4 * k4 + 3]);
      }
    }
  }
  if (ntile == 0) {
    float* up = p.upart + (int64_t)split * p.M * R;
#pragma unroll
    for (int jb = 0; jb < RB; ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * wave + 4 * (lane >> 4) + e;
        const int j = 16 * jb + (lane & 15);
        if (j < R && row < p.M) up[row * R + j] = uacc[jb][e];
      }
  }
}

template <int FMT, bool TRANS, int R>
hipError_t launch_split(const Params& p, int splits, hipStream_t s) {
  constexpr int B_EL = TRANS ? TK * (128 + 32) : 128 * SA;
  constexpr int D_EL = TRANS ? BL_ELEMS : AD_ELEMS;
  constexpr size_t smem = 2 * (size_t)(64 * SA + B_EL + D_EL) * sizeof(uint16_t);
  static_assert(smem <= 80 * 1024, "two workgroups per CU");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)qsplit_kernel<FMT, TRANS, R>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((qsplit_kernel<FMT, TRANS, R>), dim3((unsigned)((p.O + 127) / 128), (unsigned)splits),
                     dim3(256), smem, s, p);
  return hipGetLastError();
}

constexpr int MAX_SPLITS = 16;

// Split-contraction reduction and epilogue: per output element the partials
// are summed in split order (deterministic), the LoRA term s . U . up^T is
// added in fp32 (U = sum of its partials), and the sum is rounded once to
// bf16.  Column-slab 0 also writes U (forward) or V (dX).  One thread per 4
// consecutive outputs of one row.
template <int R>
__global__ __launch_bounds__(128) void split_reduce_kernel(const float* __restrict__ part,
                                                           const float* __restrict__ upart, int splits,
                                                           int64_t M, int64_t O, const uint16_t* __restrict__ up,
                                                           bool trans, float s, uint16_t* __restrict__ out,
                                                           float* __restrict__ save) {
  __shared__ float us[R];
  const int64_t m = blockIdx.y;
  const int tid = threadIdx.x;
  // splits past the last read as zero through the resource bounds
  const __amdgpu_buffer_rsrc_t rp = rsrc(part, (int64_t)splits * M * O * 4);
  const __amdgpu_buffer_rsrc_t ru = rsrc(upart, (int64_t)splits * M * R * 4);
  if (tid < R) {
    uint32_t v[MAX_SPLITS];
#pragma unroll
    for (int sp = 0; sp < MAX_SPLITS; ++sp) v[sp] = bload4(ru, (uint32_t)((((int64_t)sp * M + m) * R + tid) * 4));
    float u = 0.0f;
#pragma unroll
    for (int sp = 0; sp < MAX_SPLITS; ++sp) u += __uint_as_float(v[sp]);
    if (save && blockIdx.x == 0) save[m * R + tid] = u;
    us[tid] = s * u;
  }
  const int64_t o = (int64_t)blockIdx.x * 512 + tid * 4;
  const bool live = o < O;
  // the up-matrix entries of these 4 outputs, as bf16 pairs
  uint32_t w[4][R / 2];
  if (live) {
    if (!trans) {   // B [O, R]: 4 rows of R
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int q = 0; q < R / 8; ++q) {
          const uint4 v = *reinterpret_cast<const uint4*>(up + (o + c) * R + 8 * q);
          w[c][4 * q] = v.x; w[c][4 * q + 1] = v.y; w[c][4 * q + 2] = v.z; w[c][4 * q + 3] = v.w;
        }
    } else {        // A [R, O]: 4 consecutive entries of each row j
#pragma unroll
      for (int j = 0; j < R; j += 2) {
        const uint2 v0 = *reinterpret_cast<const uint2*>(up + (int64_t)j * O + o);
        const uint2 v1 = *reinterpret_cast<const uint2*>(up + (int64_t)(j + 1) * O + o);
        w[0][j / 2] = (v0.x & 0xFFFF) | (v1.x << 16);
        w[1][j / 2] = (v0.x >> 16) | (v1.x & 0xFFFF0000u);
        w[2][j / 2] = (v0.y & 0xFFFF) | (v1.y << 16);
        w[3][j / 2] = (v0.y >> 16) | (v1.y & 0xFFFF0000u);
      }
    }
  }
  // all partial loads in flight at once, then summed in split order
  uint4 pv[MAX_SPLITS];
#pragma unroll
  for (int sp = 0; sp < MAX_SPLITS; ++sp)
    pv[sp] = bload16(rp, live ? (uint32_t)((((int64_t)sp * M + m) * O + o) * 4) : OOB);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int sp = 0; sp < MAX_SPLITS; ++sp) {
    acc.x += __uint_as_float(pv[sp].x); acc.y += __uint_as_float(pv[sp].y);
    acc.z += __uint_as_float(pv[sp].z); acc.w += __uint_as_float(pv[sp].w);
  }
  __syncthreads();
  if (!live) return;
  float l[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int q = 0; q < R / 2; ++q) {
      l[c] += us[2 * q] * __uint_as_float(w[c][q] << 16);
      l[c] += us[2 * q + 1] * __uint_as_float(w[c][q] & 0xFFFF0000u);
    }
  const uint32_t lo = pack_bf16x2(acc.x + l[0], acc.y + l[1]);
  const uint32_t hi = pack_bf16x2(acc.z + l[2], acc.w + l[3]);
  *reinterpret_cast<uint2*>(out + m * O + o) = make_uint2(lo, hi);
}

// At most SMALL_M tokens: 64-row tiles, 128 columns wide, the contraction split
// over blockIdx.y so that up to 512 workgroups (two per CU, one round) stream
// W with at least 4 steps each, then the reduction kernel.  Otherwise 256-row tiles, 256 columns wide when that
// still gives at least one tile per CU, else 128.
constexpr int64_t SMALL_M = 64;
constexpr int STN = 128;
static_assert(MAX_SPLITS == 16, "split_reduce_kernel unrolls over 16 splits");

struct SplitPlan {
  int splits = 0, sps = 0;
  size_t upart_off = 0, total = 0;
};

SplitPlan split_plan(bool trans, int64_t m, int64_t n, int64_t k, int r) {
  SplitPlan pl;
  if (m <= 0 || m > SMALL_M) return pl;
  const int64_t O = trans ? k : n, C = trans ? n : k;
  const int64_t KT = (C + TK - 1) / TK;
  const int64_t tn = (O + STN - 1) / STN;
  int64_t sp = std::min<int64_t>({std::max<int64_t>(1, KT / 4), 512 / tn, (int64_t)MAX_SPLITS});
  if (sp < 1) sp = 1;
  pl.sps = (int)((KT + sp - 1) / sp);
  pl.splits = (int)((KT + pl.sps - 1) / pl.sps);
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  pl.upart_off = al((size_t)pl.splits * m * O * 4);
  pl.total = pl.upart_off + al((size_t)pl.splits * m * r * 4);
  return pl;
}

// Output tile width for 256-row tiles: the one with the least time in rounds
// of 256 workgroups (one per CU) times work per tile, the narrower tiles
// weighted for their lower MFMA efficiency (more LDS traffic per MFMA);
// ties go to the wider tile.
int pick_tn(int64_t m, int64_t o) {
  const int64_t mt = (m + 255) / 256;
  const int tns[3] = {256, 192, 128};
  const double eff[3] = {1.0, 0.95, 0.85};
  int best = 256;
  double best_cost = 1e300;
  for (int i = 0; i < 3; ++i) {
    const int64_t tiles = mt * ((o + tns[i] - 1) / tns[i]);
    const double cost = (double)((tiles + 255) / 256) * tns[i] / eff[i];
    if (cost < best_cost * (1 - 1e-9)) {
      best_cost = cost;
      best = tns[i];
    }
  }
  return best;
}

template <int FMT, bool TRANS, int R>
hipError_t launch_w(const Params& p, int splits, hipStream_t s) {
  if (splits > 0) {
    hipError_t e = launch_split<FMT, TRANS, R>(p, splits, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(split_reduce_kernel<R>, dim3((unsigned)((p.O + 511) / 512), (unsigned)p.M), dim3(128), 0, s,
                       (const float*)p.part, (const float*)p.upart, splits, p.M, p.O, p.up, TRANS, p.s, p.out,
                       p.save);
    return hipGetLastError();
  }
#ifndef QL_GEMM_THREADS
#define QL_GEMM_THREADS 512
#endif
  switch (pick_tn(p.M, p.O)) {
    case 256: return launch_t<FMT, TRANS, R, 256, 256, QL_GEMM_THREADS, false>(p, 1, s);
    case 192: return launch_t<FMT, TRANS, R, 256, 192, QL_GEMM_THREADS, false>(p, 1, s);
    default: return launch_t<FMT, TRANS, R, 256, 128, QL_GEMM_THREADS, false>(p, 1, s);
  }
}

template <int FMT, bool TRANS>
hipError_t launch_r(const Params& p, int r, int splits, hipStream_t s) {
  switch (r) {
    case 8: return launch_w<FMT, TRANS, 8>(p, splits, s);
    case 16: return launch_w<FMT, TRANS, 16>(p, splits, s);
    default: return launch_w<FMT, TRANS, 32>(p, splits, s);
  }
}

template <int FMT>
hipError_t launch_f(const Params& p, bool trans, int r, int splits, hipStream_t s) {
  return trans ? launch_r<FMT, true>(p, r, splits, s) : launch_r<FMT, false>(p, r, splits, s);
}

}  // namespace

// FP8 base, more than SMALL_M tokens: hi [M, C] | lo [M, C] | row scales [M]
struct Fp8Plan {
  size_t lo_off = 0, rs_off = 0, total = 0;
};
Fp8Plan fp8_plan(bool trans, int64_t m, int64_t n, int64_t k) {
  Fp8Plan pl;
  const int64_t C = trans ? n : k;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  pl.lo_off = al((size_t)m * C);
  pl.rs_off = pl.lo_off + al((size_t)m * C);
  pl.total = pl.rs_off + al((size_t)m * 4);
  return pl;
}

bool use_fp8_mfma(int32_t fmt, int64_t m) { return fmt == QL_FMT_FP8_E4M3 && m > SMALL_M; }

size_t qgemm_workspace_bytes(int32_t fmt, bool trans, int64_t m, int64_t n, int64_t k, int32_t r) {
  if (use_fp8_mfma(fmt, m)) return fp8_plan(trans, m, n, k).total;
  return split_plan(trans, m, n, k, r).total;
}

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
  if (use_fp8_mfma(c.w->format, c.m)) {
    // a1 split of the activation, the rank-r projection (U or V, written to save), fp8 GEMM
    const Fp8Plan fp = fp8_plan(c.trans, c.m, p.N, p.K);
    uint8_t* base = reinterpret_cast<uint8_t*>(c.ws);
    uint8_t* hi = base;
    uint8_t* lo = base + fp.lo_off;
    float* rs = reinterpret_cast<float*>(base + fp.rs_off);
    hipError_t e = launch_act_quant(c.act, c.m, p.C, hi, lo, rs, s);
    if (e == hipSuccess) e = launch_rproj(c.act, c.m, p.C, c.down, !c.trans, c.r, c.save, s);
    if (e != hipSuccess) return e;
    Gemm8Call g{};
    g.w = c.w;
    g.trans = c.trans;
    g.hi = hi;
    g.lo = lo;
    g.rs = rs;
    g.m = c.m;
    g.u = c.save;
    g.up = c.up;
    g.r = c.r;
    g.s = c.s;
    g.out = c.out;
    return launch_qgemm8(g, s);
  }
  const Nf4Table& t = nf4_table();
  for (int i = 0; i < 16; ++i) p.book.c[i] = t.level[i];
  const SplitPlan pl = split_plan(c.trans, c.m, p.N, p.K, c.r);
  if (pl.splits > 0) {
    p.part = reinterpret_cast<float*>(c.ws);
    p.upart = reinterpret_cast<float*>(reinterpret_cast<char*>(c.ws) + pl.upart_off);
    p.sps = pl.sps;
  }
  switch (c.w->format) {
    case QL_FMT_Q4_0: return launch_f<QL_FMT_Q4_0>(p, c.trans, c.r, pl.splits, s);
    case QL_FMT_NF4: return launch_f<QL_FMT_NF4>(p, c.trans, c.r, pl.splits, s);
    default: return launch_f<QL_FMT_FP8_E4M3>(p, c.trans, c.r, pl.splits, s);
  }
}

}  // namespace ql
