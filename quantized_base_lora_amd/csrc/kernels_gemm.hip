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
// Tiling (gfx950): the workgroup owns a 256 x TN output tile, TN = 256, 192
// or 128, whichever needs the least time counted in rounds of one workgroup
// per CU.  With 512 threads (the default) there are two waves per SIMD, so one
// wave's stalls are covered by the other's MFMAs; each wave owns a 128 x 64,
// 64 x 96 or 64 x 64 block.
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
//
// One launch can run several independent calls of one format, direction,
// token count and rank (q|k|v, gate|up of a decoder layer): a problem table
// in the kernel arguments, each problem its own run of tiles, ordered by
// contraction length so the longest tiles are dispatched first.  Each output
// element is computed exactly as in a launch of its own, whatever the tile
// shape, so grouped results are bitwise those of separate calls; what the
// group saves is the ramp-up and drain of every launch but one.
#include <algorithm>

#include "dequant.h"

namespace ql {
namespace {

// TM = 256: NTH = 256 gives four waves, one per SIMD, each owning a
// 128 x TN/2 block; NTH = 512 gives eight waves, two per SIMD, each owning a
// 128 x 64 (TN = 256), 64 x 96 (TN = 192) or 64 x 64 (TN = 128) block.
template <int TM_, int TN, int NTH> struct Shape {
  static constexpr int TM = TM_;
  static constexpr int NW = NTH / 64;
  static constexpr int A_ELEMS = TM * SA;
  static constexpr int SBT = TN + 32;                 // dX W tile [TK][TN] stride (576 / 320 B rows)
  // dX W tile: 16-byte piece p of 32-element group g in row w is stored at
  // piece p ^ wswz(w, g).  Unswizzled, the 16-byte dequantization stores of a
  // wave (8 rows x 8 groups for TN = 256) fall on a quarter of the LDS banks
  // (rows 576 B apart, groups 64 B apart), 4- to 5-way conflicts; swizzled
  // they spread over all banks, and the transposing fragment reads (4
  // consecutive bytes-8 runs of 4 rows per 16 lanes) stay conflict-free.
  __device__ static int wswz(int row, int grp) { return TN == 256 ? ((row + 2 * (grp >> 2)) & 3) : (grp & 3); }
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
  static_assert(MB >= 1 && NB >= 1 && AR >= 1 && UI >= 1, "tile shape");
};

// problems of one launch: workgroups [tile0[g], tile0[g + 1]) own the tiles of
// problem g (tile0[n] = grid size)
struct GemmArgs {
  Params p[MAX_GROUP];
  int32_t tile0[MAX_GROUP + 1];
  int32_t n;
};

template <int FMT, bool TRANS, int R, int TM_, int TN, int NTH>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(NTH / 256, NTH / 256)))
void qgemm_kernel(GemmArgs ga) {
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
  constexpr bool BYTES = byte_codes<FMT>();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / S::WAVES_N, wn = wave % S::WAVES_N;

  // ---- problem and tile: each problem's tiles in contiguous runs per XCD
  // (workgroups go round-robin over the 8 XCDs; a run of a multiple of 8
  // workgroups starting at a multiple of 8 keeps that order)
  const int bid = (int)blockIdx.x;
  int pi = 0;
  while (pi + 1 < ga.n && bid >= ga.tile0[pi + 1]) ++pi;
  const Params& p = ga.p[pi];
  const int t0 = ga.tile0[pi], tiles = ga.tile0[pi + 1] - t0;
  const int nt = (int)((p.O + TN - 1) / TN);
  int t = bid - t0;
  if ((tiles & 7) == 0 && (t0 & 7) == 0) t = (t & 7) * (tiles >> 3) + (t >> 3);
  // tiles in groups of GM row blocks, column by column within a group: the
  // 32 workgroups an XCD runs at once then cover a few row blocks by several
  // column tiles instead of one row block by 32 column tiles, so its L2 sees
  // less of W per tile (for wide layers the whole of W passed through every
  // XCD's L2 for each row block)
  constexpr int GM = 4;
  const int mt = tiles / nt;
  const int grp = t / (GM * nt), fm = grp * GM;
  const int gm = mt - fm < GM ? mt - fm : GM;        // row blocks in this group
  const int tg = t - grp * GM * nt;
  const int64_t o0 = (int64_t)(tg / gm) * TN;
  const int64_t m0 = (int64_t)(fm + tg % gm) * TM;
  const int KT = (int)((p.C + TK - 1) / TK);
  const int kbeg = 0, kend = KT, NKT = KT;          // contraction steps of this workgroup

  // ---- buffer resources (bases rebased to this tile, so 32-bit offsets suffice)
  const __amdgpu_buffer_rsrc_t ract = rsrc(p.act + m0 * p.C, (p.M - m0) * p.C * 2);
  const int64_t crow = BYTES ? p.K : p.K / 2;        // code bytes per row of W
  const int64_t wrow0 = TRANS ? 0 : o0;              // first W row this tile reads
  const int64_t wcol0 = TRANS ? (BYTES ? o0 : o0 / 2) : 0;
  const __amdgpu_buffer_rsrc_t rcode = rsrc(p.codes + wrow0 * crow + wcol0, (p.N - wrow0) * crow - wcol0);
  const int64_t srow = scales_per_row<FMT>(p.K);   // scale words per row
  const int64_t ssz = scale_bytes<FMT>();
  const __amdgpu_buffer_rsrc_t rscale =
      rsrc((const char*)p.scales + scale_offset<FMT>() + wrow0 * srow * ssz, (p.N - wrow0) * srow * ssz);
  const __amdgpu_buffer_rsrc_t rdown = rsrc(p.down, (int64_t)R * p.C * 2);

  float tscale = 0.0f;
  if constexpr (tensor_scale<FMT>()) tscale = reinterpret_cast<const float*>(p.scales)[0];

  // ---- per-thread load coordinates
  const int arow = tid >> 3, acol = (tid & 7) * 8;   // act: rows arow + ARS i, 8 columns
  constexpr int AR = S::AR, ARS = S::ARS;
  const bool wtask = !S::WPART || tid < S::WGT;     // wave-uniform
  int wr[WG], wg[WG];                                // W groups: row of the W tile, group in that row
  bool wg_in[WG];                                    // dX: the group's output columns lie inside K
  int wsx[WG];                                       // dX: piece swizzle of the group, in elements
#pragma unroll
  for (int j = 0; j < WG; ++j) {
    const int g = tid + NT * j;
    wr[j] = g / GPR;
    wg[j] = g % GPR;
    wg_in[j] = !TRANS || (o0 + 32 * (wg[j] + 1) <= p.K);
    wsx[j] = TRANS ? S::wswz(wr[j], wg[j]) << 3 : 0;
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
    // forward: a group past the end of the contraction reads as zero.  Threads
    // without a W group issue the loads too, at an out-of-range offset (no
    // traffic): every path then has the same loads in flight and the
    // compiler's wait counts stay exact.
    const bool live = wtask && (TRANS || c0 + 32 * wg[j] < p.C);
    const uint32_t coff = live ? (uint32_t)(wrow * crow + kgrp * (BYTES ? 32 : 16)) : OOB;
    wreg[j].c0 = bload16(rcode, coff);
    if constexpr (BYTES) wreg[j].c1 = bload16(rcode, live ? coff + 16 : OOB);
    if constexpr (!FP8) {
      const int64_t kabs = TRANS ? (o0 >> 5) + wg[j] : kgrp;   // group index along K
      if constexpr (two_byte_scales<FMT>()) {
        const int64_t idx = wrow * srow + kabs;
        wreg[j].sraw = bload4(rscale, live ? (uint32_t)((idx * 2) & ~3LL) : OOB);
        wreg[j].ssh = (uint32_t)(idx & 1) * 16;
      } else if constexpr (FMT == QL_FMT_MXFP4) {
        const int64_t idx = wrow * srow + kabs;
        wreg[j].sraw = bload4(rscale, live ? (uint32_t)(idx & ~3LL) : OOB);
        wreg[j].ssh = (uint32_t)(idx & 3) * 8;
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
    float s0, s1;
    group_scales<FMT>(wreg[j].sraw >> wreg[j].ssh, tscale, s0, s1);
    deq.prepare(wreg[j], wg_in[j] ? s0 : 0.0f, p.book, wg_in[j], wg_in[j] ? s1 : 0.0f);
  };
  auto store_w = [&](uint16_t* st, int j, int i) {   // elements 8i .. 8i+7 of W group j
    if (!wtask) return;
    const int po = TRANS ? (8 * i) ^ wsx[j] : 8 * i;
    uint16_t* dst = st + A_ELEMS + (TRANS ? wr[j] * S::SBT : wr[j] * SA) + wg[j] * 32 + po;
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
        const int row = ks * 16 + 8 * (b >> 1) + (sl >> 2);   // rows row and row + 4: one swizzle
        const int pcol = col ^ (S::wswz(row, col >> 5) << 3);   // bits 3-4 of col: the piece
        fb[h][j] = tr16x8(Bs + row * S::SBT + pcol, Bs + (row + 4) * S::SBT + pcol);
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
    if constexpr (TRANS && TN == 192) {
      // scheduling groups (MFMA, 20 VALU, 2 LDS reads, 1 LDS write, 1 load,
      // repeated) for the last block of this region: measured 5-8 % faster for
      // this tile; neutral or slower for the others
#pragma unroll
      for (int g = 0; g < 3 * MB * NB; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    lds_barrier();
    // slice 3
    read_frags(ns, 0);
    mfma_ks(3);
  }
  // the tile's slice of the up matrix, loaded now so the epilogue does not
  // wait for it: forward B rows o0 .. o0+TN (contiguous, 8 elements per
  // piece), dX A[j][o0 .. o0+TN] (8 columns of one row per piece; consecutive
  // lanes take consecutive rows j, so their 2-byte transposed stores into the
  // epilogue tile are adjacent instead of 8 tile rows apart)
  constexpr int UPP = TN * R / 8;                    // 16-byte pieces
  constexpr int UPT = (UPP + NT - 1) / NT;
  uint4 upv[UPT];
  {
    const __amdgpu_buffer_rsrc_t rup = TRANS ? rsrc(p.up, (int64_t)R * p.K * 2)
                                             : rsrc(p.up + o0 * R, (p.N - o0) * R * 2);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int q = tid + NT * u;
      uint32_t off = OOB;
      if constexpr (TRANS) {
        const int j = q % R, c = (q / R) * 8;
        if (q < UPP && o0 + c < p.K) off = (uint32_t)((j * p.K + o0 + c) * 2);
      } else {
        if (q < UPP) off = (uint32_t)(q * 16);
      }
      upv[u] = bload16(rup, off);
    }
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

  // ---------------------------------------------------------------- epilogue
  mfma_result_guard();   // the conditional store of U below follows the last MFMAs
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
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int q = tid + NT * u;
    if (q < UPP) {
      if constexpr (TRANS) {
        const int j = q % R, c = (q / R) * 8;
        const uint32_t w[4] = {upv[u].x, upv[u].y, upv[u].z, upv[u].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t v = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          Bx[(c + e) * SX + j] = v;
          Bx[(c + e) * SX + R + j] = v;
        }
      } else {
        const int col = q / (R / 8), j = (q % (R / 8)) * 8;
        *reinterpret_cast<uint4*>(Bx + col * SX + j) = upv[u];
        *reinterpret_cast<uint4*>(Bx + col * SX + R + j) = upv[u];
      }
    }
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
  // ---- store bf16.  Lane l holds row l % 32 and, in accumulators 4g .. 4g+3,
  // columns 8g + 4 (l / 32) .. +3.  For each pair of column groups (2p, 2p+1)
  // lanes l and l + 32 trade halves (v_permlane32_swap): lane l then holds
  // the 8 columns of group 2p, lane l + 32 those of group 2p+1, and each
  // writes them with one 16-byte store.
  const int hl = lane >> 5;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int64_t row = m0 + S::WM * wm + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const uint32_t a0 = pack_bf16x2(acc[i][j][8 * pr + 0], acc[i][j][8 * pr + 1]);
        const uint32_t a1 = pack_bf16x2(acc[i][j][8 * pr + 2], acc[i][j][8 * pr + 3]);
        const uint32_t b0 = pack_bf16x2(acc[i][j][8 * pr + 4], acc[i][j][8 * pr + 5]);
        const uint32_t b1 = pack_bf16x2(acc[i][j][8 * pr + 6], acc[i][j][8 * pr + 7]);
        // lanes >= 32 of the first operand trade places with lanes < 32 of the second
        const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
        const int64_t col = o0 + S::WN * wn + 32 * j + 8 * (2 * pr + hl);
        if (row < p.M && col < p.O)
          *reinterpret_cast<uint4*>(p.out + row * p.O + col) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
      }
  }
}

template <int FMT, bool TRANS, int R, int TM, int TN, int NTH>
hipError_t launch_t(const GemmArgs& g, hipStream_t s) {
  using S = Shape<TM, TN, NTH>;
  constexpr int B_ELEMS = TRANS ? S::BT_ELEMS : S::BF_ELEMS;
  constexpr int D_ELEMS = TRANS ? BL_ELEMS : AD_ELEMS;
  constexpr size_t smem = 2 * (size_t)(S::A_ELEMS + B_ELEMS + D_ELEMS) * sizeof(uint16_t);
  static_assert(smem <= 160 * 1024, "LDS budget");
  static_assert((size_t)(TM + TN) * (2 * R + 8) * sizeof(uint16_t) <= smem, "epilogue LDS");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)qgemm_kernel<FMT, TRANS, R, TM, TN, NTH>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  GemmArgs a = g;
  int64_t tiles = 0;
  for (int i = 0; i < a.n; ++i) {
    a.tile0[i] = (int32_t)tiles;
    tiles += ((a.p[i].O + TN - 1) / TN) * ((a.p[i].M + TM - 1) / TM);
  }
  a.tile0[a.n] = (int32_t)tiles;
  hipLaunchKernelGGL((qgemm_kernel<FMT, TRANS, R, TM, TN, NTH>), dim3((unsigned)tiles),
                     dim3(NTH), smem, s, a);
  return hipGetLastError();
}

// Output tile: the one with the least time in rounds of 256 workgroups (one
// per CU) times work per tile, each shape weighted for its MFMA efficiency
// (the narrower tiles read more LDS per MFMA); ties go to the earlier entry.
// 128x128 tiles only pay off when the 256-row tiles would leave CUs idle.
// A group counts its tiles in units of its longest contraction.
struct TilePick {
  int tm, tn;
};
TilePick pick_tile(const GemmArgs& g) {
  struct Cand {
    int tm, tn;
    double eff;
  };
  const Cand c[4] = {{256, 256, 1.0}, {256, 192, 0.95}, {256, 128, 0.85}, {128, 128, 0.6}};
  const int nc = 4;
  TilePick best{256, 256};
  double best_cost = 1e300;
  int64_t cmax = 1;
  for (int j = 0; j < g.n; ++j) cmax = std::max<int64_t>(cmax, g.p[j].C);
  for (int i = 0; i < nc; ++i) {
    int64_t work = 0;                                // tiles x contraction length
    for (int j = 0; j < g.n; ++j)
      work += ((g.p[j].M + c[i].tm - 1) / c[i].tm) * ((g.p[j].O + c[i].tn - 1) / c[i].tn) * g.p[j].C;
    const int64_t rounds = (work + 256 * cmax - 1) / (256 * cmax);
    const double cost = (double)rounds * c[i].tm * c[i].tn / c[i].eff;
    if (cost < best_cost * (1 - 1e-9)) {
      best_cost = cost;
      best = TilePick{c[i].tm, c[i].tn};
    }
  }
  return best;
}

template <int FMT, bool TRANS, int R>
hipError_t launch_w(const GemmArgs& g, hipStream_t s) {
#ifndef QL_GEMM_THREADS
#define QL_GEMM_THREADS 512
#endif
  const TilePick t = pick_tile(g);
  if (t.tm == 128) return launch_t<FMT, TRANS, R, 128, 128, QL_GEMM_THREADS>(g, s);
  switch (t.tn) {
    case 256: return launch_t<FMT, TRANS, R, 256, 256, QL_GEMM_THREADS>(g, s);
    case 192: return launch_t<FMT, TRANS, R, 256, 192, QL_GEMM_THREADS>(g, s);
    default: return launch_t<FMT, TRANS, R, 256, 128, QL_GEMM_THREADS>(g, s);
  }
}

template <int FMT, bool TRANS>
hipError_t launch_r(const GemmArgs& g, int r, hipStream_t s) {
  switch (r) {
    case 8: return launch_w<FMT, TRANS, 8>(g, s);
    case 16: return launch_w<FMT, TRANS, 16>(g, s);
    default: return launch_w<FMT, TRANS, 32>(g, s);
  }
}

template <int FMT>
hipError_t launch_f(const GemmArgs& g, bool trans, int r, hipStream_t s) {
  return trans ? launch_r<FMT, true>(g, r, s) : launch_r<FMT, false>(g, r, s);
}

hipError_t launch_tiles(int fmt, const GemmArgs& g, bool trans, int r, hipStream_t s) {
  switch (fmt) {
    case QL_FMT_Q4_0: return launch_f<QL_FMT_Q4_0>(g, trans, r, s);
    case QL_FMT_NF4: return launch_f<QL_FMT_NF4>(g, trans, r, s);
    case QL_FMT_MXFP4: return launch_f<QL_FMT_MXFP4>(g, trans, r, s);
    case QL_FMT_Q8_0: return launch_f<QL_FMT_Q8_0>(g, trans, r, s);
    case QL_FMT_NVFP4: return launch_f<QL_FMT_NVFP4>(g, trans, r, s);
    default: return launch_f<QL_FMT_FP8_E4M3>(g, trans, r, s);
  }
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

// the kernel parameters of a call on the bf16 matrix-core paths; splits > 0
// selects the small-M split path
static void make_params(const GemmCall& c, Params& p, int& splits) {
  p = Params{};
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
  if (c.w->format == QL_FMT_NVFP4) {
    // E2M1 values in code order: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, then their negatives
    static const float e2m1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    for (int i = 0; i < 8; ++i) {
      p.book.c[i] = e2m1[i];
      p.book.c[8 + i] = -e2m1[i];
    }
  } else {
    const Nf4Table& t = nf4_table();
    for (int i = 0; i < 16; ++i) p.book.c[i] = t.level[i];
  }
  const SplitPlan pl = split_plan(c.trans, c.m, p.N, p.K, c.r);
  splits = pl.splits;
  if (pl.splits > 0) {
    p.part = reinterpret_cast<float*>(c.ws);
    p.upart = reinterpret_cast<float*>(reinterpret_cast<char*>(c.ws) + pl.upart_off);
    p.sps = pl.sps;
  }
}

// FP8 base above SMALL_M: per call the a1 split of the activation (done once
// for calls that share their activation), the rank-r projection (U or V,
// written to save), then one fp8 GEMM launch for all the calls
static bool fp8_group(const GemmCall* calls, int n) {
  if (n < 1 || n > MAX_GROUP) return false;
  for (int i = 0; i < n; ++i) {
    const GemmCall& c = calls[i];
    if (!use_fp8_mfma(c.w->format, c.m) || c.grads || c.trans != calls[0].trans || c.m != calls[0].m ||
        c.r != calls[0].r)
      return false;
  }
  return true;
}

static hipError_t launch_fp8_calls(const GemmCall* calls, int n, hipStream_t s) {
  // the activation splits of the group's distinct activations, then the
  // calls' projections, each in one launch (the computations are
  // independent, so the order does not change results), then the GEMMs
  Gemm8Call g[MAX_GROUP];
  ActSplit sp[MAX_GROUP];
  Rproj pr[MAX_GROUP];
  int nsp = 0;
  for (int i = 0; i < n; ++i) {
    const GemmCall& c = calls[i];
    const int64_t N = c.w->n_out, K = c.w->k_in, C = c.trans ? N : K;
    int j = 0;
    while (j < i && !(calls[j].act == c.act && (calls[j].trans ? calls[j].w->n_out : calls[j].w->k_in) == C)) ++j;
    if (j < i) {                                     // same activation: its split is already there
      g[i].hi = g[j].hi;
      g[i].lo = g[j].lo;
      g[i].rs = g[j].rs;
    } else {
      const Fp8Plan fp = fp8_plan(c.trans, c.m, N, K);
      uint8_t* base = reinterpret_cast<uint8_t*>(c.ws);
      uint8_t* hi = base;
      uint8_t* lo = base + fp.lo_off;
      float* rs = reinterpret_cast<float*>(base + fp.rs_off);
      g[i].hi = hi;
      g[i].lo = lo;
      g[i].rs = rs;
      sp[nsp++] = ActSplit{c.act, hi, lo, rs, C};
    }
    pr[i] = Rproj{c.act, c.down, c.save, C};
    g[i].w = c.w;
    g[i].trans = c.trans;
    g[i].m = c.m;
    g[i].u = c.save;
    g[i].up = c.up;
    g[i].r = c.r;
    g[i].s = c.s;
    g[i].out = c.out;
  }
  hipError_t e = launch_act_quant_group(sp, nsp, calls[0].m, s);
  if (e != hipSuccess) return e;
  e = launch_rproj_group(pr, n, calls[0].m, !calls[0].trans, calls[0].r, s);
  if (e != hipSuccess) return e;
  return launch_qgemm8(g, n, s);
}

hipError_t launch_qgemm(const GemmCall& c, hipStream_t s) {
  if (use_fp8_mfma(c.w->format, c.m)) return launch_fp8_calls(&c, 1, s);
  Params p;
  int splits = 0;
  make_params(c, p, splits);
  // the adapter gradients ride only on the split path's reduction
  if (c.grads && (!c.trans || splits == 0)) return hipErrorInvalidValue;
  if (splits > 0) {
    SplitGroup g{};
    g.p[0] = p;
    g.splits[0] = splits;
    g.n = 1;
    return launch_split_path(c.w->format, c.trans, c.r, g, c.grads, s);
  }
  GemmArgs g{};
  g.p[0] = p;
  g.n = 1;
  return launch_tiles(c.w->format, g, c.trans, c.r, s);
}

// one launch (pair) for the group: one format, direction, token count and
// rank, and one path for all (the small-M split path, or the bf16 tile kernel;
// the FP8 base's fp8 path above SMALL_M is grouped by launch_fp8_calls)
bool qgemm_groupable(const GemmCall* calls, int n) {
  if (n < 2 || n > MAX_GROUP) return false;
  const GemmCall& c0 = calls[0];
  const bool split = split_plan(c0.trans, c0.m, c0.w->n_out, c0.w->k_in, c0.r).splits > 0;
  if (!split && (use_fp8_mfma(c0.w->format, c0.m) || c0.grads)) return false;
  for (int i = 0; i < n; ++i) {
    const GemmCall& c = calls[i];
    if (c.w->format != c0.w->format || c.trans != c0.trans || c.m != c0.m || c.r != c0.r ||
        (c.grads != nullptr) != (c0.grads != nullptr))
      return false;
    if ((split_plan(c.trans, c.m, c.w->n_out, c.w->k_in, c.r).splits > 0) != split) return false;
  }
  return true;
}

hipError_t launch_qgemm_group(const GemmCall* calls, int n, hipStream_t s) {
  if (n > 1 && fp8_group(calls, n)) return launch_fp8_calls(calls, n, s);
  if (!qgemm_groupable(calls, n)) {
    for (int i = 0; i < n; ++i) {
      hipError_t e = launch_qgemm(calls[i], s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  int splits[MAX_GROUP];
  Params ps[MAX_GROUP];
  for (int i = 0; i < n; ++i) make_params(calls[i], ps[i], splits[i]);
  if (splits[0] == 0) {
    // tile kernel: longest contraction first (stable), so its tiles start first
    int order[MAX_GROUP];
    for (int i = 0; i < n; ++i) order[i] = i;
    std::stable_sort(order, order + n, [&](int a, int b) { return ps[a].C > ps[b].C; });
    GemmArgs g{};
    g.n = n;
    for (int i = 0; i < n; ++i) g.p[i] = ps[order[i]];
    return launch_tiles(calls[0].w->format, g, calls[0].trans, calls[0].r, s);
  }
  SplitGroup g{};
  GradFuse gf[MAX_GROUP];
  g.n = n;
  for (int i = 0; i < n; ++i) {
    g.p[i] = ps[i];
    g.splits[i] = splits[i];
    if (calls[i].grads) gf[i] = *calls[i].grads;
  }
  return launch_split_path(calls[0].w->format, calls[0].trans, calls[0].r, g, calls[0].grads ? gf : nullptr, s);
}

}  // namespace ql
