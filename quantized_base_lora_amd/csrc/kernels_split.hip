// a3 / a6 for at most 64 tokens: the split-contraction path.
//
// With so few tokens the base GEMM is bound by streaming and dequantizing W;
// the contraction is split across workgroups (fp32 partials in the caller's
// workspace) and a second kernel adds the partials in split order, fuses the
// LoRA term and rounds once to bf16, so results do not depend on scheduling.
#include <algorithm>

#include "dequant.h"

namespace ql {
namespace {

// At most 64 tokens the base GEMM is bound by streaming W, and each
// workgroup sees only a few contraction steps, so every step's loads must be
// in flight long before they are needed: a ring of D register stages keeps
// the loads of steps it+1 .. it+D outstanding while step it computes.  Tile:
// all tokens (TM = 32 MBK rows: 32 when M <= 32, else 64) x 128 output
// columns, four waves side by side (TM x 32 each), the contraction split
// across workgroups; fp32 partial sums out.  One launch serves a group of
// independent problems: each workgroup finds its problem, column tile and
// split in a table in the kernel arguments.  (The forward with at most 16
// tokens and a 4-bit base runs qstream16_kernel or qsplit16_kernel below
// instead.)
//
// Forward (y = x.W^T): no W element is used by more than one wave, so W is
// not staged through LDS.  Each lane loads the codes of its own MFMA
// B-operand row (row 32 wave + lane % 32): one whole 32-element group per
// step, group h = lane / 32 of the step's two, in one 16-byte load (32 for
// FP8) with one scale, and dequantizes it straight into operand registers;
// only the shared activation tile goes through LDS.  The order in which a dot
// product runs over K is free, so slice ks of lane half h holds elements
// 32 h + 8 ks .. 32 h + 8 ks + 7 of the step (the dequantizer's pieces of the
// group in order, whatever the format's nibble layout), and the activation
// fragment is read in the same order.
template <bool TRANS> constexpr int split_b_elems() { return TRANS ? TK * (128 + 32) : 0; }

// Launch arguments of a group: the problems and the first workgroup of each.
struct SplitArgs {
  Params p[MAX_GROUP];
  int32_t unit0[MAX_GROUP + 1];   // unit0[n] = grid size
  int32_t ntiles[MAX_GROUP];
  int32_t n;
};

// Scale window (SW, forward only): the tile's scale entries over the
// workgroup's slice (at most 128 contiguous bytes a row) are loaded once into
// LDS with coalesced dword loads, after the stages, and each step reads its
// scale there instead of issuing a load that touches 32 rows with 1-4 bytes
// each.
constexpr int SWB = 144;                           // LDS row stride of the scale window (bytes)
// dwords a window row: 128 bytes (32 steps of a 4-byte scale step); MXFP4's
// one-byte scales need at most 64
template <int FMT> constexpr int sw_dw() { return FMT == QL_FMT_MXFP4 ? 16 : 32; }
template <int FMT> constexpr int scale_step64_bytes() { return FMT == QL_FMT_MXFP4 ? 2 : 4; }

template <int FMT, bool TRANS, int R, int MBK, bool SW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qsplit_kernel(SplitArgs ga) {
  static_assert(!SW || (!TRANS && FMT != QL_FMT_FP8_E4M3), "scale window: forward, scaled formats");
  constexpr int TM = 32 * MBK, TN = 128, NT = 256, D = 4;
  static_assert(D % 2 == 0, "buffer parity of a step is its position in the chunk");
  constexpr int SBT = TN + 32;
  constexpr int A_EL = TM * SA;
  constexpr int B_EL = split_b_elems<TRANS>();
  constexpr int D_EL = TRANS ? BL_ELEMS : AD_ELEMS;
  constexpr int STAGE = A_EL + B_EL + D_EL;
  constexpr int RB = (R + 15) / 16;
  constexpr int GPR = TRANS ? TN / 32 : TK / 32;
  constexpr bool FP8 = FMT == QL_FMT_FP8_E4M3;
  constexpr bool BYTES = byte_codes<FMT>();
  constexpr bool DIRECT = !TRANS;                    // forward: W straight into operand registers
  constexpr size_t STAGES_BYTES = 2 * (size_t)(TM * SA + split_b_elems<TRANS>() + (TRANS ? BL_ELEMS : AD_ELEMS)) * 2;
  static_assert(!DIRECT || TN == 4 * 32, "one 32-row W block per wave");
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint8_t* swin = reinterpret_cast<uint8_t*>(smem) + STAGES_BYTES;   // scale window (SW)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // units (column tile, split) are handed to the 8 XCDs (round robin over the
  // linear workgroup id) in contiguous runs, so adjacent column tiles of one
  // split share their XCD's L2: a dX step reads 64 of the 128 bytes of each
  // W-row line, and the neighbouring tile reads the other half
  const int bid = (int)blockIdx.x;
  int pi = 0;                                        // this workgroup's problem (uniform)
  while (pi + 1 < ga.n && bid >= ga.unit0[pi + 1]) ++pi;
  const Params& p = ga.p[pi];
  const int u0 = ga.unit0[pi], nunits = ga.unit0[pi + 1] - u0, nt = ga.ntiles[pi];
  int unit = bid - u0;
  if ((nunits & 7) == 0 && (u0 & 7) == 0) unit = (unit & 7) * (nunits >> 3) + (unit >> 3);
  const int ntile = unit % nt, split = unit / nt;
  const int64_t o0 = (int64_t)ntile * TN;
  const int KT = (int)((p.C + TK - 1) / TK);
  const int kbeg = split * p.sps;
  const int kend = min(KT, kbeg + p.sps);
  const int NKT = kend - kbeg;
  // scale window: the slice's first scale byte in its row, and its offset in
  // the dword that holds it (MXFP4, two bytes a step: 0 or 2)
  const int64_t sb0 = (int64_t)kbeg * scale_step64_bytes<FMT>();
  const int sdel = (int)(sb0 & 3);

  const __amdgpu_buffer_rsrc_t ract = rsrc(p.act, p.M * p.C * 2);
  const int64_t crow = BYTES ? p.K : p.K / 2;
  const int64_t wrow0 = TRANS ? 0 : o0;
  const int64_t wcol0 = TRANS ? (BYTES ? o0 : o0 / 2) : 0;
  const __amdgpu_buffer_rsrc_t rcode = rsrc(p.codes + wrow0 * crow + wcol0, (p.N - wrow0) * crow - wcol0);
  const int64_t srow = scales_per_row<FMT>(p.K);
  const int64_t ssz = scale_bytes<FMT>();
  const __amdgpu_buffer_rsrc_t rscale =
      rsrc((const char*)p.scales + scale_offset<FMT>() + wrow0 * srow * ssz, (p.N - wrow0) * srow * ssz);
  const __amdgpu_buffer_rsrc_t rdown = rsrc(p.down, (int64_t)R * p.C * 2);
  float tscale = 0.0f;
  if constexpr (tensor_scale<FMT>()) tscale = reinterpret_cast<const float*>(p.scales)[0];

  const int arow = tid >> 3, acol = (tid & 7) * 8;   // act rows arow (and arow + 32 when MBK = 2)
  const int wr = tid / GPR, wg = tid % GPR;          // one W group per thread per step
  const bool wg_in = !TRANS || (o0 + 32 * (wg + 1) <= p.K);
  constexpr int DPR = TRANS ? R / 8 : TK / 8;
  // the rank-r projection (U or V) is stored by column tile 0 only, so the
  // other tiles neither load the down matrix nor run its MFMAs
  const bool rank_tile = ntile == 0;
  const bool dload = tid < 8 * R && rank_tile;
  const int drow = tid / DPR, dcol = (tid % DPR) * 8;

  struct Slot {
    uint4 a0, a1, d;
    WGroup w;   // direct forward: c0 (c1 for FP8) = this lane's codes of both groups; sraw / ssh = their scales
    int kt;
  };
  const int hsel = lane >> 5;                        // direct forward: which group of the step this lane holds
  Slot ring[D];
  // loads of step kt; a step past the split's end reads zeros (no memory traffic)
  auto issue = [&](Slot& sl, int kt) {
    const bool sv = kt < kend;
    const int64_t c0 = (int64_t)kt * TK;
    const bool alive = sv && c0 + acol < p.C;
    sl.a0 = bload16(ract, alive ? (uint32_t)((arow * p.C + c0 + acol) * 2) : OOB);
    if constexpr (MBK == 2) sl.a1 = bload16(ract, alive ? (uint32_t)(((arow + 32) * p.C + c0 + acol) * 2) : OOB);
    sl.kt = kt;
    if constexpr (DIRECT) {
      const int64_t wrow = 32 * wave + (lane & 31);  // W row, relative to the tile
      const bool gl = sv && c0 + 32 * hsel < p.C;    // this lane's group lies inside K
      if constexpr (BYTES) {
        const uint32_t base = (uint32_t)(wrow * crow + c0 + 32 * hsel);
        sl.w.c0 = bload16(rcode, gl ? base : OOB);
        sl.w.c1 = bload16(rcode, gl ? base + 16 : OOB);
        const int64_t idx = wrow * srow + (c0 >> 5) + hsel;
        sl.w.sraw = (FP8 || SW) ? 0u : bload2(rscale, gl ? (uint32_t)(idx * 2) : OOB);
      } else {
        sl.w.c0 = bload16(rcode, gl ? (uint32_t)(wrow * crow + c0 / 2 + 16 * hsel) : OOB);
        sl.w.c1 = make_uint4(0, 0, 0, 0);
        const int64_t idx = wrow * srow + (c0 >> 5) + hsel;   // the group's scale index (NF4: per 64, below)
        if constexpr (SW) sl.w.sraw = 0;
        else if constexpr (FMT == QL_FMT_Q4_0 || FMT == QL_FMT_NVFP4) sl.w.sraw = bload2(rscale, gl ? (uint32_t)(idx * 2) : OOB);
        else if constexpr (FMT == QL_FMT_MXFP4) sl.w.sraw = bload1(rscale, gl ? (uint32_t)idx : OOB);
        else sl.w.sraw = bload4(rscale, gl ? (uint32_t)((wrow * srow + (c0 >> 6)) * 4) : OOB);
      }
      sl.w.ssh = 0;
    } else {
    const int64_t wrow = TRANS ? c0 + wr : wr;
    const int64_t kgrp = TRANS ? wg : (c0 >> 5) + wg;
    const bool wlive = sv && (TRANS || c0 + 32 * wg < p.C);
    const uint32_t coff = wlive ? (uint32_t)(wrow * crow + kgrp * (BYTES ? 32 : 16)) : OOB;
    sl.w.c0 = bload16(rcode, coff);
    sl.w.ssh = 0;
    sl.w.c1 = BYTES ? bload16(rcode, wlive ? coff + 16 : OOB) : make_uint4(0, 0, 0, 0);
    if constexpr (FP8) {
      sl.w.sraw = 0;
    } else {
      const int64_t kabs = TRANS ? (o0 >> 5) + wg : kgrp;
      if constexpr (two_byte_scales<FMT>()) {
        const int64_t idx = wrow * srow + kabs;
        sl.w.sraw = bload4(rscale, wlive ? (uint32_t)((idx * 2) & ~3LL) : OOB);
        sl.w.ssh = (uint32_t)(idx & 1) * 16;
      } else if constexpr (FMT == QL_FMT_MXFP4) {
        const int64_t idx = wrow * srow + kabs;
        sl.w.sraw = bload4(rscale, wlive ? (uint32_t)(idx & ~3LL) : OOB);
        sl.w.ssh = (uint32_t)(idx & 3) * 8;
      } else {
        sl.w.sraw = bload4(rscale, wlive ? (uint32_t)((wrow * srow + (kabs >> 1)) * 4) : OOB);
      }
    }
    }
    uint32_t doff;
    if constexpr (TRANS) doff = (uint32_t)(((c0 + drow) * R + dcol) * 2);
    else doff = c0 + dcol < p.C ? (uint32_t)((drow * p.C + c0 + dcol) * 2) : OOB;
    sl.d = bload16(rdown, dload && sv ? doff : OOB);
  };
  // direct forward: the lane's group of a step -> its four B operands (slices ks = 0..3)
  auto dequant_direct = [&](const Slot& sl, uint4* wb) {
    const int64_t c0 = (int64_t)sl.kt * TK;
    const bool gl = sl.kt < kend && c0 + 32 * hsel < p.C;
    uint32_t raw = sl.w.sraw;
    if constexpr (SW) {
      // step t of the slice: groups 2 t + hsel (NF4: one entry per step),
      // sdel bytes into the window row
      const uint8_t* srw = swin + (32 * wave + (lane & 31)) * SWB + sdel;
      const int t = sl.kt - kbeg;
      if constexpr (two_byte_scales<FMT>()) raw = *reinterpret_cast<const uint16_t*>(srw + 2 * (2 * t + hsel));
      else if constexpr (FMT == QL_FMT_MXFP4) raw = srw[2 * t + hsel];
      else raw = *reinterpret_cast<const uint32_t*>(srw + 4 * t);
    }
    float s0, s1;
    group_scales<FMT>(raw, tscale, s0, s1);
    Deq<FMT> dq;
    dq.prepare(sl.w, gl ? s0 : 0.0f, p.book, gl, gl ? s1 : 0.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i) wb[i] = dq.piece(i);
  };
  auto store = [&](const Slot& sl, uint16_t* st, uint4* wb) {
    *reinterpret_cast<uint4*>(st + arow * SA + acol) = sl.a0;
    if constexpr (MBK == 2) *reinterpret_cast<uint4*>(st + (arow + 32) * SA + acol) = sl.a1;
    if (dload) *reinterpret_cast<uint4*>(st + A_EL + B_EL + drow * (TRANS ? SL : SA) + dcol) = sl.d;
    if constexpr (DIRECT) {
      dequant_direct(sl, wb);
      return;
    }
    float s0, s1;
    group_scales<FMT>(sl.w.sraw >> sl.w.ssh, tscale, s0, s1);
    Deq<FMT> dq;
    dq.prepare(sl.w, wg_in ? s0 : 0.0f, p.book, wg_in, wg_in ? s1 : 0.0f);
    // dX W tile: 16-byte piece i of group wg stored at piece i ^ (wg & 3), so a
    // wave's stores (16 rows x 4 groups, rows 320 B apart) spread over all
    // banks instead of four-way conflicts (measured 56 % of LDS-active cycles)
    uint16_t* dst = st + A_EL + (TRANS ? wr * SBT : wr * SA) + wg * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(dst + 8 * (i ^ (wg & 3))) = dq.piece(i);
  };
  // every slot starts defined (the prologue may leave some unused)
#pragma unroll
  for (int u = 0; u < D; ++u) {
    ring[u].a0 = ring[u].a1 = ring[u].d = ring[u].w.c0 = ring[u].w.c1 = make_uint4(0, 0, 0, 0);
    ring[u].w.sraw = ring[u].w.ssh = 0;
    ring[u].kt = 0;
  }
  uint4 wbuf[2][4];                                  // direct forward: B operands of two steps
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) wbuf[b][i] = make_uint4(0, 0, 0, 0);

  f32x16 acc[MBK];
#pragma unroll
  for (int i = 0; i < MBK; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
  f32x4 uacc[RB];
#pragma unroll
  for (int jb = 0; jb < RB; ++jb) uacc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint16_t* st, const uint4* wb) {
    const uint16_t* As = st;
    const uint16_t* Bs = st + A_EL;
    const uint16_t* Ds = st + A_EL + B_EL;
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      bf16x8 af[MBK], bf;
      const int koff = DIRECT ? 32 * (lane >> 5) + 8 * ks : ks * 16 + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < MBK; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (32 * i + (lane & 31)) * SA + koff);
      if constexpr (DIRECT) {
        bf = __builtin_bit_cast(bf16x8, wb[ks]);
      } else {
        const int b = lane >> 4, sl = lane & 15;
        const int col = 32 * wave + 16 * (b & 1) + 4 * (sl & 3);
        const int row = ks * 16 + 8 * (b >> 1) + (sl >> 2);
        const int pcol = col ^ (((col >> 5) & 3) << 3);   // the stores' piece swizzle (bits 3-4 of col)
        bf = tr16x8(Bs + row * SBT + pcol, Bs + (row + 4) * SBT + pcol);
      }
#pragma unroll
      for (int i = 0; i < MBK; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af[i], acc[i], 0, 0, 0);
    }
    // rank-r projection of rows 16 wave .. 16 wave + 15 over this stage (waves
    // whose rows lie past the tile have none; only column tile 0 keeps it)
    if (!rank_tile || 16 * wave >= TM) return;
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
  // scale window (before the stages, so that waiting for it leaves their loads in flight):
  // each row's dwords from the one holding the slice's first scale byte
  constexpr int SW_DW = sw_dw<FMT>();
  uint32_t swv[SW ? 128 * SW_DW / 256 : 1];
  if constexpr (SW) {
#pragma unroll
    for (int i = 0; i < 128 * SW_DW / 256; ++i) {
      const int pc = tid + 256 * i, row = pc / SW_DW, dw = pc % SW_DW;
      const bool ok = 4 * dw < sdel + scale_step64_bytes<FMT>() * NKT;
      swv[i] = bload4(rscale, ok ? (uint32_t)(row * srow * ssz + sb0 - sdel + 4 * dw) : OOB);
    }
  }
  // prologue: D stages in flight, the first stored and its slot refilled
#pragma unroll
  for (int u = 0; u < D; ++u) issue(ring[u], kbeg + u);
  if constexpr (SW) {
#pragma unroll
    for (int i = 0; i < 128 * SW_DW / 256; ++i) {
      const int pc = tid + 256 * i;
      *reinterpret_cast<uint32_t*>(swin + (pc / SW_DW) * SWB + 4 * (pc % SW_DW)) = swv[i];
    }
  }
  lds_barrier();
  store(ring[0], smem, wbuf[0]);
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
      store(ring[(u + 1) % D], smem + ((u + 1) & 1) * STAGE, wbuf[(u + 1) & 1]);
      issue(ring[(u + 1) % D], kbeg + it + u + 1 + D);
      compute(smem + (u & 1) * STAGE, wbuf[u & 1]);
      lds_barrier();
    }
  }
  // the last (at most D) steps: everything they need is already in flight
#pragma unroll
  for (int u = 0; u < D; ++u) {
    if (it + u < NKT) {
      if (it + u + 1 < NKT) store(ring[(u + 1) % D], smem + ((u + 1) & 1) * STAGE, wbuf[(u + 1) & 1]);
      compute(smem + (u & 1) * STAGE, wbuf[u & 1]);
      lds_barrier();
    }
  }

  mfma_result_guard();
  // fp32 partials: lane holds row (lane & 31) of block i and 4 consecutive columns per 8
  float* pp = p.part + (int64_t)split * p.M * p.O;
#pragma unroll
  for (int i = 0; i < MBK; ++i) {
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
        if (j < R && row < p.M && 16 * wave < TM) up[row * R + j] = uacc[jb][e];
      }
  }
}

// Forward with at most 16 tokens: 16x16x32 MFMAs (no rows spent on absent
// tokens) over contraction steps of 128.  The tile is 16 tokens x 128
// columns; wave w owns columns 32 w .. 32 w + 31 as two 16-column blocks.
// Lane l feeds row l % 16 of each block with group l / 16 (32 elements, one
// 16-byte load for 4-bit codes) of the step, so a load instruction covers 16
// W rows with 64 contiguous bytes each; slice s of the MFMA takes pieces s of
// those groups, i.e. elements 32 (l / 16) + 8 s .. + 7 of the step, and the
// activation fragment is read in the same order.  Split and reduction as in
// qsplit_kernel (steps counted in 128s: sps = this kernel's steps per split).
constexpr int TK2 = 128;
constexpr int SA2 = TK2 + 8;                        // 272-byte rows

template <int FMT, int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qsplit16_kernel(SplitArgs ga) {
  constexpr int TN = 128, NT = 256, D = 4;
  constexpr int A_EL = 16 * SA2;
  constexpr int D_EL = 32 * SA2;                    // adapter A rows j < R (the rest stay zero)
  constexpr int STAGE = A_EL + D_EL;
  constexpr int RB = (R + 15) / 16;
  constexpr int DPT = (R * TK2 / 8 + NT - 1) / NT;  // 16-byte adapter pieces per thread
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bid = (int)blockIdx.x;
  int pi = 0;
  while (pi + 1 < ga.n && bid >= ga.unit0[pi + 1]) ++pi;
  const Params& p = ga.p[pi];
  const int u0 = ga.unit0[pi], nunits = ga.unit0[pi + 1] - u0, nt = ga.ntiles[pi];
  int unit = bid - u0;
  if ((nunits & 7) == 0 && (u0 & 7) == 0) unit = (unit & 7) * (nunits >> 3) + (unit >> 3);
  const int ntile = unit % nt, split = unit / nt;
  const int64_t o0 = (int64_t)ntile * TN;
  const int KT = (int)((p.C + TK2 - 1) / TK2);
  const int kbeg = split * p.sps;
  const int kend = min(KT, kbeg + p.sps);
  const int NKT = kend - kbeg;

  const __amdgpu_buffer_rsrc_t ract = rsrc(p.act, p.M * p.C * 2);
  const int64_t crow = p.K / 2;                     // 4-bit codes
  const __amdgpu_buffer_rsrc_t rcode = rsrc(p.codes + o0 * crow, (p.N - o0) * crow);
  const int64_t srow = scales_per_row<FMT>(p.K);
  const int64_t ssz = scale_bytes<FMT>();
  const __amdgpu_buffer_rsrc_t rscale =
      rsrc((const char*)p.scales + scale_offset<FMT>() + o0 * srow * ssz, (p.N - o0) * srow * ssz);
  const __amdgpu_buffer_rsrc_t rdown = rsrc(p.down, (int64_t)R * p.C * 2);
  float tscale = 0.0f;
  if constexpr (tensor_scale<FMT>()) tscale = reinterpret_cast<const float*>(p.scales)[0];

  const int arow = tid >> 4, acol = (tid & 15) * 8;  // activation: one 16-byte piece per thread
  const int q = lane >> 4;                           // this lane's group of the step
  const bool rank_tile = ntile == 0;

  struct Slot {
    uint4 a, d[DPT];
    WGroup w[2];                                     // the lane's group of block 0 and block 1
    int kt;
  };
  Slot ring[D];
  auto issue = [&](Slot& sl, int kt) {
    const bool sv = kt < kend;
    const int64_t c0 = (int64_t)kt * TK2;
    sl.kt = kt;
    sl.a = bload16(ract, sv && arow < p.M && c0 + acol < p.C ? (uint32_t)((arow * p.C + c0 + acol) * 2) : OOB);
    const bool gl = sv && c0 + 32 * q < p.C;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t wrow = 32 * wave + 16 * b + (lane & 15);   // W row, relative to the tile
      sl.w[b].c0 = bload16(rcode, gl ? (uint32_t)(wrow * crow + c0 / 2 + 16 * q) : OOB);
      sl.w[b].c1 = make_uint4(0, 0, 0, 0);
      const int64_t idx = wrow * srow + (c0 >> 5) + q;
      if constexpr (two_byte_scales<FMT>()) sl.w[b].sraw = bload2(rscale, gl ? (uint32_t)(idx * 2) : OOB);
      else if constexpr (FMT == QL_FMT_MXFP4) sl.w[b].sraw = bload1(rscale, gl ? (uint32_t)idx : OOB);
      else sl.w[b].sraw = bload4(rscale, gl ? (uint32_t)((wrow * srow + ((c0 + 32 * q) >> 6)) * 4) : OOB);
      sl.w[b].ssh = 0;
    }
#pragma unroll
    for (int t = 0; t < DPT; ++t) {
      const int pc = tid + NT * t, j = pc / (TK2 / 8), c = (pc % (TK2 / 8)) * 8;
      const bool live = rank_tile && sv && pc < R * (TK2 / 8) && c0 + c < p.C;
      sl.d[t] = bload16(rdown, live ? (uint32_t)((j * p.C + c0 + c) * 2) : OOB);
    }
  };
  // the lane's two groups of a step -> B operands wb[block][slice]
  auto store = [&](const Slot& sl, uint16_t* st, uint4 (*wb)[4]) {
    *reinterpret_cast<uint4*>(st + arow * SA2 + acol) = sl.a;
    if (rank_tile) {
#pragma unroll
      for (int t = 0; t < DPT; ++t) {
        const int pc = tid + NT * t, j = pc / (TK2 / 8), c = (pc % (TK2 / 8)) * 8;
        if (pc < R * (TK2 / 8)) *reinterpret_cast<uint4*>(st + A_EL + j * SA2 + c) = sl.d[t];
      }
    }
    const bool gl = sl.kt < kend && (int64_t)sl.kt * TK2 + 32 * q < p.C;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float s0, s1;
      group_scales<FMT>(sl.w[b].sraw, tscale, s0, s1);
      Deq<FMT> dq;
      dq.prepare(sl.w[b], gl ? s0 : 0.0f, p.book, gl, gl ? s1 : 0.0f);
#pragma unroll
      for (int i = 0; i < 4; ++i) wb[b][i] = dq.piece(i);
    }
  };
#pragma unroll
  for (int u = 0; u < D; ++u) {
    ring[u].a = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < DPT; ++t) ring[u].d[t] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      ring[u].w[b].c0 = ring[u].w[b].c1 = make_uint4(0, 0, 0, 0);
      ring[u].w[b].sraw = ring[u].w[b].ssh = 0;
    }
    ring[u].kt = 0;
  }
  uint4 wbuf[2][2][4];                               // B operands of two steps
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) wbuf[h][b][i] = make_uint4(0, 0, 0, 0);

  f32x4 acc[2], uacc[RB];
#pragma unroll
  for (int b = 0; b < 2; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jb = 0; jb < RB; ++jb) uacc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint16_t* st, uint4 (*wb)[4]) {
    const uint16_t* As = st;
    const uint16_t* Ds = st + A_EL;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(As + (lane & 15) * SA2 + 32 * q + 8 * sl);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wb[b][sl]), af, acc[b], 0, 0, 0);
    }
    // rank-r projection of the 16 tokens over this step (column tile 0, wave 0)
    if (!rank_tile || wave != 0) return;
#pragma unroll
    for (int kp = 0; kp < TK2 / 32; ++kp) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(As + (lane & 15) * SA2 + 32 * kp + 8 * q);
#pragma unroll
      for (int jb = 0; jb < RB; ++jb) {
        const bf16x8 bd = *reinterpret_cast<const bf16x8*>(Ds + (16 * jb + (lane & 15)) * SA2 + 32 * kp + 8 * q);
        uacc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bd, uacc[jb], 0, 0, 0);
      }
    }
  };

  for (int i = tid; i < STAGE; i += NT) {
    smem[i] = 0;
    smem[STAGE + i] = 0;
  }
  lds_barrier();
#pragma unroll
  for (int u = 0; u < D; ++u) issue(ring[u], kbeg + u);
  store(ring[0], smem, wbuf[0]);
  issue(ring[0], kbeg + D);
  lds_barrier();

  int it = 0;
  for (; it + D < NKT; it += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      store(ring[(u + 1) % D], smem + ((u + 1) & 1) * STAGE, wbuf[(u + 1) & 1]);
      issue(ring[(u + 1) % D], kbeg + it + u + 1 + D);
      compute(smem + (u & 1) * STAGE, wbuf[u & 1]);
      lds_barrier();
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u) {
    if (it + u < NKT) {
      if (it + u + 1 < NKT) store(ring[(u + 1) % D], smem + ((u + 1) & 1) * STAGE, wbuf[(u + 1) & 1]);
      compute(smem + (u & 1) * STAGE, wbuf[u & 1]);
      lds_barrier();
    }
  }

  mfma_result_guard();
  // fp32 partials: lane holds token lane % 16 and 4 consecutive columns of each block
  float* pp = p.part + (int64_t)split * p.M * p.O;
  const int64_t m = lane & 15;
  if (m < p.M) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = o0 + 32 * wave + 16 * b + 4 * q;
      if (col < p.O) *reinterpret_cast<float4*>(pp + m * p.O + col) = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
    }
  }
  if (rank_tile && wave == 0) {
    float* up = p.upart + (int64_t)split * p.M * R;
#pragma unroll
    for (int jb = 0; jb < RB; ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 4 * q + e;
        const int j = 16 * jb + (lane & 15);
        if (j < R && row < p.M) up[row * R + j] = uacc[jb][e];
      }
  }
}

// Forward with at most 16 tokens, streaming form.  The same tile, lane
// mapping and partial layout as qsplit16_kernel, but no workgroup barrier
// inside the contraction: the workgroup's whole activation slice (16 tokens
// x at most S16_STEPS steps of 128) is loaded into LDS once, behind the
// first W loads, and each wave then streams its 32 W rows through a ring of
// D register stages, dequantizing straight into MFMA operands, at its own
// pace.  The rank-r projection U of column tile 0 is spread over its four
// waves (wave w takes the 32-element slice w of every step, loading its
// adapter fragments in the same ring), and the four partial sums are added
// through LDS at the end.
constexpr int S16_STEPS = 8;
constexpr int XS16 = S16_STEPS * TK2 + 8;          // LDS row stride of the activation slice (bf16)
// the scale window: dwords a row (the slice's S16_STEPS steps of scale bytes)
// and the LDS row stride (a pad of 4 or 16 bytes spreads the rows over the
// banks); MXFP4's one-byte scales need half, which leaves room for four
// workgroups a CU
template <int FMT> constexpr int s16_dw() { return (FMT == QL_FMT_MXFP4 ? 4 : 8) * S16_STEPS / 4; }
template <int FMT> constexpr int s16_stride() { return 4 * s16_dw<FMT>() + (FMT == QL_FMT_MXFP4 ? 4 : 16); }
// waves a SIMD: four for MXFP4 up to rank 16 (its decode needs fewer
// registers; rank 32 would spill), three otherwise
template <int FMT, int R> constexpr int s16_waves() { return FMT == QL_FMT_MXFP4 && R <= 16 ? 4 : 3; }
// scale bytes per row and step of 128 (MXFP4: 4 one-byte entries; the others 8 bytes)
template <int FMT> constexpr int scale_step_bytes() { return FMT == QL_FMT_MXFP4 ? 4 : 8; }

template <int FMT, int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(s16_waves<FMT, R>(), s16_waves<FMT, R>())))
void qstream16_kernel(SplitArgs ga) {
  constexpr int TN = 128, D = 4;
  constexpr int RB = (R + 15) / 16;
  __shared__ __attribute__((aligned(16))) uint16_t xs[16 * XS16];
  constexpr int SW16 = s16_stride<FMT>(), SWD = s16_dw<FMT>();
  __shared__ __attribute__((aligned(16))) uint8_t sw[128 * SW16];   // the tile's scale window
  constexpr int SBS = scale_step_bytes<FMT>();

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bid = (int)blockIdx.x;
  int pi = 0;
  while (pi + 1 < ga.n && bid >= ga.unit0[pi + 1]) ++pi;
  const Params& p = ga.p[pi];
  const int u0 = ga.unit0[pi], nunits = ga.unit0[pi + 1] - u0, nt = ga.ntiles[pi];
  int unit = bid - u0;
  if ((nunits & 7) == 0 && (u0 & 7) == 0) unit = (unit & 7) * (nunits >> 3) + (unit >> 3);
  const int ntile = unit % nt, split = unit / nt;
  const int64_t o0 = (int64_t)ntile * TN;
  const int KT = (int)((p.C + TK2 - 1) / TK2);
  const int kbeg = split * p.sps;
  const int kend = min(KT, kbeg + p.sps);
  const int NKT = kend - kbeg;                       // 1 .. S16_STEPS (checked by the launcher)

  const __amdgpu_buffer_rsrc_t ract = rsrc(p.act, p.M * p.C * 2);
  const int64_t crow = p.K / 2;                     // 4-bit codes
  const __amdgpu_buffer_rsrc_t rcode = rsrc(p.codes + o0 * crow, (p.N - o0) * crow);
  const int64_t srow = scales_per_row<FMT>(p.K);
  const int64_t ssz = scale_bytes<FMT>();
  const __amdgpu_buffer_rsrc_t rscale =
      rsrc((const char*)p.scales + scale_offset<FMT>() + o0 * srow * ssz, (p.N - o0) * srow * ssz);
  const __amdgpu_buffer_rsrc_t rdown = rsrc(p.down, (int64_t)R * p.C * 2);
  float tscale = 0.0f;
  if constexpr (tensor_scale<FMT>()) tscale = reinterpret_cast<const float*>(p.scales)[0];

  const int q = lane >> 4;                           // this lane's group of a step
  const bool rank_tile = ntile == 0;

  // ---- activation slice: every load issued before any W load, so waiting
  // for it leaves the W loads in flight.  Thread t loads row t / 16, pieces
  // t % 16 + 16 s (s < S16_STEPS; pieces outside the slice read zero).
  {
    const int xr = tid >> 4, xp = (tid & 15) * 8;
    uint4 xv[S16_STEPS];
#pragma unroll
    for (int st = 0; st < S16_STEPS; ++st) {
      const int64_t col = (int64_t)(kbeg + st) * TK2 + xp;
      const bool ok = st < NKT && xr < p.M && col < p.C;
      xv[st] = bload16(ract, ok ? (uint32_t)((xr * p.C + col) * 2) : OOB);
    }
    // the scale entries of the tile's 128 rows over the slice (at most 64
    // contiguous bytes a row, 32 for MXFP4), loaded once in dwords (a
    // lane per dword of a row; no load reaches past the window) and
    // read from LDS by each step: per-step scale loads touch 16 rows with 2-8
    // bytes each and cost 7-15 % of the launch
    uint32_t sv[128 * SWD / 256];
#pragma unroll
    for (int i = 0; i < 128 * SWD / 256; ++i) {
      const int pc = tid + 256 * i, row = pc / SWD, dw = pc % SWD;
      const bool ok = 4 * dw < SBS * NKT;
      sv[i] = bload4(rscale, ok ? (uint32_t)(row * srow * ssz + (int64_t)kbeg * SBS + 4 * dw) : OOB);
    }
#pragma unroll
    for (int st = 0; st < S16_STEPS; ++st)
      *reinterpret_cast<uint4*>(xs + xr * XS16 + st * TK2 + xp) = xv[st];
#pragma unroll
    for (int i = 0; i < 128 * SWD / 256; ++i) {
      const int pc = tid + 256 * i;
      *reinterpret_cast<uint32_t*>(sw + (pc / SWD) * SW16 + 4 * (pc % SWD)) = sv[i];
    }
  }

  struct Slot {
    uint4 c[2];                                      // codes of the lane's group in W row blocks 0 and 1
    uint4 ad[RB];                                    // rank tile: adapter fragments of slice `wave` of the step
  };
  Slot ring[D];
  auto issue = [&](Slot& sl, int kt) {
    const bool sv = kt < kend;
    const int64_t c0 = (int64_t)kt * TK2;
    const bool gl = sv && c0 + 32 * q < p.C;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t wrow = 32 * wave + 16 * b + (lane & 15);   // W row, relative to the tile
      sl.c[b] = bload16(rcode, gl ? (uint32_t)(wrow * crow + c0 / 2 + 16 * q) : OOB);
    }
    const int64_t kk = c0 + 32 * wave + 8 * q;
#pragma unroll
    for (int jb = 0; jb < RB; ++jb) {
      const int j = 16 * jb + (lane & 15);
      const bool live = rank_tile && sv && j < R && kk < p.C;
      sl.ad[jb] = bload16(rdown, live ? (uint32_t)((j * p.C + kk) * 2) : OOB);
    }
  };

  f32x4 acc[2], uacc[RB];
#pragma unroll
  for (int b = 0; b < 2; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jb = 0; jb < RB; ++jb) uacc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // step t of the slice (absolute step kbeg + t) from its ring slot; refill
  // the slot with step t + D when `refill`
  auto step = [&](Slot& sl, int t, bool refill) {
    const bool gl = kbeg + t < kend && (int64_t)(kbeg + t) * TK2 + 32 * q < p.C;
    uint4 wb[2][4];
    if constexpr (FMT == QL_FMT_NF4) {
      // The lanes of rows q and q ^ 1 (16 lanes each) hold the two 32-element
      // groups of one NF4 block (64 elements, one absmax) for the same two W
      // rows, so they need the same two lookup tables: each lane builds the
      // table of row block q & 1, and one row swap per table word hands every
      // lane of the pair both (the values are those it would have built).
      const int bq = q & 1;
      const uint8_t* srw = sw + (32 * wave + 16 * bq + (lane & 15)) * SW16;
      const float a = __uint_as_float(*reinterpret_cast<const uint32_t*>(srw + 4 * (2 * t + (q >> 1))));
      uint32_t tl[4], th[4], tb[2][2][4];
      Deq<FMT>::build_table(p.book, gl ? a : 0.0f, tl, th);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const auto sl_ = __builtin_amdgcn_permlane16_swap(tl[w], tl[w], false, false);
        const auto sh_ = __builtin_amdgcn_permlane16_swap(th[w], th[w], false, false);
        tb[0][0][w] = sl_[0]; tb[1][0][w] = sl_[1];   // even row of the pair: row block 0; odd: 1
        tb[0][1][w] = sh_[0]; tb[1][1][w] = sh_[1];
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        Deq<FMT> dq;
        dq.wd[0] = sl.c[b].x; dq.wd[1] = sl.c[b].y; dq.wd[2] = sl.c[b].z; dq.wd[3] = sl.c[b].w;
#pragma unroll
        for (int w = 0; w < 4; ++w) { dq.tl[w] = tb[b][0][w]; dq.th[w] = tb[b][1][w]; }
#pragma unroll
        for (int i = 0; i < 4; ++i) wb[b][i] = dq.piece(i);
      }
    } else {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      // this group's scale entry from the window: group 4 t + q of the slice
      const uint8_t* srw = sw + (32 * wave + 16 * b + (lane & 15)) * SW16;
      uint32_t raw;
      if constexpr (two_byte_scales<FMT>()) raw = *reinterpret_cast<const uint16_t*>(srw + 2 * (4 * t + q));
      else if constexpr (FMT == QL_FMT_MXFP4) raw = srw[4 * t + q];
      else raw = *reinterpret_cast<const uint32_t*>(srw + 4 * (2 * t + (q >> 1)));   // NF4: one fp32 per 64
      WGroup g;
      g.c0 = sl.c[b];
      g.c1 = make_uint4(0, 0, 0, 0);
      g.sraw = raw;
      g.ssh = 0;
      float s0, s1;
      group_scales<FMT>(raw, tscale, s0, s1);
      Deq<FMT> dq;
      dq.prepare(g, gl ? s0 : 0.0f, p.book, gl, gl ? s1 : 0.0f);
#pragma unroll
      for (int i = 0; i < 4; ++i) wb[b][i] = dq.piece(i);
    }
    }
    const uint16_t* xrow = xs + (lane & 15) * XS16 + t * TK2;
    if (rank_tile) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(xrow + 32 * wave + 8 * q);
#pragma unroll
      for (int jb = 0; jb < RB; ++jb)
        uacc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, sl.ad[jb]), uacc[jb], 0, 0, 0);
    }
    if (refill) issue(sl, kbeg + t + D);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(xrow + 32 * q + 8 * s4);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wb[b][s4]), af, acc[b], 0, 0, 0);
    }
  };

#pragma unroll
  for (int u = 0; u < D; ++u) issue(ring[u], kbeg + u);
  lds_barrier();                                     // the activation slice is in LDS

  // whole chunks of D steps run branch-free (static slot indices), so the
  // wait for each slot counts only the loads issued after it; the last
  // chunk issues nothing
  int it = 0;
  for (; it + D < NKT; it += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) step(ring[u], it + u, true);
  }
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (it + u < NKT) step(ring[u], it + u, false);

  mfma_result_guard();
  float* pp = p.part + (int64_t)split * p.M * p.O;
  const int64_t m = lane & 15;
  if (m < p.M) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = o0 + 32 * wave + 16 * b + 4 * q;
      if (col < p.O) *reinterpret_cast<float4*>(pp + m * p.O + col) = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
    }
  }
  if (rank_tile) {
    // waves 1-3 hand their U partials to wave 0 through LDS (the slice is no longer read)
    f32x4* red = reinterpret_cast<f32x4*>(xs);
    lds_barrier();
    if (wave > 0) {
#pragma unroll
      for (int jb = 0; jb < RB; ++jb) red[((wave - 1) * RB + jb) * 64 + lane] = uacc[jb];
    }
    lds_barrier();
    if (wave == 0) {
      float* up = p.upart + (int64_t)split * p.M * R;
#pragma unroll
      for (int jb = 0; jb < RB; ++jb) {
        f32x4 t = uacc[jb];
#pragma unroll
        for (int w = 0; w < 3; ++w) {
          const f32x4 o = red[(w * RB + jb) * 64 + lane];
          t = f32x4{t[0] + o[0], t[1] + o[1], t[2] + o[2], t[3] + o[3]};
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 4 * q + e;
          const int j = 16 * jb + (lane & 15);
          if (j < R && row < p.M) up[row * R + j] = t[e];
        }
      }
    }
  }
}

// steps of 128 per split for the 16-token kernel, from the 64-step plan (never
// more splits than the plan's, so its workspace suffices); 0 if unsuited
inline int split16_plan(const Params& p, int splits, int& sps2) {
  const int KT = (int)((p.C + TK - 1) / TK);
  const int sps = (KT + splits - 1) / splits;
  sps2 = (sps + 1) / 2;
  const int KT2 = (int)((p.C + TK2 - 1) / TK2);
  const int s2 = (KT2 + sps2 - 1) / sps2;
  return s2 <= splits ? s2 : 0;
}

// the streaming 16-token kernel holds the whole activation slice in LDS (at
// most S16_STEPS steps per workgroup; measured 10 % faster per launch than the
// staged kernel, which serves longer slices), and its scale window's rows
// must start 4-byte aligned
template <int FMT> bool stream16_ok(const Params& p, int sps2) {
  return sps2 <= S16_STEPS && (p.K * scale_bytes<FMT>() / (FMT == QL_FMT_NF4 ? 64 : 32)) % 4 == 0;
}

// problems idx[0 .. n) of g on the streaming (stream) or the staged 16-token
// kernel, in steps of 128; each problem's split count set to its 128-step plan
template <int FMT, int R>
hipError_t launch_split16(SplitGroup& g, const int* idx, int n, bool stream, hipStream_t s) {
  static_assert(!byte_codes<FMT>(), "4-bit formats only");
  constexpr size_t smem = 2 * (size_t)(16 * SA2 + 32 * SA2) * sizeof(uint16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)qsplit16_kernel<FMT, R>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  SplitArgs a{};
  a.n = n;
  int32_t units = 0;
  for (int j = 0; j < n; ++j) {
    const int i = idx[j];
    int sps2 = 0;
    const int s2 = split16_plan(g.p[i], g.splits[i], sps2);
    if (s2 == 0) return hipErrorInvalidValue;
    a.p[j] = g.p[i];
    a.p[j].sps = sps2;
    g.splits[i] = s2;                                // the reduction adds this many partials
    a.ntiles[j] = (int32_t)((g.p[i].O + 127) / 128);
    a.unit0[j] = units;
    units += a.ntiles[j] * s2;
  }
  a.unit0[n] = units;
  if (stream)
    hipLaunchKernelGGL((qstream16_kernel<FMT, R>), dim3((unsigned)units), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((qsplit16_kernel<FMT, R>), dim3((unsigned)units), dim3(256), smem, s, a);
  return hipGetLastError();
}

template <int FMT, bool TRANS, int R, int MBK, bool SW>
hipError_t launch_split_m(const SplitGroup& g, hipStream_t s) {
  constexpr int B_EL = split_b_elems<TRANS>();
  constexpr int D_EL = TRANS ? BL_ELEMS : AD_ELEMS;
  constexpr size_t smem = 2 * (size_t)(32 * MBK * SA + B_EL + D_EL) * sizeof(uint16_t) + (SW ? 128 * SWB : 0);
  static_assert(smem <= 80 * 1024, "two workgroups per CU");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)qsplit_kernel<FMT, TRANS, R, MBK, SW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  SplitArgs a{};
  a.n = g.n;
  int32_t units = 0;
  for (int i = 0; i < g.n; ++i) {
    a.p[i] = g.p[i];
    a.ntiles[i] = (int32_t)((g.p[i].O + 127) / 128);
    a.unit0[i] = units;
    units += a.ntiles[i] * g.splits[i];
  }
  a.unit0[g.n] = units;
  hipLaunchKernelGGL((qsplit_kernel<FMT, TRANS, R, MBK, SW>), dim3((unsigned)units), dim3(256), smem, s, a);
  return hipGetLastError();
}

// the general split kernel: 32-row tiles when every token fits in one 32x32
// MFMA block; the scale-window variant when every problem allows it (it
// reads the same scales, so results do not depend on the choice)
template <int FMT, bool TRANS, int R>
hipError_t launch_split_general(const SplitGroup& g, hipStream_t s) {
  if constexpr (!TRANS && FMT != QL_FMT_FP8_E4M3) {
    // the scale window holds 4 sw_dw bytes a row, read in aligned dwords
    // from the one holding a slice's first scale byte (an MXFP4 slice of an
    // odd number of steps starts 2 bytes into it in every other split, so 2
    // more bytes); the rows must start 4-byte aligned
    bool sw = true;
    for (int i = 0; i < g.n; ++i) {
      const int sb = scale_step64_bytes<FMT>() * g.p[i].sps;
      sw = sw && sb + (sb % 4 ? 2 : 0) <= 4 * sw_dw<FMT>() && (g.p[i].K * scale_bytes<FMT>() / (FMT == QL_FMT_NF4 ? 64 : 32)) % 4 == 0;
    }
    if (sw)
      return g.p[0].M <= 32 ? launch_split_m<FMT, TRANS, R, 1, true>(g, s) : launch_split_m<FMT, TRANS, R, 2, true>(g, s);
  }
  return g.p[0].M <= 32 ? launch_split_m<FMT, TRANS, R, 1, false>(g, s) : launch_split_m<FMT, TRANS, R, 2, false>(g, s);
}

template <int FMT, bool TRANS, int R>
hipError_t launch_split(SplitGroup& g, hipStream_t s) {
  // the 16-token kernels hold a ring of four steps of two groups per lane:
  // 4-bit codes fit the registers, one-byte codes (FP8, Q8_0) would spill.
  // Each problem of a group runs the kernel a call of its own would run (the
  // streaming or the staged 16-token kernel, or the general split kernel:
  // their summation orders differ), one launch per kernel, so the group's
  // results stay bitwise those of single calls.
  if constexpr (!TRANS && !byte_codes<FMT>()) {
    if (g.p[0].M <= 16) {
      int ist[MAX_GROUP], isg[MAX_GROUP], ipl[MAX_GROUP], nst = 0, nsg = 0, npl = 0;
      for (int i = 0; i < g.n; ++i) {
        int sps2 = 0;
        const int s2 = split16_plan(g.p[i], g.splits[i], sps2);
        if (s2 == 0) ipl[npl++] = i;
        else if (stream16_ok<FMT>(g.p[i], sps2)) ist[nst++] = i;
        else isg[nsg++] = i;
      }
      hipError_t e = hipSuccess;
      if (nst) e = launch_split16<FMT, R>(g, ist, nst, true, s);
      if (e == hipSuccess && nsg) e = launch_split16<FMT, R>(g, isg, nsg, false, s);
      if (e != hipSuccess || npl == 0) return e;
      SplitGroup gp{};
      gp.n = npl;
      for (int j = 0; j < npl; ++j) {
        gp.p[j] = g.p[ipl[j]];
        gp.splits[j] = g.splits[ipl[j]];
      }
      return launch_split_general<FMT, TRANS, R>(gp, s);
    }
  }
  return launch_split_general<FMT, TRANS, R>(g, s);
}

// Split-contraction reduction and epilogue: per output element the partials
// are summed in split order (deterministic), the LoRA term s . U . up^T is
// added in fp32 (U = sum of its partials), and the sum is rounded once to
// bf16.  Column-slab 0 also writes U (forward) or V (dX).  One thread per 4
// consecutive outputs of MR rows: it loads their up-matrix entries once and
// the partials of all MR rows at once (SPL per row, SPL at least the split
// count; MR SPL = 16 keeps the loads in flight within the same registers), so
// with few splits the up matrix is read once per MR rows instead of per row.
struct ReduceItem {
  const float* part;
  const float* upart;
  const uint16_t* up;
  uint16_t* out;
  float* save;
  int64_t M, O;
  float s;
  int32_t splits, xblocks, blk0;   // blk0: first workgroup of this item
};
struct ReduceArgs {
  ReduceItem it[MAX_GROUP];
  int32_t n;
  int32_t trans;
};

template <int R, int SPL>
__global__ __launch_bounds__(128) void split_reduce_kernel(ReduceArgs ra) {
  constexpr int MR = MAX_SPLITS / SPL;
  __shared__ float us[MR][R];
  const int bid = (int)blockIdx.x;
  int ii = 0;
  while (ii + 1 < ra.n && bid >= ra.it[ii + 1].blk0) ++ii;
  const ReduceItem& I = ra.it[ii];
  const float* __restrict__ part = I.part;
  const float* __restrict__ upart = I.upart;
  const uint16_t* __restrict__ up = I.up;
  uint16_t* __restrict__ out = I.out;
  float* __restrict__ save = I.save;
  const int64_t M = I.M, O = I.O;
  const float s = I.s;
  const bool trans = ra.trans != 0;
  const int local = bid - I.blk0;
  const int bx = local % I.xblocks;
  const int64_t m0 = (int64_t)(local / I.xblocks) * MR;
  const int tid = threadIdx.x;
  // splits past the last read as zero through the resource bounds
  const __amdgpu_buffer_rsrc_t rp = rsrc(part, (int64_t)I.splits * M * O * 4);
  const __amdgpu_buffer_rsrc_t ru = rsrc(upart, (int64_t)I.splits * M * R * 4);
  for (int t = tid; t < MR * R; t += 128) {
    const int r = t / R, j = t % R;
    const int64_t m = m0 + r;
    uint32_t v[SPL];
#pragma unroll
    for (int sp = 0; sp < SPL; ++sp)
      v[sp] = bload4(ru, m < M ? (uint32_t)((((int64_t)sp * M + m) * R + j) * 4) : OOB);
    float u = 0.0f;
#pragma unroll
    for (int sp = 0; sp < SPL; ++sp) u += __uint_as_float(v[sp]);
    if (save && bx == 0 && m < M) save[m * R + j] = u;
    us[r][j] = s * u;
  }
  const int64_t o = (int64_t)bx * 512 + tid * 4;
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
  // all partial loads of the MR rows in flight at once, then summed in split order
  uint4 pv[MR][SPL];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int sp = 0; sp < SPL; ++sp)
      pv[r][sp] = bload16(rp, (live && m0 + r < M) ? (uint32_t)((((int64_t)sp * M + m0 + r) * O + o) * 4) : OOB);
  __syncthreads();
  if (!live) return;
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    const int64_t m = m0 + r;
    if (m < M) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int sp = 0; sp < SPL; ++sp) {
        acc.x += __uint_as_float(pv[r][sp].x); acc.y += __uint_as_float(pv[r][sp].y);
        acc.z += __uint_as_float(pv[r][sp].z); acc.w += __uint_as_float(pv[r][sp].w);
      }
      float l[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int q = 0; q < R / 2; ++q) {
          l[c] += us[r][2 * q] * __uint_as_float(w[c][q] << 16);
          l[c] += us[r][2 * q + 1] * __uint_as_float(w[c][q] & 0xFFFF0000u);
        }
      const uint32_t lo = pack_bf16x2(acc.x + l[0], acc.y + l[1]);
      const uint32_t hi = pack_bf16x2(acc.z + l[2], acc.w + l[3]);
      *reinterpret_cast<uint2*>(out + m * O + o) = make_uint2(lo, hi);
    }
  }
}

// dX reduction with the adapter gradients, at most 32 tokens (all of them in
// every workgroup).  Workgroup g owns dX columns [16 g, 16 g + 16): it adds
// the split partials in split order, adds s . V . A in fp32 (V = sum of its
// split partials, in split order) and rounds once to bf16; it writes the same
// columns of dA = s . V^T x, and rows [nb g, nb g + nb) of dB = s . dY^T U.
// Every sum over tokens runs in token order in fp32 (exact bf16 operands),
// so results are reproducible.
constexpr int RB_TC = 16;       // dX / dA columns per workgroup
constexpr int RB_NB = 64;       // at most this many dB rows per workgroup
constexpr int RB_MAXM = 32;     // tokens (host side: split_path_fuses_grads)

struct ReduceBwdItem {
  const float* part;
  const float* upart;
  const uint16_t* adA;
  uint16_t* dx;
  const uint16_t* x;
  const uint16_t* dy;
  const float* u;
  float* d_a;
  float* d_b;
  int64_t M, K, N, nb;
  float s;
  int32_t splits, accumulate, blk0;
};
struct ReduceBwdArgs {
  ReduceBwdItem it[MAX_GROUP];
  int32_t n;
};

template <int R>
__global__ __launch_bounds__(256) void split_reduce_bwd_kernel(ReduceBwdArgs ra) {
  constexpr int NT = 256, TC = RB_TC, SR = R + 1;
  const int bid = (int)blockIdx.x;
  int ii = 0;
  while (ii + 1 < ra.n && bid >= ra.it[ii + 1].blk0) ++ii;
  const ReduceBwdItem& I = ra.it[ii];
  const float* __restrict__ part = I.part;
  const float* __restrict__ upart = I.upart;
  const uint16_t* __restrict__ adA = I.adA;
  uint16_t* __restrict__ dx = I.dx;
  const uint16_t* __restrict__ x = I.x;
  const uint16_t* __restrict__ dy = I.dy;
  const float* __restrict__ u = I.u;
  float* __restrict__ d_a = I.d_a;
  float* __restrict__ d_b = I.d_b;
  const int64_t M = I.M, K = I.K, N = I.N, nb = I.nb;
  const float s = I.s;
  const int splits = I.splits, accumulate = I.accumulate;
  const int64_t gblk = bid - I.blk0;                 // this workgroup's index within its item
  __shared__ float vs[RB_MAXM * SR];                  // V [m][j]
  __shared__ float ush[RB_MAXM * SR];                 // U [m][j]
  __shared__ float as_[R * TC];                       // A [j][k0 ..]
  __shared__ uint16_t xs[RB_MAXM * TC];               // x [m][k0 ..] (bf16)
  __shared__ uint16_t ys[RB_MAXM * RB_NB];            // dY [m][n0 ..] (bf16)
  const int tid = threadIdx.x;
  const int64_t k0 = gblk * TC, n0 = gblk * nb;
  const int nn = n0 < N ? (int)(n0 + nb <= N ? nb : N - n0) : 0;   // dB rows of this workgroup
  const int kc = k0 < K ? (int)(k0 + TC <= K ? TC : K - k0) : 0;  // dX / dA columns
  const int m_ = (int)M;

  const __amdgpu_buffer_rsrc_t rp = rsrc(part, (int64_t)splits * M * K * 4);
  const __amdgpu_buffer_rsrc_t ru = rsrc(upart, (int64_t)splits * M * R * 4);
  for (int idx = tid; idx < m_ * R; idx += NT) {
    const int m = idx / R, j = idx % R;
    uint32_t v[MAX_SPLITS];
#pragma unroll
    for (int sp = 0; sp < MAX_SPLITS; ++sp) v[sp] = bload4(ru, (uint32_t)((((int64_t)sp * M + m) * R + j) * 4));
    float t = 0.0f;
#pragma unroll
    for (int sp = 0; sp < MAX_SPLITS; ++sp) t += __uint_as_float(v[sp]);
    vs[m * SR + j] = t;
    ush[m * SR + j] = u[m * R + j];
  }
  for (int idx = tid; idx < R * kc; idx += NT) {
    const int j = idx / kc, c = idx % kc;
    as_[j * TC + c] = __uint_as_float((uint32_t)adA[(int64_t)j * K + k0 + c] << 16);
  }
  for (int idx = tid; idx < m_ * kc; idx += NT) {
    const int m = idx / kc, c = idx % kc;
    xs[m * TC + c] = x[(int64_t)m * K + k0 + c];
  }
  for (int idx = tid; idx < m_ * nn; idx += NT) {
    const int m = idx / nn, c = idx % nn;
    ys[m * RB_NB + c] = dy[(int64_t)m * N + n0 + c];
  }
  __syncthreads();

  // dX: 4 consecutive columns of one token per task (K is a multiple of 32)
  for (int t = tid; t < m_ * (kc / 4); t += NT) {
    const int m = t / (kc / 4), c = (t % (kc / 4)) * 4;
    uint4 pv[MAX_SPLITS];
#pragma unroll
    for (int sp = 0; sp < MAX_SPLITS; ++sp)
      pv[sp] = bload16(rp, (uint32_t)((((int64_t)sp * M + m) * K + k0 + c) * 4));
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < MAX_SPLITS; ++sp) {
      acc[0] += __uint_as_float(pv[sp].x); acc[1] += __uint_as_float(pv[sp].y);
      acc[2] += __uint_as_float(pv[sp].z); acc[3] += __uint_as_float(pv[sp].w);
    }
    float l[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float sv = s * vs[m * SR + j];
#pragma unroll
      for (int e = 0; e < 4; ++e) l[e] += sv * as_[j * TC + c + e];
    }
    *reinterpret_cast<uint2*>(dx + m * K + k0 + c) =
        make_uint2(pack_bf16x2(acc[0] + l[0], acc[1] + l[1]), pack_bf16x2(acc[2] + l[2], acc[3] + l[3]));
  }
  // dA[j][k] = s . sum_m V[m][j] x[m][k]
  for (int t = tid; t < R * kc; t += NT) {
    const int j = t / kc, c = t % kc;
    float acc = 0.0f;
    for (int m = 0; m < m_; ++m) acc += vs[m * SR + j] * __uint_as_float((uint32_t)xs[m * TC + c] << 16);
    const int64_t o = (int64_t)j * K + k0 + c;
    const float v = s * acc;
    d_a[o] = accumulate ? d_a[o] + v : v;
  }
  // dB[n][j] = s . sum_m dY[m][n] U[m][j]
  for (int t = tid; t < nn * R; t += NT) {
    const int c = t / R, j = t % R;
    float acc = 0.0f;
    for (int m = 0; m < m_; ++m) acc += __uint_as_float((uint32_t)ys[m * RB_NB + c] << 16) * ush[m * SR + j];
    const int64_t o = (n0 + c) * R + j;
    const float v = s * acc;
    d_b[o] = accumulate ? d_b[o] + v : v;
  }
}

template <int FMT, bool TRANS, int R>
hipError_t launch_path(const SplitGroup& g0, const GradFuse* gf, hipStream_t s) {
  SplitGroup g = g0;                                 // the split launch may set how many partials each problem has
  hipError_t e = launch_split<FMT, TRANS, R>(g, s);
  if (e != hipSuccess) return e;
  if (gf) {
    ReduceBwdArgs ra{};
    ra.n = g.n;
    int32_t blocks = 0;
    for (int i = 0; i < g.n; ++i) {
      const Params& p = g.p[i];
      // enough workgroups for the dX columns and for at most RB_NB dB rows each
      const int64_t nblk = std::max((p.K + RB_TC - 1) / RB_TC, (p.N + RB_NB - 1) / RB_NB);
      ReduceBwdItem& I = ra.it[i];
      I.part = p.part;
      I.upart = p.upart;
      I.adA = p.up;
      I.dx = p.out;
      I.x = gf[i].x;
      I.dy = p.act;
      I.u = gf[i].u;
      I.d_a = gf[i].d_a;
      I.d_b = gf[i].d_b;
      I.M = p.M;
      I.K = p.K;
      I.N = p.N;
      I.nb = (p.N + nblk - 1) / nblk;
      I.s = p.s;
      I.splits = g.splits[i];
      I.accumulate = gf[i].accumulate;
      I.blk0 = blocks;
      blocks += (int32_t)nblk;
    }
    hipLaunchKernelGGL(split_reduce_bwd_kernel<R>, dim3((unsigned)blocks), dim3(256), 0, s, ra);
    return hipGetLastError();
  }
  ReduceArgs ra{};
  ra.n = g.n;
  ra.trans = TRANS ? 1 : 0;
  int32_t maxsp = 1;
  for (int i = 0; i < g.n; ++i) maxsp = std::max(maxsp, (int32_t)g.splits[i]);
  const int spl = maxsp <= 2 ? 2 : maxsp <= 4 ? 4 : maxsp <= 8 ? 8 : MAX_SPLITS;
  const int mr = MAX_SPLITS / spl;                   // rows per workgroup
  int32_t blocks = 0;
  for (int i = 0; i < g.n; ++i) {
    const Params& p = g.p[i];
    ReduceItem& I = ra.it[i];
    I.part = p.part;
    I.upart = p.upart;
    I.up = p.up;
    I.out = p.out;
    I.save = p.save;
    I.M = p.M;
    I.O = p.O;
    I.s = p.s;
    I.splits = g.splits[i];
    I.xblocks = (int32_t)((p.O + 511) / 512);
    I.blk0 = blocks;
    blocks += I.xblocks * (int32_t)((p.M + mr - 1) / mr);
  }
  switch (spl) {
    case 2: hipLaunchKernelGGL((split_reduce_kernel<R, 2>), dim3((unsigned)blocks), dim3(128), 0, s, ra); break;
    case 4: hipLaunchKernelGGL((split_reduce_kernel<R, 4>), dim3((unsigned)blocks), dim3(128), 0, s, ra); break;
    case 8: hipLaunchKernelGGL((split_reduce_kernel<R, 8>), dim3((unsigned)blocks), dim3(128), 0, s, ra); break;
    default: hipLaunchKernelGGL((split_reduce_kernel<R, MAX_SPLITS>), dim3((unsigned)blocks), dim3(128), 0, s, ra); break;
  }
  return hipGetLastError();
}

template <int FMT, bool TRANS>
hipError_t launch_r(const SplitGroup& g, int r, const GradFuse* gf, hipStream_t s) {
  switch (r) {
    case 8: return launch_path<FMT, TRANS, 8>(g, gf, s);
    case 16: return launch_path<FMT, TRANS, 16>(g, gf, s);
    default: return launch_path<FMT, TRANS, 32>(g, gf, s);
  }
}

}  // namespace

static_assert(MAX_SPLITS == 16, "split_reduce_kernel: rows x splits per thread add up to 16");

SplitPlan split_plan(bool trans, int64_t m, int64_t n, int64_t k, int r) {
  SplitPlan pl;
  if (m <= 0 || m > SMALL_M) return pl;
  const int64_t O = trans ? k : n, C = trans ? n : k;
  const int64_t KT = (C + TK - 1) / TK;
  const int64_t tn = (O + STN - 1) / STN;
  // at most 256 units (column tiles x splits) a launch, 512 for the 16-token
  // forward: fewer splits write and re-read fewer partial sums, and measured
  // 1-6 % faster layer steps at 16-64 tokens (a cap of 128, or 1024 for dX,
  // was slower); the 16-token forward's streaming kernel wants the shorter slices
  const int64_t cap = (!trans && m <= 16) ? 512 : 256;
  int64_t sp = std::min<int64_t>({std::max<int64_t>(1, KT / 4), cap / tn, (int64_t)MAX_SPLITS});
  if (sp < 1) sp = 1;
  // a wide dX output (more than 128 column tiles at two splits: fewer units
  // than CUs) takes up to 512 units, so every CU gets work (Llama-3.1-8B's
  // down projection at 16-64 tokens: 224 -> 448 units, the step 2-3 % shorter)
  if (trans && tn * sp < 256)
    sp = std::max<int64_t>(sp, std::min<int64_t>({std::max<int64_t>(1, KT / 4), 512 / tn, (int64_t)MAX_SPLITS}));
  pl.sps = (int)((KT + sp - 1) / sp);
  pl.splits = (int)((KT + pl.sps - 1) / pl.sps);
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  pl.upart_off = al((size_t)pl.splits * m * O * 4);
  pl.total = pl.upart_off + al((size_t)pl.splits * m * r * 4);
  return pl;
}


// up to 32 tokens one fused launch beats the two (measured); at 64 the
// per-token loops of the fused kernel cost more than the launch it saves
bool split_path_fuses_grads(int64_t m) { return m > 0 && m <= 32; }

bool split_path_tokens(int64_t m) { return m > 0 && m <= SMALL_M; }

hipError_t launch_split_path(int fmt, bool trans, int r, const SplitGroup& g, const GradFuse* gf, hipStream_t s) {
  if (g.n < 1 || g.n > MAX_GROUP) return hipErrorInvalidValue;
  if (gf && (!trans || !split_path_fuses_grads(g.p[0].M))) return hipErrorInvalidValue;
  for (int i = 1; i < g.n; ++i)
    if (g.p[i].M != g.p[0].M) return hipErrorInvalidValue;
  switch (fmt) {
    case QL_FMT_Q4_0: return trans ? launch_r<QL_FMT_Q4_0, true>(g, r, gf, s) : launch_r<QL_FMT_Q4_0, false>(g, r, gf, s);
    case QL_FMT_NF4: return trans ? launch_r<QL_FMT_NF4, true>(g, r, gf, s) : launch_r<QL_FMT_NF4, false>(g, r, gf, s);
    case QL_FMT_MXFP4: return trans ? launch_r<QL_FMT_MXFP4, true>(g, r, gf, s) : launch_r<QL_FMT_MXFP4, false>(g, r, gf, s);
    case QL_FMT_Q8_0: return trans ? launch_r<QL_FMT_Q8_0, true>(g, r, gf, s) : launch_r<QL_FMT_Q8_0, false>(g, r, gf, s);
    case QL_FMT_NVFP4: return trans ? launch_r<QL_FMT_NVFP4, true>(g, r, gf, s) : launch_r<QL_FMT_NVFP4, false>(g, r, gf, s);
    default: return trans ? launch_r<QL_FMT_FP8_E4M3, true>(g, r, gf, s) : launch_r<QL_FMT_FP8_E4M3, false>(g, r, gf, s);
  }
}

}  // namespace ql
