// a3 / a6 for the FP8 E4M3 base on the fp8 matrix cores (more than 64
// tokens), and the rank-r projection that these GEMMs take precomputed.
//
// The activation (x forward, dY for dX) arrives split per row into two E4M3
// terms, act ~= s_m (hi + lo / 16), s_m a power of two (a1); W's codes are
// used raw.  Each 64-deep contraction step issues, per 32 x 32 output block,
// one scaled 32x32x64 f8f6f4 MFMA on hi (unit scales) and one on lo (E8M0
// scale 2^-4 on that operand), into one fp32 accumulator.  The epilogue
// multiplies by s_w s_m (tensor scale times row scale), adds s . U . up^T on
// bf16 MFMAs (s . U split into a high and a low bf16 term, as in the bf16
// GEMM) and rounds once to bf16.
//
// dX reads W through the same [row of W][column] LDS tile with 8-bit
// transpose reads (ds_read_b64_tr_b8), so no transposed copy of the base is
// made.  512 threads, two waves per SIMD, a 256 x TN output tile per
// workgroup, double-buffered LDS.  The two waves of a SIMD take turns (a
// ping-pong schedule): while one issues the MFMAs of a step on fragments it
// holds in registers, the other stages data and reads its next fragments, so
// the matrix cores do not wait for LDS traffic.  Counted in GPU cycles this
// took the forward GEMM from 62 % to 80 % MFMA busy; at that load the chip's
// power limit lowers the clock (≈ 1.95 -> 1.65 GHz in the counter runs), so
// wall time fell by less than the cycles.
#include <algorithm>

#include "common.h"
#include "device.h"

namespace ql {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int TM = 256, TK = 64, NT = 512;
constexpr int SB = 80;                 // act planes and forward W tile: row stride in bytes

template <int TN, bool TRANS> struct Shape8 {
  static constexpr int WAVES_N = 2;                  // wave blocks 64 x TN/2: the two activation planes are the larger operand
  static constexpr int WAVES_M = 8 / WAVES_N;
  static constexpr int WM = TM / WAVES_M, WN = TN / WAVES_N;
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int SBT = TN + 32;              // dX W tile [TK][TN]: row stride in bytes (transposing reads conflict-free)
  static constexpr int A_BYTES = TM * SB;          // one activation plane
  static constexpr int W_BYTES = TRANS ? TK * SBT : TN * SB;
  static constexpr int STAGE = 2 * A_BYTES + W_BYTES;
  static constexpr int CPR = TN / 16;              // dX: pieces per W-tile row
};

struct P8 {
  const uint8_t* hi;       // [M, C] E4M3
  const uint8_t* lo;       // [M, C] E4M3, 16x finer
  const float* rs;         // [M] row scales (powers of two)
  const uint8_t* codes;    // W [N, K] E4M3
  const float* wscale;     // [1] tensor scale of W
  const float* u;          // [M, R] rank-r projection (U forward, V for dX)
  const uint16_t* up;      // forward: B [N, R]; dX: A [R, K]
  uint16_t* out;           // [M, O] bf16
  int64_t M, N, K, C, O;
  float s;
};

__device__ __forceinline__ v8i frag_b128x2(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  v8i r = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  return r;
}

__device__ __forceinline__ v2i tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)p);
}

// problems of one launch: workgroups [tile0[g], tile0[g + 1]) own the tiles
// of problem g (tile0[n] = grid size)
struct Args8 {
  P8 p[QL_GROUP_MAX];
  int32_t tile0[QL_GROUP_MAX + 1];
  int32_t n;
};

template <bool TRANS, int R, int TN>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void qgemm8_kernel(Args8 ga) {
  using S = Shape8<TN, TRANS>;
  extern __shared__ __attribute__((aligned(16))) uint8_t sm8[];
  constexpr int MB = S::MB, NB = S::NB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / S::WAVES_N, wn = wave % S::WAVES_N;

  // problem and tile: each problem's tiles in contiguous runs per XCD
  // (workgroups go round-robin over the 8 XCDs; a run of a multiple of 8
  // workgroups starting at a multiple of 8 keeps that order)
  const int bid = (int)blockIdx.x;
  int pi = 0;
  while (pi + 1 < ga.n && bid >= ga.tile0[pi + 1]) ++pi;
  const P8& p = ga.p[pi];
  const int t0 = ga.tile0[pi], tiles = ga.tile0[pi + 1] - t0;
  const int nt = (int)((p.O + TN - 1) / TN);
  const int mt = tiles / nt;
  int t = bid - t0;
  if ((tiles & 7) == 0 && (t0 & 7) == 0) t = (t & 7) * (tiles >> 3) + (t >> 3);
  // tiles in groups of GM row blocks, column by column within a group, so the
  // workgroups an XCD runs at once share W panels as well as activation panels
  constexpr int GM = 2;
  const int grp = t / (GM * nt), fm = grp * GM;
  const int gm = mt - fm < GM ? mt - fm : GM;
  const int tg = t - grp * GM * nt;
  const int64_t o0 = (int64_t)(tg / gm) * TN;
  const int64_t m0 = (int64_t)(fm + tg % gm) * TM;
  const int KT = (int)((p.C + TK - 1) / TK);

  const __amdgpu_buffer_rsrc_t rhi = rsrc(p.hi + m0 * p.C, (p.M - m0) * p.C);
  const __amdgpu_buffer_rsrc_t rlo = rsrc(p.lo + m0 * p.C, (p.M - m0) * p.C);
  const __amdgpu_buffer_rsrc_t rcode =
      TRANS ? rsrc(p.codes + o0, p.N * p.K - o0) : rsrc(p.codes + o0 * p.K, (p.N - o0) * p.K);

  // ---- ping-pong schedule.  Waves 0-3 (group 0) and 4-7 (group 1), one of
  // each per SIMD, alternate between a memory phase (store the staged half of
  // the next step, issue the loads of the half after it, read this step's
  // fragments into registers) and a compute phase (this step's MFMAs on those
  // registers); group 1 runs one phase behind group 0 and every phase ends at
  // a workgroup barrier, so while one wave of a SIMD issues MFMAs the other
  // moves data.  Group 0 stages the hi plane and the first half of the W tile,
  // group 1 the lo plane and the second half.
  const int pg = __builtin_amdgcn_readfirstlane(tid >> 8);   // wave-uniform, in a scalar register
  const int gt = tid & 255;
  constexpr int WP = TRANS ? TK * S::CPR : TN * 4;          // 16-byte W pieces a step
  constexpr int WH = WP / NT;                               // per thread of a group (half each)
  static_assert(WP % NT == 0, "W tile pieces split evenly over the two groups");
  const __amdgpu_buffer_rsrc_t rpl = pg ? rlo : rhi;
  int arow[4], acol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = gt + 256 * i;
    arow[i] = q >> 2;
    acol[i] = (q & 3) * 16;
  }
  int wrow[WH], wcol[WH];
#pragma unroll
  for (int i = 0; i < WH; ++i) {
    const int q = pg * (WP / 2) + gt + 256 * i;
    wrow[i] = TRANS ? q / S::CPR : q >> 2;
    wcol[i] = TRANS ? (q % S::CPR) * 16 : (q & 3) * 16;
  }
  // per-thread load offsets and limits, formed once: the loop then reads no
  // field of the problem table (a field reloaded from it in the loop waits for
  // this wave's LDS traffic as well, the two sharing one counter)
  const int32_t C32 = (int32_t)p.C, K32 = (int32_t)p.K;
  uint32_t aoff[4];
  int32_t alim[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    aoff[i] = (uint32_t)(arow[i] * C32 + acol[i]);
    alim[i] = C32 - acol[i];                     // column c0 + acol < C
  }
  uint32_t woff[WH];
  int32_t wlim[WH];
#pragma unroll
  for (int i = 0; i < WH; ++i) {
    woff[i] = (uint32_t)(wrow[i] * K32 + wcol[i]);
    // forward: column c0 + wcol < K; dX: the piece's columns o0 + wcol lie inside K (all steps)
    wlim[i] = TRANS ? (o0 + wcol[i] < p.K ? 0x7FFFFFFF : 0) : K32 - wcol[i];
  }
  uint32_t kstep = TRANS ? (uint32_t)(TK * K32) : (uint32_t)TK;   // W offset advance per step
  asm volatile("" : "+s"(kstep));
  auto load = [&](int kt, uint4 (&da)[4], uint4 (&dw)[WH]) {
    const int32_t c0 = kt * TK;
#pragma unroll
    for (int i = 0; i < 4; ++i) da[i] = bload16(rpl, c0 < alim[i] ? aoff[i] + (uint32_t)c0 : OOB);
    // W rows past N lie outside the resource (dX: rows c0 + wrow; forward: o0 + wrow)
#pragma unroll
    for (int i = 0; i < WH; ++i) dw[i] = bload16(rcode, c0 < wlim[i] ? woff[i] + (uint32_t)kt * kstep : OOB);
  };
  auto store = [&](uint8_t* st, const uint4 (&da)[4], const uint4 (&dw)[WH]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(st + pg * S::A_BYTES + arow[i] * SB + acol[i]) = da[i];
#pragma unroll
    for (int i = 0; i < WH; ++i)
      *reinterpret_cast<uint4*>(st + 2 * S::A_BYTES + wrow[i] * (TRANS ? S::SBT : SB) + wcol[i]) = dw[i];
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  v8i wf[NB], hf[MB], lf[MB];
  auto read_frags = [&](const uint8_t* st) {
    const uint8_t* Hs = st;
    const uint8_t* Ls = st + S::A_BYTES;
    const uint8_t* Ws = st + 2 * S::A_BYTES;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if constexpr (TRANS) {
        // lane: output column (row of the A operand) within the block, 32 contraction rows
        const int b = lane >> 4, s = lane & 15;
        const int col = S::WN * wn + 32 * j + 16 * (b & 1) + 8 * (s & 1);
        const int row = 32 * (b >> 1) + (s >> 1);
        const v2i t0 = tr8(Ws + (row + 0) * S::SBT + col);
        const v2i t1 = tr8(Ws + (row + 8) * S::SBT + col);
        const v2i t2 = tr8(Ws + (row + 16) * S::SBT + col);
        const v2i t3 = tr8(Ws + (row + 24) * S::SBT + col);
        v8i r = {t0.x, t0.y, t1.x, t1.y, t2.x, t2.y, t3.x, t3.y};
        wf[j] = r;
      } else {
        wf[j] = frag_b128x2(Ws + (S::WN * wn + 32 * j + (lane & 31)) * SB + 32 * (lane >> 5));
      }
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int off = (S::WM * wm + 32 * i + (lane & 31)) * SB + 32 * (lane >> 5);
      hf[i] = frag_b128x2(Hs + off);
      lf[i] = frag_b128x2(Ls + off);
    }
  };
  auto mfmas = [&]() {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], hf[i], acc[i][j], 0, 0, 0, 127, 0, 127);
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], lf[i], acc[i][j], 0, 0, 0, 127, 0, 123);
      }
  };

  // epilogue operands: row scales, the tile's rows of U (fp32, contiguous)
  // and its slice of the up matrix (forward B rows o0 .. o0+TN; dX
  // A[j][o0 .. o0+TN]), loaded in the last memory phase
  constexpr int UQ = TM * R / 4, UQT = UQ / NT > 0 ? UQ / NT : 1;   // 16-byte U pieces
  constexpr int UPP = TN * R / 8;
  constexpr int UPT = (UPP + NT - 1) / NT;
  float rsv[MB];
  uint4 uv[UQT], upv[UPT];
  auto load_epilogue = [&]() {
    const __amdgpu_buffer_rsrc_t rrs = rsrc(p.rs + m0, (p.M - m0) * 4);
    const __amdgpu_buffer_rsrc_t ru = rsrc(p.u + m0 * R, (p.M - m0) * R * 4);
    const __amdgpu_buffer_rsrc_t rup = TRANS ? rsrc(p.up, (int64_t)R * p.K * 2)
                                             : rsrc(p.up + o0 * R, (p.N - o0) * R * 2);
#pragma unroll
    for (int i = 0; i < MB; ++i)
      rsv[i] = __uint_as_float(bload4(rrs, (uint32_t)((S::WM * wm + 32 * i + (lane & 31)) * 4)));
#pragma unroll
    for (int u = 0; u < UQT; ++u) {
      const int q = tid + NT * u;
      uv[u] = bload16(ru, q < UQ ? (uint32_t)(q * 16) : OOB);
    }
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int q = tid + NT * u;
      uint32_t off = OOB;
      if constexpr (TRANS) {
        const int j = q / (TN / 8), c = (q % (TN / 8)) * 8;
        if (q < UPP && o0 + c < p.K) off = (uint32_t)((j * p.K + o0 + c) * 2);
      } else {
        if (q < UPP) off = (uint32_t)(q * 16);
      }
      upv[u] = bload16(rup, off);
    }
  };

  // prologue: step 0 whole in LDS, this group's half of step 1 staged
  uint4 ra[4], rw[WH];
  {
    uint4 a0[4], w0[WH];
    load(0, a0, w0);
    if (KT > 1) load(1, ra, rw);
    store(sm8, a0, w0);
  }
  lds_barrier();
  // every wave passes the same number of barriers: group 1 one extra before
  // the loop, group 0 one extra after it
  if (pg) __builtin_amdgcn_s_barrier();
  for (int kt = 0; kt < KT; ++kt) {
    // memory phase
    if (kt + 1 < KT) store(sm8 + ((kt + 1) & 1) * S::STAGE, ra, rw);
    if (kt + 2 < KT) load(kt + 2, ra, rw);
    if (kt + 1 == KT) load_epilogue();
    read_frags(sm8 + (kt & 1) * S::STAGE);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // compute phase
    mfmas();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!pg) __builtin_amdgcn_s_barrier();

  mfma_result_guard();
  // ---- epilogue: scales, then s . U . up^T on bf16 MFMAs, one rounding to bf16
  const float sw = *p.wscale;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const float sc = sw * rsv[i];                    // rows past M read 0
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] *= sc;
  }
  constexpr int SX = 2 * R + 8;
  uint16_t* Ax = reinterpret_cast<uint16_t*>(sm8);
  uint16_t* Bx = Ax + TM * SX;
  // s.U split into high and low bf16 parts (rows past M read 0)
#pragma unroll
  for (int u = 0; u < UQT; ++u) {
    const int q = tid + NT * u;
    if (q < UQ) {
      const int row = q / (R / 4), j = (q % (R / 4)) * 4;
      const float uu[4] = {__uint_as_float(uv[u].x), __uint_as_float(uv[u].y), __uint_as_float(uv[u].z),
                           __uint_as_float(uv[u].w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float su = p.s * uu[e];
        const __bf16 h = (__bf16)su;
        const __bf16 l = (__bf16)(su - (float)h);
        Ax[row * SX + j + e] = __builtin_bit_cast(uint16_t, h);
        Ax[row * SX + R + j + e] = __builtin_bit_cast(uint16_t, l);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int q = tid + NT * u;
    if (q < UPP) {
      if constexpr (TRANS) {
        const int j = q / (TN / 8), c = (q % (TN / 8)) * 8;
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
  // bf16 stores: lanes l and l + 32 trade column halves (v_permlane32_swap)
  // so each writes 8 consecutive columns of its row with one 16-byte store
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
        const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
        const int64_t col = o0 + S::WN * wn + 32 * j + 8 * (2 * pr + hl);
        if (row < p.M && col < p.O)
          *reinterpret_cast<uint4*>(p.out + row * p.O + col) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
      }
  }
}

template <bool TRANS, int R, int TN>
hipError_t launch8_t(Args8& a, hipStream_t s) {
  using S = Shape8<TN, TRANS>;
  constexpr size_t smem = 2 * (size_t)S::STAGE;
  static_assert(smem <= 160 * 1024, "LDS budget");
  static_assert((size_t)(TM + TN) * (2 * R + 8) * 2 <= smem, "epilogue LDS");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)qgemm8_kernel<TRANS, R, TN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  int32_t tiles = 0;
  for (int i = 0; i < a.n; ++i) {
    a.tile0[i] = tiles;
    tiles += (int32_t)(((a.p[i].O + TN - 1) / TN) * ((a.p[i].M + TM - 1) / TM));
  }
  a.tile0[a.n] = tiles;
  hipLaunchKernelGGL((qgemm8_kernel<TRANS, R, TN>), dim3((unsigned)tiles), dim3(NT), smem, s, a);
  return hipGetLastError();
}

// 256-wide tiles when the launch has at least one workgroup per CU of them
template <bool TRANS, int R>
hipError_t launch8_w(Args8& a, hipStream_t s) {
  int64_t tiles256 = 0;
  for (int i = 0; i < a.n; ++i) tiles256 += ((a.p[i].O + 255) / 256) * ((a.p[i].M + TM - 1) / TM);
  if (tiles256 >= 256) return launch8_t<TRANS, R, 256>(a, s);
  return launch8_t<TRANS, R, 128>(a, s);
}

// ------------------------------------------------------------------ rank-r projection
// out[m][j] = sum_c act[m][c] D(c, j), D(c, j) = A[j][c] (A layout, [R, C]) or
// B[c][j] (B layout, [C, R]), fp32 accumulation on 32x32x16 bf16 MFMAs.  A
// workgroup owns 32 rows; its eight waves (two per SIMD) take the 64-wide
// contraction chunks round robin, each with the loads of its next three
// chunks in flight, and their partial sums are added in wave order (fixed).
// Global loads are coalesced: eight lanes cover one 128-byte row piece of a
// chunk (activation rows, and A rows in the A layout), four loads a chunk,
// and each wave puts them through its own LDS tile, from which it reads the
// MFMA fragments (one wave's LDS operations complete in order, so no barrier
// is needed).  Loading the fragments straight from global memory touched 32
// rows with 32 bytes each per load instruction and ran 1.5x slower.  A
// B-layout chunk is contiguous already and goes through the wave's LDS tile
// with transposing reads.
constexpr int RP_NW = 8;        // waves per rank-r projection workgroup

// up to QL_GROUP_MAX projections of one token count, rank and layout in one
// launch; each workgroup finds its problem in a table in the kernel
// arguments.  Workgroup b runs row block 8 (s / n) + b % 8 of problem s % n,
// s = b / 8: workgroups are dealt to the eight XCDs in turn, so the n
// problems' workgroups for one row block run side by side on one XCD, and
// problems that project the same activation (q|k|v, gate|up) read it from
// that XCD's L2 instead of once each from memory.
struct RprojJob {
  const uint16_t* act;
  const uint16_t* d;
  float* out;
  int64_t C;
};
struct RprojJobs {
  RprojJob j[QL_GROUP_MAX];
  int32_t n;
  int32_t per;           // row blocks of 32 per problem
  int64_t M;
};

template <int R, bool ALAYOUT>
__global__ __launch_bounds__(64 * RP_NW) void rproj_kernel(RprojJobs jobs) {
  const int bid = (int)blockIdx.x;
  const int slot = bid >> 3;
  const int ji = slot % jobs.n;
  const int blk = (slot / jobs.n) * 8 + (bid & 7);
  if (blk >= jobs.per) return;                       // whole workgroup, before any barrier
  const uint16_t* __restrict__ act = jobs.j[ji].act;
  const uint16_t* __restrict__ d = jobs.j[ji].d;
  float* __restrict__ out = jobs.j[ji].out;
  const int64_t M = jobs.M, C = jobs.j[ji].C;
  constexpr int SLD = 48, SX = 72, D = 3, NW = RP_NW, NT = 64 * NW;
  constexpr int DP = ALAYOUT ? 4 : R / 8;            // adapter pieces per lane and chunk
  __shared__ __attribute__((aligned(16))) uint16_t xt[NW][32 * SX];                       // activation chunk
  __shared__ __attribute__((aligned(16))) uint16_t dl[NW][ALAYOUT ? 32 * SX : 64 * SLD];  // adapter chunk
  __shared__ float red[NW][32][33];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the chunk loop is not divergent
  const int64_t m0 = (int64_t)blk * 32;
  const __amdgpu_buffer_rsrc_t ract = rsrc(act + m0 * C, (M - m0) * C * 2);
  const __amdgpu_buffer_rsrc_t rd = rsrc(d, (int64_t)R * C * 2);
  if constexpr (!ALAYOUT)
    for (int i = lane; i < 64 * SLD; i += 64) dl[wave][i] = 0;   // columns past r stay zero
  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  // wave w takes chunks c0 = 64 w + 64 NW i; a ring of D chunks of loads is in
  // flight (chunks past C read zero through out-of-range offsets)
  const int nit = (int)((C - 64 * wave + 64 * NW - 1) / (64 * NW));
  const int prow = lane >> 3, pcol = (lane & 7) * 8;   // coalesced piece: rows prow + 8 i, 8 columns
  struct Slot {
    uint4 a[4];
    uint4 d[DP];
  };
  Slot ring[D];
  auto issue = [&](Slot& sl, int it) {
    const int64_t c0 = 64 * (int64_t)wave + 64 * NW * (int64_t)it;
    const int64_t k = c0 + pcol;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = prow + 8 * i;
      sl.a[i] = bload16(ract, k < C ? (uint32_t)((row * C + k) * 2) : OOB);
      if constexpr (ALAYOUT) sl.d[i] = bload16(rd, (row < R && k < C) ? (uint32_t)((row * C + k) * 2) : OOB);
    }
    if constexpr (!ALAYOUT) {
#pragma unroll
      for (int t = 0; t < DP; ++t) {
        const int q = lane + 64 * t;
        const int row = q / (R / 8), col = (q % (R / 8)) * 8;
        sl.d[t] = bload16(rd, c0 + row < C ? (uint32_t)(((c0 + row) * R + col) * 2) : OOB);
      }
    }
  };
  auto consume = [&](const Slot& sl) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(&xt[wave][(prow + 8 * i) * SX + pcol]) = sl.a[i];
      if constexpr (ALAYOUT) *reinterpret_cast<uint4*>(&dl[wave][(prow + 8 * i) * SX + pcol]) = sl.d[i];
    }
    if constexpr (!ALAYOUT) {
      // the chunk of B [C, R] through this wave's LDS tile
#pragma unroll
      for (int t = 0; t < DP; ++t) {
        const int q = lane + 64 * t;
        const int row = q / (R / 8), col = (q % (R / 8)) * 8;
        *reinterpret_cast<uint4*>(&dl[wave][row * SLD + col]) = sl.d[t];
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int fo = (lane & 31) * SX + 16 * ks + 8 * (lane >> 5);
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(&xt[wave][fo]);
      bf16x8 df;
      if constexpr (ALAYOUT) {
        df = *reinterpret_cast<const bf16x8*>(&dl[wave][fo]);
      } else {
        const int b = lane >> 4, sl_ = lane & 15;
        const int col = 16 * (b & 1) + 4 * (sl_ & 3);
        const int row = 16 * ks + 8 * (b >> 1) + (sl_ >> 2);
        df = tr16x8(&dl[wave][row * SLD + col], &dl[wave][(row + 4) * SLD + col]);
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, df, acc, 0, 0, 0);
    }
  };
  // slot by slot in refill order, and a scheduling barrier after each refill,
  // so that each chunk waits only for its own loads
#pragma unroll
  for (int u = 0; u < D; ++u) {
    issue(ring[u], u);
    __builtin_amdgcn_sched_barrier(0);
  }
  int it = 0;
  for (; it + D <= nit; it += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      consume(ring[u]);
      issue(ring[u], it + u + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (it + u < nit) consume(ring[u]);
  mfma_result_guard();
  // lane: column j = lane & 31, rows 8 (e / 4) + 4 (lane / 32) + e % 4
#pragma unroll
  for (int e = 0; e < 16; ++e) red[wave][8 * (e / 4) + 4 * (lane >> 5) + (e % 4)][lane & 31] = acc[e];
  __syncthreads();
  for (int i = tid; i < 32 * R; i += NT) {
    const int m = i / R, j = i % R;
    if (m0 + m < M) {
      float t = red[0][m][j];
#pragma unroll
      for (int w = 1; w < NW; ++w) t += red[w][m][j];   // wave order
      out[(m0 + m) * R + j] = t;
    }
  }
}

}  // namespace

hipError_t launch_rproj_group(const Rproj* pr, int n, int64_t m, bool a_layout, int32_t r, hipStream_t s) {
  if (m == 0 || n == 0) return hipSuccess;
  if (n > QL_GROUP_MAX) return hipErrorInvalidValue;
  RprojJobs a{};
  a.n = n;
  a.M = m;
  a.per = (int32_t)((m + 31) / 32);
  for (int i = 0; i < n; ++i) a.j[i] = RprojJob{pr[i].act, pr[i].d, pr[i].out, pr[i].c};
  const dim3 grid((unsigned)((a.per + 7) / 8 * 8 * n));
#define QL_RPROJ(RR)                                                                                 \
  if (a_layout) hipLaunchKernelGGL((rproj_kernel<RR, true>), grid, dim3(64 * RP_NW), 0, s, a);      \
  else hipLaunchKernelGGL((rproj_kernel<RR, false>), grid, dim3(64 * RP_NW), 0, s, a);
  switch (r) {
    case 8: QL_RPROJ(8) break;
    case 16: QL_RPROJ(16) break;
    default: QL_RPROJ(32) break;
  }
#undef QL_RPROJ
  return hipGetLastError();
}

hipError_t launch_rproj(const uint16_t* act, int64_t m, int64_t c, const uint16_t* d, bool a_layout, int32_t r,
                        float* out, hipStream_t s) {
  const Rproj pr{act, d, out, c};
  return launch_rproj_group(&pr, 1, m, a_layout, r, s);
}

hipError_t launch_qgemm8(const Gemm8Call* c, int n, hipStream_t s) {
  if (n < 1 || n > QL_GROUP_MAX) return hipErrorInvalidValue;
  // longest contraction first (stable), so its tiles start first
  int order[QL_GROUP_MAX];
  for (int i = 0; i < n; ++i) order[i] = i;
  auto clen = [&](int i) { return c[i].trans ? c[i].w->n_out : c[i].w->k_in; };
  std::stable_sort(order, order + n, [&](int x, int y) { return clen(x) > clen(y); });
  Args8 a{};
  a.n = n;
  for (int i = 0; i < n; ++i) {
    const Gemm8Call& ci = c[order[i]];
    if (ci.trans != c[0].trans || ci.r != c[0].r) return hipErrorInvalidValue;
    P8& p = a.p[i];
    p.hi = ci.hi;
    p.lo = ci.lo;
    p.rs = ci.rs;
    p.codes = ci.w->codes;
    p.wscale = reinterpret_cast<const float*>(ci.w->scales);
    p.u = ci.u;
    p.up = ci.up;
    p.out = ci.out;
    p.M = ci.m;
    p.N = ci.w->n_out;
    p.K = ci.w->k_in;
    p.C = ci.trans ? p.N : p.K;
    p.O = ci.trans ? p.K : p.N;
    p.s = ci.s;
  }
  switch (c[0].r) {
    case 8: return c[0].trans ? launch8_w<true, 8>(a, s) : launch8_w<false, 8>(a, s);
    case 16: return c[0].trans ? launch8_w<true, 16>(a, s) : launch8_w<false, 16>(a, s);
    default: return c[0].trans ? launch8_w<true, 32>(a, s) : launch8_w<false, 32>(a, s);
  }
}

}  // namespace ql
