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
// the same contraction loop on 16x16x32 MFMAs; the "up" product is one more
// short MFMA contraction over 2r bf16 columns (s.U split into a high and a
// low bf16 term, so the epilogue keeps ~16 bits of U) before the single
// bf16 rounding of the output.  The base is never written.
//
// Dequantized tile values are bf16_RNE(fl32 value): Q4_0 (q - 8) * d is exact
// in fp32; NF4 uses a per-thread 16-entry table of bf16_RNE(fl32(c[q] * a))
// looked up with byte permutes; FP8 decodes with the hardware E4M3 convert
// and multiplies by the tensor scale.
//
// Tiling (gfx950, wave64): a 256-thread workgroup owns a 256 x 128 output
// tile; its four waves each own 128 x 64 (4 x 2 MFMA 32x32x16 blocks).  The
// contraction advances 64 at a time through double-buffered LDS, so the
// dequantization and LDS stores for tile t+1 overlap the MFMAs of tile t,
// and global loads for tile t+2 are in flight meanwhile.
#include "common.h"

namespace ql {
namespace {

constexpr int TM = 256, TN = 128, TK = 64;
constexpr int NTHREADS = 256;
constexpr int SA = TK + 8;          // act tile row stride (bf16): 144 B, conflict-free b128 reads
constexpr int SBF = TK + 8;         // forward W tile [TN][TK] stride
constexpr int SBT = TN + 32;        // dX W tile [TK][TN] stride: 320 B rows for transpose reads
constexpr int A_ELEMS = TM * SA;
constexpr int BF_ELEMS = TN * SBF;
constexpr int BT_ELEMS = TK * SBT;

struct Book { float c[16]; };

typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// ------------------------------------------------------------------ W tile registers
// Each thread handles one 32-element group of one row of W per contraction tile.
template <int FMT>
struct WRegs {
  uint4 c0;          // 4-bit: 16 bytes of codes; fp8: first 16 bytes
  uint4 c1;          // fp8: second 16 bytes
  float scale;       // Q4_0: d; NF4: absmax; FP8: unused (tensor scale)
  bool valid;
};

template <int FMT>
__device__ __forceinline__ void load_w(WRegs<FMT>& r, const uint8_t* __restrict__ codes,
                                       const void* __restrict__ scales, int64_t n, int64_t kg,
                                       int64_t N, int64_t K) {
  r.valid = (n < N) && (kg * 32 < K);
  if (!r.valid) return;
  if constexpr (FMT == QL_FMT_FP8_E4M3) {
    const uint4* p = reinterpret_cast<const uint4*>(codes + n * K + kg * 32);
    r.c0 = p[0];
    r.c1 = p[1];
  } else {
    r.c0 = *reinterpret_cast<const uint4*>(codes + n * (K / 2) + kg * 16);
    if constexpr (FMT == QL_FMT_Q4_0) {
      uint16_t h = reinterpret_cast<const uint16_t*>(scales)[n * (K / 32) + kg];
      uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
      float v = (e == 0) ? (float)m * 5.9604644775390625e-08f
                         : __uint_as_float(((e + 112u) << 23) | (m << 13));
      r.scale = (h & 0x8000) ? -v : v;
    } else {
      r.scale = reinterpret_cast<const float*>(scales)[n * (K / 64) + (kg >> 1)];
    }
  }
}

// NF4 lookup: 4 codes (one per byte, 0..15) -> 2 dwords of bf16 pairs, from
// byte-plane tables tl/th (entry e's low / high byte at byte e%4 of word e/4).
__device__ __forceinline__ void nf4_lookup4(uint32_t q4, const uint32_t* tl, const uint32_t* th,
                                            uint32_t& out01, uint32_t& out23) {
  uint32_t s3 = q4 & 0x07070707u;
  uint32_t s8 = ((q4 >> 1) & 0x04040404u) | 0x03020100u;
  uint32_t l = __builtin_amdgcn_perm(__builtin_amdgcn_perm(tl[3], tl[2], s3),
                                     __builtin_amdgcn_perm(tl[1], tl[0], s3), s8);
  uint32_t h = __builtin_amdgcn_perm(__builtin_amdgcn_perm(th[3], th[2], s3),
                                     __builtin_amdgcn_perm(th[1], th[0], s3), s8);
  out01 = __builtin_amdgcn_perm(h, l, 0x05010400u);
  out23 = __builtin_amdgcn_perm(h, l, 0x07030602u);
}

// Dequantize one 32-element group into 16 dwords (bf16 pairs in element order).
template <int FMT>
__device__ __forceinline__ void dequant_group(const WRegs<FMT>& r, const Book& book, float tscale,
                                              uint32_t* out) {
  if (!r.valid) {
#pragma unroll
    for (int i = 0; i < 16; ++i) out[i] = 0u;
    return;
  }
  if constexpr (FMT == QL_FMT_FP8_E4M3) {
    uint32_t wd[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], false);
      f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[i], true);
      out[2 * i] = pack_bf16x2(a.x * tscale, a.y * tscale);
      out[2 * i + 1] = pack_bf16x2(b.x * tscale, b.y * tscale);
    }
  } else {
    uint32_t wd[4] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w};
    if constexpr (FMT == QL_FMT_Q4_0) {
      const float d = r.scale, nd8 = -8.0f * r.scale;    // (q - 8) d = fma(q, d, -8d), exact
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t lo = wd[i] & 0x0F0F0F0Fu, hi = (wd[i] >> 4) & 0x0F0F0F0Fu;
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
      for (int i = 0; i < 8; ++i) pr[i] = pack_bf16x2(book.c[2 * i] * r.scale, book.c[2 * i + 1] * r.scale);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        tl[w] = __builtin_amdgcn_perm(pr[2 * w + 1], pr[2 * w], 0x06040200u);
        th[w] = __builtin_amdgcn_perm(pr[2 * w + 1], pr[2 * w], 0x07050301u);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t lo = wd[i] & 0x0F0F0F0Fu, hi = (wd[i] >> 4) & 0x0F0F0F0Fu;
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
  const uint16_t* down;  // [R, C]
  const uint16_t* up;    // fwd: [N, R]; dX: [R, K]
  uint16_t* out;         // [M, O]
  float* save;           // [M, R] or null
  int64_t M, N, K, C, O;
  float s;
  Book book;
};

__device__ __forceinline__ uint4 ld_act(const uint16_t* __restrict__ act, int64_t row, int64_t col,
                                        int64_t M, int64_t C) {
  if (row < M && col < C) return *reinterpret_cast<const uint4*>(act + row * C + col);
  return make_uint4(0, 0, 0, 0);
}

template <int FMT, bool TRANS, int R>
__global__ __launch_bounds__(NTHREADS) void qgemm_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  constexpr int B_ELEMS = TRANS ? BT_ELEMS : BF_ELEMS;
  constexpr int STAGE = A_ELEMS + B_ELEMS;
  constexpr int RB = (R + 15) / 16;                  // 16-column blocks of the rank-r projection

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t o0 = (int64_t)blockIdx.x * TN;       // output column tile
  const int64_t m0 = (int64_t)blockIdx.y * TM;       // output row tile
  const int64_t KT = (p.C + TK - 1) / TK;
  float tscale = 0.0f;
  if constexpr (FMT == QL_FMT_FP8_E4M3) tscale = reinterpret_cast<const float*>(p.scales)[0];

  // ---- per-thread load coordinates
  const int arow = tid >> 3, acol = (tid & 7) * 8;   // act: 8 rows apart by 32
  // W group handled by this thread: forward (row n, group kg); dX (row n = contraction)
  const int wr = TRANS ? (tid >> 2) : (tid >> 1);
  const int wgi = TRANS ? (tid & 3) : (tid & 1);

  uint4 areg[8];
  WRegs<FMT> wreg;
  uint4 dreg[2][RB];                                   // down-projection B fragments (16 x 32 per kp)

  auto issue_loads = [&](int64_t kt) {
    const int64_t c0 = kt * TK;
#pragma unroll
    for (int i = 0; i < 8; ++i) areg[i] = ld_act(p.act, m0 + 32 * i + arow, c0 + acol, p.M, p.C);
    if constexpr (TRANS) {
      load_w<FMT>(wreg, p.codes, p.scales, c0 + wr, (o0 >> 5) + wgi, p.N, p.K);
    } else {
      load_w<FMT>(wreg, p.codes, p.scales, o0 + wr, (c0 >> 5) + wgi, p.N, p.K);
    }
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
      for (int jb = 0; jb < RB; ++jb) {
        const int j = 16 * jb + (lane & 15);
        const int64_t c = c0 + 32 * kp + 8 * (lane >> 4);
        dreg[kp][jb] = (j < R && c < p.C) ? *reinterpret_cast<const uint4*>(p.down + (int64_t)j * p.C + c)
                                          : make_uint4(0, 0, 0, 0);
      }
  };

  auto store_tile = [&](int stage) {
    uint16_t* As = smem + stage * STAGE;
    uint16_t* Bs = As + A_ELEMS;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(As + (32 * i + arow) * SA + acol) = areg[i];
    uint32_t v[16];
    dequant_group<FMT>(wreg, p.book, tscale, v);
    uint16_t* dst = TRANS ? (Bs + wr * SBT + wgi * 32) : (Bs + wr * SBF + wgi * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(dst + 8 * i) = make_uint4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  f32x4 uacc[4][RB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jb = 0; jb < RB; ++jb) uacc[i][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 dcur[2][RB];

  issue_loads(0);
  store_tile(0);
#pragma unroll
  for (int kp = 0; kp < 2; ++kp)
#pragma unroll
    for (int jb = 0; jb < RB; ++jb) dcur[kp][jb] = dreg[kp][jb];
  if (KT > 1) issue_loads(1);
  __syncthreads();

  for (int64_t kt = 0; kt < KT; ++kt) {
    const int cur = (int)(kt & 1);
    const uint16_t* As = smem + cur * STAGE;
    const uint16_t* Bs = As + A_ELEMS;

    // -- main MFMAs on the current stage
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (128 * wm + 32 * i + (lane & 31)) * SA + ks * 16 + 8 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (TRANS) {
          const int b = lane >> 4, sl = lane & 15;
          const int g = b >> 1;
          const int col = 64 * wn + 32 * j + 16 * (b & 1) + 4 * (sl & 3);
          s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(Bs + (ks * 16 + 8 * g + (sl >> 2)) * SBT + col));
          s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(Bs + (ks * 16 + 8 * g + 4 + (sl >> 2)) * SBT + col));
          typedef short s16x8 __attribute__((ext_vector_type(8)));
          s16x8 t = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          bfr[j] = __builtin_bit_cast(bf16x8, t);
        } else {
          bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + (64 * wn + 32 * j + (lane & 31)) * SBF + ks * 16 + 8 * (lane >> 5));
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    // -- rank-r down projection on this wave's 64 rows
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(As + (64 * wave + 16 * i + (lane & 15)) * SA + 32 * kp + 8 * (lane >> 4));
#pragma unroll
        for (int jb = 0; jb < RB; ++jb)
          uacc[i][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, dcur[kp][jb]), uacc[i][jb], 0, 0, 0);
      }
    }
    // -- stage the next tile while the MFMAs drain
    if (kt + 1 < KT) {
      store_tile(cur ^ 1);
#pragma unroll
      for (int kp = 0; kp < 2; ++kp)
#pragma unroll
        for (int jb = 0; jb < RB; ++jb) dcur[kp][jb] = dreg[kp][jb];
      if (kt + 2 < KT) issue_loads(kt + 2);
    }
    __syncthreads();
  }

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
          if (p.save && blockIdx.x == 0 && m0 + row < p.M) p.save[(m0 + row) * R + j] = u;
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
    if (o0 + col < p.O)
      v = TRANS ? p.up[(int64_t)j * p.K + o0 + col] : p.up[(o0 + col) * R + j];
    Bx[col * SX + j] = v;
    Bx[col * SX + R + j] = v;
  }
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < (2 * R) / 16; ++ks) {
    bf16x8 af[4], bfr[2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(Ax + (128 * wm + 32 * i + (lane & 31)) * SX + ks * 16 + 8 * (lane >> 5));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(Bx + (64 * wn + 32 * j + (lane & 31)) * SX + ks * 16 + 8 * (lane >> 5));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  }
  // ---- store bf16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + 128 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int64_t col = o0 + 64 * wn + 32 * j + (lane & 31);
        if (row < p.M && col < p.O) {
          const __bf16 h = (__bf16)acc[i][j][e];
          p.out[row * p.O + col] = __builtin_bit_cast(uint16_t, h);
        }
      }
}

template <int FMT, bool TRANS, int R>
hipError_t launch_t(const Params& p, hipStream_t s) {
  constexpr int B_ELEMS = TRANS ? BT_ELEMS : BF_ELEMS;
  constexpr size_t smem = 2 * (size_t)(A_ELEMS + B_ELEMS) * sizeof(uint16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)qgemm_kernel<FMT, TRANS, R>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((unsigned)((p.O + TN - 1) / TN), (unsigned)((p.M + TM - 1) / TM));
  hipLaunchKernelGGL((qgemm_kernel<FMT, TRANS, R>), grid, dim3(NTHREADS), smem, s, p);
  return hipGetLastError();
}

template <int FMT, bool TRANS>
hipError_t launch_r(const Params& p, int r, hipStream_t s) {
  switch (r) {
    case 8: return launch_t<FMT, TRANS, 8>(p, s);
    case 16: return launch_t<FMT, TRANS, 16>(p, s);
    default: return launch_t<FMT, TRANS, 32>(p, s);
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
