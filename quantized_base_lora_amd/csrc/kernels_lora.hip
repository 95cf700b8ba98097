// a8 / a9: adapter gradients, reduced over the M tokens.
//
//   dA = s . V^T . x   [r, K]      dB = s . dY^T . U   [N, r]
//
// Both have the form out[p][j] = s . sum_m X[m][p] . Q[m][j] with X a bf16
// activation ([M, K] or [M, N]) and Q an fp32 rank-r projection ([M, r]).
// grad_partial computes per-partition sums on 16x16x32 bf16 MFMAs: X tiles
// sit in LDS as [m][p] and reach the MFMA A operand through LDS transpose
// reads; Q is split into a high and a low bf16 term (about 16 bits kept) and
// read the same way.  The M range is cut into a fixed number of partitions
// and grad_reduce adds the partials in partition order, so the result does
// not depend on scheduling (no float atomics).
#include "common.h"

namespace ql {
namespace {

constexpr int NT = 256;
constexpr int TP = 128;         // p columns per workgroup
constexpr int TMC = 64;         // m rows per step
constexpr int SX = TP + 32;     // X tile stride (bf16)
constexpr int SQ = 32 + 16;     // Q tile stride (bf16), up to 32 columns

__global__ __launch_bounds__(NT) void transpose_rn_kernel(const uint16_t* __restrict__ b, int64_t n,
                                                          int r, uint16_t* __restrict__ bt) {
  int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (i >= n * r) return;
  int64_t row = i / r;
  int j = (int)(i % r);
  bt[(int64_t)j * n + row] = b[i];
}

// out[m][j] = sum_c x[m][c] * p[j][c]; one workgroup per row.
template <int R>
__global__ __launch_bounds__(NT) void down_proj_kernel(const uint16_t* __restrict__ x, int64_t c,
                                                       const uint16_t* __restrict__ pm,
                                                       float* __restrict__ out) {
  __shared__ float red[NT / 64][R];
  const int64_t row = blockIdx.x;
  float acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = 0.0f;
  for (int64_t k = threadIdx.x; k < c; k += NT) {
    float xv = __uint_as_float((uint32_t)x[row * c + k] << 16);
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j] = fmaf(xv, __uint_as_float((uint32_t)pm[(int64_t)j * c + k] << 16), acc[j]);
  }
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc[j] += __shfl_xor(acc[j], off);
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int j = 0; j < R; ++j) red[threadIdx.x >> 6][j] = acc[j];
  __syncthreads();
  if (threadIdx.x < R) {
    const int j = threadIdx.x;
    out[row * R + j] = (red[0][j] + red[1][j]) + (red[2][j] + red[3][j]);
  }
}

template <int R>
__global__ __launch_bounds__(NT) void grad_partial_kernel(const uint16_t* __restrict__ x, int64_t m,
                                                          int64_t pdim, const float* __restrict__ q,
                                                          int64_t chunk, float* __restrict__ part) {
  constexpr int RB = (R + 15) / 16;
  __shared__ __attribute__((aligned(16))) uint16_t Xs[TMC * SX];
  __shared__ __attribute__((aligned(16))) uint16_t Qh[TMC * SQ];
  __shared__ __attribute__((aligned(16))) uint16_t Ql[TMC * SQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t p0 = (int64_t)blockIdx.x * TP;
  const int64_t mq0 = (int64_t)blockIdx.y * chunk;
  const int64_t mq1 = mq0 + chunk < m ? mq0 + chunk : m;

  // columns R..16*RB-1 of the Q tiles stay zero
  for (int i = tid; i < TMC * SQ; i += NT) { Qh[i] = 0; Ql[i] = 0; }

  f32x4 acc[2][RB];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int jb = 0; jb < RB; ++jb) acc[a][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int xr = tid >> 4, xc = (tid & 15) * 8;      // X: rows xr + 16 i, 8 columns
  constexpr int QPT = R / 4;                         // Q floats per thread
  const int qr = tid >> 2, qc = (tid & 3) * QPT;

  for (int64_t mc = mq0; mc < mq1; mc += TMC) {
    uint4 xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = mc + xr + 16 * i, col = p0 + xc;
      xv[i] = (row < mq1 && col < pdim) ? *reinterpret_cast<const uint4*>(x + row * pdim + col)
                                        : make_uint4(0, 0, 0, 0);
    }
    float qv[QPT];
    {
      const int64_t row = mc + qr;
#pragma unroll
      for (int t = 0; t < QPT; ++t) qv[t] = (row < mq1) ? q[row * R + qc + t] : 0.0f;
    }
    __syncthreads();   // previous step's readers are done
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(Xs + (xr + 16 * i) * SX + xc) = xv[i];
#pragma unroll
    for (int t = 0; t < QPT; ++t) {
      const __bf16 h = (__bf16)qv[t];
      const __bf16 l = (__bf16)(qv[t] - (float)h);
      Qh[qr * SQ + qc + t] = __builtin_bit_cast(uint16_t, h);
      Ql[qr * SQ + qc + t] = __builtin_bit_cast(uint16_t, l);
    }
    __syncthreads();
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      const int b = lane >> 4, sl = lane & 15;
      const int rbase = 32 * kp + 8 * b + (sl >> 2);
      bf16x8 bh[RB], bl[RB];
#pragma unroll
      for (int jb = 0; jb < RB; ++jb) {
        const int col = 16 * jb + 4 * (sl & 3);
        s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(Qh + rbase * SQ + col));
        s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(Qh + (rbase + 4) * SQ + col));
        s16x4 l0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(Ql + rbase * SQ + col));
        s16x4 l1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(Ql + (rbase + 4) * SQ + col));
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        s16x8 th = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        s16x8 tl = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        bh[jb] = __builtin_bit_cast(bf16x8, th);
        bl[jb] = __builtin_bit_cast(bf16x8, tl);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int col = 16 * (2 * wave + a) + 4 * (sl & 3);
        s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(Xs + rbase * SX + col));
        s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(Xs + (rbase + 4) * SX + col));
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        s16x8 tx = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        bf16x8 af = __builtin_bit_cast(bf16x8, tx);
#pragma unroll
        for (int jb = 0; jb < RB; ++jb) {
          acc[a][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bh[jb], acc[a][jb], 0, 0, 0);
          acc[a][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bl[jb], acc[a][jb], 0, 0, 0);
        }
      }
    }
  }
  // partial[q][p][j]: lane holds column j = 16 jb + lane%16, rows 4 (lane/16) + e
  float* dst = part + (int64_t)blockIdx.y * pdim * R;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int jb = 0; jb < RB; ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t prow = p0 + 16 * (2 * wave + a) + 4 * (lane >> 4) + e;
        const int j = 16 * jb + (lane & 15);
        if (prow < pdim && j < R) dst[prow * R + j] = acc[a][jb][e];
      }
}

__global__ __launch_bounds__(NT) void grad_reduce_kernel(const float* __restrict__ part, int nparts,
                                                         int64_t pdim, int r, float s,
                                                         float* __restrict__ out, int transpose_out,
                                                         int accumulate) {
  int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (i >= pdim * r) return;
  float sum = 0.0f;
  for (int q = 0; q < nparts; ++q) sum += part[(int64_t)q * pdim * r + i];
  const int64_t pi = i / r;
  const int j = (int)(i % r);
  const int64_t o = transpose_out ? (int64_t)j * pdim + pi : i;
  const float v = s * sum;
  out[o] = accumulate ? out[o] + v : v;
}

inline unsigned blocks(int64_t n) { return (unsigned)((n + NT - 1) / NT); }

}  // namespace

int32_t grad_parts(int64_t m) {
  int64_t p = (m + 255) / 256;
  if (p < 1) p = 1;
  if (p > 64) p = 64;
  return (int32_t)p;
}

hipError_t launch_transpose_rn(const uint16_t* b, int64_t n, int32_t r, uint16_t* bt, hipStream_t s) {
  hipLaunchKernelGGL(transpose_rn_kernel, dim3(blocks(n * r)), dim3(NT), 0, s, b, n, r, bt);
  return hipGetLastError();
}

hipError_t launch_down_proj(const uint16_t* x, int64_t m, int64_t c, const uint16_t* p, int32_t r,
                            float* out, hipStream_t s) {
  if (m == 0) return hipSuccess;
  switch (r) {
    case 8: hipLaunchKernelGGL(down_proj_kernel<8>, dim3((unsigned)m), dim3(NT), 0, s, x, c, p, out); break;
    case 16: hipLaunchKernelGGL(down_proj_kernel<16>, dim3((unsigned)m), dim3(NT), 0, s, x, c, p, out); break;
    default: hipLaunchKernelGGL(down_proj_kernel<32>, dim3((unsigned)m), dim3(NT), 0, s, x, c, p, out); break;
  }
  return hipGetLastError();
}

hipError_t launch_grad_partial(const uint16_t* x, int64_t m, int64_t pdim, const float* v, int32_t r,
                               float* part, int32_t nparts, hipStream_t s) {
  int64_t chunk = (m + nparts - 1) / nparts;
  chunk = (chunk + TMC - 1) / TMC * TMC;
  dim3 grid((unsigned)((pdim + TP - 1) / TP), (unsigned)nparts);
  switch (r) {
    case 8: hipLaunchKernelGGL(grad_partial_kernel<8>, grid, dim3(NT), 0, s, x, m, pdim, v, chunk, part); break;
    case 16: hipLaunchKernelGGL(grad_partial_kernel<16>, grid, dim3(NT), 0, s, x, m, pdim, v, chunk, part); break;
    default: hipLaunchKernelGGL(grad_partial_kernel<32>, grid, dim3(NT), 0, s, x, m, pdim, v, chunk, part); break;
  }
  return hipGetLastError();
}

hipError_t launch_grad_reduce(const float* part, int32_t nparts, int64_t pdim, int32_t r, float s,
                              float* out, bool transpose_out, bool accumulate, hipStream_t st) {
  hipLaunchKernelGGL(grad_reduce_kernel, dim3(blocks(pdim * r)), dim3(NT), 0, st, part, nparts, pdim, r,
                     s, out, transpose_out ? 1 : 0, accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace ql
