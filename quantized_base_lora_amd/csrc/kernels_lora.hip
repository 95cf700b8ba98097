// a8 / a9: adapter gradients, reduced over the M tokens.
//
//   dA = s . V^T . x   [r, K]      dB = s . dY^T . U   [N, r]
//
// Both have the form out[p][j] = s . sum_m X[m][p] . Q[m][j] with X a bf16
// activation ([M, K] or [M, N]) and Q an fp32 rank-r projection ([M, r]);
// one launch serves both, for up to QL_GROUP_MAX calls at once (a problem
// table in the kernel arguments).  A workgroup owns 64 columns p (128 at
// rank 32) and one of P fixed partitions of M; it streams its rows through
// LDS in steps of 64 (loads running ahead in a ring of register sets) and
// accumulates on 16x16x32 bf16
// MFMAs, with X reaching the A operand through LDS transpose reads and Q
// split into a high and a low bf16 term (about 16 bits kept).  Each
// workgroup writes its partial sums; a second launch adds the P partials in
// partition order, so the sum order is fixed per shape and the result
// bitwise reproducible (no float atomics).  The hand-off between the two is
// a kernel boundary: an in-kernel "last workgroup reduces" scheme would need
// an agent-scope fence per workgroup, which on a multi-XCD part writes back
// and invalidates the XCD's L2 each time.
#include "common.h"
#include "device.h"

namespace ql {
namespace {

constexpr int NT = 256;
constexpr int TMC = 64;         // m rows per step
constexpr int SQ = 32 + 16;     // Q tile stride (bf16), up to 32 columns
constexpr int CHUNK = 512;      // rows per partition
// p columns per workgroup: 16 per wave up to rank 16; 32 per wave (two MFMA
// column blocks sharing each Q fragment) at rank 32, which halves the Q loads,
// splits and LDS reads per X byte
template <int R> constexpr int grad_cpw() { return R == 32 ? 2 : 1; }
template <int R> constexpr int grad_tp() { return 64 * grad_cpw<R>(); }

struct GradProb {
  const uint16_t* x;
  const float* q;
  float* out;
  float* part;
  int64_t pdim;
  int32_t transpose_out;
  float s;
  int32_t accumulate;
  int32_t blk0;          // first workgroup of this problem's run (below)
  int32_t rblk0;         // first workgroup of this problem in the reduction launch
  int32_t nblk;          // workgroups of this problem: tiles x partitions
  int32_t nrun, ridx;    // size of its run, its index in the run
};
// Problems that read the same input with the same width (dA of calls with one
// activation: q|k|v, gate|up) form a run.  Workgroup b of a run of n takes
// workgroup 8 (s / n) + b % 8 of its problem s % n, s = b / 8: workgroups are
// dealt to the eight XCDs in turn, so the run's workgroups for one tile and
// partition run side by side on one XCD and read the input from its L2
// instead of once each from memory.

// dA and dB of up to QL_GROUP_MAX calls with one token count and rank: the
// problems of a launch share m, the partition plan and r.
constexpr int MAX_PROB = 2 * QL_GROUP_MAX;
struct GradArgs {
  GradProb prob[MAX_PROB];
  int32_t nprob;
  int64_t m;
  int64_t chunk;
  int32_t nparts;
  int32_t r;
};

// four workgroups per CU (register budget of four waves per SIMD) for ranks up
// to 16; rank 32 needs more registers (three)
template <int R> constexpr int grad_waves() { return R <= 16 ? 4 : 3; }

template <int R>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(grad_waves<R>(), grad_waves<R>())))
void grad_kernel(GradArgs a) {
  constexpr int RB = (R + 15) / 16;
  constexpr int QPT = R / 4;                         // Q floats per thread per step
  constexpr int CPW = grad_cpw<R>(), TP = grad_tp<R>();
  constexpr int SX = TP + 32;                        // X tile stride (bf16)
  constexpr int XPT = TP / 32;                       // X pieces (8 columns) per thread per step
  __shared__ __attribute__((aligned(16))) uint16_t Xs[TMC * SX];
  __shared__ __attribute__((aligned(16))) uint16_t Qh[TMC * SQ];
  __shared__ __attribute__((aligned(16))) uint16_t Ql[TMC * SQ];

  const int bid = (int)blockIdx.x;
  int pi = 0;                                        // this workgroup's problem (uniform)
  while (pi + 1 < a.nprob && bid >= a.prob[pi + 1].blk0) ++pi;   // the last problem of its run
  int local = bid - a.prob[pi].blk0;
  if (a.prob[pi].nrun > 1) {
    const int nrun = a.prob[pi].nrun, slot = local >> 3;
    pi += slot % nrun - a.prob[pi].ridx;
    local = (slot / nrun) * 8 + (local & 7);
    if (local >= a.prob[pi].nblk) return;             // whole workgroup, before any barrier
  }
  const GradProb& pr = a.prob[pi];
  const int part = local % a.nparts;                 // partition of M
  const int64_t p0 = (int64_t)(local / a.nparts) * TP;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t mq0 = (int64_t)part * a.chunk;
  const int64_t mq1 = mq0 + a.chunk < a.m ? mq0 + a.chunk : a.m;

  for (int i = tid; i < TMC * SQ; i += NT) { Qh[i] = 0; Ql[i] = 0; }

  f32x4 acc[CPW][RB];
#pragma unroll
  for (int cb = 0; cb < CPW; ++cb)
#pragma unroll
    for (int jb = 0; jb < RB; ++jb) acc[cb][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // X: rows xr + (256 / (TP / 8)) i, 8 columns at xc
  constexpr int XROWS = NT / (TP / 8);
  const int xr = tid / (TP / 8), xc = (tid % (TP / 8)) * 8;
  const int qr = tid >> 2, qc = (tid & 3) * QPT;

  // loads run DEPTH - 1 steps ahead of the LDS stores (a ring of register sets).
  // Reads past the partition or past the last column go to an out-of-range
  // buffer offset and return zero, so no loaded value is inspected at issue.
  // ring depth that fits the register budget (the rank-32 tile's X pieces
  // are twice as many)
  constexpr int DEPTH = R == 32 ? 2 : 3;
  const __amdgpu_buffer_rsrc_t rx = rsrc(pr.x + mq0 * pr.pdim, (mq1 - mq0) * pr.pdim * 2);
  const __amdgpu_buffer_rsrc_t rq = rsrc(pr.q + mq0 * R, (mq1 - mq0) * R * 4);
  const int NS = (int)((mq1 - mq0 + TMC - 1) / TMC);
  uint4 xv[DEPTH][XPT];
  uint32_t qv[DEPTH][QPT];
  auto load = [&](int slot, int step) {
    const int64_t r0 = (int64_t)step * TMC;            // first row of the step, partition-relative
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int64_t row = r0 + xr + XROWS * i, col = p0 + xc;
      xv[slot][i] = bload16(rx, col < pr.pdim ? (uint32_t)((row * pr.pdim + col) * 2) : OOB);
    }
    const uint32_t qoff = (uint32_t)(((r0 + qr) * R + qc) * 4);
#pragma unroll
    for (int t = 0; t < QPT; t += 4) {
      if constexpr (QPT >= 4) {
        const uint4 v = bload16(rq, qoff + 4 * t);
        qv[slot][t] = v.x; qv[slot][t + 1] = v.y; qv[slot][t + 2] = v.z; qv[slot][t + 3] = v.w;
      }
    }
    if constexpr (QPT < 4) {
#pragma unroll
      for (int t = 0; t < QPT; ++t) qv[slot][t] = bload4(rq, qoff + 4 * t);
    }
  };
  auto step = [&](int u) {
    lds_barrier();                                    // previous step's readers are done
#pragma unroll
    for (int i = 0; i < XPT; ++i) *reinterpret_cast<uint4*>(Xs + (xr + XROWS * i) * SX + xc) = xv[u][i];
    // this thread's QPT consecutive Q values as hi / lo bf16 pairs, packed into
    // 32-bit words and stored 8 bytes at a time (4 for rank 8)
    uint32_t hw[QPT / 2], lw[QPT / 2];
#pragma unroll
    for (int t = 0; t < QPT; t += 2) {
      const float q0 = __uint_as_float(qv[u][t]), q1 = __uint_as_float(qv[u][t + 1]);
      const float h0 = (float)(__bf16)q0, h1 = (float)(__bf16)q1;
      hw[t / 2] = pack_bf16x2(h0, h1);
      lw[t / 2] = pack_bf16x2(q0 - h0, q1 - h1);
    }
    if constexpr (QPT == 2) {
      *reinterpret_cast<uint32_t*>(Qh + qr * SQ + qc) = hw[0];
      *reinterpret_cast<uint32_t*>(Ql + qr * SQ + qc) = lw[0];
    } else {
#pragma unroll
      for (int t = 0; t < QPT / 2; t += 2) {
        *reinterpret_cast<uint2*>(Qh + qr * SQ + qc + 2 * t) = make_uint2(hw[t], hw[t + 1]);
        *reinterpret_cast<uint2*>(Ql + qr * SQ + qc + 2 * t) = make_uint2(lw[t], lw[t + 1]);
      }
    }
    lds_barrier();
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      const int b = lane >> 4, sl = lane & 15;
      const int rbase = 32 * kp + 8 * b + (sl >> 2);
      bf16x8 af[CPW];
#pragma unroll
      for (int cb = 0; cb < CPW; ++cb) {
        const int xcol = 16 * (CPW * wave + cb) + 4 * (sl & 3);
        af[cb] = tr16x8(Xs + rbase * SX + xcol, Xs + (rbase + 4) * SX + xcol);
      }
#pragma unroll
      for (int jb = 0; jb < RB; ++jb) {
        const int col = 16 * jb + 4 * (sl & 3);
        const bf16x8 th = tr16x8(Qh + rbase * SQ + col, Qh + (rbase + 4) * SQ + col);
        const bf16x8 tl = tr16x8(Ql + rbase * SQ + col, Ql + (rbase + 4) * SQ + col);
#pragma unroll
        for (int cb = 0; cb < CPW; ++cb) {
          acc[cb][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[cb], th, acc[cb][jb], 0, 0, 0);
          acc[cb][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[cb], tl, acc[cb][jb], 0, 0, 0);
        }
      }
    }
  };

#pragma unroll
  for (int u = 0; u < DEPTH - 1; ++u) load(u, u);
  // whole chunks of DEPTH steps run branch-free with static ring slots
  int st = 0;
  for (; st + DEPTH <= NS; st += DEPTH) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      load((u + DEPTH - 1) % DEPTH, st + u + DEPTH - 1);
      step(u);
    }
  }
#pragma unroll
  for (int u = 0; u < DEPTH; ++u) {
    if (st + u < NS) {
      load((u + DEPTH - 1) % DEPTH, st + u + DEPTH - 1);
      step(u);
    }
  }
  mfma_result_guard();
  // lane holds column j = 16 jb + lane%16, rows 4 (lane/16) + e.  With one
  // partition the sum is complete: scale and write the result (out[p][j] or
  // out[j][p]); otherwise write partial[q][p][j] for the reduction launch.
  const bool final_out = a.nparts == 1;
  float* dst = pr.part + (int64_t)part * pr.pdim * R;
#pragma unroll
  for (int cb = 0; cb < CPW; ++cb)
#pragma unroll
    for (int jb = 0; jb < RB; ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t prow = p0 + 16 * (CPW * wave + cb) + 4 * (lane >> 4) + e;
        const int j = 16 * jb + (lane & 15);
        if (prow < pr.pdim && j < R) {
          if (final_out) {
            const int64_t o = pr.transpose_out ? (int64_t)j * pr.pdim + prow : prow * R + j;
            const float v = pr.s * acc[cb][jb][e];
            pr.out[o] = pr.accumulate ? pr.out[o] + v : v;
          } else {
            dst[prow * R + j] = acc[cb][jb][e];
          }
        }
      }
}

// out[p][j] (or out[j][p]) = s * sum_q part[q][p][j], q in partition order; one
// thread per output element, the partials read 8 at a time.
__global__ __launch_bounds__(NT) void grad_reduce_kernel(GradArgs a) {
  const int bid = (int)blockIdx.x;
  int pb = 0;
  while (pb + 1 < a.nprob && bid >= a.prob[pb + 1].rblk0) ++pb;
  const GradProb& pr = a.prob[pb];
  const int64_t total = pr.pdim * a.r;
  const int64_t i = (int64_t)(bid - pr.rblk0) * NT + threadIdx.x;
  if (i >= total) return;
  const float* src = pr.part + i;
  float sum = 0.0f;
  int q = 0;
  for (; q + 8 <= a.nparts; q += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[(int64_t)(q + u) * total];
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  for (; q < a.nparts; ++q) sum += src[(int64_t)q * total];
  const int64_t pi = i / a.r;
  const int j = (int)(i % a.r);
  const int64_t o = pr.transpose_out ? (int64_t)j * pr.pdim + pi : i;
  const float v = pr.s * sum;
  pr.out[o] = pr.accumulate ? pr.out[o] + v : v;
}

// out[m][j] = sum_c x[m][c] * b[c][j]; one workgroup per row (used when dX is not wanted).
template <int R>
__global__ __launch_bounds__(NT) void down_proj_kernel(const uint16_t* __restrict__ x, int64_t c,
                                                       const uint16_t* __restrict__ b,
                                                       float* __restrict__ out) {
  __shared__ float red[NT / 64][R];
  const int64_t row = blockIdx.x;
  float acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = 0.0f;
  for (int64_t k = threadIdx.x; k < c; k += NT) {
    const float xv = __uint_as_float((uint32_t)x[row * c + k] << 16);
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j] = fmaf(xv, __uint_as_float((uint32_t)b[k * R + j] << 16), acc[j]);
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

}  // namespace

int32_t grad_parts(int64_t m) {
  int64_t p = (m + CHUNK - 1) / CHUNK;
  if (p < 1) p = 1;
  if (p > 64) p = 64;
  return (int32_t)p;
}

int64_t grad_tiles(int64_t pdim, int32_t r) {
  const int64_t tp = r == 32 ? grad_tp<32>() : grad_tp<16>();
  return (pdim + tp - 1) / tp;
}

hipError_t launch_down_proj(const uint16_t* x, int64_t m, int64_t c, const uint16_t* b, int32_t r,
                            float* out, hipStream_t s) {
  if (m == 0) return hipSuccess;
  switch (r) {
    case 8: hipLaunchKernelGGL(down_proj_kernel<8>, dim3((unsigned)m), dim3(NT), 0, s, x, c, b, out); break;
    case 16: hipLaunchKernelGGL(down_proj_kernel<16>, dim3((unsigned)m), dim3(NT), 0, s, x, c, b, out); break;
    default: hipLaunchKernelGGL(down_proj_kernel<32>, dim3((unsigned)m), dim3(NT), 0, s, x, c, b, out); break;
  }
  return hipGetLastError();
}

hipError_t launch_grad_reduce(GradReduceSet& d, hipStream_t s) {
  if (d.n == 0) return hipSuccess;
  GradArgs a{};
  a.nprob = d.n;
  a.r = d.r;
  a.nparts = d.nparts;
  int32_t rblocks = 0;
  for (int i = 0; i < d.n; ++i) {
    const GradReduceSet::Item& it = d.item[i];
    a.prob[i] = GradProb{nullptr, nullptr, it.out, const_cast<float*>(it.part), it.pdim, it.transpose_out,
                         it.s, it.accumulate, 0, rblocks, 0, 1, 0};
    rblocks += (int32_t)((it.pdim * d.r + NT - 1) / NT);
  }
  d.n = 0;
  hipLaunchKernelGGL(grad_reduce_kernel, dim3((unsigned)rblocks), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grads_group(const GradLaunch* g, int n, hipStream_t s, GradReduceSet* defer) {
  if (n < 1 || n > QL_GROUP_MAX) return hipErrorInvalidValue;
  GradArgs a{};
  a.nprob = 2 * n;
  a.r = g[0].r;
  a.m = g[0].m;
  a.nparts = g[0].nparts;
  int64_t chunk = (g[0].m + g[0].nparts - 1) / g[0].nparts;
  a.chunk = (chunk + TMC - 1) / TMC * TMC;
  int32_t blocks = 0, rblocks = 0;
  GradProb src[MAX_PROB];
  for (int i = 0; i < n; ++i) {
    if (g[i].m != a.m || g[i].r != a.r || g[i].nparts != a.nparts) return hipErrorInvalidValue;
    const float sc = g[i].s;
    const int32_t acc = g[i].accumulate;
    src[2 * i] = GradProb{g[i].x, g[i].v, g[i].d_a, g[i].part_a, g[i].k, 1, sc, acc, 0, 0, 0, 1, 0};
    src[2 * i + 1] = GradProb{g[i].dy, g[i].u, g[i].d_b, g[i].part_b, g[i].n, 0, sc, acc, 0, 0, 0, 1, 0};
  }
  // runs of problems with one input and width, in order of first appearance
  bool taken[MAX_PROB] = {};
  int np = 0;
  for (int i = 0; i < a.nprob; ++i) {
    if (taken[i]) continue;
    const int first = np;
    for (int j = i; j < a.nprob; ++j)
      if (!taken[j] && src[j].x == src[i].x && src[j].pdim == src[i].pdim) {
        taken[j] = true;
        a.prob[np++] = src[j];
      }
    const int nrun = np - first;
    const int32_t w = (int32_t)grad_tiles(src[i].pdim, a.r) * a.nparts;
    for (int j = first; j < np; ++j) {
      GradProb& pr = a.prob[j];
      pr.blk0 = blocks;
      pr.nblk = w;
      pr.nrun = nrun;
      pr.ridx = j - first;
      pr.rblk0 = rblocks;
      rblocks += (int32_t)((pr.pdim * a.r + NT - 1) / NT);
    }
    blocks += nrun == 1 ? w : (w + 7) / 8 * 8 * nrun;
  }
  const bool held = defer && a.m > 0 && a.nparts > 1;
  if (held && defer->n > 0 &&
      (defer->r != a.r || defer->nparts != a.nparts || defer->n + a.nprob > MAX_PROB)) {
    hipError_t e = launch_grad_reduce(*defer, s);
    if (e != hipSuccess) return e;
  }
  if (a.m > 0) {
    switch (a.r) {
      case 8: hipLaunchKernelGGL(grad_kernel<8>, dim3((unsigned)blocks), dim3(NT), 0, s, a); break;
      case 16: hipLaunchKernelGGL(grad_kernel<16>, dim3((unsigned)blocks), dim3(NT), 0, s, a); break;
      default: hipLaunchKernelGGL(grad_kernel<32>, dim3((unsigned)blocks), dim3(NT), 0, s, a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nparts == 1) return e;   // one partition: the kernel wrote dA, dB
    if (held) {
      defer->r = a.r;
      defer->nparts = a.nparts;
      for (int i = 0; i < a.nprob; ++i) {
        const GradProb& pr = a.prob[i];
        defer->item[defer->n++] = GradReduceSet::Item{pr.part, pr.out, pr.pdim, pr.transpose_out, pr.s, pr.accumulate};
      }
      return hipSuccess;
    }
  } else {
    a.nparts = 0;                                     // no tokens: dA = dB = 0 (or unchanged)
  }
  hipLaunchKernelGGL(grad_reduce_kernel, dim3((unsigned)rblocks), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grads(const GradLaunch& g, hipStream_t s) { return launch_grads_group(&g, 1, s); }

hipError_t launch_grad_kernels(GradKernelSet& k, hipStream_t s, GradReduceSet* defer) {
  if (k.n == 0) return hipSuccess;
  const int n = k.n;
  k.n = 0;
  return launch_grads_group(k.g, n, s, defer);
}

}  // namespace ql
