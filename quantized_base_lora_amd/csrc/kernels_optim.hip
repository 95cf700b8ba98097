// AdamW step on the LoRA adapters, all tensors of a call in one launch.
//
// The Surogate README page lists "AdamW 8-bit" among its optimizers and the
// GGUF-recipe page ("How it works") trains its adapters with 8-bit AdamW; the
// update is decoupled weight decay (Loshchilov & Hutter, "Decoupled Weight
// Decay Regularization", Algorithm 2) in the convention PyTorch and
// bitsandbytes share: the decay is scaled by the learning rate and applied
// before the Adam term.  Moments are fp32 (the pages do not define the 8-bit
// state format).  Per element, with g = grad * grad_scale:
//   p *= 1 - lr * wd;  m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
//   p -= (lr / (1 - b1^t)) * m / (sqrt(v) / sqrt(1 - b2^t) + eps);
//   bf16 copy = bf16_RNE(p) (the adapter the next forward reads).
// HBM-bound: 16 bytes read and 12 (+2 for the copy) written per element.
#include "common.h"
#include "device.h"
#include "dyn8.h"

namespace ql {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;                       // elements per thread: one 16-byte piece per array, so a
constexpr int kBlockElems = kThreads * kVec;  // layer's adapters give several workgroups per CU

struct AdamwKernelArgs {
  ql_adamw_tensor t[QL_ADAMW_MAX_TENSORS];
  int64_t blk0[QL_ADAMW_MAX_TENSORS + 1];     // first block of each tensor, blk0[nt] = grid size
  int32_t nt;
  float decay, b1, omb1, b2, omb2, step_size, inv_bc2_sqrt, eps, gs;
};

__global__ __launch_bounds__(kThreads) void adamw_kernel(AdamwKernelArgs a) {
  const int64_t b = blockIdx.x;
  int ti = 0;
  while (ti + 1 < a.nt && b >= a.blk0[ti + 1]) ++ti;   // uniform over the block
  const ql_adamw_tensor& T = a.t[ti];
  const int64_t e = (b - a.blk0[ti]) * kBlockElems + (int64_t)threadIdx.x * 4;   // n % 4 == 0
  {
    if (e >= T.n) return;
    float4 p = *reinterpret_cast<const float4*>(T.param + e);
    const float4 g4 = *reinterpret_cast<const float4*>(T.grad + e);
    float4 m = *reinterpret_cast<const float4*>(T.exp_avg + e);
    float4 v = *reinterpret_cast<const float4*>(T.exp_avg_sq + e);
    float* pp = &p.x;
    float* mp = &m.x;
    float* vp = &v.x;
    const float* gp = &g4.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g = gp[i] * a.gs;
      float th = pp[i] * a.decay;
      mp[i] = a.b1 * mp[i] + a.omb1 * g;
      vp[i] = a.b2 * vp[i] + a.omb2 * (g * g);
      const float denom = sqrtf(vp[i]) * a.inv_bc2_sqrt + a.eps;
      th = th - a.step_size * (mp[i] / denom);
      pp[i] = th;
    }
    *reinterpret_cast<float4*>(T.param + e) = p;
    *reinterpret_cast<float4*>(T.exp_avg + e) = m;
    *reinterpret_cast<float4*>(T.exp_avg_sq + e) = v;
    if (T.param_bf16)
      *reinterpret_cast<uint2*>(T.param_bf16 + e) = make_uint2(pack_bf16x2(p.x, p.y), pack_bf16x2(p.z, p.w));
  }
}

// ---------------------------------------------------------------- 8-bit moments
// The same update with each moment stored as 8-bit codes of the dynamic tree
// type in blocks of kAdamw8Block elements with one fp32 largest magnitude per
// block (dyn8.h): the moments are dequantized (level * absmax), updated in
// fp32, the parameter moves with the fp32 moments, and each moment is
// quantized again with its block's new largest magnitude: r = m / absmax
// (IEEE divide), code = number of thresholds below |r| (a value equal to a
// threshold takes the lower code), sign bit for a negative first moment with
// a non-zero code.  One workgroup per block, eight elements per thread.  The
// codes are integer decisions taken in fp32, so every operation is written
// with its own rounding and in a fixed order (no fused multiply-add): the
// results are reproducible bit for bit.  HBM-bound: 4 + 4 + 1 + 1 bytes read
// and 4 + 1 + 1 (+2 for the copy) written per element.
// fp32 operations rounded one by one: defined with contraction off, so no
// multiply and add of the update are fused into one rounding, wherever they
// are inlined
#pragma clang fp contract(off)
__device__ __forceinline__ float mul_rn(float a, float b) { return a * b; }
__device__ __forceinline__ float add_rn(float a, float b) { return a + b; }
__device__ __forceinline__ float sub_rn(float a, float b) { return a - b; }
#pragma clang fp contract(on)

__constant__ Dyn8Table kDynS = make_dyn8(true);
__constant__ Dyn8Table kDynU = make_dyn8(false);

constexpr int kThreads8 = kAdamw8Block / 8;

struct Adamw8KernelArgs {
  ql_adamw8_tensor t[QL_ADAMW_MAX_TENSORS];
  int64_t blk0[QL_ADAMW_MAX_TENSORS + 1];
  int32_t nt;
  float decay, b1, omb1, b2, omb2, step_size, inv_bc2_sqrt, eps, gs;
};

// number of the ascending thresholds thr[0 .. 2^bits - 2] strictly below x
// (0 and NaN -> 0): an estimate from the level formula (decade z from log10,
// then the nearest of the decade's 2^f levels), moved down while the
// threshold below it is not below x and up while the one above it is, so
// the result is the rank by definition whatever the estimate (usually one
// or two comparisons instead of a binary search's eight dependent lookups)
__device__ __forceinline__ uint32_t dyn8_rank(const float* thr, int bits, float x) {
  if (!(x > 0.0f)) return 0u;
  const int last = (1 << bits) - 1;
  int z = (int)(-__log10f(x));
  z = z < 0 ? 0 : (z > bits - 1 ? bits - 1 : z);
  const int f = bits - 1 - z;
  float y = x;
#pragma unroll
  for (int i = 0; i < 7; ++i)
    if (i < z) y *= 10.0f;
  int q = (int)rintf((y - 0.1f) * ((float)(1 << f) / 0.9f)) - 1;
  q = q < 0 ? 0 : (q > (1 << f) - 1 ? (1 << f) - 1 : q);
  int c = (1 << f) + q;
  while (c > 0 && !(thr[c - 1] < x)) --c;
  while (c < last && thr[c] < x) ++c;
  return (uint32_t)c;
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kThreads8 / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

__global__ __launch_bounds__(kThreads8) void adamw8_kernel(Adamw8KernelArgs a) {
  __shared__ float red_m[kThreads8 / 64], red_v[kThreads8 / 64];
  // the level and threshold tables in LDS (lane-divergent lookups)
  __shared__ float lvl_s[128], lvl_u[256], thr_s[127], thr_u[255];
  static_assert(kThreads8 == 256, "one table entry per thread");
  {
    const int t = threadIdx.x;
    lvl_u[t] = kDynU.level[t];
    if (t < 255) thr_u[t] = kDynU.thresh[t];
    if (t < 128) lvl_s[t] = kDynS.level[t];
    if (t < 127) thr_s[t] = kDynS.thresh[t];
  }
  __syncthreads();
  const int64_t b = blockIdx.x;
  int ti = 0;
  while (ti + 1 < a.nt && b >= a.blk0[ti + 1]) ++ti;   // uniform over the block
  const ql_adamw8_tensor& T = a.t[ti];
  const int64_t blk = b - a.blk0[ti];
  const int64_t e = blk * kAdamw8Block + (int64_t)threadIdx.x * 8;   // n % 8 == 0: all 8 live or none
  const bool live = e < T.n;
  float p[8] = {}, g[8] = {}, m[8], v[8];
  uint32_t mc[2] = {0, 0}, vc[2] = {0, 0};
  if (live) {
    const float4* pp = reinterpret_cast<const float4*>(T.param + e);
    const float4* gp = reinterpret_cast<const float4*>(T.grad + e);
    const float4 p0 = pp[0], p1 = pp[1], g0 = gp[0], g1 = gp[1];
    p[0] = p0.x; p[1] = p0.y; p[2] = p0.z; p[3] = p0.w; p[4] = p1.x; p[5] = p1.y; p[6] = p1.z; p[7] = p1.w;
    g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w; g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
    const uint2 mcv = *reinterpret_cast<const uint2*>(T.exp_avg + e);
    const uint2 vcv = *reinterpret_cast<const uint2*>(T.exp_avg_sq + e);
    mc[0] = mcv.x; mc[1] = mcv.y; vc[0] = vcv.x; vc[1] = vcv.y;
  }
  const float am = live ? T.exp_avg_absmax[blk] : 0.0f;
  const float av = live ? T.exp_avg_sq_absmax[blk] : 0.0f;
  float mmax = 0.0f, vmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t cm = (mc[i >> 2] >> (8 * (i & 3))) & 0xFF, cv = (vc[i >> 2] >> (8 * (i & 3))) & 0xFF;
    const float mag = mul_rn(lvl_s[cm & 0x7F], am);
    const float mo = (cm & 0x80) ? -mag : mag;
    const float vo = mul_rn(lvl_u[cv], av);
    const float gi = mul_rn(g[i], a.gs);
    const float th = mul_rn(p[i], a.decay);
    m[i] = add_rn(mul_rn(a.b1, mo), mul_rn(a.omb1, gi));
    v[i] = add_rn(mul_rn(a.b2, vo), mul_rn(a.omb2, mul_rn(gi, gi)));
    // sqrtf is correctly rounded here (the native square root alone is not)
    const float denom = add_rn(mul_rn(sqrtf(v[i]), a.inv_bc2_sqrt), a.eps);
    p[i] = sub_rn(th, mul_rn(a.step_size, __fdiv_rn(m[i], denom)));
    if (live) {
      mmax = fmaxf(mmax, fabsf(m[i]));
      vmax = fmaxf(vmax, fabsf(v[i]));
    }
  }
  const float am2 = block_max(mmax, red_m);
  const float av2 = block_max(vmax, red_v);
  if (!live) return;
  uint32_t om[2] = {0, 0}, ov[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t km = 0, kv = 0;
    if (am2 > 0.0f) {
      const float r = __fdiv_rn(m[i], am2);
      km = dyn8_rank(thr_s, 7, fabsf(r));
      if (r < 0.0f && km > 0) km |= 0x80;
    }
    if (av2 > 0.0f) kv = dyn8_rank(thr_u, 8, fabsf(__fdiv_rn(v[i], av2)));
    om[i >> 2] |= km << (8 * (i & 3));
    ov[i >> 2] |= kv << (8 * (i & 3));
  }
  float4* pp = reinterpret_cast<float4*>(T.param + e);
  pp[0] = make_float4(p[0], p[1], p[2], p[3]);
  pp[1] = make_float4(p[4], p[5], p[6], p[7]);
  *reinterpret_cast<uint2*>(T.exp_avg + e) = make_uint2(om[0], om[1]);
  *reinterpret_cast<uint2*>(T.exp_avg_sq + e) = make_uint2(ov[0], ov[1]);
  if (threadIdx.x == 0) {
    T.exp_avg_absmax[blk] = am2;
    T.exp_avg_sq_absmax[blk] = av2;
  }
  if (T.param_bf16)
    *reinterpret_cast<uint4*>(T.param_bf16 + e) = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                                             pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
}

template <class Args>
void fill_constants(Args& a, const ql_adamw_hparams& hp) {
  const double t = hp.step;
  a.decay = (float)(1.0 - hp.lr * hp.weight_decay);
  a.b1 = (float)hp.beta1;
  a.omb1 = (float)(1.0 - hp.beta1);
  a.b2 = (float)hp.beta2;
  a.omb2 = (float)(1.0 - hp.beta2);
  a.step_size = (float)(hp.lr / (1.0 - pow(hp.beta1, t)));
  a.inv_bc2_sqrt = (float)(1.0 / sqrt(1.0 - pow(hp.beta2, t)));
  a.eps = (float)hp.eps;
  a.gs = (float)hp.grad_scale;
}

}  // namespace

const Dyn8Table& dyn8_table(bool is_signed) {
  static const Dyn8Table s = make_dyn8(true), u = make_dyn8(false);
  return is_signed ? s : u;
}

hipError_t launch_adamw8(const ql_adamw8_tensor* ts, int32_t nt, const ql_adamw_hparams& hp, hipStream_t s) {
  Adamw8KernelArgs a{};
  int64_t blocks = 0;
  int32_t k = 0;
  for (int32_t i = 0; i < nt; ++i) {
    if (ts[i].n == 0) continue;
    a.t[k] = ts[i];
    a.blk0[k] = blocks;
    blocks += (ts[i].n + kAdamw8Block - 1) / kAdamw8Block;
    ++k;
  }
  if (k == 0) return hipSuccess;
  a.blk0[k] = blocks;
  a.nt = k;
  fill_constants(a, hp);
  hipLaunchKernelGGL(adamw8_kernel, dim3((unsigned)blocks), dim3(kThreads8), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_adamw(const ql_adamw_tensor* ts, int32_t nt, const ql_adamw_hparams& hp, hipStream_t s) {
  AdamwKernelArgs a{};
  int64_t blocks = 0;
  int32_t k = 0;
  for (int32_t i = 0; i < nt; ++i) {
    if (ts[i].n == 0) continue;                // empty tensors take no block
    a.t[k] = ts[i];
    a.blk0[k] = blocks;
    blocks += (ts[i].n + kBlockElems - 1) / kBlockElems;
    ++k;
  }
  if (k == 0) return hipSuccess;
  a.blk0[k] = blocks;
  a.nt = k;
  const double t = hp.step;
  a.decay = (float)(1.0 - hp.lr * hp.weight_decay);
  a.b1 = (float)hp.beta1;
  a.omb1 = (float)(1.0 - hp.beta1);
  a.b2 = (float)hp.beta2;
  a.omb2 = (float)(1.0 - hp.beta2);
  a.step_size = (float)(hp.lr / (1.0 - pow(hp.beta1, t)));
  a.inv_bc2_sqrt = (float)(1.0 / sqrt(1.0 - pow(hp.beta2, t)));
  a.eps = (float)hp.eps;
  a.gs = (float)hp.grad_scale;
  hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ql
