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

}  // namespace

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
