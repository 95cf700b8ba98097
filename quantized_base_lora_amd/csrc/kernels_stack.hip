// Stacked adapters: frozen lower adapters under one trainable top adapter
// (the Surogate review page's stacked LoRA, adapters trained on top of
// other adapters without an offline merge).  The sum
//   sum_i s_i . (x . A_i^T) . B_i^T
// is one adapter of rank R = sum_i r_i with A = [A_1; ...; A_top] and
// B = [c_1 B_1, ..., B_top], c_i = s_i / s_top, at the top's scale s_top, so
// the layer's own kernels run the stack unchanged; the top adapter's
// gradients are the last r_top rows of dA and columns of dB.  This kernel
// builds the two concatenated factors (one pass, bf16 in and out; the frozen
// blocks of B are scaled in fp32 and rounded once, the top block is copied).
#include <algorithm>

#include "common.h"
#include "device.h"

namespace ql {
namespace {

constexpr int kThreads = 256;

struct StackArgs {
  const uint16_t* a[QL_STACK_MAX];
  const uint16_t* b[QL_STACK_MAX];
  float c[QL_STACK_MAX];           // s_i / s_top (1 for the top)
  int32_t r[QL_STACK_MAX];
  int32_t off[QL_STACK_MAX + 1];   // first row of adapter i in A (first column in B)
  int32_t n;
  int32_t R;
  int64_t K, N;
  uint16_t* a_cat;                 // [R, K]
  uint16_t* b_cat;                 // [N, R]
};

__global__ __launch_bounds__(kThreads) void stack_kernel(StackArgs s) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t na = (int64_t)s.R * s.K, nb = s.N * s.R;
  if (i < na) {                                    // A: rows of the adapters in order
    const int row = (int)(i / s.K);
    int a = 0;
    while (a + 1 < s.n && row >= s.off[a + 1]) ++a;
    s.a_cat[i] = s.a[a][(int64_t)(row - s.off[a]) * s.K + i % s.K];
  }
  if (i < nb) {                                    // B: column blocks, the frozen ones scaled
    const int64_t nrow = i / s.R;
    const int col = (int)(i % s.R);
    int a = 0;
    while (a + 1 < s.n && col >= s.off[a + 1]) ++a;
    const uint16_t v = s.b[a][nrow * s.r[a] + (col - s.off[a])];
    if (a == s.n - 1) {
      s.b_cat[i] = v;
    } else {
      const float f = __uint_as_float((uint32_t)v << 16) * s.c[a];
      s.b_cat[i] = __builtin_bit_cast(uint16_t, (__bf16)f);   // nearest even
    }
  }
}

}  // namespace

hipError_t launch_stack(const ql_adapter* ad, int32_t n, int64_t n_out, int64_t k_in, uint16_t* a_cat,
                        uint16_t* b_cat, float* alpha_cat, hipStream_t st) {
  StackArgs s{};
  s.n = n;
  s.K = k_in;
  s.N = n_out;
  s.a_cat = a_cat;
  s.b_cat = b_cat;
  const double s_top = (double)ad[n - 1].alpha / (double)ad[n - 1].r;
  int32_t off = 0;
  for (int i = 0; i < n; ++i) {
    s.a[i] = ad[i].lora_a;
    s.b[i] = ad[i].lora_b;
    s.r[i] = ad[i].r;
    s.c[i] = i == n - 1 ? 1.0f : (float)(((double)ad[i].alpha / (double)ad[i].r) / s_top);
    s.off[i] = off;
    off += ad[i].r;
  }
  s.off[n] = off;
  s.R = off;
  *alpha_cat = (float)s_top * (float)off;          // alpha_cat / R == fl32(s_top): R is a power of two
  const int64_t total = std::max<int64_t>((int64_t)s.R * k_in, n_out * (int64_t)s.R);
  hipLaunchKernelGGL(stack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, s);
  return hipGetLastError();
}

}  // namespace ql
