// Internal declarations shared by the library's translation units.
// gfx950 (CDNA4) only: wave64, bf16 and fp8 MFMA, LDS transpose reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qlora.h"

namespace ql {

// ----------------------------------------------------------------- vector types
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------- barriers
// Workgroup barrier for LDS hand-offs only.  __syncthreads() is a release /
// acquire fence at workgroup scope, which on gfx9 waits for every outstanding
// vector-memory operation, loads included (vmcnt covers both), and so would
// drain the prefetches of later tiles at every step.  Here only this wave's
// LDS operations are completed before the barrier; global loads stay in
// flight.  The memory clobber keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ----------------------------------------------------------------- NF4 levels
// The 16 levels (fp32, ascending) and the 15 decision thresholds
// m_i = fl32(fl32(c_i + c_{i+1}) * 0.5), built once on the host.
struct Nf4Table {
  float level[16];
  float mid[15];
};
const Nf4Table& nf4_table();

// ----------------------------------------------------------------- errors
int set_error(int code, const char* fmt, ...);
int hip_error(hipError_t e, const char* what);
#define QL_HIP(call)                                   \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) return ::ql::hip_error(e_, #call); \
  } while (0)

// ----------------------------------------------------------------- launchers
// All take already-validated arguments and enqueue on `stream`.

// pack / dequant / activation split (kernels_pack.hip)
// block formats (Q4_0, NF4, MXFP4, Q8_0): one thread per 32-element group
hipError_t launch_pack_blocks(int fmt, const float* w, int64_t n, int64_t k,
                              uint8_t* codes, void* scales, uint32_t* status,
                              hipStream_t s);
hipError_t launch_pack_fp8(const float* w, int64_t n, int64_t k, uint8_t* codes,
                           float* scale, uint32_t* ws, hipStream_t s);
hipError_t launch_pack_nvfp4(const float* w, int64_t n, int64_t k, uint8_t* codes, void* scales,
                             uint32_t* ws, hipStream_t s);
hipError_t launch_dequant(const ql_qweight& w, float* out_f32, uint16_t* out_bf16,
                          hipStream_t s);
hipError_t launch_act_quant(const uint16_t* x, int64_t m, int64_t k, uint8_t* hi,
                            uint8_t* lo, float* scale, hipStream_t s);
// the split of n (1 .. QL_GROUP_MAX) activations of m rows each: one launch
// per split kernel used
struct ActSplit {
  const uint16_t* x;
  uint8_t* hi;
  uint8_t* lo;
  float* scale;
  int64_t k;
};
hipError_t launch_act_quant_group(const ActSplit* sp, int n, int64_t m, hipStream_t s);
hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s);
// one streaming read of bytes (a multiple of 16) at buf; sink [QL_STREAM_READ_THREADS]
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t s);

// fused base GEMM + LoRA (kernels_gemm.hip)
// dX with few tokens (split_path_fuses_grads): the reduction launch of the
// split path also computes the adapter gradients (one launch instead of two)
struct GradFuse {
  const uint16_t* x;       // [M, K] layer input
  const float* u;          // [M, r] U saved by the forward
  float* d_a;              // [r, K]
  float* d_b;              // [N, r]
  int32_t accumulate;
};
bool split_path_fuses_grads(int64_t m);
// the small-token (split-contraction) path serves this many tokens
bool split_path_tokens(int64_t m);

struct GemmCall {
  const ql_qweight* w;
  bool trans;              // false: y = act . W^T (contract K); true: dX = act . W (contract N)
  const uint16_t* act;     // [M, C] bf16, C = contraction length
  int64_t m;
  const uint16_t* down;    // forward: A [r, K]; backward: B [N, r]
  const uint16_t* up;      // forward: B [N, r]; backward: A [r, K]
  int32_t r;
  float s;                 // alpha / r
  uint16_t* out;           // [M, O] bf16, O = output columns
  float* save;             // [M, r] fp32 rank-r projection (U or V), may be null
  void* ws;                // scratch of qgemm_workspace_bytes(trans, m, n, k, r) bytes (small-M path)
  const GradFuse* grads;   // dX only, with split_path_fuses_grads(m): also write dA, dB (else null)
};
hipError_t launch_qgemm(const GemmCall& c, hipStream_t s);
// independent calls of one format, direction, token count and rank: on the
// small-M split path one split launch and one reduction launch for all of
// them, on the bf16 tile path one launch, for the FP8 base above SMALL_M one
// fp8 GEMM launch (with one activation split per distinct activation); all
// bitwise the results of separate calls.  Other call sets are launched one
// by one
bool qgemm_groupable(const GemmCall* calls, int n);
hipError_t launch_qgemm_group(const GemmCall* calls, int n, hipStream_t s);
// scratch the GEMM needs: split-contraction partials when m is small; for the
// FP8 base with more tokens, the activation split (hi, lo planes and row scales)
size_t qgemm_workspace_bytes(int32_t fmt, bool trans, int64_t m, int64_t n, int64_t k, int32_t r);

// FP8 base on fp8 matrix cores (kernels_fp8.hip): the activation arrives split
// (a1), the rank-r projection precomputed
struct Gemm8Call {
  const ql_qweight* w;
  bool trans;
  const uint8_t* hi;       // [M, C] E4M3
  const uint8_t* lo;       // [M, C] E4M3
  const float* rs;         // [M] row scales
  int64_t m;
  const float* u;          // [M, r] U (forward) or V (dX)
  const uint16_t* up;      // forward: B [N, r]; dX: A [r, K]
  int32_t r;
  float s;
  uint16_t* out;           // [M, O] bf16
};
// one launch for n (1 .. QL_GROUP_MAX) independent calls of one direction and rank
hipError_t launch_qgemm8(const Gemm8Call* c, int n, hipStream_t s);
// out [m, r] fp32 = act [m, c] . D, D = A^T (a_layout, A [r, c]) or B ([c, r])
hipError_t launch_rproj(const uint16_t* act, int64_t m, int64_t c, const uint16_t* d, bool a_layout, int32_t r,
                        float* out, hipStream_t s);
// n (1 .. QL_GROUP_MAX) projections of m rows each, one layout and rank: one launch
struct Rproj {
  const uint16_t* act;
  const uint16_t* d;
  float* out;
  int64_t c;
};
hipError_t launch_rproj_group(const Rproj* pr, int n, int64_t m, bool a_layout, int32_t r, hipStream_t s);

// stacked adapters -> one concatenated adapter (kernels_stack.hip); arguments already validated
hipError_t launch_stack(const ql_adapter* ad, int32_t n, int64_t n_out, int64_t k_in, uint16_t* a_cat,
                        uint16_t* b_cat, float* alpha_cat, hipStream_t st);

// adapter optimizer step (kernels_optim.hip); arguments already validated
hipError_t launch_adamw(const ql_adamw_tensor* ts, int32_t nt, const ql_adamw_hparams& hp, hipStream_t s);
hipError_t launch_adamw8(const ql_adamw8_tensor* ts, int32_t nt, const ql_adamw_hparams& hp, hipStream_t s);
// the levels of the 8-bit state type (dyn8.h), built at compile time
struct Dyn8Table;
const Dyn8Table& dyn8_table(bool is_signed);

// LoRA-side kernels (kernels_lora.hip)
// out[m][j] = sum_c x[m][c] * b[c][j]     (fp32), b is [C, r]
hipError_t launch_down_proj(const uint16_t* x, int64_t m, int64_t c, const uint16_t* b,
                            int32_t r, float* out, hipStream_t s);
// dA = s V^T x and dB = s dY^T U: one launch for both partial sums, one to reduce them in fixed order
struct GradLaunch {
  const uint16_t* x;       // [M, K]
  const uint16_t* dy;      // [M, N]
  const float* v;          // [M, r]
  const float* u;          // [M, r]
  float* d_a;              // [r, K]
  float* d_b;              // [N, r]
  float* part_a;           // [P, K, r]
  float* part_b;           // [P, N, r]
  int64_t m, k, n;
  int32_t r, nparts;
  float s;
  int32_t accumulate;
};
hipError_t launch_grads(const GradLaunch& g, hipStream_t s);
// Reductions of adapter-gradient partials held back so that those of
// consecutive backward calls run as one launch (a launch plan gathers them).
// The items of a set share the rank and the partition count.
struct GradReduceSet {
  struct Item {
    const float* part;       // [nparts, pdim, r]
    float* out;              // [pdim, r], or [r, pdim] with transpose_out
    int64_t pdim;
    int32_t transpose_out;
    float s;
    int32_t accumulate;
  };
  Item item[2 * QL_GROUP_MAX];
  int32_t n = 0, r = 0, nparts = 0;
};
// the gradients of n calls with one token count, rank and partition plan in
// one launch (and one reduction launch).  With `defer`, a reduction that is
// needed (M > 0, more than one partition) is added to the set instead of
// launched; a set it does not fit is launched first.
hipError_t launch_grads_group(const GradLaunch* g, int n, hipStream_t s, GradReduceSet* defer = nullptr);
// launches the set's reductions as one launch (nothing if it is empty) and empties it
hipError_t launch_grad_reduce(GradReduceSet& d, hipStream_t s);
// Adapter-gradient launches held back by a launch plan, so that those of
// consecutive backward steps run as one grad_kernel launch; the calls of a
// set share the token count (> 0), rank and partition plan.
struct GradKernelSet {
  GradLaunch g[QL_GROUP_MAX];
  int32_t n = 0;
  bool fits(const GradLaunch& x) const {
    return n == 0 || (n < QL_GROUP_MAX && x.m == g[0].m && x.r == g[0].r && x.nparts == g[0].nparts);
  }
};
// launches the set's calls as one group (reductions into `defer` as
// launch_grads_group does) and empties it
hipError_t launch_grad_kernels(GradKernelSet& k, hipStream_t s, GradReduceSet* defer);
int32_t grad_parts(int64_t m);
int64_t grad_tiles(int64_t pdim, int32_t r);

}  // namespace ql
