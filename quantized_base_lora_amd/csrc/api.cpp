// C ABI entry points (include/qlora.h): argument validation, workspace
// layout, and the launch sequence of each call.  No device memory is
// allocated here; scratch comes from the caller's workspace.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.h"

namespace ql {

static thread_local char g_err[512];

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_error(hipError_t e, const char* what) {
  return set_error(QL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

namespace {

constexpr size_t kAlign = 256;
inline size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int block_of(int32_t fmt) { return fmt == QL_FMT_NF4 ? 64 : 32; }

int check_sticky() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_error(e, "pending HIP error");
  return QL_OK;
}

int check_shape(int32_t fmt, int64_t n, int64_t k) {
  if (fmt != QL_FMT_Q4_0 && fmt != QL_FMT_NF4 && fmt != QL_FMT_FP8_E4M3 && fmt != QL_FMT_MXFP4)
    return set_error(QL_EUNSUPPORTED, "unknown format %d", fmt);
  if (n <= 0 || k <= 0) return set_error(QL_EINVAL, "n_out and k_in must be positive");
  if (k % block_of(fmt)) return set_error(QL_EINVAL, "k_in=%lld is not a multiple of %d", (long long)k, block_of(fmt));
  if (n % 32) return set_error(QL_EINVAL, "n_out=%lld is not a multiple of 32", (long long)n);
  return QL_OK;
}

int check_weight(const ql_qweight* w) {
  if (!w) return set_error(QL_EINVAL, "null weight");
  int rc = check_shape(w->format, w->n_out, w->k_in);
  if (rc) return rc;
  if (w->reserved != 0) return set_error(QL_EINVAL, "weight.reserved must be 0");
  if (!w->codes || !w->scales) return set_error(QL_EINVAL, "null codes or scales");
  if (!aligned16(w->codes)) return set_error(QL_EINVAL, "codes not 16-byte aligned");
  if (((uintptr_t)w->scales & 3u) != 0) return set_error(QL_EINVAL, "scales not 4-byte aligned");
  return QL_OK;
}

int check_rank(int32_t r) {
  if (r != 8 && r != 16 && r != 32) return set_error(QL_EUNSUPPORTED, "rank %d not in {8,16,32}", r);
  return QL_OK;
}

// backward workspace: V [M, r] fp32 | partials for dA [P, K, r] | for dB [P, N, r] |
// the dX GEMM's own scratch (split-contraction partials, small M only)
struct BwdLayout {
  size_t v, pa, pb, g, total;
  int32_t parts;
};

BwdLayout bwd_layout(int32_t fmt, int64_t n, int64_t k, int64_t m, int32_t r) {
  BwdLayout l{};
  l.parts = grad_parts(m);
  l.v = 0;
  l.pa = l.v + up((size_t)m * r * 4);
  l.pb = l.pa + up((size_t)l.parts * k * r * 4);
  l.g = l.pb + up((size_t)l.parts * n * r * 4);
  l.total = l.g + up(qgemm_workspace_bytes(fmt, true, m, n, k, r));
  return l;
}

}  // namespace
}  // namespace ql

using namespace ql;

extern "C" {

const char* ql_last_error(void) { return g_err; }

int32_t ql_version(void) { return 1; }

int ql_nf4_levels(float* out) {
  if (!out) return set_error(QL_EINVAL, "null output");
  memcpy(out, nf4_table().level, 16 * sizeof(float));
  return QL_OK;
}

size_t qlora_workspace_bytes(int32_t op, int32_t format, int64_t n_out, int64_t k_in, int64_t m,
                             int32_t r) {
  switch (op) {
    case QL_OP_PACK: return 256;
    case QL_OP_FWD: return qgemm_workspace_bytes(format, false, m < 0 ? 0 : m, n_out, k_in, r);
    case QL_OP_BWD: return bwd_layout(format, n_out, k_in, m < 0 ? 0 : m, r).total;
    default: return 0;
  }
}

int quant_pack(int32_t format, const float* w, int64_t n_out, int64_t k_in, uint8_t* codes,
               void* scales, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(format, n_out, k_in);
  if (rc) return rc;
  if (!w || !codes || !scales || !ws) return set_error(QL_EINVAL, "null pointer");
  if (!aligned16(w) || !aligned16(codes) || ((uintptr_t)scales & 3u) || ((uintptr_t)ws & 3u))
    return set_error(QL_EINVAL, "misaligned pointer");
  if (ws_bytes < 256) return set_error(QL_EWORKSPACE, "pack needs 256 bytes of workspace");
  if ((rc = check_sticky())) return rc;
  hipStream_t s = as_stream(stream);
  uint32_t* st = reinterpret_cast<uint32_t*>(ws);
  hipError_t e;
  if (format == QL_FMT_FP8_E4M3) {
    e = launch_pack_fp8(w, n_out, k_in, codes, reinterpret_cast<float*>(scales), st, s);
  } else {
    e = launch_zero_u32(st, 2, s);
    if (e == hipSuccess) e = launch_pack_4bit(format, w, n_out, k_in, codes, scales, st + 1, s);
  }
  if (e != hipSuccess) return hip_error(e, "quant_pack launch");
  QL_HIP(hipStreamSynchronize(s));
  uint32_t flags[2] = {0, 0};
  QL_HIP(hipMemcpy(flags, ws, sizeof flags, hipMemcpyDeviceToHost));
  uint32_t f = flags[1];
  if (f & 1u) return set_error(QL_ENONFINITE, "base weight holds NaN or Inf");
  if (f & 2u) return set_error(QL_EOVERFLOW, "a Q4_0 block scale overflows fp16");
  return QL_OK;
}

int qlora_dequant(const ql_qweight* w, float* out_f32, uint16_t* out_bf16, void* stream) {
  int rc = check_weight(w);
  if (rc) return rc;
  if ((out_f32 && !aligned16(out_f32)) || (out_bf16 && !aligned16(out_bf16)))
    return set_error(QL_EINVAL, "misaligned output");
  if (!out_f32 && !out_bf16) return QL_OK;
  if ((rc = check_sticky())) return rc;
  hipError_t e = launch_dequant(*w, out_f32, out_bf16, as_stream(stream));
  if (e != hipSuccess) return hip_error(e, "dequant launch");
  return QL_OK;
}

int ql_act_quant_e4m3(const uint16_t* x, int64_t m, int64_t k, uint8_t* hi, uint8_t* lo,
                      float* scale, void* stream) {
  if (m < 0 || k <= 0 || k % 16) return set_error(QL_EINVAL, "need m >= 0 and k a positive multiple of 16");
  if (m == 0) return QL_OK;
  if (!x || !hi || !lo || !scale) return set_error(QL_EINVAL, "null pointer");
  if (!aligned16(x) || !aligned16(hi) || !aligned16(lo)) return set_error(QL_EINVAL, "misaligned pointer");
  int rc = check_sticky();
  if (rc) return rc;
  hipError_t e = launch_act_quant(x, m, k, hi, lo, scale, as_stream(stream));
  if (e != hipSuccess) return hip_error(e, "act quant launch");
  return QL_OK;
}

int ql_adamw_step(const ql_adamw_tensor* tensors, int32_t n_tensors, const ql_adamw_hparams* hp,
                  void* stream) {
  if (n_tensors < 0 || n_tensors > QL_ADAMW_MAX_TENSORS)
    return set_error(QL_EINVAL, "n_tensors=%d outside [0, %d]", n_tensors, QL_ADAMW_MAX_TENSORS);
  if (!hp || (n_tensors > 0 && !tensors)) return set_error(QL_EINVAL, "null pointer");
  if (hp->step < 1) return set_error(QL_EINVAL, "step must be >= 1");
  if (hp->reserved != 0) return set_error(QL_EINVAL, "hparams.reserved must be 0");
  const double f[6] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->grad_scale};
  for (double v : f)
    if (!(v - v == 0.0)) return set_error(QL_EINVAL, "non-finite hyperparameter");
  if (hp->lr < 0.0 || hp->eps < 0.0 || hp->weight_decay < 0.0)
    return set_error(QL_EINVAL, "lr, eps and weight_decay must be >= 0");
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0 && hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return set_error(QL_EINVAL, "beta1 and beta2 must lie in [0, 1)");
  for (int32_t i = 0; i < n_tensors; ++i) {
    const ql_adamw_tensor& t = tensors[i];
    if (t.n < 0 || t.n % 4) return set_error(QL_EINVAL, "tensor %d: n=%lld is not a multiple of 4", i, (long long)t.n);
    if (t.n == 0) continue;
    if (!t.param || !t.grad || !t.exp_avg || !t.exp_avg_sq)
      return set_error(QL_EINVAL, "tensor %d: null pointer", i);
    if (!aligned16(t.param) || !aligned16(t.grad) || !aligned16(t.exp_avg) || !aligned16(t.exp_avg_sq) ||
        (t.param_bf16 && !aligned16(t.param_bf16)))
      return set_error(QL_EINVAL, "tensor %d: misaligned pointer", i);
  }
  int rc = check_sticky();
  if (rc) return rc;
  hipError_t e = launch_adamw(tensors, n_tensors, *hp, as_stream(stream));
  if (e != hipSuccess) return hip_error(e, "adamw launch");
  return QL_OK;
}

int qlora_linear_fwd(const ql_qweight* w, const uint16_t* x, int64_t m, const uint16_t* lora_a,
                     const uint16_t* lora_b, int32_t r, float alpha, uint16_t* y, float* u_save,
                     void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_weight(w)) || (rc = check_rank(r))) return rc;
  if (m < 0) return set_error(QL_EINVAL, "m < 0");
  if (m == 0) return QL_OK;
  if (!x || !lora_a || !lora_b || !y || !u_save) return set_error(QL_EINVAL, "null pointer");
  if (!aligned16(x) || !aligned16(lora_a) || !aligned16(lora_b) || !aligned16(y) || !aligned16(u_save))
    return set_error(QL_EINVAL, "misaligned pointer");
  size_t need = qlora_workspace_bytes(QL_OP_FWD, w->format, w->n_out, w->k_in, m, r);
  if (ws_bytes < need) return set_error(QL_EWORKSPACE, "forward needs %zu workspace bytes", need);
  if (need && (!ws || !aligned16(ws))) return set_error(QL_EINVAL, "null or misaligned workspace");
  if ((rc = check_sticky())) return rc;
  GemmCall c{};
  c.w = w;
  c.trans = false;
  c.act = x;
  c.m = m;
  c.down = lora_a;
  c.up = lora_b;
  c.r = r;
  c.s = alpha / (float)r;
  c.out = y;
  c.save = u_save;
  c.ws = ws;
  hipError_t e = launch_qgemm(c, as_stream(stream));
  if (e != hipSuccess) return hip_error(e, "forward launch");
  return QL_OK;
}

int qlora_linear_bwd(const ql_qweight* w, const uint16_t* x, const uint16_t* dy, const float* u_save,
                     int64_t m, const uint16_t* lora_a, const uint16_t* lora_b, int32_t r, float alpha,
                     uint16_t* dx, float* d_a, float* d_b, int32_t accumulate, void* ws,
                     size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_weight(w)) || (rc = check_rank(r))) return rc;
  if (m < 0) return set_error(QL_EINVAL, "m < 0");
  // with m == 0 the token-dimension buffers may be empty (null); dA and dB are still written
  if ((m > 0 && (!x || !dy || !u_save)) || !lora_a || !lora_b || !d_a || !d_b || !ws)
    return set_error(QL_EINVAL, "null pointer");
  if (!aligned16(x) || !aligned16(dy) || !aligned16(u_save) || !aligned16(lora_a) || !aligned16(lora_b) ||
      (dx && !aligned16(dx)) || !aligned16(d_a) || !aligned16(d_b) || !aligned16(ws))
    return set_error(QL_EINVAL, "misaligned pointer");
  const int64_t n = w->n_out, k = w->k_in;
  BwdLayout L = bwd_layout(w->format, n, k, m, r);
  if (ws_bytes < L.total) return set_error(QL_EWORKSPACE, "backward needs %zu workspace bytes", L.total);
  if ((rc = check_sticky())) return rc;
  hipStream_t s = as_stream(stream);
  char* base = reinterpret_cast<char*>(ws);
  float* v = reinterpret_cast<float*>(base + L.v);
  float* pa = reinterpret_cast<float*>(base + L.pa);
  float* pb = reinterpret_cast<float*>(base + L.pb);
  const float sc = alpha / (float)r;
  hipError_t e = hipSuccess;
  // at most 64 tokens the dX reduction launch also writes dA and dB
  const bool fuse = m > 0 && dx && split_path_fuses_grads(m);
  GradFuse gf{x, u_save, d_a, d_b, accumulate != 0};
  if (m > 0 && dx) {
    GemmCall c{};
    c.w = w;
    c.trans = true;
    c.act = dy;
    c.m = m;
    c.down = lora_b;
    c.up = lora_a;
    c.r = r;
    c.s = sc;
    c.out = dx;
    c.save = v;
    c.ws = base + L.g;
    c.grads = fuse ? &gf : nullptr;
    e = launch_qgemm(c, s);
  } else if (m > 0) {
    e = launch_down_proj(dy, m, n, lora_b, r, v, s);
  }
  if (e == hipSuccess && !fuse) {
    GradLaunch g{};
    g.x = x;
    g.dy = dy;
    g.v = v;
    g.u = u_save;
    g.d_a = d_a;
    g.d_b = d_b;
    g.part_a = pa;
    g.part_b = pb;
    g.m = m;
    g.k = k;
    g.n = n;
    g.r = r;
    g.nparts = L.parts;
    g.s = sc;
    g.accumulate = accumulate != 0;
    e = launch_grads(g, s);
  }
  if (e != hipSuccess) return hip_error(e, "backward launch");
  return QL_OK;
}

}  // extern "C"
