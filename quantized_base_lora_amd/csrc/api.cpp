// C ABI entry points (include/qlora.h): argument validation, workspace
// layout, and the launch sequence of each call.  No device memory is
// allocated here; scratch comes from the caller's workspace.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <vector>

#include "common.h"
#include "dyn8.h"

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
  if (fmt != QL_FMT_Q4_0 && fmt != QL_FMT_NF4 && fmt != QL_FMT_FP8_E4M3 && fmt != QL_FMT_MXFP4 && fmt != QL_FMT_Q8_0 &&
      fmt != QL_FMT_NVFP4)
    return set_error(QL_EUNSUPPORTED, "unknown format %d", fmt);
  if (n <= 0 || k <= 0) return set_error(QL_EINVAL, "n_out and k_in must be positive");
  if (k % block_of(fmt)) return set_error(QL_EINVAL, "k_in=%lld is not a multiple of %d", (long long)k, block_of(fmt));
  if (n % 32) return set_error(QL_EINVAL, "n_out=%lld is not a multiple of 32", (long long)n);
  // every buffer offset a kernel forms must fit 31 bits: rows of at most
  // QL_MAX_FEATURES elements (a 256-row tile, a 512-row gradient partition and
  // 16 split partials of 64 tokens stay below 2 GiB) and codes below 2 GiB
  if (n > QL_MAX_FEATURES || k > QL_MAX_FEATURES)
    return set_error(QL_EUNSUPPORTED, "n_out=%lld, k_in=%lld: at most %d features per side", (long long)n,
                     (long long)k, QL_MAX_FEATURES);
  const int64_t code_bytes = (fmt == QL_FMT_FP8_E4M3 || fmt == QL_FMT_Q8_0) ? n * k : n * k / 2;
  if (code_bytes > 0x7FFFFFFFLL)
    return set_error(QL_EUNSUPPORTED, "codes of %lld bytes: at most 2 GiB - 1 per weight", (long long)code_bytes);
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


// Arguments of one forward / backward call; the weight descriptor is copied.
struct FwdArgs {
  ql_qweight w;
  const uint16_t* x;
  int64_t m;
  const uint16_t *a, *b;
  int32_t r;
  float alpha;
  uint16_t* y;
  float* u;
  void* ws;
  size_t ws_bytes;
};
struct BwdArgs {
  ql_qweight w;
  const uint16_t *x, *dy;
  const float* u;
  int64_t m;
  const uint16_t *a, *b;
  int32_t r;
  float alpha;
  uint16_t* dx;
  float *da, *db;
  int32_t accumulate;
  void* ws;
  size_t ws_bytes;
};

int check_fwd(const ql_qweight* wp, const FwdArgs& a) {
  int rc;
  if ((rc = check_weight(wp)) || (rc = check_rank(a.r))) return rc;
  if (a.m < 0) return set_error(QL_EINVAL, "m < 0");
  if (a.m == 0) return QL_OK;
  if (!a.x || !a.a || !a.b || !a.y || !a.u) return set_error(QL_EINVAL, "null pointer");
  if (!aligned16(a.x) || !aligned16(a.a) || !aligned16(a.b) || !aligned16(a.y) || !aligned16(a.u))
    return set_error(QL_EINVAL, "misaligned pointer");
  const size_t need = qgemm_workspace_bytes(a.w.format, false, a.m, a.w.n_out, a.w.k_in, a.r);
  if (a.ws_bytes < need) return set_error(QL_EWORKSPACE, "forward needs %zu workspace bytes", need);
  if (need && (!a.ws || !aligned16(a.ws))) return set_error(QL_EINVAL, "null or misaligned workspace");
  return QL_OK;
}

GemmCall fwd_gemm(const FwdArgs& a) {
  GemmCall c{};
  c.w = &a.w;
  c.trans = false;
  c.act = a.x;
  c.m = a.m;
  c.down = a.a;
  c.up = a.b;
  c.r = a.r;
  c.s = a.alpha / (float)a.r;
  c.out = a.y;
  c.save = a.u;
  c.ws = a.ws;
  return c;
}

int enqueue_fwd(const FwdArgs& a, hipStream_t s) {
  if (a.m == 0) return QL_OK;
  hipError_t e = launch_qgemm(fwd_gemm(a), s);
  if (e != hipSuccess) return hip_error(e, "forward launch");
  return QL_OK;
}

int check_bwd(const ql_qweight* wp, const BwdArgs& a) {
  int rc;
  if ((rc = check_weight(wp)) || (rc = check_rank(a.r))) return rc;
  if (a.m < 0) return set_error(QL_EINVAL, "m < 0");
  // with m == 0 the token-dimension buffers may be empty (null); dA and dB are still written
  if ((a.m > 0 && (!a.x || !a.dy || !a.u)) || !a.a || !a.b || !a.da || !a.db || !a.ws)
    return set_error(QL_EINVAL, "null pointer");
  if (!aligned16(a.x) || !aligned16(a.dy) || !aligned16(a.u) || !aligned16(a.a) || !aligned16(a.b) ||
      (a.dx && !aligned16(a.dx)) || !aligned16(a.da) || !aligned16(a.db) || !aligned16(a.ws))
    return set_error(QL_EINVAL, "misaligned pointer");
  const BwdLayout L = bwd_layout(a.w.format, a.w.n_out, a.w.k_in, a.m, a.r);
  if (a.ws_bytes < L.total) return set_error(QL_EWORKSPACE, "backward needs %zu workspace bytes", L.total);
  return QL_OK;
}

// The pieces of a backward call: the dX GEMM (with V and, at most 32 tokens,
// dA and dB fused into its reduction) and the separate adapter-gradient
// launch otherwise.
struct BwdParts {
  BwdLayout L;
  float *v, *pa, *pb;
  bool fuse;
  GradFuse gf;
  GemmCall gemm;
};

void bwd_parts(const BwdArgs& a, BwdParts& b) {
  const int64_t n = a.w.n_out, k = a.w.k_in, m = a.m;
  b.L = bwd_layout(a.w.format, n, k, m, a.r);
  char* base = reinterpret_cast<char*>(a.ws);
  b.v = reinterpret_cast<float*>(base + b.L.v);
  b.pa = reinterpret_cast<float*>(base + b.L.pa);
  b.pb = reinterpret_cast<float*>(base + b.L.pb);
  b.fuse = m > 0 && a.dx && split_path_fuses_grads(m);
  b.gf = GradFuse{a.x, a.u, a.da, a.db, a.accumulate != 0};
  b.gemm = GemmCall{};
  GemmCall& c = b.gemm;
  c.w = &a.w;
  c.trans = true;
  c.act = a.dy;
  c.m = m;
  c.down = a.b;
  c.up = a.a;
  c.r = a.r;
  c.s = a.alpha / (float)a.r;
  c.out = a.dx;
  c.save = b.v;
  c.ws = base + b.L.g;
  c.grads = b.fuse ? &b.gf : nullptr;
}

GradLaunch grad_launch(const BwdArgs& a, const BwdParts& b) {
  GradLaunch g{};
  g.x = a.x;
  g.dy = a.dy;
  g.v = b.v;
  g.u = a.u;
  g.d_a = a.da;
  g.d_b = a.db;
  g.part_a = b.pa;
  g.part_b = b.pb;
  g.m = a.m;
  g.k = a.w.k_in;
  g.n = a.w.n_out;
  g.r = a.r;
  g.nparts = b.L.parts;
  g.s = a.alpha / (float)a.r;
  g.accumulate = a.accumulate != 0;
  return g;
}

// the adapter gradients of n calls: launched now, or (kdefer, launch plans)
// added to the held-back set, which is launched first if they do not fit it.
// Held back only on the small-token path, where a launch costs more than its
// work (the 64-token Llama-3.1-8B step 5 % shorter); with many tokens each
// launch right after its dX GEMM finds dY still in the last-level cache
// (held back to the end of the step, the Qwen3-0.6B layer at 8192 tokens
// ran 1.7 % slower).
hipError_t grads_now_or_held(const GradLaunch* g, int n, hipStream_t s, GradReduceSet* defer,
                             GradKernelSet* kdefer) {
  if (!kdefer || !split_path_tokens(g[0].m)) return launch_grads_group(g, n, s, defer);
  for (int i = 0; i < n; ++i) {
    if (!kdefer->fits(g[i])) {
      hipError_t e = launch_grad_kernels(*kdefer, s, defer);
      if (e != hipSuccess) return e;
    }
    kdefer->g[kdefer->n++] = g[i];
  }
  return hipSuccess;
}

hipError_t bwd_grads(const BwdArgs& a, const BwdParts& b, hipStream_t s, GradReduceSet* defer,
                     GradKernelSet* kdefer) {
  if (b.fuse) return hipSuccess;
  const GradLaunch g = grad_launch(a, b);
  return grads_now_or_held(&g, 1, s, defer, kdefer);
}

// defer: hold the gradient reduction back in that set; kdefer: hold the
// gradient launch itself back (launch plans)
int enqueue_bwd(const BwdArgs& a, hipStream_t s, GradReduceSet* defer = nullptr, GradKernelSet* kdefer = nullptr) {
  BwdParts b;
  bwd_parts(a, b);
  hipError_t e = hipSuccess;
  if (a.m > 0 && a.dx) e = launch_qgemm(b.gemm, s);
  else if (a.m > 0) e = launch_down_proj(a.dy, a.m, a.w.n_out, a.b, a.r, b.v, s);
  if (e == hipSuccess) e = bwd_grads(a, b, s, defer, kdefer);
  if (e != hipSuccess) return hip_error(e, "backward launch");
  return QL_OK;
}

// ---- groups of independent calls (one token count and rank)
bool overlaps(const void* p, size_t pn, const void* q, size_t qn) {
  if (!p || !q || !pn || !qn) return false;
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + qn && b < a + pn;
}

struct Span {
  const void* p;
  size_t n;
};

// every buffer a call reads or writes, and which of them it writes
void fwd_spans(const FwdArgs& a, Span* all, int& na, Span* out, int& no) {
  const int64_t m = a.m, k = a.w.k_in, n = a.w.n_out, r = a.r;
  na = no = 0;
  all[na++] = {a.x, (size_t)(m * k * 2)};
  all[na++] = {a.a, (size_t)(r * k * 2)};
  all[na++] = {a.b, (size_t)(n * r * 2)};
  out[no++] = all[na++] = {a.y, (size_t)(m * n * 2)};
  out[no++] = all[na++] = {a.u, (size_t)(m * r * 4)};
  out[no++] = all[na++] = {a.ws, a.ws_bytes};
}
void bwd_spans(const BwdArgs& a, Span* all, int& na, Span* out, int& no) {
  const int64_t m = a.m, k = a.w.k_in, n = a.w.n_out, r = a.r;
  na = no = 0;
  all[na++] = {a.x, (size_t)(m * k * 2)};
  all[na++] = {a.dy, (size_t)(m * n * 2)};
  all[na++] = {a.u, (size_t)(m * r * 4)};
  all[na++] = {a.a, (size_t)(r * k * 2)};
  all[na++] = {a.b, (size_t)(n * r * 2)};
  out[no++] = all[na++] = {a.dx, a.dx ? (size_t)(m * k * 2) : 0};
  out[no++] = all[na++] = {a.da, (size_t)(r * k * 4)};
  out[no++] = all[na++] = {a.db, (size_t)(n * r * 4)};
  out[no++] = all[na++] = {a.ws, a.ws_bytes};
}

template <class Args, class SpanFn>
int check_independent(const Args* a, int n, SpanFn spans) {
  for (int i = 0; i < n; ++i) {
    Span ai[10], ao[6];
    int nai, nao;
    spans(a[i], ai, nai, ao, nao);
    for (int j = 0; j < n; ++j) {
      if (j == i) continue;
      Span bj[10], bo[6];
      int nbj, nbo;
      spans(a[j], bj, nbj, bo, nbo);
      for (int x = 0; x < nao; ++x)
        for (int y = 0; y < nbj; ++y)
          if (overlaps(ao[x].p, ao[x].n, bj[y].p, bj[y].n))
            return set_error(QL_EINVAL, "group calls %d and %d are not independent (an output of %d overlaps a buffer of %d)",
                             i, j, i, j);
    }
  }
  return QL_OK;
}

int enqueue_fwd_group(const FwdArgs* a, int n, hipStream_t s) {
  if (n <= 0 || a[0].m == 0) return QL_OK;
  GemmCall c[QL_GROUP_MAX];
  for (int i = 0; i < n; ++i) c[i] = fwd_gemm(a[i]);
  hipError_t e = launch_qgemm_group(c, n, s);
  if (e != hipSuccess) return hip_error(e, "grouped forward launch");
  return QL_OK;
}

int enqueue_bwd_group(const BwdArgs* a, int n, hipStream_t s, GradReduceSet* defer = nullptr,
                      GradKernelSet* kdefer = nullptr) {
  bool all_dx = true;
  for (int i = 0; i < n; ++i) all_dx = all_dx && a[i].dx;
  if (n <= 1 || a[0].m == 0 || !all_dx) {
    for (int i = 0; i < n; ++i) {
      int rc = enqueue_bwd(a[i], s, defer, kdefer);
      if (rc) return rc;
    }
    return QL_OK;
  }
  BwdParts b[QL_GROUP_MAX];
  GemmCall c[QL_GROUP_MAX];
  for (int i = 0; i < n; ++i) {
    bwd_parts(a[i], b[i]);
    c[i] = b[i].gemm;
  }
  hipError_t e = launch_qgemm_group(c, n, s);
  if (e == hipSuccess && !b[0].fuse) {   // one token count: all fused or none
    GradLaunch g[QL_GROUP_MAX];
    for (int i = 0; i < n; ++i) g[i] = grad_launch(a[i], b[i]);
    e = grads_now_or_held(g, n, s, defer, kdefer);
  }
  if (e != hipSuccess) return hip_error(e, "grouped backward launch");
  return QL_OK;
}

struct PlanStep {
  enum Kind { FWD, BWD, EVENT, FWD_GROUP, BWD_GROUP } kind;
  FwdArgs fwd;
  BwdArgs bwd;
  hipEvent_t event;
  std::vector<FwdArgs> fwds;
  std::vector<BwdArgs> bwds;
};

FwdArgs fwd_args(const ql_fwd_call& c, int64_t m, int32_t r) {
  return FwdArgs{c.w ? *c.w : ql_qweight{}, c.x, m, c.lora_a, c.lora_b, r, c.alpha, c.y, c.u_save, c.ws, c.ws_bytes};
}
BwdArgs bwd_args(const ql_bwd_call& c, int64_t m, int32_t r) {
  return BwdArgs{c.w ? *c.w : ql_qweight{}, c.x, c.dy, c.u_save, m, c.lora_a, c.lora_b, r, c.alpha,
                 c.dx, c.d_a, c.d_b, c.accumulate, c.ws, c.ws_bytes};
}

// validates a group: count, every call as a single call, one format, and independence
int check_fwd_group(const ql_fwd_call* calls, int32_t n, int64_t m, int32_t r, std::vector<FwdArgs>& out) {
  if (n < 1 || n > QL_GROUP_MAX) return set_error(QL_EINVAL, "group size %d outside [1, %d]", n, QL_GROUP_MAX);
  if (!calls) return set_error(QL_EINVAL, "null calls");
  out.clear();
  for (int i = 0; i < n; ++i) {
    if (calls[i].reserved != 0) return set_error(QL_EINVAL, "call %d: reserved must be 0", i);
    out.push_back(fwd_args(calls[i], m, r));
    int rc = check_fwd(calls[i].w, out.back());
    if (rc) return rc;
    if (out.back().w.format != out[0].w.format) return set_error(QL_EINVAL, "group mixes base formats");
  }
  return check_independent(out.data(), n, fwd_spans);
}
int check_bwd_group(const ql_bwd_call* calls, int32_t n, int64_t m, int32_t r, std::vector<BwdArgs>& out) {
  if (n < 1 || n > QL_GROUP_MAX) return set_error(QL_EINVAL, "group size %d outside [1, %d]", n, QL_GROUP_MAX);
  if (!calls) return set_error(QL_EINVAL, "null calls");
  out.clear();
  for (int i = 0; i < n; ++i) {
    out.push_back(bwd_args(calls[i], m, r));
    int rc = check_bwd(calls[i].w, out.back());
    if (rc) return rc;
    if (out.back().w.format != out[0].w.format) return set_error(QL_EINVAL, "group mixes base formats");
  }
  return check_independent(out.data(), n, bwd_spans);
}

}  // namespace
}  // namespace ql

using namespace ql;

struct ql_plan {
  std::vector<PlanStep> steps;
};

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
  } else if (format == QL_FMT_NVFP4) {
    e = launch_pack_nvfp4(w, n_out, k_in, codes, scales, st, s);
  } else {
    e = launch_zero_u32(st, 2, s);
    if (e == hipSuccess) e = launch_pack_blocks(format, w, n_out, k_in, codes, scales, st + 1, s);
  }
  if (e != hipSuccess) return hip_error(e, "quant_pack launch");
  QL_HIP(hipStreamSynchronize(s));
  uint32_t flags[2] = {0, 0};
  QL_HIP(hipMemcpy(flags, ws, sizeof flags, hipMemcpyDeviceToHost));
  uint32_t f = flags[1];
  if (f & 1u) return set_error(QL_ENONFINITE, "base weight holds NaN or Inf");
  if (f & 2u) return set_error(QL_EOVERFLOW, "a block scale overflows fp16");
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

int ql_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return set_error(QL_EINVAL, "null pointer");
  if (bytes <= 0 || bytes % 16) return set_error(QL_EINVAL, "bytes=%lld: need a positive multiple of 16", (long long)bytes);
  if (!aligned16(buf) || ((uintptr_t)sink & 3u)) return set_error(QL_EINVAL, "misaligned pointer");
  int rc = check_sticky();
  if (rc) return rc;
  hipError_t e = launch_stream_read(buf, bytes, sink, as_stream(stream));
  if (e != hipSuccess) return hip_error(e, "stream read launch");
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

int ql_stack_adapters(const ql_adapter* adapters, int32_t n, int64_t n_out, int64_t k_in, uint16_t* a_cat,
                      uint16_t* b_cat, float* alpha_cat, void* stream) {
  if (n < 2 || n > QL_STACK_MAX) return set_error(QL_EINVAL, "stack of %d adapters outside [2, %d]", n, QL_STACK_MAX);
  if (!adapters || !a_cat || !b_cat || !alpha_cat) return set_error(QL_EINVAL, "null pointer");
  if (n_out <= 0 || k_in <= 0) return set_error(QL_EINVAL, "n_out and k_in must be positive");
  if (!aligned16(a_cat) || !aligned16(b_cat)) return set_error(QL_EINVAL, "misaligned output");
  int32_t R = 0;
  for (int i = 0; i < n; ++i) {
    const ql_adapter& a = adapters[i];
    if (!a.lora_a || !a.lora_b || !aligned16(a.lora_a) || !aligned16(a.lora_b))
      return set_error(QL_EINVAL, "adapter %d: null or misaligned pointer", i);
    if (a.r < 1 || a.r > 32) return set_error(QL_EINVAL, "adapter %d: rank %d", i, a.r);
    if (!(a.alpha > 0.0f) || !(a.alpha - a.alpha == 0.0f))
      return set_error(QL_EINVAL, "adapter %d: alpha must be finite and positive", i);
    R += a.r;
  }
  if (R != 8 && R != 16 && R != 32) return set_error(QL_EUNSUPPORTED, "stacked rank %d not in {8,16,32}", R);
  int rc = check_sticky();
  if (rc) return rc;
  hipError_t e = launch_stack(adapters, n, n_out, k_in, a_cat, b_cat, alpha_cat, as_stream(stream));
  if (e != hipSuccess) return hip_error(e, "stack launch");
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

// hyperparameters shared by both AdamW variants
static int check_adamw_hparams(const ql_adamw_hparams* hp) {
  if (hp->step < 1) return set_error(QL_EINVAL, "step must be >= 1");
  if (hp->reserved != 0) return set_error(QL_EINVAL, "hparams.reserved must be 0");
  const double f[6] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->grad_scale};
  for (double v : f)
    if (!(v - v == 0.0)) return set_error(QL_EINVAL, "non-finite hyperparameter");
  if (hp->lr < 0.0 || hp->eps < 0.0 || hp->weight_decay < 0.0)
    return set_error(QL_EINVAL, "lr, eps and weight_decay must be >= 0");
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0 && hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return set_error(QL_EINVAL, "beta1 and beta2 must lie in [0, 1)");
  return QL_OK;
}

int ql_adamw8_step(const ql_adamw8_tensor* tensors, int32_t n_tensors, const ql_adamw_hparams* hp,
                   void* stream) {
  if (n_tensors < 0 || n_tensors > QL_ADAMW_MAX_TENSORS)
    return set_error(QL_EINVAL, "n_tensors=%d outside [0, %d]", n_tensors, QL_ADAMW_MAX_TENSORS);
  if (!hp || (n_tensors > 0 && !tensors)) return set_error(QL_EINVAL, "null pointer");
  int rc = check_adamw_hparams(hp);
  if (rc) return rc;
  for (int32_t i = 0; i < n_tensors; ++i) {
    const ql_adamw8_tensor& t = tensors[i];
    if (t.n < 0 || t.n % 8) return set_error(QL_EINVAL, "tensor %d: n=%lld is not a multiple of 8", i, (long long)t.n);
    if (t.n == 0) continue;
    if (!t.param || !t.grad || !t.exp_avg || !t.exp_avg_absmax || !t.exp_avg_sq || !t.exp_avg_sq_absmax)
      return set_error(QL_EINVAL, "tensor %d: null pointer", i);
    if (!aligned16(t.param) || !aligned16(t.grad) || (t.param_bf16 && !aligned16(t.param_bf16)) ||
        ((uintptr_t)t.exp_avg & 7u) || ((uintptr_t)t.exp_avg_sq & 7u) || ((uintptr_t)t.exp_avg_absmax & 3u) ||
        ((uintptr_t)t.exp_avg_sq_absmax & 3u))
      return set_error(QL_EINVAL, "tensor %d: misaligned pointer", i);
  }
  if ((rc = check_sticky())) return rc;
  hipError_t e = launch_adamw8(tensors, n_tensors, *hp, as_stream(stream));
  if (e != hipSuccess) return hip_error(e, "adamw8 launch");
  return QL_OK;
}

int ql_dyn8_levels(int32_t is_signed, float* out) {
  if (!out) return set_error(QL_EINVAL, "null output");
  const Dyn8Table& t = dyn8_table(is_signed != 0);
  memcpy(out, t.level, (size_t)t.count * sizeof(float));
  return QL_OK;
}

int qlora_linear_fwd(const ql_qweight* w, const uint16_t* x, int64_t m, const uint16_t* lora_a,
                     const uint16_t* lora_b, int32_t r, float alpha, uint16_t* y, float* u_save,
                     void* ws, size_t ws_bytes, void* stream) {
  FwdArgs a{w ? *w : ql_qweight{}, x, m, lora_a, lora_b, r, alpha, y, u_save, ws, ws_bytes};
  int rc = check_fwd(w, a);
  if (rc || m == 0) return rc;
  if ((rc = check_sticky())) return rc;
  return enqueue_fwd(a, as_stream(stream));
}

int qlora_linear_bwd(const ql_qweight* w, const uint16_t* x, const uint16_t* dy, const float* u_save,
                     int64_t m, const uint16_t* lora_a, const uint16_t* lora_b, int32_t r, float alpha,
                     uint16_t* dx, float* d_a, float* d_b, int32_t accumulate, void* ws,
                     size_t ws_bytes, void* stream) {
  BwdArgs a{w ? *w : ql_qweight{}, x, dy, u_save, m, lora_a, lora_b, r, alpha, dx, d_a, d_b, accumulate, ws,
            ws_bytes};
  int rc = check_bwd(w, a);
  if (rc) return rc;
  if ((rc = check_sticky())) return rc;
  return enqueue_bwd(a, as_stream(stream));
}

int qlora_linear_fwd_group(const ql_fwd_call* calls, int32_t n, int64_t m, int32_t r, void* stream) {
  std::vector<FwdArgs> a;
  int rc = check_fwd_group(calls, n, m, r, a);
  if (rc || m == 0) return rc;
  if ((rc = check_sticky())) return rc;
  return enqueue_fwd_group(a.data(), n, as_stream(stream));
}

int qlora_linear_bwd_group(const ql_bwd_call* calls, int32_t n, int64_t m, int32_t r, void* stream) {
  std::vector<BwdArgs> a;
  int rc = check_bwd_group(calls, n, m, r, a);
  if (rc) return rc;
  if ((rc = check_sticky())) return rc;
  return enqueue_bwd_group(a.data(), n, as_stream(stream));
}

// ---------------------------------------------------------------- launch plans
int ql_plan_create(ql_plan** plan) {
  if (!plan) return set_error(QL_EINVAL, "null plan pointer");
  *plan = new (std::nothrow) ql_plan();
  if (!*plan) return set_error(QL_EINVAL, "out of host memory");
  return QL_OK;
}

int ql_plan_add_fwd(ql_plan* plan, const ql_qweight* w, const uint16_t* x, int64_t m,
                    const uint16_t* lora_a, const uint16_t* lora_b, int32_t r, float alpha, uint16_t* y,
                    float* u_save, void* ws, size_t ws_bytes) {
  if (!plan) return set_error(QL_EINVAL, "null plan");
  FwdArgs a{w ? *w : ql_qweight{}, x, m, lora_a, lora_b, r, alpha, y, u_save, ws, ws_bytes};
  int rc = check_fwd(w, a);
  if (rc) return rc;
  PlanStep st{};
  st.kind = PlanStep::FWD;
  st.fwd = a;
  plan->steps.push_back(st);
  return QL_OK;
}

int ql_plan_add_bwd(ql_plan* plan, const ql_qweight* w, const uint16_t* x, const uint16_t* dy,
                    const float* u_save, int64_t m, const uint16_t* lora_a, const uint16_t* lora_b, int32_t r,
                    float alpha, uint16_t* dx, float* d_a, float* d_b, int32_t accumulate, void* ws,
                    size_t ws_bytes) {
  if (!plan) return set_error(QL_EINVAL, "null plan");
  BwdArgs a{w ? *w : ql_qweight{}, x, dy, u_save, m, lora_a, lora_b, r, alpha, dx, d_a, d_b, accumulate, ws,
            ws_bytes};
  int rc = check_bwd(w, a);
  if (rc) return rc;
  PlanStep st{};
  st.kind = PlanStep::BWD;
  st.bwd = a;
  plan->steps.push_back(st);
  return QL_OK;
}

int ql_plan_add_fwd_group(ql_plan* plan, const ql_fwd_call* calls, int32_t n, int64_t m, int32_t r) {
  if (!plan) return set_error(QL_EINVAL, "null plan");
  PlanStep st{};
  st.kind = PlanStep::FWD_GROUP;
  int rc = check_fwd_group(calls, n, m, r, st.fwds);
  if (rc) return rc;
  plan->steps.push_back(std::move(st));
  return QL_OK;
}

int ql_plan_add_bwd_group(ql_plan* plan, const ql_bwd_call* calls, int32_t n, int64_t m, int32_t r) {
  if (!plan) return set_error(QL_EINVAL, "null plan");
  PlanStep st{};
  st.kind = PlanStep::BWD_GROUP;
  int rc = check_bwd_group(calls, n, m, r, st.bwds);
  if (rc) return rc;
  plan->steps.push_back(std::move(st));
  return QL_OK;
}

int ql_plan_add_event(ql_plan* plan, void* event) {
  if (!plan || !event) return set_error(QL_EINVAL, "null plan or event");
  PlanStep st{};
  st.kind = PlanStep::EVENT;
  st.event = reinterpret_cast<hipEvent_t>(event);
  plan->steps.push_back(st);
  return QL_OK;
}

int ql_plan_size(const ql_plan* plan) { return plan ? (int)plan->steps.size() : 0; }

int ql_plan_run(ql_plan* plan, void* stream) {
  if (!plan) return set_error(QL_EINVAL, "null plan");
  int rc = check_sticky();
  if (rc) return rc;
  hipStream_t s = as_stream(stream);
  // The adapter-gradient launches of backward steps, and their reductions,
  // are held back and run as one launch each: before the first later step
  // that touches a buffer they write (dA, dB, partials in a backward
  // workspace) or writes a buffer they read (x, dY, U, and V in a backward
  // workspace), before an event, and at the end of the plan.  They are the
  // same kernels on the same data (a problem's result does not depend on the
  // others in a launch), so results are bitwise those of the calls made one
  // by one.
  GradReduceSet pend;
  GradKernelSet kpend;
  for (const PlanStep& st : plan->steps) {
    bool kflush = st.kind == PlanStep::EVENT;
    if (!kflush && kpend.n > 0) {
      std::vector<Span> all, out;
      auto add = [&](const Span* ai, int na, const Span* ao, int no) {
        all.insert(all.end(), ai, ai + na);
        out.insert(out.end(), ao, ao + no);
      };
      Span ai[10], ao[6];
      int na, no;
      if (st.kind == PlanStep::FWD) { fwd_spans(st.fwd, ai, na, ao, no); add(ai, na, ao, no); }
      if (st.kind == PlanStep::BWD) { bwd_spans(st.bwd, ai, na, ao, no); add(ai, na, ao, no); }
      for (const FwdArgs& f : st.fwds) { fwd_spans(f, ai, na, ao, no); add(ai, na, ao, no); }
      for (const BwdArgs& b : st.bwds) { bwd_spans(b, ai, na, ao, no); add(ai, na, ao, no); }
      for (int i = 0; i < kpend.n && !kflush; ++i) {
        const GradLaunch& g = kpend.g[i];
        const size_t r4 = (size_t)g.r * 4;
        const Span reads[4] = {{g.x, (size_t)(g.m * g.k * 2)}, {g.dy, (size_t)(g.m * g.n * 2)},
                               {g.v, (size_t)g.m * r4}, {g.u, (size_t)g.m * r4}};
        const Span writes[4] = {{g.d_a, (size_t)g.k * r4}, {g.d_b, (size_t)g.n * r4},
                                {g.part_a, g.nparts > 1 ? (size_t)g.nparts * g.k * r4 : 0},
                                {g.part_b, g.nparts > 1 ? (size_t)g.nparts * g.n * r4 : 0}};
        for (const Span& x : out)
          for (const Span& y : reads) kflush = kflush || overlaps(x.p, x.n, y.p, y.n);
        for (const Span& x : all)
          for (const Span& y : writes) kflush = kflush || overlaps(x.p, x.n, y.p, y.n);
      }
    }
    if (kflush && kpend.n > 0) {
      hipError_t e = launch_grad_kernels(kpend, s, &pend);
      if (e != hipSuccess) return hip_error(e, "plan gradient launch");
    }
    bool flush = st.kind == PlanStep::EVENT;
    if (!flush && pend.n > 0) {
      std::vector<Span> all, out;
      auto add_fwd = [&](const FwdArgs& f) {
        Span ai[10], ao[6];
        int na, no;
        fwd_spans(f, ai, na, ao, no);
        all.insert(all.end(), ai, ai + na);
        out.insert(out.end(), ao, ao + no);
      };
      auto add_bwd = [&](const BwdArgs& b) {
        Span ai[10], ao[6];
        int na, no;
        bwd_spans(b, ai, na, ao, no);
        all.insert(all.end(), ai, ai + na);
        out.insert(out.end(), ao, ao + no);
      };
      if (st.kind == PlanStep::FWD) add_fwd(st.fwd);
      if (st.kind == PlanStep::BWD) add_bwd(st.bwd);
      for (const FwdArgs& f : st.fwds) add_fwd(f);
      for (const BwdArgs& b : st.bwds) add_bwd(b);
      for (int i = 0; i < pend.n && !flush; ++i) {
        const GradReduceSet::Item& it = pend.item[i];
        const size_t ob = (size_t)it.pdim * pend.r * 4, pb = ob * pend.nparts;
        for (const Span& x : all) flush = flush || overlaps(x.p, x.n, it.out, ob);
        for (const Span& x : out) flush = flush || overlaps(x.p, x.n, it.part, pb);
      }
    }
    if (flush && pend.n > 0) {
      hipError_t e = launch_grad_reduce(pend, s);
      if (e != hipSuccess) return hip_error(e, "plan gradient reduction");
    }
    switch (st.kind) {
      case PlanStep::FWD: rc = enqueue_fwd(st.fwd, s); break;
      case PlanStep::BWD: rc = enqueue_bwd(st.bwd, s, &pend, &kpend); break;
      case PlanStep::FWD_GROUP: rc = enqueue_fwd_group(st.fwds.data(), (int)st.fwds.size(), s); break;
      case PlanStep::BWD_GROUP: rc = enqueue_bwd_group(st.bwds.data(), (int)st.bwds.size(), s, &pend, &kpend); break;
      default: {
        hipError_t e = hipEventRecord(st.event, s);
        rc = e == hipSuccess ? QL_OK : hip_error(e, "plan event record");
      }
    }
    if (rc) return rc;
  }
  hipError_t e = launch_grad_kernels(kpend, s, &pend);
  if (e != hipSuccess) return hip_error(e, "plan gradient launch");
  e = launch_grad_reduce(pend, s);
  return e == hipSuccess ? QL_OK : hip_error(e, "plan gradient reduction");
}

int ql_plan_destroy(ql_plan* plan) {
  delete plan;
  return QL_OK;
}

}  // extern "C"
