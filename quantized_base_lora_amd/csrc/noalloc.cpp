// qlora_linear_bwd_noalloc: the backward call for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its scratch (V, the adapter-gradient
// partials and the dX GEMM's split partials) lives in a file-scope device
// array of fixed size instead of a caller-supplied workspace; the kernels
// and their launch configuration are those of qlora_linear_bwd.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, from module load until the process ends.  Host code never uses
// the array's name as an address (on the host it is only a stand-in for the
// symbol): the device address is looked up once per device with
// hipGetSymbolAddress and kept.  Every call on a GPU shares that GPU's
// array, so calls that overlap in time on one GPU (different streams, or
// host threads) race on it; the caller must order them.  The backward
// kernels write every scratch element they later read, so nothing needs
// clearing between calls.
#include <mutex>

#include "common.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[QL_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// the current device's address of `scratch`, looked up on the first call on
// that device (with it current) and kept
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ql::hip_error(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return ql::set_error(QL_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return ql::hip_error(e, "hipGetSymbolAddress(scratch)");
    if (!p) return ql::set_error(QL_EHIP, "hipGetSymbolAddress(scratch) returned null");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return QL_OK;
}

}  // namespace

extern "C" int qlora_linear_bwd_noalloc(const ql_qweight* w, const uint16_t* x, const uint16_t* dy,
                                        const float* u_save, int64_t m, const uint16_t* lora_a,
                                        const uint16_t* lora_b, int32_t r, float alpha, uint16_t* dx,
                                        float* d_a, float* d_b, int32_t accumulate, void* stream) {
  if (!w) return ql::set_error(QL_EINVAL, "null weight");
  if (m < 0) return ql::set_error(QL_EINVAL, "m < 0");
  const size_t need = qlora_workspace_bytes(QL_OP_BWD, w->format, w->n_out, w->k_in, m, r);
  if (need > (size_t)QL_NOALLOC_SCRATCH_BYTES)
    return ql::set_error(QL_EUNSUPPORTED,
                         "backward of this shape needs %zu scratch bytes; the allocation-free call has %d",
                         need, QL_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  int rc = scratch_address(&ws);
  if (rc) return rc;
  return qlora_linear_bwd(w, x, dy, u_save, m, lora_a, lora_b, r, alpha, dx, d_a, d_b, accumulate, ws,
                          (size_t)QL_NOALLOC_SCRATCH_BYTES, stream);
}
