// a10: per-layer stream of the frozen base from pinned host memory into a
// small pool of pre-allocated VRAM slots, one layer ahead, on a side stream
// (Soup page, opening paragraph: the base is only read, so it only has to
// arrive before the matmul that uses it; peak VRAM becomes one layer per
// slot instead of the whole model).
//
// Ordering is carried by two events per slot: `ready` (recorded on the copy
// stream after the copy into the slot) and `freed` (recorded on the compute
// stream when the slot's readers have been enqueued).  A copy into a slot
// waits for its `freed` event; a reader waits for its `ready` event.  The
// pool never allocates device or host memory.
#include <chrono>
#include <thread>
#include <vector>

#include "common.h"

namespace ql {
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t s);
}

using namespace ql;

namespace {
enum SlotState { EMPTY, PENDING, ACQUIRED, RELEASED };

struct Slot {
  int layer = -1;
  SlotState state = EMPTY;
  hipEvent_t ready = nullptr;
  hipEvent_t freed = nullptr;
  bool freed_recorded = false;
  uint64_t release_tick = 0;
};

// test hook: the delay travels in the pointer argument itself, so the host
// function reads no pool memory (the pool may be gone by the time it runs)
void sleep_host(void* arg) {
  const int us = (int)reinterpret_cast<intptr_t>(arg);
  std::this_thread::sleep_for(std::chrono::microseconds(us));
}
}  // namespace

struct ql_pool {
  std::vector<void*> slot_dev;
  size_t slot_bytes = 0;
  std::vector<const void*> layer_host;
  std::vector<size_t> layer_bytes;
  std::vector<Slot> slots;
  std::vector<int> layer_slot;
  uint64_t tick = 0;
  int64_t hits = 0, copies = 0, bytes = 0;
  int delay_us = 0, poison = 0, skip_wait = 0;
};

extern "C" {

int ql_pool_create(ql_pool** pool, int32_t n_slots, void* const* slot_dev, size_t slot_bytes,
                   int32_t n_layers, const void* const* layer_host, const size_t* layer_bytes) {
  if (!pool) return set_error(QL_EINVAL, "null pool out-pointer");
  *pool = nullptr;
  if (n_slots < 1 || n_layers < 1 || !slot_dev || !layer_host || !layer_bytes || slot_bytes == 0)
    return set_error(QL_EINVAL, "bad pool arguments");
  for (int i = 0; i < n_slots; ++i)
    if (!slot_dev[i] || ((uintptr_t)slot_dev[i] & 255u)) return set_error(QL_EINVAL, "slot %d null or not 256-byte aligned", i);
  for (int l = 0; l < n_layers; ++l) {
    if (!layer_host[l]) return set_error(QL_EINVAL, "layer %d host image is null", l);
    if (layer_bytes[l] > slot_bytes) return set_error(QL_EINVAL, "layer %d (%zu B) exceeds slot size", l, layer_bytes[l]);
  }
  ql_pool* p = new ql_pool();
  p->slot_dev.assign(slot_dev, slot_dev + n_slots);
  p->slot_bytes = slot_bytes;
  p->layer_host.assign(layer_host, layer_host + n_layers);
  p->layer_bytes.assign(layer_bytes, layer_bytes + n_layers);
  p->slots.resize(n_slots);
  p->layer_slot.assign(n_layers, -1);
  for (auto& s : p->slots) {
    hipError_t e = hipEventCreateWithFlags(&s.ready, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&s.freed, hipEventDisableTiming);
    if (e != hipSuccess) {
      ql_pool_destroy(p);
      return hip_error(e, "pool event create");
    }
  }
  *pool = p;
  return QL_OK;
}

int layer_stream_prefetch(ql_pool* p, int32_t layer, void* copy_stream) {
  if (!p) return set_error(QL_EINVAL, "null pool");
  if (layer < 0 || layer >= (int)p->layer_slot.size()) return set_error(QL_EINVAL, "layer %d out of range", layer);
  int si = p->layer_slot[layer];
  if (si >= 0) {                                        // resident or in flight
    Slot& s = p->slots[si];
    if (s.state == RELEASED) s.state = PENDING;         // protect it from eviction until used
    ++p->hits;
    return QL_OK;
  }
  int pick = -1;
  for (int i = 0; i < (int)p->slots.size(); ++i)
    if (p->slots[i].state == EMPTY) { pick = i; break; }
  if (pick < 0)
    for (int i = 0; i < (int)p->slots.size(); ++i)
      if (p->slots[i].state == RELEASED && (pick < 0 || p->slots[i].release_tick < p->slots[pick].release_tick)) pick = i;
  if (pick < 0) return set_error(QL_ESTATE, "no free slot for layer %d: every slot is pending or acquired", layer);
  Slot& s = p->slots[pick];
  hipStream_t cs = reinterpret_cast<hipStream_t>(copy_stream);
  if (s.freed_recorded) QL_HIP(hipStreamWaitEvent(cs, s.freed, 0));
  if (s.layer >= 0) p->layer_slot[s.layer] = -1;
  if (p->poison) {
    hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(p->slot_dev[pick]),
                                   (int64_t)(p->slot_bytes / 4), 0xFFFFFFFFu, cs);
    if (e != hipSuccess) return hip_error(e, "pool poison fill");
  }
  if (p->delay_us > 0)
    QL_HIP(hipLaunchHostFunc(cs, sleep_host, reinterpret_cast<void*>((intptr_t)p->delay_us)));
  const size_t nb = p->layer_bytes[layer];
  QL_HIP(hipMemcpyAsync(p->slot_dev[pick], p->layer_host[layer], nb, hipMemcpyHostToDevice, cs));
  QL_HIP(hipEventRecord(s.ready, cs));
  s.layer = layer;
  s.state = PENDING;
  p->layer_slot[layer] = pick;
  ++p->copies;
  p->bytes += (int64_t)nb;
  return QL_OK;
}

int ql_pool_acquire(ql_pool* p, int32_t layer, void* compute_stream, void** slot_dev) {
  if (!p || !slot_dev) return set_error(QL_EINVAL, "null argument");
  if (layer < 0 || layer >= (int)p->layer_slot.size()) return set_error(QL_EINVAL, "layer %d out of range", layer);
  int si = p->layer_slot[layer];
  if (si < 0) return set_error(QL_ESTATE, "layer %d was not prefetched", layer);
  Slot& s = p->slots[si];
  if (s.state == ACQUIRED) return set_error(QL_ESTATE, "layer %d is already acquired", layer);
  if (!p->skip_wait) QL_HIP(hipStreamWaitEvent(reinterpret_cast<hipStream_t>(compute_stream), s.ready, 0));
  s.state = ACQUIRED;
  *slot_dev = p->slot_dev[si];
  return QL_OK;
}

int ql_pool_release(ql_pool* p, int32_t layer, void* compute_stream) {
  if (!p) return set_error(QL_EINVAL, "null pool");
  if (layer < 0 || layer >= (int)p->layer_slot.size()) return set_error(QL_EINVAL, "layer %d out of range", layer);
  int si = p->layer_slot[layer];
  if (si < 0 || p->slots[si].state != ACQUIRED) return set_error(QL_ESTATE, "layer %d is not acquired", layer);
  Slot& s = p->slots[si];
  QL_HIP(hipEventRecord(s.freed, reinterpret_cast<hipStream_t>(compute_stream)));
  s.freed_recorded = true;
  s.state = RELEASED;
  s.release_tick = ++p->tick;
  return QL_OK;
}

int ql_pool_stats(const ql_pool* p, int64_t* out3) {
  if (!p || !out3) return set_error(QL_EINVAL, "null argument");
  out3[0] = p->hits;
  out3[1] = p->copies;
  out3[2] = p->bytes;
  return QL_OK;
}

int ql_pool_debug(ql_pool* p, int32_t delay_us, int32_t poison, int32_t skip_wait) {
  if (!p) return set_error(QL_EINVAL, "null pool");
  if (delay_us < 0 || delay_us > 10000000) return set_error(QL_EINVAL, "delay_us out of range");
  p->delay_us = delay_us;
  p->poison = poison;
  p->skip_wait = skip_wait;
  return QL_OK;
}

// Waits until every copy the pool enqueued has finished (each slot's last
// ready event), so no queued copy or test hook outlives the pool's events.
int ql_pool_destroy(ql_pool* p) {
  if (!p) return QL_OK;
  hipError_t first = hipSuccess;
  for (auto& s : p->slots)
    if (s.ready && s.state != EMPTY) {
      hipError_t e = hipEventSynchronize(s.ready);
      if (first == hipSuccess) first = e;
    }
  for (auto& s : p->slots) {
    if (s.ready) (void)hipEventDestroy(s.ready);
    if (s.freed) (void)hipEventDestroy(s.freed);
  }
  delete p;
  return first == hipSuccess ? QL_OK : hip_error(first, "pool destroy: waiting for queued copies");
}

}  // extern "C"
