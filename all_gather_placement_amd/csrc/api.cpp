// Entry points of the reduce-scatter and all-gather placement: argument checks, the per-call
// device pointer table, and dispatch to the gfx950 kernels or to the DMA engines.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <utility>
#include <vector>

#include "../../include/tide.h"
#include "layout.h"

namespace tide {
namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

// True when some output range overlaps another output range or any input range.  Inputs may
// overlap each other (C identical contributors are legal).
bool outputs_overlap(std::vector<Range> outs, const std::vector<Range>& ins) {
  std::sort(outs.begin(), outs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < outs.size(); ++i)
    if (outs[i].lo < outs[i - 1].hi) return true;
  for (const Range& in : ins) {
    // first output whose end is beyond in.lo
    auto it = std::upper_bound(outs.begin(), outs.end(), in.lo,
                               [](uintptr_t v, const Range& r) { return v < r.hi; });
    // outs are sorted and disjoint, so their `hi` values are sorted too
    if (it != outs.end() && it->lo < in.hi) return true;
  }
  return false;
}

tide_status hip_fail(int err) {
  set_last_hip_error(err);
  return err == hipErrorOutOfMemory ? TIDE_ERR_NOMEM : TIDE_ERR_HIP;
}

// Stage `n` device pointers for a launch on `stream`; returns the slot that holds them.
int acquire_ptrs(DeviceState* st, void* const* ptrs, size_t n, hipStream_t stream, PtrSlot** out) {
  // A slot that already holds this exact table and was last used on this stream can be reused
  // without a copy: stream order keeps its earlier readers ahead of the new launch.  Calls that
  // alternate between tables (an RS and an AG on the same group) hit different slots.
  for (int k = 0; k < kPtrSlots; ++k) {
    PtrSlot& s = st->slots[k];
    if (s.n == n && s.host != nullptr && s.stream == stream &&
        std::memcmp(s.host, ptrs, n * sizeof(void*)) == 0) {
      *out = &s;
      return hipSuccess;
    }
  }
  const int idx = st->next;
  PtrSlot& s = st->slots[idx];
  hipError_t e;
  if (s.pending) {
    if ((e = hipEventSynchronize(s.done)) != hipSuccess) return e;
    s.pending = false;
  }
  if (s.done == nullptr) {
    if ((e = hipEventCreateWithFlags(&s.done, hipEventDisableTiming)) != hipSuccess) return e;
  }
  if (s.cap < n) {
    if (s.dev) (void)hipFree(s.dev);
    if (s.host) (void)hipHostFree(s.host);
    s.dev = nullptr;
    s.host = nullptr;
    s.cap = 0;
    size_t cap = std::max<size_t>(n, 256);
    if ((e = hipMalloc(reinterpret_cast<void**>(&s.dev), cap * sizeof(void*))) != hipSuccess) return e;
    if ((e = hipHostMalloc(reinterpret_cast<void**>(&s.host), cap * sizeof(void*), hipHostMallocDefault)) !=
        hipSuccess) {
      (void)hipFree(s.dev);
      s.dev = nullptr;
      return e;
    }
    s.cap = cap;
  }
  std::memcpy(s.host, ptrs, n * sizeof(void*));
  s.n = n;
  s.stream = stream;
  if ((e = hipMemcpyAsync(s.dev, s.host, n * sizeof(void*), hipMemcpyHostToDevice, stream)) != hipSuccess) {
    s.n = 0;
    return e;
  }
  st->next = (idx + 1) % kPtrSlots;
  *out = &s;
  return hipSuccess;
}

int release_ptrs(PtrSlot* s, hipStream_t stream) {
  hipError_t e = hipEventRecord(s->done, stream);
  if (e == hipSuccess) s->pending = true;
  return e;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Create the internal copy streams and their fork/join events on first use (layout mutex held).
int ensure_dma(DeviceState* st) {
  hipError_t e;
  if (st->dma_fork == nullptr &&
      (e = hipEventCreateWithFlags(&st->dma_fork, hipEventDisableTiming)) != hipSuccess)
    return e;
  for (int k = 0; k < kDmaStreams; ++k) {
    if (st->dma[k] == nullptr && (e = hipStreamCreateWithFlags(&st->dma[k], hipStreamNonBlocking)) != hipSuccess)
      return e;
    if (st->dma_join[k] == nullptr &&
        (e = hipEventCreateWithFlags(&st->dma_join[k], hipEventDisableTiming)) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

// Launch plan for `count` work items: cu_budget 0 = one item per workgroup in one launch;
// B > 0 = grids of at most `max_wgs` workgroups, each taking `bounded_items` items and exiting
// (bounded_items 0: one launch, workgroups walk every item).
struct Plan {
  int grid;
  int items;
  int64_t per_launch;
};

Plan plan_for(int64_t count, int32_t cu_budget, int64_t max_wgs, int bounded_items) {
  if (cu_budget <= 0) {
    const int64_t cap = kPersistentWorkgroups > 0 ? kPersistentWorkgroups : (int64_t(1) << 30);
    const int64_t g = std::min<int64_t>(count, cap);
    const int items = int((count + g - 1) / g);
    return Plan{int(g), items, int64_t(g) * items};
  }
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(count, max_wgs));
  const int64_t items = bounded_items > 0 ? bounded_items : (count + grid - 1) / grid;
  return Plan{int(grid), int(items), grid * items};
}

}  // namespace
}  // namespace tide

using tide::Range;

extern "C" {

tide_status tide_rs_bf16_to_fp32(const tide_layout* layout, int32_t C, const void* const* grads,
                                 float* const* shards, int32_t cu_budget, void* stream) {
  if (layout == nullptr || grads == nullptr || shards == nullptr || C < 1 || cu_budget < 0)
    return TIDE_ERR_INVALID;
  const int32_t P = layout->P, R = layout->R;
  const int64_t S = layout->S;
  if (int64_t(C) * P > (int64_t(1) << 24)) return TIDE_ERR_INVALID;

  bool vec = true;
  std::vector<Range> ins, outs;
  ins.reserve(size_t(C) * P);
  outs.reserve(R);
  for (int32_t c = 0; c < C; ++c) {
    for (int32_t p = 0; p < P; ++p) {
      const void* g = grads[size_t(c) * P + p];
      const int64_t n = layout->params[p].numel;
      if (n == 0) continue;
      if (g == nullptr || !tide::aligned(g, 2)) return TIDE_ERR_INVALID;
      vec = vec && tide::aligned(g, 16);
      const uintptr_t lo = reinterpret_cast<uintptr_t>(g);
      ins.push_back(Range{lo, lo + uintptr_t(n) * 2});
    }
  }
  for (int32_t r = 0; r < R; ++r) {
    const float* s = shards[r];
    if (S == 0) continue;
    if (s == nullptr || !tide::aligned(s, 4)) return TIDE_ERR_INVALID;
    vec = vec && tide::aligned(s, 16);
    const uintptr_t lo = reinterpret_cast<uintptr_t>(s);
    outs.push_back(Range{lo, lo + uintptr_t(S) * 4});
  }
  if (tide::outputs_overlap(outs, ins)) return TIDE_ERR_INVALID;
  const int64_t count = int64_t(layout->rs_chunks.size());
  if (count == 0) return TIDE_OK;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(layout->mu);
  tide::DeviceState* st = nullptr;
  int e = tide::device_state(layout, &st);
  if (e != hipSuccess) return tide::hip_fail(e);

  // Pointer table: C*P gradient pointers, then R shard pointers.
  std::vector<void*> table(size_t(C) * P + R);
  for (size_t i = 0; i < size_t(C) * P; ++i) table[i] = const_cast<void*>(grads[i]);
  for (int32_t r = 0; r < R; ++r) table[size_t(C) * P + r] = shards[r];
  tide::PtrSlot* slot = nullptr;
  if ((e = tide::acquire_ptrs(st, table.data(), table.size(), hs, &slot)) != hipSuccess) return tide::hip_fail(e);

  const tide::Plan plan = tide::plan_for(count, cu_budget, cu_budget, tide::kRsBoundedItems);
  for (int64_t first = 0; first < count; first += plan.per_launch) {
    const int64_t n = std::min<int64_t>(plan.per_launch, count - first);
    const int grid = int(std::min<int64_t>(plan.grid, n));
    e = tide::launch_rs(st->rs, first, n, grid, plan.items, const_cast<const void* const*>(slot->dev), P, C, S,
                        /*flat=*/false, vec, hs);
    if (e != hipSuccess) {
      (void)tide::release_ptrs(slot, hs);
      return tide::hip_fail(e);
    }
  }
  if ((e = tide::release_ptrs(slot, hs)) != hipSuccess) return tide::hip_fail(e);
  return TIDE_OK;
}

tide_status tide_ag_place(const tide_layout* layout, const void* stage, void* const* params, int32_t mode,
                          int32_t cu_budget, void* stream) {
  if (layout == nullptr || params == nullptr || cu_budget < 0) return TIDE_ERR_INVALID;
  if (mode != TIDE_AG_KERNEL && mode != TIDE_AG_SDMA && mode != TIDE_AG_COPY2D) return TIDE_ERR_INVALID;
  const int32_t P = layout->P, R = layout->R;
  const int64_t S = layout->S;
  const int64_t stage_n = int64_t(R) * S;
  if (stage_n > 0 && (stage == nullptr || !tide::aligned(stage, 2))) return TIDE_ERR_INVALID;
  bool vec = stage_n == 0 || tide::aligned(stage, 16);
  std::vector<Range> ins, outs;
  if (stage_n > 0) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(stage);
    ins.push_back(Range{lo, lo + uintptr_t(stage_n) * 2});
  }
  for (int32_t p = 0; p < P; ++p) {
    const int64_t n = layout->params[p].numel;
    if (n == 0) continue;
    const void* q = params[p];
    if (q == nullptr || !tide::aligned(q, 2)) return TIDE_ERR_INVALID;
    vec = vec && tide::aligned(q, 16);
    const uintptr_t lo = reinterpret_cast<uintptr_t>(q);
    outs.push_back(Range{lo, lo + uintptr_t(n) * 2});
  }
  if (tide::outputs_overlap(outs, ins)) return TIDE_ERR_INVALID;
  hipStream_t hs = static_cast<hipStream_t>(stream);

  if (mode == TIDE_AG_COPY2D) {
    // One 2-D copy per parameter covers the ranks whose slice is full (rows of the copy = ranks,
    // source pitch = one stage slot, destination pitch = one slice), plus one copy for the rank
    // whose slice is partly padding.  The runtime chooses the engine.
    for (int32_t p = 0; p < P; ++p) {
      const tide::ParamGeom& g = layout->params[p];
      if (g.numel == 0) continue;
      const int64_t full = g.rows / g.m;  // ranks with v == m_p
      const char* src = static_cast<const char*>(stage) + 2 * g.o;
      char* dst = static_cast<char*>(params[p]);
      hipError_t e = hipSuccess;
      if (full > 0)
        e = hipMemcpy2DAsync(dst, size_t(2 * g.e), src, size_t(2 * S), size_t(2 * g.e), size_t(full),
                             hipMemcpyDeviceToDevice, hs);
      if (e == hipSuccess && full < R) {
        const int64_t v = g.rows - full * g.m;
        if (v > 0) e = hipMemcpyAsync(dst + 2 * full * g.e, src + 2 * full * S, size_t(2 * v * g.L),
                                      hipMemcpyDeviceToDevice, hs);
      }
      if (e == hipErrorInvalidValue || e == hipErrorNotSupported) {
        tide::set_last_hip_error(e);
        return TIDE_ERR_UNSUPPORTED;
      }
      if (e != hipSuccess) return tide::hip_fail(e);
    }
    return TIDE_OK;
  }

  if (mode == TIDE_AG_SDMA) {
    // DMA engines only: the runtime sends 1-D device-to-device copies of the "no compute unit"
    // kind to the SDMA engines (2-D copies become shader kernels), so each (parameter, rank)
    // segment -- contiguous on both sides -- is one copy.  Copies alternate over the internal
    // copy streams, which fork from and join back into the caller's stream.
    std::lock_guard<std::mutex> lock(layout->mu);
    tide::DeviceState* st = nullptr;
    int e = tide::device_state(layout, &st);
    if (e != hipSuccess) return tide::hip_fail(e);
    if ((e = tide::ensure_dma(st)) != hipSuccess) return tide::hip_fail(e);
    if ((e = hipEventRecord(st->dma_fork, hs)) != hipSuccess) return tide::hip_fail(e);
    for (int k = 0; k < tide::kDmaStreams; ++k)
      if ((e = hipStreamWaitEvent(st->dma[k], st->dma_fork, 0)) != hipSuccess) return tide::hip_fail(e);
    int64_t issued = 0;
    for (int32_t p = 0; p < P && e == hipSuccess; ++p) {
      const tide::ParamGeom& g = layout->params[p];
      if (g.numel == 0) continue;
      for (int32_t r = 0; r < R; ++r) {
        const int64_t v = std::min<int64_t>(g.m, std::max<int64_t>(0, g.rows - int64_t(r) * g.m));
        if (v == 0) break;
        const char* src = static_cast<const char*>(stage) + 2 * (int64_t(r) * S + g.o);
        char* dst = static_cast<char*>(params[p]) + 2 * int64_t(r) * g.e;
        e = hipMemcpyAsync(dst, src, size_t(2 * v * g.L), hipMemcpyDeviceToDeviceNoCU,
                           st->dma[issued % tide::kDmaStreams]);
        if (e != hipSuccess) break;
        ++issued;
      }
    }
    // Join even after a failed copy, so the caller's stream never runs ahead of issued copies.
    int ej = hipSuccess;
    for (int k = 0; k < tide::kDmaStreams; ++k) {
      if (ej == hipSuccess) ej = hipEventRecord(st->dma_join[k], st->dma[k]);
      if (ej == hipSuccess) ej = hipStreamWaitEvent(hs, st->dma_join[k], 0);
    }
    if (e == hipErrorInvalidValue || e == hipErrorNotSupported) {
      tide::set_last_hip_error(e);
      return TIDE_ERR_UNSUPPORTED;
    }
    if (e != hipSuccess) return tide::hip_fail(e);
    if (ej != hipSuccess) return tide::hip_fail(ej);
    return TIDE_OK;
  }

  const int64_t count = int64_t(layout->ag_chunks.size());
  if (count == 0) return TIDE_OK;
  std::lock_guard<std::mutex> lock(layout->mu);
  tide::DeviceState* st = nullptr;
  int e = tide::device_state(layout, &st);
  if (e != hipSuccess) return tide::hip_fail(e);
  tide::PtrSlot* slot = nullptr;
  if ((e = tide::acquire_ptrs(st, params, size_t(P), hs, &slot)) != hipSuccess) return tide::hip_fail(e);
  const int64_t ag_wgs = int64_t(cu_budget) * tide::kThreads / tide::kAgThreads;
  const tide::Plan plan = tide::plan_for(count, cu_budget, ag_wgs, tide::kAgBoundedItems);
  for (int64_t first = 0; first < count; first += plan.per_launch) {
    const int64_t n = std::min<int64_t>(plan.per_launch, count - first);
    const int grid = int(std::min<int64_t>(plan.grid, n));
    e = tide::launch_ag(st->ag, first, n, grid, plan.items, const_cast<void*>(stage),
                        const_cast<const void* const*>(slot->dev), /*pack=*/false, vec, hs);
    if (e != hipSuccess) {
      (void)tide::release_ptrs(slot, hs);
      return tide::hip_fail(e);
    }
  }
  if ((e = tide::release_ptrs(slot, hs)) != hipSuccess) return tide::hip_fail(e);
  return TIDE_OK;
}

tide_status tide_slot_pack(const tide_layout* layout, const void* const* grads, void* slot, int32_t cu_budget,
                           void* stream) {
  if (layout == nullptr || grads == nullptr || cu_budget < 0) return TIDE_ERR_INVALID;
  const int32_t P = layout->P, R = layout->R;
  const int64_t S = layout->S;
  const int64_t slot_n = int64_t(R) * S;
  if (slot_n > 0 && (slot == nullptr || !tide::aligned(slot, 2))) return TIDE_ERR_INVALID;
  bool vec = slot_n == 0 || tide::aligned(slot, 16);
  std::vector<Range> ins, outs;
  if (slot_n > 0) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(slot);
    outs.push_back(Range{lo, lo + uintptr_t(slot_n) * 2});
  }
  for (int32_t p = 0; p < P; ++p) {
    const int64_t n = layout->params[p].numel;
    if (n == 0) continue;
    const void* g = grads[p];
    if (g == nullptr || !tide::aligned(g, 2)) return TIDE_ERR_INVALID;
    vec = vec && tide::aligned(g, 16);
    const uintptr_t lo = reinterpret_cast<uintptr_t>(g);
    ins.push_back(Range{lo, lo + uintptr_t(n) * 2});
  }
  if (tide::outputs_overlap(outs, ins)) return TIDE_ERR_INVALID;
  if (slot_n == 0) return TIDE_OK;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(layout->mu);
  tide::DeviceState* st = nullptr;
  int e = tide::device_state(layout, &st);
  if (e != hipSuccess) return tide::hip_fail(e);
  const int64_t count = int64_t(layout->ag_chunks.size());
  if (count > 0) {
    tide::PtrSlot* pslot = nullptr;
    if ((e = tide::acquire_ptrs(st, const_cast<void* const*>(grads), size_t(P), hs, &pslot)) != hipSuccess)
      return tide::hip_fail(e);
    const int64_t ag_wgs = int64_t(cu_budget) * tide::kThreads / tide::kAgThreads;
    const tide::Plan plan = tide::plan_for(count, cu_budget, ag_wgs, tide::kAgBoundedItems);
    for (int64_t first = 0; first < count && e == hipSuccess; first += plan.per_launch) {
      const int64_t n = std::min<int64_t>(plan.per_launch, count - first);
      const int grid = int(std::min<int64_t>(plan.grid, n));
      e = tide::launch_ag(st->ag, first, n, grid, plan.items, slot, const_cast<const void* const*>(pslot->dev),
                          /*pack=*/true, vec, hs);
    }
    const int er = tide::release_ptrs(pslot, hs);
    if (e != hipSuccess) return tide::hip_fail(e);
    if (er != hipSuccess) return tide::hip_fail(er);
  }
  e = tide::launch_fill_zero(st->slot_pad, int64_t(layout->slot_pad_items.size()), slot, hs);
  if (e != hipSuccess) return tide::hip_fail(e);
  return TIDE_OK;
}

tide_status tide_rs_slots_bf16_to_fp32(const tide_layout* layout, int32_t C, const void* const* slots,
                                       float* const* shards, int32_t cu_budget, void* stream) {
  if (layout == nullptr || slots == nullptr || shards == nullptr || C < 1 || cu_budget < 0)
    return TIDE_ERR_INVALID;
  const int32_t R = layout->R;
  const int64_t S = layout->S;
  if (C > (1 << 24)) return TIDE_ERR_INVALID;
  if (S == 0) return TIDE_OK;
  bool vec = true;
  std::vector<Range> ins, outs;
  for (int32_t c = 0; c < C; ++c) {
    const void* g = slots[c];
    if (g == nullptr || !tide::aligned(g, 2)) return TIDE_ERR_INVALID;
    vec = vec && tide::aligned(g, 16);
    const uintptr_t lo = reinterpret_cast<uintptr_t>(g);
    ins.push_back(Range{lo, lo + uintptr_t(int64_t(R) * S) * 2});
  }
  for (int32_t r = 0; r < R; ++r) {
    const float* s = shards[r];
    if (s == nullptr || !tide::aligned(s, 4)) return TIDE_ERR_INVALID;
    vec = vec && tide::aligned(s, 16);
    const uintptr_t lo = reinterpret_cast<uintptr_t>(s);
    outs.push_back(Range{lo, lo + uintptr_t(S) * 4});
  }
  if (tide::outputs_overlap(outs, ins)) return TIDE_ERR_INVALID;
  const int64_t count = int64_t(layout->rs_chunks.size());
  hipStream_t hs = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(layout->mu);
  tide::DeviceState* st = nullptr;
  int e = tide::device_state(layout, &st);
  if (e != hipSuccess) return tide::hip_fail(e);
  std::vector<void*> table(size_t(C) + R);
  for (int32_t c = 0; c < C; ++c) table[c] = const_cast<void*>(slots[c]);
  for (int32_t r = 0; r < R; ++r) table[size_t(C) + r] = shards[r];
  tide::PtrSlot* pslot = nullptr;
  if ((e = tide::acquire_ptrs(st, table.data(), table.size(), hs, &pslot)) != hipSuccess) return tide::hip_fail(e);
  const tide::Plan plan = tide::plan_for(count, cu_budget, cu_budget, tide::kRsBoundedItems);
  for (int64_t first = 0; first < count && e == hipSuccess; first += plan.per_launch) {
    const int64_t n = std::min<int64_t>(plan.per_launch, count - first);
    const int grid = int(std::min<int64_t>(plan.grid, n));
    e = tide::launch_rs(st->rs, first, n, grid, plan.items, const_cast<const void* const*>(pslot->dev), 1, C, S,
                        /*flat=*/true, vec, hs);
  }
  const int er = tide::release_ptrs(pslot, hs);
  if (e != hipSuccess) return tide::hip_fail(e);
  if (er != hipSuccess) return tide::hip_fail(er);
  return TIDE_OK;
}

}  // extern "C"
