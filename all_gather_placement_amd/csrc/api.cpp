// Entry points of the reduce-scatter, the all-gather placement and Slot-Reuse: argument checks,
// device pointer tables, and dispatch to the gfx950 kernels or to the DMA engines.
//
// Every entry point first turns its arguments into a validated Request (the host table of device
// pointers the kernels read, plus launch parameters).  Immediate calls stage that table through
// the layout's ring of pointer-table slots; prepared calls (tide_*_prepare) give it a device
// buffer of its own, so tide_call_launch only enqueues kernels.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <utility>
#include <vector>

#include "../../include/tide.h"
#include "layout.h"

namespace tide {
namespace {

static_assert(TIDE_CU_EXCLUSIVE_MAX_ITEMS == 2 * kRsCuMaxGroups && rs_cu_items_ok(4, 2),
              "header and kernels agree on the widest CU-exclusive RS workgroup");

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
    // first output whose end is beyond in.lo (outs are sorted and disjoint, so their ends are too)
    auto it = std::upper_bound(outs.begin(), outs.end(), in.lo,
                               [](uintptr_t v, const Range& r) { return v < r.hi; });
    if (it != outs.end() && it->lo < in.hi) return true;
  }
  return false;
}

tide_status hip_fail(int err) {
  set_last_hip_error(err);
  return err == hipErrorOutOfMemory ? TIDE_ERR_NOMEM : TIDE_ERR_HIP;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + uintptr_t(bytes)};
}

// ---------------------------------------------------------------------------------------------
// Validated requests
// ---------------------------------------------------------------------------------------------

enum Kind { kRs = 0, kAg = 1, kPack = 2, kRsSlots = 3 };

struct Request {
  Kind kind = kRs;
  int32_t C = 0;          // contributors (RS kinds)
  int32_t mode = TIDE_AG_KERNEL;
  int32_t form = TIDE_LAUNCH_DEFAULT;  // launch form and count (include/tide.h tide_launch_form)
  int32_t count = 0;
  bool vec = true;        // every base pointer 16-byte aligned
  void* stage = nullptr;  // AG stage / packed slot
  // Device pointers the kernels read, host copy:
  //   kRs [C*P gradients][R shards]; kAg, kPack [P parameters/gradients]; kRsSlots [C slots][R shards]
  std::vector<void*> table;
};

tide_status validate_rs(const tide_layout* L, int32_t C, const void* const* grads, float* const* shards,
                        int32_t form, int32_t count, Request* q) {
  if (L == nullptr || grads == nullptr || shards == nullptr || C < 1 || !rs_launch_ok(C, form, count))
    return TIDE_ERR_INVALID;
  const int32_t P = L->P, R = L->R;
  const int64_t S = L->S;
  if (int64_t(C) * P > (int64_t(1) << 24)) return TIDE_ERR_INVALID;
  q->kind = kRs;
  q->C = C;
  q->form = form;
  q->count = count;
  q->vec = true;
  std::vector<Range> ins, outs;
  ins.reserve(size_t(C) * P);
  for (int32_t c = 0; c < C; ++c) {
    for (int32_t p = 0; p < P; ++p) {
      const void* g = grads[size_t(c) * P + p];
      const int64_t n = L->params[p].numel;
      if (n == 0) continue;
      if (g == nullptr || !aligned(g, 2)) return TIDE_ERR_INVALID;
      q->vec = q->vec && aligned(g, 16);
      ins.push_back(range_of(g, n * 2));
    }
  }
  for (int32_t r = 0; r < R; ++r) {
    if (S == 0) continue;
    if (shards[r] == nullptr || !aligned(shards[r], 4)) return TIDE_ERR_INVALID;
    q->vec = q->vec && aligned(shards[r], 16);
    outs.push_back(range_of(shards[r], S * 4));
  }
  if (outputs_overlap(outs, ins)) return TIDE_ERR_INVALID;
  q->table.assign(size_t(C) * P + R, nullptr);
  for (size_t i = 0; i < size_t(C) * P; ++i) q->table[i] = const_cast<void*>(grads[i]);
  for (int32_t r = 0; r < R; ++r) q->table[size_t(C) * P + r] = shards[r];
  return TIDE_OK;
}

tide_status validate_rs_slots(const tide_layout* L, int32_t C, const void* const* slots, float* const* shards,
                              int32_t form, int32_t count, Request* q) {
  if (L == nullptr || slots == nullptr || shards == nullptr || C < 1 || !rs_launch_ok(C, form, count))
    return TIDE_ERR_INVALID;
  if (C > (1 << 24)) return TIDE_ERR_INVALID;
  const int32_t R = L->R;
  const int64_t S = L->S;
  q->kind = kRsSlots;
  q->C = C;
  q->form = form;
  q->count = count;
  q->vec = true;
  std::vector<Range> ins, outs;
  if (S > 0) {
    for (int32_t c = 0; c < C; ++c) {
      if (slots[c] == nullptr || !aligned(slots[c], 2)) return TIDE_ERR_INVALID;
      q->vec = q->vec && aligned(slots[c], 16);
      ins.push_back(range_of(slots[c], int64_t(R) * S * 2));
    }
    for (int32_t r = 0; r < R; ++r) {
      if (shards[r] == nullptr || !aligned(shards[r], 4)) return TIDE_ERR_INVALID;
      q->vec = q->vec && aligned(shards[r], 16);
      outs.push_back(range_of(shards[r], S * 4));
    }
  }
  if (outputs_overlap(outs, ins)) return TIDE_ERR_INVALID;
  q->table.assign(size_t(C) + R, nullptr);
  for (int32_t c = 0; c < C; ++c) q->table[c] = const_cast<void*>(slots[c]);
  for (int32_t r = 0; r < R; ++r) q->table[size_t(C) + r] = shards[r];
  return TIDE_OK;
}

// AG placement (pack = false: stage -> params) and Slot-Reuse packing (pack = true: params ->
// slot) share one layout of arguments: a stage/slot of R*S bf16 and P per-parameter tensors.
tide_status validate_ag(const tide_layout* L, const void* stage, void* const* params, int32_t mode,
                        int32_t form, int32_t count, bool pack, Request* q) {
  if (L == nullptr || params == nullptr) return TIDE_ERR_INVALID;
  if (!pack && mode != TIDE_AG_KERNEL && mode != TIDE_AG_SDMA && mode != TIDE_AG_COPY2D) return TIDE_ERR_INVALID;
  // launch forms shape the kernel only: the DMA modes take the default
  if (!ag_launch_ok(form, count) || (!pack && mode != TIDE_AG_KERNEL && form != TIDE_LAUNCH_DEFAULT))
    return TIDE_ERR_INVALID;
  const int32_t P = L->P, R = L->R;
  const int64_t stage_n = int64_t(R) * L->S;
  if (stage_n > 0 && (stage == nullptr || !aligned(stage, 2))) return TIDE_ERR_INVALID;
  q->kind = pack ? kPack : kAg;
  q->mode = pack ? TIDE_AG_KERNEL : mode;
  q->form = form;
  q->count = count;
  q->vec = stage_n == 0 || aligned(stage, 16);
  q->stage = const_cast<void*>(stage);
  std::vector<Range> stage_r, tensors;
  if (stage_n > 0) stage_r.push_back(range_of(stage, stage_n * 2));
  for (int32_t p = 0; p < P; ++p) {
    const int64_t n = L->params[p].numel;
    if (n == 0) continue;
    if (params[p] == nullptr || !aligned(params[p], 2)) return TIDE_ERR_INVALID;
    q->vec = q->vec && aligned(params[p], 16);
    tensors.push_back(range_of(params[p], n * 2));
  }
  // placement writes the parameters (outputs) from the stage; packing writes the slot
  if (pack ? outputs_overlap(stage_r, tensors) : outputs_overlap(tensors, stage_r)) return TIDE_ERR_INVALID;
  q->table.assign(params, params + P);
  return TIDE_OK;
}

// ---------------------------------------------------------------------------------------------
// Pointer-table ring (immediate calls)
// ---------------------------------------------------------------------------------------------

// Stage `n` device pointers for a launch on `stream`; returns the slot that holds them.
int acquire_ptrs(DeviceState* st, void* const* ptrs, size_t n, hipStream_t stream, PtrSlot** out) {
  // A slot that already holds this exact table and was last used on this stream can be reused
  // without a refill: stream order keeps its earlier readers ahead of the new launch.  Calls that
  // alternate between tables (an RS and an AG on the same group) hit different slots.
  for (int k = 0; k < kPtrSlots; ++k) {
    PtrSlot& s = st->slots[k];
    if (s.n == n && s.dev != nullptr && s.stream == stream && std::memcmp(s.host.data(), ptrs, n * sizeof(void*)) == 0) {
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
    dev_free(s.dev, st->aux);  // not pending: nothing reads it any more
    s.dev = nullptr;
    s.cap = 0;
    s.n = 0;
    const size_t cap = std::max<size_t>(n, 256);
    void* p = nullptr;
    if ((e = static_cast<hipError_t>(dev_alloc_copy(st->aux, nullptr, cap * sizeof(void*), &p))) != hipSuccess) return e;
    s.dev = static_cast<void**>(p);
    s.cap = cap;
  }
  s.host.assign(ptrs, ptrs + n);
  s.n = n;
  s.stream = stream;
  if ((e = static_cast<hipError_t>(launch_put_ptrs(s.dev, ptrs, int64_t(n), stream))) != hipSuccess) {
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

// Create the internal copy streams and their fork/join events on first use (layout mutex held).
int ensure_dma(DeviceState* st) {
  hipError_t e;
  if (st->dma_fork == nullptr && (e = hipEventCreateWithFlags(&st->dma_fork, hipEventDisableTiming)) != hipSuccess)
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

// ---------------------------------------------------------------------------------------------
// Enqueueing validated work
// ---------------------------------------------------------------------------------------------

// Kernels of a table-driven request (RS, RS from slots, AG kernel, slot pack), reading the device
// pointer table `dev_table`.  Only kernel launches: nothing is allocated, copied or recorded.
int enqueue_kernels(const tide_layout* L, const DeviceState* st, const Request& q, void* const* dev_table,
                    hipStream_t hs) {
  const void* const* tbl = const_cast<const void* const*>(dev_table);
  const bool bounded = q.form == TIDE_LAUNCH_BOUNDED;
  int e = hipSuccess;
  if (q.kind == kRs || q.kind == kRsSlots) {
    const int64_t count = int64_t(L->rs_chunks.size());
    const bool flat = q.kind == kRsSlots;
    if (const int n = rs_cu_launch_items(q.C, q.form, q.count)) {
      // one launch of CU-exclusive workgroups of n items (the table's order: items are rank-major)
      return launch_rs_cu(st->rs, count, rs_cu_groups(n), rs_cu_items_per_group(n), tbl, flat ? 1 : L->P, q.C, L->S,
                          flat, q.vec, cu_exclusive_lds(*st), hs);
    }
    const int64_t rs_wgs = bounded ? int64_t(q.count) * kBudgetThreads / kThreads : 0;
    const Plan plan = plan_for(count, bounded, rs_wgs, kRsBoundedItems);
    // single-item workgroups under a per-CU cap, or bounded launches (capped by their budget)
    const int lds = rs_launch_lds(*st, q.C, q.form, q.count);
    for (int64_t first = 0; first < count && e == hipSuccess; first += plan.per_launch) {
      const int64_t n = std::min<int64_t>(plan.per_launch, count - first);
      e = launch_rs(st->rs, first, n, int(std::min<int64_t>(plan.grid, n)), plan.items, tbl, flat ? 1 : L->P, q.C,
                    L->S, flat, q.vec, lds, hs);
    }
    return e;
  }
  const int64_t count = int64_t(L->ag_chunks.size());
  if (q.form == TIDE_LAUNCH_CU_EXCLUSIVE) {
    if (count > 0)
      e = launch_ag_cu(st->ag, count, q.count, q.stage, tbl, q.kind == kPack, q.vec, cu_exclusive_lds(*st), hs);
    if (e == hipSuccess && q.kind == kPack)
      e = launch_fill_zero(st->slot_pad, int64_t(L->slot_pad_items.size()), q.stage, hs);
    return e;
  }
  const int64_t ag_wgs = bounded ? int64_t(q.count) * kBudgetThreads / kAgThreads : 0;
  const Plan plan = plan_for(count, bounded, ag_wgs, kAgBoundedItems);
  // Few workgroups per CU (small budgets): each loads two items at a time.
  const int batch = bounded && ag_wgs <= int64_t(kAgBatchMaxWgsPerCu) * std::max(st->cus, 1) ? 2 : 1;
  for (int64_t first = 0; first < count && e == hipSuccess; first += plan.per_launch) {
    const int64_t n = std::min<int64_t>(plan.per_launch, count - first);
    e = launch_ag(st->ag, first, n, int(std::min<int64_t>(plan.grid, n)), plan.items, batch, q.stage, tbl,
                  q.kind == kPack, q.vec, hs);
  }
  if (e == hipSuccess && q.kind == kPack)
    e = launch_fill_zero(st->slot_pad, int64_t(L->slot_pad_items.size()), q.stage, hs);
  return e;
}

bool needs_kernels(const tide_layout* L, const Request& q) {
  if (q.kind == kRs || q.kind == kRsSlots) return !L->rs_chunks.empty();
  if (q.kind == kPack) return int64_t(L->R) * L->S > 0;
  return !L->ag_chunks.empty();
}

// One 2-D copy per parameter covers the ranks whose slice is full (rows of the copy = ranks,
// source pitch = one stage slot, destination pitch = one slice), plus one copy for the rank whose
// slice is partly padding.  The runtime chooses the engine.
tide_status enqueue_ag_copy2d(const tide_layout* L, const Request& q, hipStream_t hs) {
  const int64_t S = L->S;
  for (int32_t p = 0; p < L->P; ++p) {
    const ParamGeom& g = L->params[p];
    if (g.numel == 0) continue;
    const int64_t full = g.rows / g.m;  // ranks with v == m_p
    const char* src = static_cast<const char*>(q.stage) + 2 * g.o;
    char* dst = static_cast<char*>(q.table[p]);
    hipError_t e = hipSuccess;
    if (full > 0)
      e = hipMemcpy2DAsync(dst, size_t(2 * g.e), src, size_t(2 * S), size_t(2 * g.e), size_t(full),
                           hipMemcpyDeviceToDevice, hs);
    if (e == hipSuccess && full < L->R) {
      const int64_t v = g.rows - full * g.m;
      if (v > 0)
        e = hipMemcpyAsync(dst + 2 * full * g.e, src + 2 * full * S, size_t(2 * v * g.L), hipMemcpyDeviceToDevice, hs);
    }
    if (e == hipErrorInvalidValue || e == hipErrorNotSupported) {
      set_last_hip_error(e);
      return TIDE_ERR_UNSUPPORTED;
    }
    if (e != hipSuccess) return hip_fail(e);
  }
  return TIDE_OK;
}

// DMA engines only: the runtime sends 1-D device-to-device copies of the "no compute unit" kind
// to the SDMA engines (2-D copies become shader kernels), so each (parameter, rank) segment --
// contiguous on both sides -- is one copy.  Copies alternate over the internal copy streams, which
// fork from and join back into the caller's stream.  Layout mutex held.
tide_status enqueue_ag_sdma(const tide_layout* L, DeviceState* st, const Request& q, hipStream_t hs) {
  int e = ensure_dma(st);
  if (e != hipSuccess) return hip_fail(e);
  if ((e = hipEventRecord(st->dma_fork, hs)) != hipSuccess) return hip_fail(e);
  for (int k = 0; k < kDmaStreams; ++k)
    if ((e = hipStreamWaitEvent(st->dma[k], st->dma_fork, 0)) != hipSuccess) return hip_fail(e);
  const int64_t S = L->S;
  int64_t issued = 0;
  for (int32_t p = 0; p < L->P && e == hipSuccess; ++p) {
    const ParamGeom& g = L->params[p];
    if (g.numel == 0) continue;
    for (int32_t r = 0; r < L->R; ++r) {
      const int64_t v = std::min<int64_t>(g.m, std::max<int64_t>(0, g.rows - int64_t(r) * g.m));
      if (v == 0) break;
      const char* src = static_cast<const char*>(q.stage) + 2 * (int64_t(r) * S + g.o);
      char* dst = static_cast<char*>(q.table[p]) + 2 * int64_t(r) * g.e;
      e = hipMemcpyAsync(dst, src, size_t(2 * v * g.L), hipMemcpyDeviceToDeviceNoCU, st->dma[issued % kDmaStreams]);
      if (e != hipSuccess) break;
      ++issued;
    }
  }
  // Join even after a failed copy, so the caller's stream never runs ahead of issued copies.
  int ej = hipSuccess;
  for (int k = 0; k < kDmaStreams; ++k) {
    if (ej == hipSuccess) ej = hipEventRecord(st->dma_join[k], st->dma[k]);
    if (ej == hipSuccess) ej = hipStreamWaitEvent(hs, st->dma_join[k], 0);
  }
  if (e == hipErrorInvalidValue || e == hipErrorNotSupported) {
    set_last_hip_error(e);
    return TIDE_ERR_UNSUPPORTED;
  }
  if (e != hipSuccess) return hip_fail(e);
  if (ej != hipSuccess) return hip_fail(ej);
  return TIDE_OK;
}

// Immediate execution of a validated request.
tide_status run_now(const tide_layout* L, const Request& q, void* stream) {
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (q.kind == kAg && q.mode == TIDE_AG_COPY2D) return enqueue_ag_copy2d(L, q, hs);
  if (!(q.kind == kAg && q.mode == TIDE_AG_SDMA) && !needs_kernels(L, q)) return TIDE_OK;
  std::lock_guard<std::mutex> lock(L->mu);
  DeviceState* st = nullptr;
  int e = device_state(L, &st);
  if (e != hipSuccess) return hip_fail(e);
  if (q.kind == kAg && q.mode == TIDE_AG_SDMA) return enqueue_ag_sdma(L, st, q, hs);
  PtrSlot* slot = nullptr;
  if ((e = acquire_ptrs(st, q.table.data(), q.table.size(), hs, &slot)) != hipSuccess) return hip_fail(e);
  e = enqueue_kernels(L, st, q, slot->dev, hs);
  const int er = release_ptrs(slot, hs);
  if (e != hipSuccess) return hip_fail(e);
  if (er != hipSuccess) return hip_fail(er);
  return TIDE_OK;
}

}  // namespace
}  // namespace tide

// A prepared call: a validated request with a device pointer table of its own.
struct tide_call {
  const tide_layout* layout = nullptr;
  tide::Request q;
  int device = -1;
  void** dev_table = nullptr;
  tide::DeviceState* st = nullptr;  // node of layout->devices; std::map nodes do not move
  // Completion marks of the kernel launches: one event per stream the call was launched on,
  // recorded again after each launch, so that destroying the call (or its layout) waits for this
  // call's work and nothing else.  A launch captured into a graph, or one whose stream could not be
  // queried, cannot be tracked that way: `untracked` makes destroy wait for the whole device.
  std::mutex mu;
  std::vector<std::pair<hipStream_t, hipEvent_t>> marks;
  bool untracked = false;
};

namespace tide {
namespace {

// Record the completion mark of a kernel launch on `hs` (see tide_call::marks).
int mark_launch(tide_call* call, hipStream_t hs) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t q = hipStreamIsCapturing(hs, &cs);
  // a failed query (the legacy stream while another stream captures, say) leaves the thread's last
  // error set, which the next launch would report as its own: clear it, and wait for the device then
  if (q != hipSuccess) (void)hipGetLastError();
  std::lock_guard<std::mutex> lock(call->mu);
  if (q != hipSuccess || cs != hipStreamCaptureStatusNone) {
    call->untracked = true;
    return hipSuccess;
  }
  for (auto& m : call->marks)
    if (m.first == hs) return hipEventRecord(m.second, hs);
  hipEvent_t ev = nullptr;
  hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e != hipSuccess) return e;
  call->marks.emplace_back(hs, ev);
  return hipEventRecord(ev, hs);
}

// Wait until every launch of `call` has finished (the call's device current).
void wait_call(tide_call* call) {
  std::lock_guard<std::mutex> lock(call->mu);
  if (call->untracked) {
    (void)hipDeviceSynchronize();
    call->untracked = false;
  }
  for (auto& m : call->marks) (void)hipEventSynchronize(m.second);
}

}  // namespace

void wait_for_calls(const tide_layout* layout) {
  int cur = 0;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  for (tide_call* call : layout->calls) {
    if (have && call->device != cur) (void)hipSetDevice(call->device);
    wait_call(call);
    if (have && call->device != cur) (void)hipSetDevice(cur);
  }
}

}  // namespace tide

namespace {

tide_status prepare(const tide_layout* L, tide::Request&& q, tide_call** out) {
  if (out == nullptr) return TIDE_ERR_INVALID;
  tide_call* call = new (std::nothrow) tide_call();
  if (call == nullptr) return TIDE_ERR_NOMEM;
  call->layout = L;
  call->q = std::move(q);
  int e = hipGetDevice(&call->device);
  if (e == hipSuccess) {
    std::lock_guard<std::mutex> lock(L->mu);
    e = tide::device_state(L, &call->st);
  }
  // The DMA placement modes address parameters from the host table; only kernels read a device one.
  const bool kernels = !(call->q.kind == tide::kAg && call->q.mode != TIDE_AG_KERNEL);
  if (e == hipSuccess && kernels && !call->q.table.empty()) {
    const size_t bytes = call->q.table.size() * sizeof(void*);
    void* p = nullptr;
    e = tide::dev_alloc_copy(call->st->aux, call->q.table.data(), bytes, &p);
    call->dev_table = static_cast<void**>(p);
  }
  if (e != hipSuccess) {
    delete call;
    return tide::hip_fail(e);
  }
  {
    std::lock_guard<std::mutex> lock(L->mu);
    L->calls.push_back(call);
  }
  *out = call;
  return TIDE_OK;
}

}  // namespace

extern "C" {

tide_status tide_rs_bf16_to_fp32(const tide_layout* layout, int32_t C, const void* const* grads,
                                 float* const* shards, int32_t launch_form, int32_t launch_count, void* stream) {
  tide::Request q;
  const tide_status s = tide::validate_rs(layout, C, grads, shards, launch_form, launch_count, &q);
  return s != TIDE_OK ? s : tide::run_now(layout, q, stream);
}

tide_status tide_ag_place(const tide_layout* layout, const void* stage, void* const* params, int32_t mode,
                          int32_t launch_form, int32_t launch_count, void* stream) {
  tide::Request q;
  const tide_status s =
      tide::validate_ag(layout, stage, params, mode, launch_form, launch_count, /*pack=*/false, &q);
  return s != TIDE_OK ? s : tide::run_now(layout, q, stream);
}

tide_status tide_slot_pack(const tide_layout* layout, const void* const* grads, void* slot, int32_t launch_form,
                           int32_t launch_count, void* stream) {
  tide::Request q;
  const tide_status s = tide::validate_ag(layout, slot, const_cast<void* const*>(grads), TIDE_AG_KERNEL, launch_form,
                                          launch_count, /*pack=*/true, &q);
  return s != TIDE_OK ? s : tide::run_now(layout, q, stream);
}

tide_status tide_rs_slots_bf16_to_fp32(const tide_layout* layout, int32_t C, const void* const* slots,
                                       float* const* shards, int32_t launch_form, int32_t launch_count,
                                       void* stream) {
  tide::Request q;
  const tide_status s = tide::validate_rs_slots(layout, C, slots, shards, launch_form, launch_count, &q);
  return s != TIDE_OK ? s : tide::run_now(layout, q, stream);
}

tide_status tide_rs_bf16_to_fp32_noalloc(const tide_layout* layout, int32_t C, const void* const* grads,
                                         float* const* shards, int32_t launch_form, int32_t launch_count,
                                         void* stream) {
  tide::Request q;
  tide_status s = tide::validate_rs(layout, C, grads, shards, launch_form, launch_count, &q);
  if (s != TIDE_OK) return s;
  if (int64_t(q.table.size()) > int64_t(TIDE_NOALLOC_MAX_PTRS)) return TIDE_ERR_INVALID;
  if (!tide::needs_kernels(layout, q)) return TIDE_OK;
  int dev = 0;
  int e = hipGetDevice(&dev);
  if (e != hipSuccess) return tide::hip_fail(e);
  const tide::DeviceState* st = nullptr;
  {
    // the device tables must exist already: creating them here would allocate
    std::lock_guard<std::mutex> lock(layout->mu);
    auto it = layout->devices.find(dev);
    if (it == layout->devices.end()) return TIDE_ERR_INVALID;
    st = &it->second;  // std::map nodes do not move; the state is never erased before destroy
  }
  if (st->scratch == nullptr || int64_t(q.table.size()) > st->scratch_ptrs) return TIDE_ERR_INVALID;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  e = tide::launch_put_ptrs(st->scratch, q.table.data(), int64_t(q.table.size()), hs);
  if (e == hipSuccess) e = tide::enqueue_kernels(layout, st, q, static_cast<void* const*>(st->scratch), hs);
  return e == hipSuccess ? TIDE_OK : tide::hip_fail(e);
}

tide_status tide_rs_prepare(const tide_layout* layout, int32_t C, const void* const* grads, float* const* shards,
                            int32_t launch_form, int32_t launch_count, tide_call** out) {
  tide::Request q;
  const tide_status s = tide::validate_rs(layout, C, grads, shards, launch_form, launch_count, &q);
  return s != TIDE_OK ? s : prepare(layout, std::move(q), out);
}

tide_status tide_ag_prepare(const tide_layout* layout, const void* stage, void* const* params, int32_t mode,
                            int32_t launch_form, int32_t launch_count, tide_call** out) {
  tide::Request q;
  const tide_status s =
      tide::validate_ag(layout, stage, params, mode, launch_form, launch_count, /*pack=*/false, &q);
  return s != TIDE_OK ? s : prepare(layout, std::move(q), out);
}

tide_status tide_slot_pack_prepare(const tide_layout* layout, const void* const* grads, void* slot,
                                   int32_t launch_form, int32_t launch_count, tide_call** out) {
  tide::Request q;
  const tide_status s = tide::validate_ag(layout, slot, const_cast<void* const*>(grads), TIDE_AG_KERNEL, launch_form,
                                          launch_count, /*pack=*/true, &q);
  return s != TIDE_OK ? s : prepare(layout, std::move(q), out);
}

tide_status tide_rs_slots_prepare(const tide_layout* layout, int32_t C, const void* const* slots,
                                  float* const* shards, int32_t launch_form, int32_t launch_count, tide_call** out) {
  tide::Request q;
  const tide_status s = tide::validate_rs_slots(layout, C, slots, shards, launch_form, launch_count, &q);
  return s != TIDE_OK ? s : prepare(layout, std::move(q), out);
}

tide_status tide_call_launch(const tide_call* call, void* stream) {
  if (call == nullptr) return TIDE_ERR_INVALID;
  int dev = -1;
  int e = hipGetDevice(&dev);
  if (e != hipSuccess) return tide::hip_fail(e);
  if (dev != call->device) return TIDE_ERR_INVALID;
  const tide::Request& q = call->q;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (q.kind == tide::kAg && q.mode == TIDE_AG_COPY2D) return tide::enqueue_ag_copy2d(call->layout, q, hs);
  if (q.kind == tide::kAg && q.mode == TIDE_AG_SDMA) {
    std::lock_guard<std::mutex> lock(call->layout->mu);
    return tide::enqueue_ag_sdma(call->layout, call->st, q, hs);
  }
  if (!tide::needs_kernels(call->layout, q)) return TIDE_OK;
  e = tide::enqueue_kernels(call->layout, call->st, q, call->dev_table, hs);
  if (e == hipSuccess) e = tide::mark_launch(const_cast<tide_call*>(call), hs);
  return e == hipSuccess ? TIDE_OK : tide::hip_fail(e);
}

tide_status tide_rs_launch_shape(int32_t C, int32_t launch_form, int32_t launch_count, int32_t* threads,
                                 int32_t* items_per_workgroup, int32_t* item_outputs, int32_t* lds_bytes) {
  if (C < 1 || !tide::rs_launch_ok(C, launch_form, launch_count)) return TIDE_ERR_INVALID;
  tide::DeviceState st;
  int dev = 0;
  int e = hipGetDevice(&dev);
  if (e == hipSuccess) e = tide::rs_device_info(dev, &st);
  if (e != hipSuccess) return tide::hip_fail(e);
  int th = tide::kThreads, items = 1, lds = 0;
  if (const int n = tide::rs_cu_launch_items(C, launch_form, launch_count)) {
    th = tide::kThreads * tide::rs_cu_groups(n);
    items = n;
    lds = tide::cu_exclusive_lds(st);
  } else {
    if (launch_form == TIDE_LAUNCH_BOUNDED) items = tide::kRsBoundedItems;
    lds = (C <= tide::kRsMaxCt ? st.rs_static_lds_ct : st.rs_static_lds_rt) +
          tide::rs_launch_lds(st, C, launch_form, launch_count);
  }
  if (threads) *threads = th;
  if (items_per_workgroup) *items_per_workgroup = items;
  if (item_outputs) *item_outputs = int32_t(tide::kRsChunk);
  if (lds_bytes) *lds_bytes = lds;
  return TIDE_OK;
}

void tide_call_destroy(tide_call* call) {
  if (call == nullptr) return;
  {
    std::lock_guard<std::mutex> lock(call->layout->mu);
    auto& v = call->layout->calls;
    v.erase(std::remove(v.begin(), v.end(), call), v.end());
  }
  int cur = 0;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  if (have && cur != call->device) (void)hipSetDevice(call->device);
  // this call's own launches only (their marks); other work on the device is not waited for
  tide::wait_call(call);
  for (auto& m : call->marks) (void)hipEventDestroy(m.second);
  tide::dev_free(call->dev_table, call->st->aux);  // stream-ordered: waits for no other work
  if (have && cur != call->device) (void)hipSetDevice(cur);
  delete call;
}

}  // extern "C"
