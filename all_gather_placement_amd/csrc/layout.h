// Host-side layout object: geometry, segment work-item tables, per-device state.
#pragma once

#include <hip/hip_runtime_api.h>

#include <map>
#include <mutex>
#include <vector>

#include "tide_internal.h"

namespace tide {

struct ParamGeom {
  int64_t rows;  // dim 0
  int64_t L;     // row length: product of the trailing dims
  int64_t m;     // padded per-rank rows: ceil(rows / R)
  int64_t e;     // per-rank shard elements: m * L
  int64_t o;     // prefix offset inside a rank's flat shard
  int64_t numel; // rows * L
};

// A ring of device pointer tables.  Each RS/AG call needs its C*P + R (or P) device pointers in
// device memory; a slot is refilled by small kernels on the caller's stream that carry the pointers
// as kernel arguments (no host staging buffer), and a call whose pointers equal the previous call's
// on the same stream reuses that slot with no refill.
struct PtrSlot {
  std::vector<void*> host;  // host copy of what the slot holds (to recognise a repeated table)
  void** dev = nullptr;
  size_t cap = 0;         // pointers
  size_t n = 0;           // pointers currently held
  hipEvent_t done = nullptr;
  hipStream_t stream = nullptr;
  bool pending = false;   // `done` has been recorded after the slot's last use
};

constexpr int kPtrSlots = 8;

// Internal streams for DMA-engine copies (created on first use, default priority).  Two streams
// measured twice the copy bandwidth of one on MI355X; more streams added little.
constexpr int kDmaStreams = 2;

struct DeviceState {
  // Internal stream of the library's own device memory: tables are allocated from the device's
  // stream-ordered pool and freed on it, so freeing them waits for nothing else (hipFree and
  // hipHostFree synchronise the whole device).
  hipStream_t aux = nullptr;
  RsChunk* rs = nullptr;
  AgChunk* ag = nullptr;
  AgChunk* slot_pad = nullptr;
  PtrSlot slots[kPtrSlots];
  int next = 0;
  hipStream_t dma[kDmaStreams] = {};
  hipEvent_t dma_fork = nullptr;
  hipEvent_t dma_join[kDmaStreams] = {};
  int cus = 0;              // compute units of the device
  int lds_per_cu = 0;       // local memory per CU (bytes)
  int lds_per_wg = 0;       // largest local memory one workgroup may request (bytes)
  int rs_static_lds_ct = 0; // static local memory of the RS kernel, C <= kRsMaxCt
  int rs_static_lds_rt = 0; // static local memory of the RS kernel, C > kRsMaxCt
  int rs_static_lds_cu = 0; // static local memory of the CU-exclusive RS kernel
  // Device address of the library's fixed pointer-table scratch array on this device (allocation-free
  // RS entry point), obtained once at set-up, and its size in pointers.
  void* scratch = nullptr;
  int64_t scratch_ptrs = 0;
};

// cu_budget values TIDE_RS_CU_EXCLUSIVE(W) (TIDE_AG_CU_EXCLUSIVE(W) for the placement kernel and the
// packing): the number of items per CU-exclusive workgroup, else 0.
inline int cu_exclusive_items(int cu_budget) {
  const int w = -cu_budget - TIDE_RS_MAX_WGS_PER_CU;
  return w >= 1 && w <= TIDE_RS_CU_EXCLUSIVE_MAX_ITEMS ? w : 0;
}

// Dynamic local memory of a CU-exclusive RS workgroup: together with its static local memory, the
// most one workgroup may request (all of a CU's on MI355X), so no second one fits beside it.
inline int rs_cu_launch_lds(const DeviceState& st) {
  const int cap = st.lds_per_wg < st.lds_per_cu ? st.lds_per_wg : st.lds_per_cu;
  const int dyn = cap - st.rs_static_lds_cu;
  return dyn > 0 ? dyn : 0;
}
// Default RS launch (cu_budget 0) in the CU-exclusive form with the widest workgroups (kRsCuMaxItems
// items) instead of single-item workgroups under a per-CU cap, where it measured faster on MI355X
// (Llama-3.1-8B shapes, R = 8, HIP-event means): C = 8, compiled (the four layer groups: +0.2 to
// +1.5% over three interleaved sessions), and C >= 12 in its runtime-C form (C = 12 / 16 / 20 / 24 /
// 32: +2.3 / +5.2 / +1.9 / +1.8 / +1.6%).  Elsewhere the cap stays: C = 9 / 10 -3.1 / -1.4% (a
// compiled capped kernel against the runtime-C form), C <= 4 -4 to -26% (a CU then holds too few
// bytes in flight).  The CU-exclusive default also leaves a concurrent one-wave GEMM its CUs
// (+12-15% instead of waiting for the whole call).
constexpr int kRsCuDefaultMinC = 12;
inline bool rs_cu_default(int C) { return C == 8 || C >= kRsCuDefaultMinC; }

// Items per CU-exclusive RS workgroup for C contributors at cu_budget, or 0 for the other forms.
inline int rs_cu_launch_items(int C, int cu_budget) {
  if (const int w = cu_exclusive_items(cu_budget)) return w;
  return cu_budget == 0 && rs_cu_default(C) ? kRsCuMaxItems : 0;
}

inline int ag_cu_launch_lds(const DeviceState& st) {  // the AG kernels have no static local memory
  return st.lds_per_wg < st.lds_per_cu ? st.lds_per_wg : st.lds_per_cu;
}

// Dynamic local memory of an RS launch with C contributors at `cu_budget` on this device: 0 caps
// the RS workgroups per CU at rs_wgs_per_cu(C), -N at N; bounded launches (> 0) add none.  Needs
// lds_per_cu, lds_per_wg and the static sizes filled in (rs_device_info).
inline int rs_launch_lds(const DeviceState& st, int C, int cu_budget) {
  if (cu_budget > 0) return 0;
  if (rs_cu_launch_items(C, cu_budget) > 0) return rs_cu_launch_lds(st);
  const int wgs = cu_budget < 0 ? -cu_budget : rs_wgs_per_cu(C);
  const int static_lds = C <= kRsMaxCt ? st.rs_static_lds_ct : st.rs_static_lds_rt;
  const int dyn = rs_dynamic_lds(st.lds_per_cu, static_lds, wgs);
  // caps below what one workgroup's local memory can express become the smallest that it can
  const int room = st.lds_per_wg - static_lds;
  return dyn < room ? dyn : (room > 0 ? room : 0);
}

// Fills cus, lds_per_cu, lds_per_wg and the RS kernel's static local memory for `device`.
// Returns a hipError_t.
int rs_device_info(int device, DeviceState* st);

// `bytes` of device memory from the device's stream-ordered pool, allocated on `aux` and filled from
// `host` (if not NULL); usable from every stream once this returns (it waits for `aux`).
int dev_alloc_copy(hipStream_t aux, const void* host, size_t bytes, void** out);
// Stream-ordered free on `aux`, for memory that nothing reads any more (the caller has waited).
void dev_free(void* p, hipStream_t aux);

}  // namespace tide

struct tide_call;

struct tide_layout {
  int32_t P = 0;
  int32_t R = 0;
  int64_t S = 0;
  std::vector<tide::ParamGeom> params;
  std::vector<tide::RsChunk> rs_chunks;
  std::vector<tide::AgChunk> ag_chunks;
  // Padding ranges of a packed rank-major slot (src = slot element offset, n), for Slot-Reuse.
  std::vector<tide::AgChunk> slot_pad_items;
  mutable std::mutex mu;
  mutable std::map<int, tide::DeviceState> devices;
  // Prepared calls made from this layout and not yet destroyed (guarded by mu): their launches
  // read the layout's device tables, so destroying the layout waits for them too.
  mutable std::vector<tide_call*> calls;
};

namespace tide {
// Returns the device state for the current device, uploading the tables on first use.
// Must be called with layout->mu held.  Returns a hipError_t.
int device_state(const tide_layout* layout, DeviceState** out);
// Reorders the work-item tables into the order workgroups take them.
void order_items(tide_layout* layout);
void set_last_hip_error(int err);
// Waits for the launches of every prepared call still registered with the layout (layout->mu held).
void wait_for_calls(const tide_layout* layout);
}  // namespace tide
