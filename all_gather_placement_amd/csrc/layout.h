// Host-side layout object: geometry, segment work-item tables, per-device state.
#pragma once

#include <hip/hip_runtime_api.h>

#include <map>
#include <mutex>
#include <vector>

#include "../../include/tide.h"
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
  // Device address of the library's fixed pointer-table scratch array on this device (allocation-free
  // RS entry point), obtained once at set-up, and its size in pointers.
  void* scratch = nullptr;
  int64_t scratch_ptrs = 0;
};

// Launch forms (include/tide.h tide_launch_form).
//
// TIDE_LAUNCH_DEFAULT for the RS with C contributors: CU-exclusive workgroups of 8 groups of 128
// threads, each group keeping 2 items' loads in flight for C <= 3 (16 items) and 1 item for C >= 4
// (8 items): the most items whose traffic, (2C + 4) KiB each, stays within the 160 KiB of a C = 8
// workgroup, so no workgroup lives longer than one at C = 8.  Measured on MI355X (Llama-3.1-8B
// shapes; HIP-event means): C = 1 / 2 / 3 / 4 / 5 / 6 / 7 / 8 stream 5.9 / 6.12 / 6.17 / 6.14 / 6.28 /
// 6.32 / 6.34 / 6.30 TB/s, against 6.29 / 6.39 / 6.42 / 6.34 / 6.32 / 6.31 / 6.26 / 6.20 for
// single-item workgroups under their best per-CU cap, which never empties a CU during the call: a
// concurrent one-wave GEMM then waits for the whole RS (+236% at C = 4) instead of +7.9% (C = 4)
// or +13.5% (C = 8, the Llama-3.1-70B group).
constexpr int rs_default_items(int C) { return C <= 3 ? 2 * kRsCuMaxGroups : kRsCuMaxGroups; }

// Groups per workgroup and items per group of a CU-exclusive RS workgroup taking n items.
inline int rs_cu_groups(int n) { return n <= kRsCuMaxGroups ? n : kRsCuMaxGroups; }
inline int rs_cu_items_per_group(int n) { return n <= kRsCuMaxGroups ? 1 : n / kRsCuMaxGroups; }

// Whether (form, count) is a valid RS launch for C contributors.
inline bool rs_launch_ok(int C, int form, int count) {
  switch (form) {
    case TIDE_LAUNCH_DEFAULT: return count == 0;
    case TIDE_LAUNCH_BOUNDED: return count >= 1;
    case TIDE_LAUNCH_CU_EXCLUSIVE:
      if (count >= 1 && count <= kRsCuMaxGroups) return true;
      return count == 2 * kRsCuMaxGroups && rs_cu_items_ok(C > kRsMaxCt ? 0 : C, 2);
    case TIDE_LAUNCH_PER_CU_CAP: return count >= 1 && count <= TIDE_MAX_WGS_PER_CU;
    default: return false;
  }
}
// Whether (form, count) is a valid launch of the placement kernel or the slot packing.
inline bool ag_launch_ok(int form, int count) {
  switch (form) {
    case TIDE_LAUNCH_DEFAULT: return count == 0;
    case TIDE_LAUNCH_BOUNDED: return count >= 1;
    case TIDE_LAUNCH_CU_EXCLUSIVE: return count >= 1 && count <= kAgCuMaxItems;
    default: return false;
  }
}

// Items per CU-exclusive RS workgroup of a valid launch, or 0 for the other forms.
inline int rs_cu_launch_items(int C, int form, int count) {
  if (form == TIDE_LAUNCH_CU_EXCLUSIVE) return count;
  if (form == TIDE_LAUNCH_DEFAULT) return rs_default_items(C > kRsMaxCt ? kRsCuMaxGroups : C);
  return 0;
}

// Local memory a CU-exclusive workgroup requests: the most one workgroup may (all of a CU's on
// MI355X), so no second one fits beside it.  The kernels have no static local memory.
inline int cu_exclusive_lds(const DeviceState& st) { return st.lds_per_wg < st.lds_per_cu ? st.lds_per_wg : st.lds_per_cu; }

// Dynamic local memory of an RS launch of single-item workgroups (bounded launches and per-CU caps):
// TIDE_LAUNCH_PER_CU_CAP N requests 1/N of the CU's local memory; bounded launches none.  Needs
// lds_per_cu, lds_per_wg and the static sizes filled in (rs_device_info).
inline int rs_launch_lds(const DeviceState& st, int C, int form, int count) {
  if (form != TIDE_LAUNCH_PER_CU_CAP) return 0;
  const int static_lds = C <= kRsMaxCt ? st.rs_static_lds_ct : st.rs_static_lds_rt;
  const int dyn = rs_dynamic_lds(st.lds_per_cu, static_lds, count);
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
