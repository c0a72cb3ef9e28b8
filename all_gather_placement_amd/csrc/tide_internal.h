// Internal declarations shared by the host layout code, the entry points and the gfx950 kernels.
#pragma once

#include <stdint.h>

#include <cstddef>

namespace tide {

// Kernel shape.  The defaults were chosen by measurement on MI355X (HBM GB/s over the Llama-3.1
// 8B/70B, Qwen3-30B-A3B and Wan2.2 layer groups); each can be overridden at build time.
//
// RS: 128 threads (2 wave64 waves) per workgroup; one work item is 1024 outputs, i.e. 8 per
// thread: one 16-byte load per contributor per lane on full items.  A workgroup moves
// 1024 * (2C + 4) bytes (20 KiB at C = 8) and exits.
// AG: 128 threads per workgroup; one work item is 2048 bf16 elements (8 KiB moved), i.e. one or
// two 16-byte vectors per thread.
// Short-lived workgroups of this size streamed HBM faster than larger items (4K-64K elements),
// more groups in flight per thread, or a persistent grid.
#ifndef TIDE_THREADS
#define TIDE_THREADS 128
#endif
#ifndef TIDE_AG_THREADS
#define TIDE_AG_THREADS 128
#endif
#ifndef TIDE_RS_CHUNK
#define TIDE_RS_CHUNK 1024
#endif
#ifndef TIDE_AG_CHUNK
#define TIDE_AG_CHUNK 2048
#endif
// RS single-item workgroups under a per-CU cap (TIDE_LAUNCH_PER_CU_CAP N): at most N RS workgroups
// per CU, enforced by the local-memory size each launch requests (the CU's LDS divided by N).
// Fewer requests in flight stream HBM better than a full CU, and a workgroup's traffic grows with
// C (2C + 4 bytes per output), so the best count falls as C grows.  Measured with 128-thread
// workgroups on the Llama-3.1-8B group: C = 8: 6 per CU beat 3, 4, 5, 7, 8 and no cap by 1-5%;
// C = 4: 8 beat 6, 12 and 16 (+2.4% over 6); C = 2 and 1: 12 beat 8, 16 and no cap (C = 1: 4.1
// TB/s at 6 -> 6.4 TB/s); C = 12: 6 beat 3, 4, 5 and no cap (5.93 TB/s); C = 16: 4 and 5 beat 2,
// 3 and no cap (5.82 TB/s).  Contributor counts up to kRsMaxCt are compiled in; above, the
// runtime-C kernel's full items load the contributors in blocks of 8: C = 20: 6 per CU 5.80 TB/s
// (3: 4.51, 4: 5.61, 5: 5.73, 8: 5.69, no cap 5.61); C = 32: 4 per CU 5.74 TB/s (3: 4.87, 5: 5.73,
// 6: 5.71, 8: 5.60, no cap 5.58).
constexpr int kRsMaxCt = 16;
#ifndef TIDE_RS_NQ
#define TIDE_RS_NQ 2
#endif
// RS, full aligned items: 0 = 8-byte loads in 4-output lane groups; 1 = 16-byte loads, 8 sums per
// lane, fp32 results redistributed through LDS for lane-contiguous stores (+1% measured on all
// four layer groups; the group path still serves partial and unaligned items).
#ifndef TIDE_RS_WIDE
#define TIDE_RS_WIDE 1
#endif
// Cache policy of the wide path's HBM accesses: -1 = global loads/stores with the non-temporal
// hint; >= 0 = raw buffer loads/stores with this cache-policy field (gfx950: bit 0 sc0, bit 1 nt,
// bit 4 sc1), each bounded in hardware by its work item's byte range.  Measured: without nt -5%;
// loads nt (2) and stores nt + sc1 (18) +0.6-1.6% over global non-temporal accesses.
#ifndef TIDE_RS_LOAD_AUX
#define TIDE_RS_LOAD_AUX 2
#endif
#ifndef TIDE_RS_STORE_AUX
#define TIDE_RS_STORE_AUX 18
#endif
// AG vector path: -1 = global non-temporal accesses; >= 0 = raw buffer accesses with this
// cache-policy field (stores add TIDE_AG_STORE_EXTRA).  Measured: no better than -1 for the copy.
#ifndef TIDE_AG_BUF_AUX
#define TIDE_AG_BUF_AUX -1
#endif
#ifndef TIDE_AG_STORE_EXTRA
#define TIDE_AG_STORE_EXTRA 0
#endif
#ifndef TIDE_AG_VECS
#define TIDE_AG_VECS 4
#endif
// AG, bounded launches: with at most this many AG workgroups per CU, a workgroup loads two full
// items before storing them (more bytes in flight where few waves are resident).  Measured on the
// Llama-3.1-8B and Qwen3 groups: budget 256 2.4-2.7 -> 4.1-4.9 TB/s, 512 4.2-4.5 -> 5.4-5.5 TB/s;
// at 6 or more workgroups per CU pairing was 3-10% slower, and batches of 4 or 8 slower still.
#ifndef TIDE_AG_BATCH_MAX_WGS_PER_CU
#define TIDE_AG_BATCH_MAX_WGS_PER_CU 4
#endif
constexpr int kAgBatchMaxWgsPerCu = TIDE_AG_BATCH_MAX_WGS_PER_CU;
// Non-temporal (streaming) hints on HBM loads and stores.
#ifndef TIDE_LOAD_NT
#define TIDE_LOAD_NT 1
#endif
#ifndef TIDE_STORE_NT
#define TIDE_STORE_NT 1
#endif
// One-launch single-item forms (default placement, per-CU caps): 0 = one workgroup per work item; N > 0 = at most N
// workgroups, each walking items with a grid stride.
#ifndef TIDE_PERSISTENT_WGS
#define TIDE_PERSISTENT_WGS 0
#endif

// Work-item order and XCD-aware renumbering (layout.cpp order_items, kernels.hip item_of).
// Measured: the RS streams best rank-major (each shard written front to back) with each of the 8
// XCDs of an MI355X walking one contiguous range of items; the AG copy best parameter-major with
// plain round-robin dispatch.  Orders: 0 parameter-major, 1 rank-major, 2 interleaved.
#ifndef TIDE_RS_ITEM_ORDER
#define TIDE_RS_ITEM_ORDER 1
#endif
#ifndef TIDE_AG_ITEM_ORDER
#define TIDE_AG_ITEM_ORDER 0
#endif
#ifndef TIDE_RS_XCD_REMAP
#define TIDE_RS_XCD_REMAP 1
#endif
#ifndef TIDE_AG_XCD_REMAP
#define TIDE_AG_XCD_REMAP 0
#endif
constexpr int64_t kXcds = 8;

constexpr int kThreads = TIDE_THREADS;
constexpr int kAgThreads = TIDE_AG_THREADS;
// Unit of TIDE_LAUNCH_BOUNDED: B admits B * kBudgetThreads threads of resident communication workgroups.
constexpr int kBudgetThreads = 256;
static_assert(kBudgetThreads % kThreads == 0 && kBudgetThreads % TIDE_AG_THREADS == 0,
              "a budget slot holds whole workgroups");
constexpr int64_t kRsChunk = TIDE_RS_CHUNK;
constexpr int64_t kAgChunk = TIDE_AG_CHUNK;
constexpr int64_t kPersistentWorkgroups = TIDE_PERSISTENT_WGS;
// Work items are whole 16-byte source vectors, so every item after a segment's first starts on a
// 16-byte source boundary.
static_assert(kRsChunk % 8 == 0 && kAgChunk % 8 == 0, "work items must be whole 16-byte vectors");
static_assert(kRsChunk < (int64_t(1) << 31) && kAgChunk < (int64_t(1) << 31), "item sizes are int32");
static_assert(kAgChunk % (8 * TIDE_AG_THREADS) == 0, "a full AG item is whole vectors for every lane");

// Bounded launches (TIDE_LAUNCH_BOUNDED B): at most B * kBudgetThreads threads of RS (or AG) workgroups
// are resident; each workgroup takes this many work items and exits, and the call issues as many
// launches as it needs.  0 = a single launch whose workgroups walk all items (resident for the
// whole call).
// Measured on MI355X against a concurrent one-wave bf16 GEMM (hipBLASLt, one 256x256 tile per
// CU): the GEMM's waves cannot share a SIMD with a resident RS wave, so a GEMM workgroup waits
// until the RS workgroups on its CU exit.  Workgroups that live for the whole call (0) slowed the
// GEMM ~7x even at B = 256; 64 items 0.5-2.5x; 16 items 4-27%; 4 items 4-8%.  Short-lived it is.
#ifndef TIDE_RS_BOUNDED_ITEMS
#define TIDE_RS_BOUNDED_ITEMS 4
#endif
// AG: 8 items (64 KiB of traffic per workgroup, like the RS's 80 KiB).  Measured on the Llama-3.1-70B group
// at budget 512 against the one-wave GEMM: 16 items 5.55 TB/s, GEMM +10.9%; 8 items 4.94 TB/s, +3.7%;
// 4 items 4.06 TB/s, +5.5%.
#ifndef TIDE_AG_BOUNDED_ITEMS
#define TIDE_AG_BOUNDED_ITEMS 8
#endif
constexpr int kRsBoundedItems = TIDE_RS_BOUNDED_ITEMS;

// CU-exclusive RS launches (TIDE_LAUNCH_CU_EXCLUSIVE N): one launch of workgroups of W = min(N, 8)
// 128-thread groups taking N/W work items each, and the largest local memory a workgroup may
// request, so each CU holds one RS workgroup and is empty whenever it exits.  Measured on MI355X (one flat
// C = 8 parameter, 2^27 outputs, beside the one-wave bf16 GEMM): W = 2 5.04 TB/s, GEMM +2.5%;
// 4: 6.25 TB/s, +4.4%; 6: 6.27, +7.9%; 8: 6.36, +10.5%; bounded budget 512 (same resident threads
// as W = 4): 5.33 TB/s, -0.2%; W = 4 with only its own local memory (several per CU): +261%.
constexpr int kRsCuMaxGroups = 8;  // 128-thread groups per CU-exclusive RS workgroup
constexpr int kAgCuMaxItems = 8;   // AG placement / Slot-Reuse packing in the same CU-exclusive form
static_assert(kThreads * kRsCuMaxGroups <= 1024, "a CU-exclusive workgroup fits the workgroup size limit");
// Items per group of a CU-exclusive RS workgroup: 1, or 2 for C <= 4 (compiled contributor counts):
// all of a group's loads stay in registers at once.  Measured on MI355X (Llama-3.1-8B shapes, one
// 8-group workgroup per CU): 2 items per group over 1 at C = 1 / 2 / 3 / 4: 5.9 / 6.12 / 6.17 / 6.19
// against 4.76 / 5.54 / 6.03 / 6.14 TB/s; 4 items per group at C = 1 / 2: 5.66 / 5.78, and 2 items per
// group at C = 8 (16 in flight per CU): 6.02 against 6.34 TB/s for 8 items (Llama-3.1-70B), not kept.
constexpr int kRsCuKi2MaxC = 4;
constexpr bool rs_cu_items_ok(int C, int ki) { return ki == 1 || (ki == 2 && C >= 1 && C <= kRsCuKi2MaxC); }
// Local memory of the exchange slots of a CU-exclusive RS workgroup: 4 KiB per item in flight.
constexpr int rs_cu_xfer_bytes(int groups, int ki) { return groups * ki * 2 * kThreads * 16; }
static_assert(rs_cu_xfer_bytes(kRsCuMaxGroups, 2) <= 64 * 1024, "the widest CU-exclusive RS workgroup fits a CU");
constexpr int kAgBoundedItems = TIDE_AG_BOUNDED_ITEMS;

// Index maps shared by the kernels and the host (one definition, so host-side checks see exactly
// what the kernels compute).
#if defined(__HIP__)
#define TIDE_HD __attribute__((host)) __attribute__((device))
#else
#define TIDE_HD
#endif

// Work item taken by workgroup `block` of a `grid`-workgroup launch over `count` items, at step j of
// its loop (it takes items while the result is below `count`).  Workgroups are dispatched
// round-robin over the XCDs (workgroup b runs on XCD b mod kXcds).  With `remap`, when the grid has
// one workgroup per item, the items are renumbered so that every XCD walks one contiguous range of
// the table, keeping its L2 and TLB on one stream of pages (a bijection on [0, count)); such a grid
// has no item for j > 0 (a launch may still pass more items per workgroup, e.g. a bounded launch's
// short tail), so every item is taken exactly once.  Otherwise items stride by the grid.
TIDE_HD inline int64_t item_index(bool remap, int64_t grid, int64_t block, int j, int64_t count) {
  if (remap && grid == count) {
    if (j > 0) return count;
    const int64_t x = block % kXcds, i = block / kXcds;
    return x * (count / kXcds) + (x < count % kXcds ? x : count % kXcds) + i;
  }
  return block + static_cast<int64_t>(j) * grid;
}

// Workgroup slot of workgroup `block` in a one-launch grid of `grid` workgroups: each XCD walks one
// contiguous range of slots (a bijection on [0, grid)).
TIDE_HD inline int64_t xcd_slot(int64_t grid, int64_t block) {
  const int64_t x = block % kXcds, i = block / kXcds;
  return x * (grid / kXcds) + (x < grid % kXcds ? x : grid % kXcds) + i;
}

// Launch plan for `count` work items: bounded = grids of at most `max_wgs` workgroups, each taking
// `bounded_items` items and exiting (bounded_items 0: one launch, workgroups walk every item);
// otherwise one launch of single-item workgroups (or kPersistentWorkgroups walking them).  Launch k
// covers items [k*per_launch, min((k+1)*per_launch, count)) with min(grid, its item count) workgroups.
struct Plan {
  int grid;
  int items;
  int64_t per_launch;
};

inline Plan plan_for(int64_t count, bool bounded, int64_t max_wgs, int bounded_items) {
  if (!bounded) {
    const int64_t cap = kPersistentWorkgroups > 0 ? kPersistentWorkgroups : (int64_t(1) << 30);
    const int64_t g = count < cap ? count : cap;
    const int items = int((count + g - 1) / g);
    return Plan{int(g), items, int64_t(g) * items};
  }
  const int64_t lim = count < max_wgs ? count : max_wgs;
  const int64_t grid = lim > 1 ? lim : 1;
  const int64_t items = bounded_items > 0 ? bounded_items : (count + grid - 1) / grid;
  return Plan{int(grid), int(items), grid * items};
}

// One RS work item: nvalid summed elements of parameter p, starting at element `src` of the
// parameter's storage, written to shard r at element `dst`; then npad zeros at dst + nvalid.
struct RsChunk {
  int64_t src;
  int64_t dst;
  int32_t p;
  int32_t r;
  int32_t nvalid;
  int32_t npad;
};
static_assert(sizeof(RsChunk) == 32, "RsChunk is two 16-byte scalar loads");

// One AG work item: n bf16 elements from stage element `src` to parameter p's element `dst`.
struct AgChunk {
  int64_t src;
  int64_t dst;
  int32_t p;
  int32_t n;
  int64_t reserved;
};
static_assert(sizeof(AgChunk) == 32, "AgChunk is two 16-byte scalar loads");

// Kernel launchers (kernels.hip).  `hip_stream` is a hipStream_t.  They return a hipError_t.
// launch_rs: flat = false reads per-parameter gradients (table [C*P grads][R shards]); flat = true
// reads C packed slots of R*S elements (table [C slots][R shards]).
// launch_ag: pack = false places stage -> parameters; pack = true packs parameters -> stage slot.
// launch_fill_zero: zeros the slot ranges of `items` (src = slot element offset, n).
// `dyn_lds` is the dynamic local memory each RS workgroup requests (occupancy cap; 0 = none);
// `batch` (1 or 2) is the number of full AG items a workgroup loads before storing.
// rs_lds_info: the local memory per CU of `device` and the static local memory of the RS kernel
// for C <= kRsMaxCt (compile-time contributor count) and above (runtime count).
// rs_dynamic_lds: the dynamic local memory that admits at most `wgs_per_cu` RS workgroups per CU
// (0 = no cap, or when it cannot be met).
int launch_rs(const RsChunk* chunks, int64_t first, int64_t count, int grid, int items_per_wg,
              const void* const* dev_ptrs, int32_t P, int32_t C, int64_t S, bool flat, bool vec, int dyn_lds,
              void* hip_stream);
int rs_lds_info(int device, int* lds_per_cu, int* static_lds_ct, int* static_lds_rt);
// launch_rs_cu: the CU-exclusive RS over all `count` items in one launch, `groups` (1 ..
// kRsCuMaxGroups) groups of 128 threads per workgroup, each taking `items_per_group` items
// (rs_cu_items_ok); `lds` is the dynamic local memory each workgroup requests (at least
// rs_cu_xfer_bytes; the whole CU's to keep it exclusive).  The kernel has no static local memory.
int launch_rs_cu(const RsChunk* chunks, int64_t count, int groups, int items_per_group, const void* const* dev_ptrs,
                 int32_t P, int32_t C, int64_t S, bool flat, bool vec, int lds, void* hip_stream);
// launch_ag_cu: the CU-exclusive AG placement (pack = false) or packing (pack = true) over all
// `count` items in one launch, items_per_wg (1 .. kAgCuMaxItems) items per workgroup.
int launch_ag_cu(const AgChunk* chunks, int64_t count, int items_per_wg, void* stage, const void* const* dev_params,
                 bool pack, bool vec, int dyn_lds, void* hip_stream);
inline int rs_dynamic_lds(int lds_per_cu, int static_lds, int wgs_per_cu) {
  if (wgs_per_cu <= 0 || lds_per_cu <= 0) return 0;
  // rounded down to 512 bytes per workgroup, so wgs_per_cu of them fit in a CU (and, for counts up
  // to 16, one more does not)
  const int dyn = (lds_per_cu / wgs_per_cu) / 512 * 512 - static_lds;
  return dyn > 0 ? dyn : 0;
}
int launch_ag(const AgChunk* chunks, int64_t first, int64_t count, int grid, int items_per_wg, int batch,
              void* stage, const void* const* dev_params, bool pack, bool vec, void* hip_stream);
int launch_fill_zero(const AgChunk* items, int64_t count, void* slot, void* hip_stream);
// Device address of the fixed pointer-table scratch array of the allocation-free RS entry point on
// the current device (hipGetSymbolAddress once per device, then cached); `max_ptrs` gets its size.
int noalloc_scratch(int device, void** out, int64_t* max_ptrs);
// Writes the n pointers `ptrs` (host) into the device array `dst` with kernel launches on
// `hip_stream` (the values travel as kernel arguments: no copy from host memory, no allocation).
int launch_put_ptrs(void* dst, void* const* ptrs, int64_t n, void* hip_stream);

}  // namespace tide
