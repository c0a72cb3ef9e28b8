// Internal declarations shared by the host layout code, the entry points and the gfx950 kernels.
#pragma once

#include <stdint.h>

#include <cstddef>

namespace tide {

// Threads per workgroup of every kernel (default: 4 wave64 waves, one per SIMD of a CDNA4 CU).
#ifndef TIDE_THREADS
#define TIDE_THREADS 256
#endif
constexpr int kThreads = TIDE_THREADS;

// Work-item sizes, in elements.  One RS work item is 2048 outputs: with 256 threads each thread
// sums exactly one 8-output vector (one 16-byte load per contributor, two 16-byte stores), and a
// workgroup moves 2048 * (2C + 4) bytes (40 KiB at C = 8) and exits.  One AG work item is 4096
// elements (16 KiB moved).  Measured on MI355X, such short-lived workgroups stream HBM faster than
// larger items or a persistent grid.  Both sizes are multiples of 8, so every work item after a
// segment's first starts on a 16-byte source boundary.
#ifndef TIDE_RS_CHUNK
#define TIDE_RS_CHUNK 2048
#endif
#ifndef TIDE_AG_CHUNK
#define TIDE_AG_CHUNK 4096
#endif
constexpr int64_t kRsChunk = TIDE_RS_CHUNK;
constexpr int64_t kAgChunk = TIDE_AG_CHUNK;
static_assert(kRsChunk % 8 == 0 && kAgChunk % 8 == 0, "work items must be whole 16-byte vectors");

// Work items a workgroup takes per launch when the caller bounds the resident workgroups.
constexpr int kItemsPerBoundedWorkgroup = 4;

// Unbounded launches (cu_budget 0): 0 = one workgroup per work item; N > 0 = at most N
// workgroups, each walking items with a grid stride.
#ifndef TIDE_PERSISTENT_WGS
#define TIDE_PERSISTENT_WGS 0
#endif
constexpr int64_t kPersistentWorkgroups = TIDE_PERSISTENT_WGS;

// Kernel shape: 8-output (RS) / 16-byte (AG) vectors each thread keeps in flight per step, and
// whether HBM accesses carry the non-temporal (streaming) hint.
#ifndef TIDE_RS_VECS
#define TIDE_RS_VECS 1
#endif
#ifndef TIDE_AG_VECS
#define TIDE_AG_VECS 4
#endif
#ifndef TIDE_LOAD_NT
#define TIDE_LOAD_NT 1
#endif
#ifndef TIDE_STORE_NT
#define TIDE_STORE_NT 1
#endif

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
int launch_rs(const RsChunk* chunks, int64_t first, int64_t count, int grid, int items_per_wg,
              const void* const* dev_ptrs, int32_t P, int32_t C, bool vec, void* hip_stream);
int launch_ag(const AgChunk* chunks, int64_t first, int64_t count, int grid, int items_per_wg,
              const void* stage, const void* const* dev_params, bool vec, void* hip_stream);

}  // namespace tide
