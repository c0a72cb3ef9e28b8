// Internal declarations shared by the host layout code, the entry points and the gfx950 kernels.
#pragma once

#include <stdint.h>

#include <cstddef>

namespace tide {

// Threads per workgroup of every kernel: 4 wave64 waves, one per SIMD of a CDNA4 CU.
constexpr int kThreads = 256;

// Work-item sizes, in elements.  An RS work item of 16384 outputs moves 16384 * (2C + 4) bytes
// (320 KiB at C = 8); an AG work item of 32768 elements moves 128 KiB.  Both are multiples of 8,
// so every work item after a segment's first starts on a 16-byte source boundary.
#ifndef TIDE_RS_CHUNK
#define TIDE_RS_CHUNK 16384
#endif
#ifndef TIDE_AG_CHUNK
#define TIDE_AG_CHUNK 32768
#endif
constexpr int64_t kRsChunk = TIDE_RS_CHUNK;
constexpr int64_t kAgChunk = TIDE_AG_CHUNK;
static_assert(kRsChunk % 8 == 0 && kAgChunk % 8 == 0, "work items must be whole 16-byte vectors");

// Work items a workgroup takes per launch when the caller bounds the resident workgroups.
constexpr int kItemsPerBoundedWorkgroup = 4;

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
