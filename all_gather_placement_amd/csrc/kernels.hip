// gfx950 kernels of the layout-aware reduce-scatter and all-gather placement.
//
// Both kernels walk a host-built table of work items (tide_internal.h).  A work item lies inside
// one (parameter, rank) segment, so a workgroup reads its item descriptor and the item's source
// pointers once, as wave-uniform scalar loads into SGPRs, and then streams contiguous memory: no
// per-element index search, no atomics, no inter-workgroup communication.  Every output element
// has exactly one writer, and every workgroup is short-lived: one work item (a few in bounded
// launches), then exit.
//
// RS ([Endgame] Figure 6a, node-local fp32 sums; abstract, bf16 gradients reduced into fp32
// shards): every output is the sum of its C contributors' bf16 inputs, each widened exactly to
// fp32 and added in ascending contributor order (C-1 IEEE binary32 adds).  On a full, aligned work
// item a lane loads one 16-byte vector (8 bf16) per contributor, so each wave load instruction
// covers 1 KiB of one contributor; the 8 fp32 sums per lane are exchanged through LDS so that each
// wave store instruction covers 1 KiB of whole cache lines.  Partial items (segment heads and
// tails) take 4-output lane groups (8-byte loads, 16-byte stores).  At C = 8 an output costs
// 20 bytes of HBM traffic and 7 adds: the kernel is HBM-bound by two orders of magnitude, so it
// is shaped for bytes in flight and clean traffic, not arithmetic (no matrix cores: nothing here
// is a contraction).
//
// AG ([Endgame] Figure 5b, each parameter filled by a single strided copy; Table 7, direct landing): a bit copy
// of each rank's valid rows from the rank-major stage into the parameter's storage, 16 bytes per
// lane per access when source and destination share their 16-byte phase.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "../../include/tide.h"
#include "tide_internal.h"

namespace tide {
namespace {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Every buffer the kernels touch is in HBM.  Pointers that arrive through a table would otherwise
// be generic (flat) pointers; accesses go through global-address-space casts to get global_*
// instructions instead of flat_* ones.
#define TIDE_GLOBAL __attribute__((address_space(1)))

// Streaming (non-temporal) accesses: every input byte is read once and every output byte written
// once, so nothing is worth keeping in the caches.
template <typename T>
__device__ __forceinline__ T load_hbm(const T* p) {
#if TIDE_LOAD_NT
  return __builtin_nontemporal_load((const TIDE_GLOBAL T*)p);
#else
  return *(const TIDE_GLOBAL T*)p;
#endif
}
template <typename T>
__device__ __forceinline__ void store_hbm(T* p, T v) {
#if TIDE_STORE_NT
  __builtin_nontemporal_store(v, (TIDE_GLOBAL T*)p);
#else
  *(TIDE_GLOBAL T*)p = v;
#endif
}

// bf16 -> fp32 is exact: the 16 bf16 bits become the upper half of the binary32.
__device__ __forceinline__ float widen_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float widen_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float widen1(unsigned short b) { return __uint_as_float(static_cast<unsigned int>(b) << 16); }

// acc[0..3] (+)= the 4 bf16 of x (element 0 in the low half of x.x).
__device__ __forceinline__ void widen4(u32x2 x, float acc[4]) {
  acc[0] = widen_lo(x.x); acc[1] = widen_hi(x.x); acc[2] = widen_lo(x.y); acc[3] = widen_hi(x.y);
}
__device__ __forceinline__ void add4(u32x2 x, float acc[4]) {
  acc[0] += widen_lo(x.x); acc[1] += widen_hi(x.x); acc[2] += widen_lo(x.y); acc[3] += widen_hi(x.y);
}
__device__ __forceinline__ void store4(float* d, const float a[4], bool dst16) {
  if (dst16) {
    store_hbm(reinterpret_cast<f32x4*>(d), f32x4{a[0], a[1], a[2], a[3]});
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) store_hbm(d + k, a[k]);
  }
}

// Work item taken by this workgroup at step j of its loop (item_index, tide_internal.h).
template <bool REMAP>
__device__ __forceinline__ int64_t item_of(int j, int64_t count) {
  return item_index(REMAP, gridDim.x, blockIdx.x, j, count);
}

// One output element, fixed ascending contributor order (heads, tails, unaligned bases).
template <int CT>
__device__ __forceinline__ float sum1(const unsigned short* const* src, int C, int64_t i) {
  const int n = CT > 0 ? CT : C;
  float acc = widen1(load_hbm(src[0] + i));
  for (int c = 1; c < n; ++c) acc += widen1(load_hbm(src[c] + i));
  return acc;
}

// Address = wave-uniform base (SGPRs) + 32-bit per-lane byte offset, which maps onto the
// global_load/store "saddr + voffset" form and keeps 64-bit addresses out of VGPRs.
template <typename T, typename B>
__device__ __forceinline__ const T* at_bytes(const B* base, uint32_t byte_off) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}
template <typename T, typename B>
__device__ __forceinline__ T* at_bytes(B* base, uint32_t byte_off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + byte_off);
}

// NQ groups of 4 outputs, kThreads groups apart, starting at element i0 of the item (i0 < 2^30,
// item-relative).  All NQ*C loads are issued before the first add.
template <int CT, int NQ>
__device__ __forceinline__ void sum_groups(const unsigned short* const* src, uint32_t i0, float* dst, bool dst16) {
  u32x2 x[NQ][CT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int k = 0; k < NQ; ++k) x[k][c] = load_hbm(at_bytes<u32x2>(src[c], 2u * (i0 + 4u * kThreads * k)));
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    float a[4];
    widen4(x[k][0], a);
#pragma unroll
    for (int c = 1; c < CT; ++c) add4(x[k][c], a);
    store4(at_bytes<float>(dst, 4u * (i0 + 4u * kThreads * k)), a, dst16);
  }
}

// Runtime contributor count (C > kRsMaxCt): same mapping, contributors loaded one at a time.
__device__ __forceinline__ void sum_group_rt(const unsigned short* const* gptr, int32_t P, int32_t p, int C,
                                             int64_t e, float* d, bool dst16) {
  float a[4];
  widen4(load_hbm(reinterpret_cast<const u32x2*>(gptr[p] + e)), a);
  for (int c = 1; c < C; ++c) add4(load_hbm(reinterpret_cast<const u32x2*>(gptr[static_cast<int64_t>(c) * P + p] + e)), a);
  store4(d, a, dst16);
}

// Element path for the runtime contributor count.
__device__ __forceinline__ float sum1_rt(const unsigned short* const* gptr, int32_t P, int32_t p, int C, int64_t e) {
  float acc = widen1(load_hbm(gptr[p] + e));
  for (int c = 1; c < C; ++c) acc += widen1(load_hbm(gptr[static_cast<int64_t>(c) * P + p] + e));
  return acc;
}

// Full work item: kThreads * 8 valid outputs, 16-byte-aligned source and destination offsets
// (so every lane takes whole 16-byte vectors), no padding.  Most items of a layer group are full.
__device__ __forceinline__ bool full_item(const RsChunk& ch) {
  return ch.nvalid == kThreads * 8 && ch.npad == 0 && (ch.src & 7) == 0 && (ch.dst & 3) == 0;
}

// Full item, step 1: one 16-byte load per contributor per lane, so each wave load instruction
// covers 1 KiB of one contributor.  Raw buffer loads are bounded in hardware to the item's bytes.
template <int CT>
__device__ __forceinline__ void full_item_load(const unsigned short* const* src, int tid, u32x4 x[CT]) {
#if TIDE_RS_LOAD_AUX >= 0
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(src[c]), 0, 16 * kThreads, 0x00020000);
    x[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * tid, 0, TIDE_RS_LOAD_AUX));
  }
#else
#pragma unroll
  for (int c = 0; c < CT; ++c) x[c] = load_hbm(at_bytes<u32x4>(src[c], 16u * tid));
#endif
}

// Full item, step 2: 8 sums per lane in ascending contributor order, then the fp32 results are
// exchanged through LDS so that each 16-byte store instruction of a wave covers 1 KiB of whole
// cache lines.  All threads of the workgroup call it (it synchronises the workgroup).
template <int CT>
__device__ __forceinline__ void full_item_sums(const u32x4 x[CT], float a[8]) {
  a[0] = widen_lo(x[0].x); a[1] = widen_hi(x[0].x); a[2] = widen_lo(x[0].y); a[3] = widen_hi(x[0].y);
  a[4] = widen_lo(x[0].z); a[5] = widen_hi(x[0].z); a[6] = widen_lo(x[0].w); a[7] = widen_hi(x[0].w);
#pragma unroll
  for (int c = 1; c < CT; ++c) {
    a[0] += widen_lo(x[c].x); a[1] += widen_hi(x[c].x); a[2] += widen_lo(x[c].y); a[3] += widen_hi(x[c].y);
    a[4] += widen_lo(x[c].z); a[5] += widen_hi(x[c].z); a[6] += widen_lo(x[c].w); a[7] += widen_hi(x[c].w);
  }
}

// A lane's 8 sums into the exchange buffer: outputs 8*tid .. 8*tid+7 of the item.
__device__ __forceinline__ void full_item_put(const float a[8], f32x4* xfer, int tid) {
  xfer[2 * tid] = f32x4{a[0], a[1], a[2], a[3]};
  xfer[2 * tid + 1] = f32x4{a[4], a[5], a[6], a[7]};
}

// The item's 1024 fp32 outputs from the exchange buffer: two 16-byte stores per lane, so each wave
// store instruction covers 1 KiB of whole cache lines.
__device__ __forceinline__ void full_item_store(const f32x4* xfer, float* dst, int tid) {
#if TIDE_RS_STORE_AUX >= 0
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(dst, 0, 32 * kThreads, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, xfer[tid]), rsrc, 16 * tid, 0, TIDE_RS_STORE_AUX);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, xfer[tid + kThreads]), rsrc, 16 * (tid + kThreads),
                                         0, TIDE_RS_STORE_AUX);
#else
  store_hbm(at_bytes<f32x4>(dst, 16u * tid), xfer[tid]);
  store_hbm(at_bytes<f32x4>(dst, 16u * (tid + kThreads)), xfer[tid + kThreads]);
#endif
}

// Wave-local form of the exchange: a full item's wave w computed outputs 512*w .. 512*w + 511
// itself, so it can redistribute them through its own 2 KiB of the group's slot and store them as
// two 1 KiB wave instructions with no workgroup barrier: every wave stores as soon as its sums are
// done.  LDS instructions of one wave execute in order; the wavefront-scope fences only keep the
// compiler from moving the reads above the writes (or the next item's writes above these reads).
// Measured on MI355X against the workgroup-wide exchange (one barrier, then every group's stores):
// single-item workgroups (bounded launches, per-CU caps) +0.9% / +-0%; CU-exclusive workgroups of
// W = 2 / 3 / 4 groups +1.8 / +2.0 / +2.5%, 5 +-0%, 6 / 7 / 8 -4 / -4 / -1.4% (Llama-3.1-70B group,
// two runs each): wide workgroups stream better when all their stores leave together.
constexpr int kRsCuWaveMaxGroups = 4;  // CU-exclusive workgroups of at most this many groups store wave by wave
__device__ __forceinline__ void full_item_wave_store(const float a[8], f32x4* xfer, float* dst, int tid) {
  const int w = tid >> 6, l = tid & 63;
  f32x4* xw = xfer + w * 128;
  xw[2 * l] = f32x4{a[0], a[1], a[2], a[3]};
  xw[2 * l + 1] = f32x4{a[4], a[5], a[6], a[7]};
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const f32x4 v0 = xw[l], v1 = xw[64 + l];
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(dst + 512 * w, 0, 2048, 0x00020000);
  constexpr int aux = TIDE_RS_STORE_AUX >= 0 ? TIDE_RS_STORE_AUX : 18;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v0), rsrc, 16 * l, 0, aux);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v1), rsrc, 16 * (64 + l), 0, aux);
  // the next item's writes to this slot come after these reads (program order within the wave)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
}

template <int CT>
__device__ __forceinline__ void full_item_finish(const u32x4 x[CT], float* dst, f32x4* xfer, int tid) {
  float a[8];
  full_item_sums<CT>(x, a);
  full_item_wave_store(a, xfer, dst, tid);
}

// Full work item, runtime contributor count (C > kRsMaxCt): contributors in blocks of 8, each
// block's 8 loads issued together (a lane past C gets a zero-sized buffer range and its value is
// never added), sums in ascending contributor order, then the same exchange and stores as above.
constexpr int kRtLoadAux = TIDE_RS_LOAD_AUX >= 0 ? TIDE_RS_LOAD_AUX : 2;     // nt
constexpr int kRtStoreAux = TIDE_RS_STORE_AUX >= 0 ? TIDE_RS_STORE_AUX : 18;  // nt sc1
__device__ __forceinline__ void full_item_rt_sums(void* const* gptr, int32_t P, const RsChunk& ch, int C, int tid,
                                                  float out[8]) {
  constexpr int B = 8;
  float a[8] = {};
  for (int c0 = 0; c0 < C; c0 += B) {
    const int nb = min(B, C - c0);
    u32x4 x[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int c = k < nb ? c0 + k : c0;
      const unsigned short* src =
          reinterpret_cast<const unsigned short*>(gptr[static_cast<int64_t>(c) * P + ch.p]) + ch.src;
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(src), 0,
                                                                           k < nb ? 16 * kThreads : 0, 0x00020000);
      x[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * tid, 0, kRtLoadAux));
    }
    // keep all B loads ahead of their first use: without this the compiler moves each load next to
    // its conditional add below, one round trip per contributor (emits no instruction)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < B; ++k) {
      if (k >= nb) break;
      const float v[8] = {widen_lo(x[k].x), widen_hi(x[k].x), widen_lo(x[k].y), widen_hi(x[k].y),
                          widen_lo(x[k].z), widen_hi(x[k].z), widen_lo(x[k].w), widen_hi(x[k].w)};
      if (c0 + k == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = v[e];  // start from x_0 itself (keeps -0.0)
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += v[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = a[e];
}

__device__ __forceinline__ void full_item_rt_store(const f32x4* xfer, float* dst, int tid) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(dst, 0, 32 * kThreads, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, xfer[tid]), rsrc, 16 * tid, 0, kRtStoreAux);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, xfer[tid + kThreads]), rsrc, 16 * (tid + kThreads),
                                         0, kRtStoreAux);
}

__device__ __forceinline__ void full_item_rt(void* const* gptr, int32_t P, const RsChunk& ch, int C, float* dst,
                                             f32x4* xfer, int tid) {
  float a[8];
  full_item_rt_sums(gptr, P, ch, C, tid, a);
  full_item_wave_store(a, xfer, dst, tid);
}

// RS kernel.  CT in 1..kRsMaxCt: contributor count fixed at compile time; CT == 0: any C >= 1.
// VEC: all source and shard base pointers are 16-byte aligned (checked on the host), so the
// alignment of an element depends only on its offset inside its buffer.
// FLAT = false: sources are the per-parameter gradients, pointer table [C*P grads][R shards],
//   item source at gradient (c, p), element ch.src (in-place read).
// FLAT = true: sources are C packed rank-major slots of R*S elements (Slot-Reuse), pointer table
//   [C slots][R shards] (P = 1), item source at slot c, element ch.r * S + ch.dst.
template <int CT, bool VEC, bool FLAT>
__global__ __launch_bounds__(kThreads) void rs_kernel(const RsChunk* __restrict__ chunks, int64_t first,
                                                      int64_t count, int items_per_wg,
                                                      void* const* __restrict__ ptrs, int32_t P, int32_t C,
                                                      int64_t S) {
  const int tid = threadIdx.x;
  const unsigned short* const* __restrict__ gptr = reinterpret_cast<const unsigned short* const*>(ptrs);
  float* const* __restrict__ sptr = reinterpret_cast<float* const*>(ptrs + static_cast<int64_t>(C) * P);
  const int nc = CT > 0 ? CT : C;

#if TIDE_RS_WIDE
  __shared__ f32x4 xfer[2 * kThreads];
#endif

  for (int j = 0; j < items_per_wg; ++j) {
    const int64_t item = item_of<TIDE_RS_XCD_REMAP != 0>(j, count);
    if (item >= count) break;
    RsChunk ch = chunks[first + item];
    if (FLAT) {
      ch.src = static_cast<int64_t>(ch.r) * S + ch.dst;
      ch.p = 0;
    }
    float* dst = sptr[ch.r] + ch.dst;
    const int n = ch.nvalid;

    if (VEC) {
      // head: elements before the first 16-byte source boundary; then whole 4-output groups
      // (2 per 8 elements); tail: fewer than 8 elements.
      const int head = min(n, static_cast<int>((-ch.src) & 7));
      const int nb = (n - head) >> 3;
      const int ng = 2 * nb;
      const int tail = (n - head) & 7;
      const bool dst16 = ((ch.dst + head) & 3) == 0;
      if constexpr (CT > 0) {
        // Per-item source pointers (wave-uniform, SGPRs): contributor c's element ch.src of p.
        const unsigned short* src[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) src[c] = gptr[static_cast<int64_t>(c) * P + ch.p] + ch.src;
#if TIDE_RS_WIDE
        if (full_item(ch)) {
          u32x4 x[CT];
          full_item_load<CT>(src, tid, x);
          full_item_finish<CT>(x, dst, xfer, tid);
          continue;  // no tail, no padding in a full item
        }
#endif
        if (tid < head) store_hbm(dst + tid, sum1<CT>(src, nc, tid));
        constexpr int NQ = TIDE_RS_NQ;
        int q = tid;
        for (; q + (NQ - 1) * kThreads < ng; q += NQ * kThreads)
          sum_groups<CT, NQ>(src, static_cast<uint32_t>(head + 4 * q), dst, dst16);
        for (; q < ng; q += kThreads) sum_groups<CT, 1>(src, static_cast<uint32_t>(head + 4 * q), dst, dst16);
        if (tid < tail) {
          const int64_t k = head + 8 * static_cast<int64_t>(nb) + tid;
          store_hbm(dst + k, sum1<CT>(src, nc, k));
        }
      } else {
#if TIDE_RS_WIDE
        if (full_item(ch)) {
          full_item_rt(ptrs, P, ch, nc, dst, xfer, tid);
          continue;  // no tail, no padding in a full item
        }
#endif
        for (int i = tid; i < head; i += kThreads) store_hbm(dst + i, sum1_rt(gptr, P, ch.p, nc, ch.src + i));
        for (int q = tid; q < ng; q += kThreads) {
          const int64_t k = head + 4 * static_cast<int64_t>(q);
          sum_group_rt(gptr, P, ch.p, nc, ch.src + k, dst + k, dst16);
        }
        for (int i = tid; i < tail; i += kThreads) {
          const int64_t k = head + 8 * static_cast<int64_t>(nb) + i;
          store_hbm(dst + k, sum1_rt(gptr, P, ch.p, nc, ch.src + k));
        }
      }
    } else {
      // Element path: any 2-byte-aligned gradients and 4-byte-aligned shards.
      for (int i = tid; i < n; i += kThreads) store_hbm(dst + i, sum1_rt(gptr, P, ch.p, nc, ch.src + i));
    }

    // Padding rows of this rank's slice: +0.0.
    for (int i = tid; i < ch.npad; i += kThreads) store_hbm(dst + n + i, 0.0f);
  }
}

// The CT contributor base pointers of parameter p, all loaded before any is used: one scalar-load
// batch and one wait (an empty asm statement that takes every pointer as an SGPR operand keeps the
// compiler from pairing each load with its first use, which would serialise them; it emits no
// instruction).
template <int CT>
__device__ __forceinline__ void load_bases(const unsigned short* const* __restrict__ gptr, int32_t P, int32_t p,
                                           const unsigned short* (&b)[CT]) {
#pragma unroll
  for (int c = 0; c < CT; ++c) b[c] = gptr[static_cast<int64_t>(c) * P + p];
  if constexpr (CT == 1) {
    asm volatile("" : "+s"(b[0]));
  } else if constexpr (CT == 2) {
    asm volatile("" : "+s"(b[0]), "+s"(b[1]));
  } else if constexpr (CT == 4) {
    asm volatile("" : "+s"(b[0]), "+s"(b[1]), "+s"(b[2]), "+s"(b[3]));
  } else if constexpr (CT == 8) {
    asm volatile("" : "+s"(b[0]), "+s"(b[1]), "+s"(b[2]), "+s"(b[3]), "+s"(b[4]), "+s"(b[5]), "+s"(b[6]),
                 "+s"(b[7]));
  }
}

// One RS work item of a CU-exclusive workgroup's group (the per-item work of rs_kernel): with `wave`,
// a full item is stored through the wave-local exchange and nullptr returned; otherwise it leaves its
// sums in the group's exchange slot `xfer` and returns the destination to store them to after the
// workgroup barrier.  Any other item is written directly and returns nullptr.
template <int CT, bool VEC, bool FLAT>
__device__ __forceinline__ float* rs_cu_item(const RsChunk* __restrict__ chunks, int64_t item,
                                             void* const* __restrict__ ptrs, int32_t P, int32_t C, int64_t S,
                                             f32x4* xfer, int tid, bool wave) {
  const unsigned short* const* __restrict__ gptr = reinterpret_cast<const unsigned short* const*>(ptrs);
  float* const* __restrict__ sptr = reinterpret_cast<float* const*>(ptrs + static_cast<int64_t>(C) * P);
  const int nc = CT > 0 ? CT : C;
  RsChunk ch = chunks[item];
  if (FLAT) {
    ch.src = static_cast<int64_t>(ch.r) * S + ch.dst;
    ch.p = 0;
  }
  float* dst = sptr[ch.r] + ch.dst;
  const int n = ch.nvalid;
  float* full_dst = nullptr;

  if (VEC) {
    const int head = min(n, static_cast<int>((-ch.src) & 7));
    const int nb = (n - head) >> 3;
    const int ng = 2 * nb;
    const int tail = (n - head) & 7;
    const bool dst16 = ((ch.dst + head) & 3) == 0;
    if constexpr (CT > 0) {
      const unsigned short* src[CT];
      load_bases<CT>(gptr, P, ch.p, src);
#pragma unroll
      for (int c = 0; c < CT; ++c) src[c] += ch.src;
#if TIDE_RS_WIDE
      if (full_item(ch)) {
        u32x4 x[CT];
        float a[8];
        full_item_load<CT>(src, tid, x);
        full_item_sums<CT>(x, a);
        if (wave) {
          full_item_wave_store(a, xfer, dst, tid);
        } else {
          full_item_put(a, xfer, tid);
          full_dst = dst;
        }
      } else
#endif
      {
        if (tid < head) store_hbm(dst + tid, sum1<CT>(src, nc, tid));
        constexpr int NQ = TIDE_RS_NQ;
        int q = tid;
        for (; q + (NQ - 1) * kThreads < ng; q += NQ * kThreads)
          sum_groups<CT, NQ>(src, static_cast<uint32_t>(head + 4 * q), dst, dst16);
        for (; q < ng; q += kThreads) sum_groups<CT, 1>(src, static_cast<uint32_t>(head + 4 * q), dst, dst16);
        if (tid < tail) {
          const int64_t k = head + 8 * static_cast<int64_t>(nb) + tid;
          store_hbm(dst + k, sum1<CT>(src, nc, k));
        }
      }
    } else {
#if TIDE_RS_WIDE
      if (full_item(ch)) {
        float a[8];
        full_item_rt_sums(ptrs, P, ch, nc, tid, a);
        if (wave) {
          full_item_wave_store(a, xfer, dst, tid);
        } else {
          full_item_put(a, xfer, tid);
          full_dst = dst;
        }
      } else
#endif
      {
        for (int i = tid; i < head; i += kThreads) store_hbm(dst + i, sum1_rt(gptr, P, ch.p, nc, ch.src + i));
        for (int q = tid; q < ng; q += kThreads) {
          const int64_t k = head + 4 * static_cast<int64_t>(q);
          sum_group_rt(gptr, P, ch.p, nc, ch.src + k, dst + k, dst16);
        }
        for (int i = tid; i < tail; i += kThreads) {
          const int64_t k = head + 8 * static_cast<int64_t>(nb) + i;
          store_hbm(dst + k, sum1_rt(gptr, P, ch.p, nc, ch.src + k));
        }
      }
    }
  } else {
    for (int i = tid; i < n; i += kThreads) store_hbm(dst + i, sum1_rt(gptr, P, ch.p, nc, ch.src + i));
  }
  // padding rows of this rank's slice (a full item has none)
  for (int i = tid; i < ch.npad; i += kThreads) store_hbm(dst + n + i, 0.0f);
  return full_dst;
}

// CU-exclusive RS kernel: one launch over all work items in workgroups of W = blockDim.x / 128
// groups of 128 threads (W <= kRsCuMaxGroups), each group taking KI consecutive items; group g of
// workgroup slot s takes items (s*W + g)*KI .. +KI-1, with the same per-item work as rs_kernel.  The
// host gives every workgroup the largest local memory one may request (here all of it dynamic: the
// W*KI exchange slots of 4 KiB and the rest unused), so a CU holds a single RS workgroup and is empty
// again whenever it exits: a concurrent kernel's workgroup waiting for a whole CU (a one-wave GEMM's,
// for instance) takes it within one RS workgroup lifetime, while the RS itself runs as one launch
// with W*KI items resident per CU.  With KI > 1 (few contributors, whose items carry few bytes), a
// group whose KI items are all full issues every load of all of them before its first sum, so the
// CU keeps as many bytes in flight as with more contributors.  Workgroups of more than
// kRsCuWaveMaxGroups groups have one workgroup barrier, outside every per-group branch: full items
// leave their sums in their exchange slots and are stored after it, all together; the others are
// finished before it.  Narrower workgroups store each full item wave by wave, with no barrier.
template <int CT, int KI, bool VEC, bool FLAT>
__global__ __launch_bounds__(kThreads * kRsCuMaxGroups) void rs_cu_kernel(const RsChunk* __restrict__ chunks,
                                                                          int64_t count,
                                                                          void* const* __restrict__ ptrs,
                                                                          int32_t P, int32_t C, int64_t S) {
  extern __shared__ f32x4 xfer_dyn[];  // W*KI exchange slots of 2*kThreads vectors
  const int W = static_cast<int>(blockDim.x) / kThreads;
  const int grp = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kThreads);
  const int tid = static_cast<int>(threadIdx.x) % kThreads;
  // workgroup slots, one per grid position: each XCD walks one contiguous range of them
  const int64_t slot = TIDE_RS_XCD_REMAP != 0 ? xcd_slot(gridDim.x, blockIdx.x) : static_cast<int64_t>(blockIdx.x);
  const int64_t first = (slot * W + grp) * KI;
  f32x4* xfer = xfer_dyn + static_cast<int64_t>(grp) * KI * 2 * kThreads;
  const bool wave = W <= kRsCuWaveMaxGroups;  // uniform over the workgroup
  float* full_dst[KI];
#pragma unroll
  for (int k = 0; k < KI; ++k) full_dst[k] = nullptr;

  bool done = false;
#if TIDE_RS_WIDE
  if constexpr (KI > 1 && CT > 0 && VEC) {
    // all KI items full: every load of every item in flight before the first sum
    if (first + KI <= count) {
      RsChunk ch[KI];
      bool all_full = true;
#pragma unroll
      for (int k = 0; k < KI; ++k) {
        ch[k] = chunks[first + k];
        if (FLAT) {
          ch[k].src = static_cast<int64_t>(ch[k].r) * S + ch[k].dst;
          ch[k].p = 0;
        }
        all_full = all_full && full_item(ch[k]);
      }
      if (all_full) {
        const unsigned short* const* __restrict__ gptr = reinterpret_cast<const unsigned short* const*>(ptrs);
        float* const* __restrict__ sptr = reinterpret_cast<float* const*>(ptrs + static_cast<int64_t>(C) * P);
        u32x4 x[KI][CT];
#pragma unroll
        for (int k = 0; k < KI; ++k) {
          const unsigned short* src[CT];
          load_bases<CT>(gptr, P, ch[k].p, src);
#pragma unroll
          for (int c = 0; c < CT; ++c) src[c] += ch[k].src;
          full_item_load<CT>(src, tid, x[k]);
          full_dst[k] = sptr[ch[k].r] + ch[k].dst;
        }
#pragma unroll
        for (int k = 0; k < KI; ++k) {
          float a[8];
          full_item_sums<CT>(x[k], a);
          if (wave) {
            full_item_wave_store(a, xfer + k * 2 * kThreads, full_dst[k], tid);
            full_dst[k] = nullptr;
          } else {
            full_item_put(a, xfer + k * 2 * kThreads, tid);
          }
        }
        done = true;
      }
    }
  }
#endif
  if (!done) {
#pragma unroll
    for (int k = 0; k < KI; ++k) {
      if (first + k < count)
        full_dst[k] = rs_cu_item<CT, VEC, FLAT>(chunks, first + k, ptrs, P, C, S, xfer + k * 2 * kThreads, tid, wave);
    }
  }

#if TIDE_RS_WIDE
  if (!wave) {
    __syncthreads();  // every group's exchange slots are written
#pragma unroll
    for (int k = 0; k < KI; ++k) {
      if (full_dst[k] != nullptr) {
        if (CT > 0)
          full_item_store(xfer + k * 2 * kThreads, full_dst[k], tid);
        else
          full_item_rt_store(xfer + k * 2 * kThreads, full_dst[k], tid);
      }
    }
  }
#endif
}

// AG kernel: bit copy of n bf16 elements per item.  VEC: stage and parameter bases are 16-byte
// aligned, so an item whose source and destination offsets agree mod 8 elements copies 16-byte
// vectors after a short head.
// PACK = false: placement, stage -> parameters.  PACK = true: the inverse (Slot-Reuse packing),
// parameters -> stage slot, over the same items.
//
// Bounded launches with few workgroups per CU leave a copy with one vector in flight per lane
// latency-bound: with batch = 2, two full items (whole 16-byte vectors, kAgChunk elements) are
// loaded together before either is stored.  batch = 1 copies one item at a time.
template <bool VEC, bool PACK>
__global__ __launch_bounds__(kAgThreads) void ag_kernel(const AgChunk* __restrict__ chunks, int64_t first,
                                                        int64_t count, int items_per_wg, int batch,
                                                        unsigned short* __restrict__ stage,
                                                        unsigned short* const* __restrict__ params) {
  const int tid = threadIdx.x;
  for (int j = 0; j < items_per_wg; ++j) {
    if (VEC && batch == 2 && j + 2 <= items_per_wg) {
      constexpr int G = 2;
      constexpr int NV = kAgChunk / 8 / kAgThreads;  // vectors per lane of a full item
      const u32x4* bs[G];
      u32x4* bd[G];
      bool full = true;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int64_t it = item_of<TIDE_AG_XCD_REMAP != 0>(j + g, count);
        full = full && it < count;
        if (full) {
          const AgChunk c = chunks[first + it];
          full = c.n == kAgChunk && (c.src & 7) == 0 && (c.dst & 7) == 0;
          bs[g] = reinterpret_cast<const u32x4*>(PACK ? params[c.p] + c.dst : stage + c.src);
          bd[g] = reinterpret_cast<u32x4*>(PACK ? stage + c.src : params[c.p] + c.dst);
        }
      }
      if (full) {
        u32x4 x[G][NV];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int k = 0; k < NV; ++k) x[g][k] = load_hbm(at_bytes<u32x4>(bs[g], 16u * (tid + k * kAgThreads)));
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int k = 0; k < NV; ++k) store_hbm(at_bytes<u32x4>(bd[g], 16u * (tid + k * kAgThreads)), x[g][k]);
        j += G - 1;
        continue;
      }
    }
    const int64_t item = item_of<TIDE_AG_XCD_REMAP != 0>(j, count);
    if (item >= count) break;
    const AgChunk ch = chunks[first + item];
    const unsigned short* src = PACK ? params[ch.p] + ch.dst : stage + ch.src;
    unsigned short* dst = PACK ? stage + ch.src : params[ch.p] + ch.dst;
    const int64_t src_off = PACK ? ch.dst : ch.src;
    const int n = ch.n;
    if (VEC && ((ch.src - ch.dst) & 7) == 0) {
      const int head = min(n, static_cast<int>((-src_off) & 7));
      const int nb = (n - head) >> 3;
      const int tail = (n - head) & 7;
      if (tid < head) store_hbm(dst + tid, load_hbm(src + tid));
      const u32x4* s = reinterpret_cast<const u32x4*>(src + head);
      u32x4* d = reinterpret_cast<u32x4*>(dst + head);
      int v = tid;
#if TIDE_AG_BUF_AUX >= 0
      // Raw buffer accesses bounded to the item's vectors, cache policy TIDE_AG_BUF_AUX.
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4*>(s), 0, 16 * nb, 0x00020000);
      const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(d, 0, 16 * nb, 0x00020000);
      for (; v < nb; v += kAgThreads)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_amdgcn_raw_buffer_load_b128(rs, 16 * v, 0, TIDE_AG_BUF_AUX),
                                               rd, 16 * v, 0, TIDE_AG_BUF_AUX | TIDE_AG_STORE_EXTRA);
#else
      constexpr int NV = TIDE_AG_VECS;
      for (; v + (NV - 1) * kAgThreads < nb; v += NV * kAgThreads) {
        u32x4 x[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) x[k] = load_hbm(at_bytes<u32x4>(s, 16u * (v + k * kAgThreads)));
#pragma unroll
        for (int k = 0; k < NV; ++k) store_hbm(at_bytes<u32x4>(d, 16u * (v + k * kAgThreads)), x[k]);
      }
      for (; v < nb; v += kAgThreads) store_hbm(at_bytes<u32x4>(d, 16u * v), load_hbm(at_bytes<u32x4>(s, 16u * v)));
#endif
      if (tid < tail) {
        const int k = head + 8 * nb + tid;
        store_hbm(dst + k, load_hbm(src + k));
      }
    } else {
      for (int i = tid; i < n; i += kAgThreads) store_hbm(dst + i, load_hbm(src + i));
    }
  }
}

// CU-exclusive AG kernel (placement, or Slot-Reuse packing with PACK): one launch over all items in
// workgroups of W = blockDim.x / 128 groups of 128 threads (W <= kAgCuMaxItems); group g of
// workgroup b copies item b*W + g.  Like the CU-exclusive RS, every workgroup is given the largest
// local memory one may request, so a CU holds one and is empty whenever it exits (a concurrent
// one-wave GEMM takes it then).  A full item's two 16-byte vectors per lane are both loaded before
// either is stored; other items take the same head / vector / tail path as ag_kernel.  No barrier.
template <bool VEC, bool PACK>
__global__ __launch_bounds__(kAgThreads * kAgCuMaxItems) void ag_cu_kernel(const AgChunk* __restrict__ chunks,
                                                                          int64_t count,
                                                                          unsigned short* __restrict__ stage,
                                                                          unsigned short* const* __restrict__ params) {
  const int W = static_cast<int>(blockDim.x) / kAgThreads;
  const int grp = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kAgThreads);
  const int tid = static_cast<int>(threadIdx.x) % kAgThreads;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * W + grp;
  if (item >= count) return;
  const AgChunk ch = chunks[item];
  const unsigned short* src = PACK ? params[ch.p] + ch.dst : stage + ch.src;
  unsigned short* dst = PACK ? stage + ch.src : params[ch.p] + ch.dst;
  const int64_t src_off = PACK ? ch.dst : ch.src;
  const int n = ch.n;
  if (VEC && n == kAgChunk && (ch.src & 7) == 0 && (ch.dst & 7) == 0) {
    constexpr int NV = kAgChunk / 8 / kAgThreads;  // vectors per lane of a full item
    u32x4 x[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) x[k] = load_hbm(at_bytes<u32x4>(src, 16u * (tid + k * kAgThreads)));
#pragma unroll
    for (int k = 0; k < NV; ++k) store_hbm(at_bytes<u32x4>(dst, 16u * (tid + k * kAgThreads)), x[k]);
  } else if (VEC && ((ch.src - ch.dst) & 7) == 0) {
    const int head = min(n, static_cast<int>((-src_off) & 7));
    const int nb = (n - head) >> 3;
    const int tail = (n - head) & 7;
    if (tid < head) store_hbm(dst + tid, load_hbm(src + tid));
    const u32x4* sv = reinterpret_cast<const u32x4*>(src + head);
    u32x4* dv = reinterpret_cast<u32x4*>(dst + head);
    for (int v = tid; v < nb; v += kAgThreads) store_hbm(at_bytes<u32x4>(dv, 16u * v), load_hbm(at_bytes<u32x4>(sv, 16u * v)));
    if (tid < tail) {
      const int k = head + 8 * nb + tid;
      store_hbm(dst + k, load_hbm(src + k));
    }
  } else {
    for (int i = tid; i < n; i += kAgThreads) store_hbm(dst + i, load_hbm(src + i));
  }
}

// Pointer-table scratch of the allocation-free RS entry point: one fixed array per device, held by
// the library until the process ends.  Host code never passes `scratch` itself to a kernel (in host
// code the name is only a stand-in for the symbol); it uses the device address that
// noalloc_scratch() obtains once per device with hipGetSymbolAddress.
constexpr int64_t kNoAllocMaxPtrs = TIDE_NOALLOC_MAX_PTRS;
static __device__ __align__(256) unsigned long long scratch[kNoAllocMaxPtrs];

// One batch of pointers as a kernel argument (2 KiB), written by one workgroup with vector stores.
constexpr int kPutPtrsBatch = 256;
struct PtrBatch {
  unsigned long long v[kPutPtrsBatch];
};

__global__ __launch_bounds__(kPutPtrsBatch) void put_ptrs_kernel(unsigned long long* __restrict__ dst, PtrBatch b,
                                                                 int n) {
  const int i = threadIdx.x;
  if (i < n) dst[i] = b.v[i];
}

// Zero-fill kernel for the padding of a packed slot: items (src = slot element offset, n).
__global__ __launch_bounds__(kAgThreads) void fill_zero_kernel(const AgChunk* __restrict__ items, int64_t count,
                                                                unsigned short* __restrict__ slot) {
  const int64_t item = blockIdx.x;
  if (item >= count) return;
  const AgChunk ch = items[item];
  for (int i = threadIdx.x; i < ch.n; i += kAgThreads) store_hbm(slot + ch.src + i, static_cast<unsigned short>(0));
}

template <int CT, bool FLAT>
hipError_t launch_rs_ct(const RsChunk* chunks, int64_t first, int64_t count, int grid, int items,
                        void* const* ptrs, int32_t P, int32_t C, int64_t S, bool vec, int lds, hipStream_t s) {
  if (vec)
    hipLaunchKernelGGL((rs_kernel<CT, true, FLAT>), dim3(grid), dim3(kThreads), lds, s, chunks, first, count, items,
                       ptrs, P, C, S);
  else
    hipLaunchKernelGGL((rs_kernel<CT, false, FLAT>), dim3(grid), dim3(kThreads), lds, s, chunks, first, count, items,
                       ptrs, P, C, S);
  return hipGetLastError();
}

template <bool FLAT>
hipError_t launch_rs_c(const RsChunk* chunks, int64_t first, int64_t count, int grid, int items, void* const* ptrs,
                       int32_t P, int32_t C, int64_t S, bool vec, int lds, hipStream_t s) {
  switch (C) {
    case 1: return launch_rs_ct<1, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 2: return launch_rs_ct<2, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 3: return launch_rs_ct<3, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 4: return launch_rs_ct<4, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 5: return launch_rs_ct<5, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 6: return launch_rs_ct<6, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 7: return launch_rs_ct<7, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 8: return launch_rs_ct<8, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 9: return launch_rs_ct<9, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 10: return launch_rs_ct<10, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 11: return launch_rs_ct<11, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 12: return launch_rs_ct<12, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 13: return launch_rs_ct<13, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 14: return launch_rs_ct<14, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 15: return launch_rs_ct<15, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    case 16: return launch_rs_ct<16, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
    default: return launch_rs_ct<0, FLAT>(chunks, first, count, grid, items, ptrs, P, C, S, vec, lds, s);
  }
}

template <int CT, int KI, bool FLAT>
hipError_t launch_rs_cu_ct(const RsChunk* chunks, int64_t count, int grid, int threads, void* const* ptrs, int32_t P,
                           int32_t C, int64_t S, bool vec, int lds, hipStream_t s) {
  if (vec)
    hipLaunchKernelGGL((rs_cu_kernel<CT, KI, true, FLAT>), dim3(grid), dim3(threads), lds, s, chunks, count, ptrs, P,
                       C, S);
  else
    hipLaunchKernelGGL((rs_cu_kernel<CT, KI, false, FLAT>), dim3(grid), dim3(threads), lds, s, chunks, count, ptrs, P,
                       C, S);
  return hipGetLastError();
}

// Items per group: 1 for every C; 2 for C <= 4, whose items carry few bytes (rs_cu_items_ok).
template <int CT, bool FLAT>
hipError_t launch_rs_cu_ki(int ki, const RsChunk* chunks, int64_t count, int grid, int threads, void* const* ptrs,
                           int32_t P, int32_t C, int64_t S, bool vec, int lds, hipStream_t s) {
  if constexpr (CT >= 1 && CT <= kRsCuKi2MaxC) {
    if (ki == 2) return launch_rs_cu_ct<CT, 2, FLAT>(chunks, count, grid, threads, ptrs, P, C, S, vec, lds, s);
  }
  if (ki != 1) return hipErrorInvalidValue;
  return launch_rs_cu_ct<CT, 1, FLAT>(chunks, count, grid, threads, ptrs, P, C, S, vec, lds, s);
}

// The CU-exclusive kernel is compiled for C = 1 .. kRsMaxCt; any other C takes its runtime-C form.
template <bool FLAT>
hipError_t launch_rs_cu_c(int ki, const RsChunk* chunks, int64_t count, int grid, int threads, void* const* ptrs,
                          int32_t P, int32_t C, int64_t S, bool vec, int lds, hipStream_t s) {
#define TIDE_RS_CU_CASE(N) \
  case N: return launch_rs_cu_ki<N, FLAT>(ki, chunks, count, grid, threads, ptrs, P, C, S, vec, lds, s);
  switch (C) {
    TIDE_RS_CU_CASE(1) TIDE_RS_CU_CASE(2) TIDE_RS_CU_CASE(3) TIDE_RS_CU_CASE(4) TIDE_RS_CU_CASE(5)
    TIDE_RS_CU_CASE(6) TIDE_RS_CU_CASE(7) TIDE_RS_CU_CASE(8) TIDE_RS_CU_CASE(9) TIDE_RS_CU_CASE(10)
    TIDE_RS_CU_CASE(11) TIDE_RS_CU_CASE(12) TIDE_RS_CU_CASE(13) TIDE_RS_CU_CASE(14) TIDE_RS_CU_CASE(15)
    TIDE_RS_CU_CASE(16)
    default: return launch_rs_cu_ki<0, FLAT>(ki, chunks, count, grid, threads, ptrs, P, C, S, vec, lds, s);
  }
#undef TIDE_RS_CU_CASE
}

}  // namespace

int launch_rs_cu(const RsChunk* chunks, int64_t count, int groups, int items_per_group, const void* const* dev_ptrs,
                 int32_t P, int32_t C, int64_t S, bool flat, bool vec, int lds, void* hip_stream) {
  if (groups < 1 || groups > kRsCuMaxGroups || !rs_cu_items_ok(C, items_per_group) || count < 1)
    return hipErrorInvalidValue;
  if (lds < rs_cu_xfer_bytes(groups, items_per_group)) return hipErrorInvalidValue;
  const int64_t per_wg = int64_t(groups) * items_per_group;
  const int64_t grid = (count + per_wg - 1) / per_wg;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  void* const* ptrs = const_cast<void* const*>(dev_ptrs);
  const int threads = kThreads * groups;
  if (flat)
    return launch_rs_cu_c<true>(items_per_group, chunks, count, int(grid), threads, ptrs, 1, C, S, vec, lds, s);
  return launch_rs_cu_c<false>(items_per_group, chunks, count, int(grid), threads, ptrs, P, C, S, vec, lds, s);
}

int launch_ag_cu(const AgChunk* chunks, int64_t count, int items_per_wg, void* stage, const void* const* dev_params,
                 bool pack, bool vec, int dyn_lds, void* hip_stream) {
  if (items_per_wg < 1 || items_per_wg > kAgCuMaxItems || count < 1) return hipErrorInvalidValue;
  const int64_t grid = (count + items_per_wg - 1) / items_per_wg;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  unsigned short* st = static_cast<unsigned short*>(stage);
  unsigned short* const* pp = reinterpret_cast<unsigned short* const*>(const_cast<void* const*>(dev_params));
  const dim3 g(static_cast<unsigned>(grid)), b(kAgThreads * items_per_wg);
  if (pack) {
    if (vec)
      hipLaunchKernelGGL((ag_cu_kernel<true, true>), g, b, dyn_lds, s, chunks, count, st, pp);
    else
      hipLaunchKernelGGL((ag_cu_kernel<false, true>), g, b, dyn_lds, s, chunks, count, st, pp);
  } else {
    if (vec)
      hipLaunchKernelGGL((ag_cu_kernel<true, false>), g, b, dyn_lds, s, chunks, count, st, pp);
    else
      hipLaunchKernelGGL((ag_cu_kernel<false, false>), g, b, dyn_lds, s, chunks, count, st, pp);
  }
  return hipGetLastError();
}

int launch_rs(const RsChunk* chunks, int64_t first, int64_t count, int grid, int items_per_wg,
              const void* const* dev_ptrs, int32_t P, int32_t C, int64_t S, bool flat, bool vec, int dyn_lds,
              void* hip_stream) {
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  void* const* ptrs = const_cast<void* const*>(dev_ptrs);
  if (flat) return launch_rs_c<true>(chunks, first, count, grid, items_per_wg, ptrs, 1, C, S, vec, dyn_lds, s);
  return launch_rs_c<false>(chunks, first, count, grid, items_per_wg, ptrs, P, C, S, vec, dyn_lds, s);
}

int rs_lds_info(int device, int* lds_per_cu, int* static_lds_ct, int* static_lds_rt) {
  hipError_t e = hipDeviceGetAttribute(lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, device);
  if (e != hipSuccess) return e;
  hipFuncAttributes attr;
  if ((e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&rs_kernel<8, true, false>))) != hipSuccess)
    return e;
  *static_lds_ct = static_cast<int>(attr.sharedSizeBytes);
  if ((e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&rs_kernel<0, true, false>))) != hipSuccess)
    return e;
  *static_lds_rt = static_cast<int>(attr.sharedSizeBytes);
  return hipSuccess;
}

int launch_ag(const AgChunk* chunks, int64_t first, int64_t count, int grid, int items_per_wg, int batch,
              void* stage, const void* const* dev_params, bool pack, bool vec, void* hip_stream) {
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  unsigned short* st = static_cast<unsigned short*>(stage);
  unsigned short* const* pp = reinterpret_cast<unsigned short* const*>(const_cast<void* const*>(dev_params));
  if (pack) {
    if (vec)
      hipLaunchKernelGGL((ag_kernel<true, true>), dim3(grid), dim3(kAgThreads), 0, s, chunks, first, count,
                         items_per_wg, batch, st, pp);
    else
      hipLaunchKernelGGL((ag_kernel<false, true>), dim3(grid), dim3(kAgThreads), 0, s, chunks, first, count,
                         items_per_wg, batch, st, pp);
  } else {
    if (vec)
      hipLaunchKernelGGL((ag_kernel<true, false>), dim3(grid), dim3(kAgThreads), 0, s, chunks, first, count,
                         items_per_wg, batch, st, pp);
    else
      hipLaunchKernelGGL((ag_kernel<false, false>), dim3(grid), dim3(kAgThreads), 0, s, chunks, first, count,
                         items_per_wg, batch, st, pp);
  }
  return hipGetLastError();
}

int noalloc_scratch(int device, void** out, int64_t* max_ptrs) {
  static std::mutex mu;
  static std::map<int, void*> addr;  // device -> address of `scratch` on it
  std::lock_guard<std::mutex> lock(mu);
  *max_ptrs = kNoAllocMaxPtrs;
  auto it = addr.find(device);
  if (it != addr.end()) {
    *out = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  addr.emplace(device, p);
  *out = p;
  return hipSuccess;
}

int launch_put_ptrs(void* dst, void* const* ptrs, int64_t n, void* hip_stream) {
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  unsigned long long* d = static_cast<unsigned long long*>(dst);
  for (int64_t first = 0; first < n; first += kPutPtrsBatch) {
    const int k = static_cast<int>(n - first < kPutPtrsBatch ? n - first : kPutPtrsBatch);
    PtrBatch b;
    for (int i = 0; i < kPutPtrsBatch; ++i)
      b.v[i] = i < k ? static_cast<unsigned long long>(reinterpret_cast<uintptr_t>(ptrs[first + i])) : 0ull;
    hipLaunchKernelGGL(put_ptrs_kernel, dim3(1), dim3(kPutPtrsBatch), 0, s, d + first, b, k);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int launch_fill_zero(const AgChunk* items, int64_t count, void* slot, void* hip_stream) {
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(count)), dim3(kAgThreads), 0, s, items, count,
                     static_cast<unsigned short*>(slot));
  return hipGetLastError();
}

}  // namespace tide
