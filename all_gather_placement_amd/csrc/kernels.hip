// gfx950 kernels of the layout-aware reduce-scatter and all-gather placement.
//
// Both kernels walk a host-built table of work items (tide_internal.h).  A work item lies inside
// one (parameter, rank) segment, so a workgroup reads its item descriptor and the item's C source
// pointers once, as wave-uniform scalar loads, and then streams contiguous memory: no per-element
// index search, no atomics, no inter-workgroup communication.  Every output element has exactly
// one writer.
//
// RS ([Endgame] Figure 6a, node-local fp32 sums; abstract, bf16 gradients reduced into fp32
// shards): each thread takes 8 consecutive outputs at a time -- one 16-byte bf16x8 load from each
// contributor, an exact widen to fp32, C-1 IEEE fp32 adds in ascending contributor order, and two
// 16-byte non-temporal fp32 stores.  At C = 8 that is 20 bytes of HBM traffic per output and 7
// adds: far below any ALU or matrix-core limit, so the kernel is HBM-bound and is shaped for
// bytes in flight (two 8-output vectors per thread per step, non-temporal streaming accesses).
//
// AG ([Endgame] Figure 5b, one strided copy per parameter; Table 7, direct landing): a bit copy
// of each rank's valid rows from the rank-major stage into the parameter's storage, 16 bytes per
// thread per access when source and destination share their 16-byte phase.
#include <hip/hip_runtime.h>

#include "tide_internal.h"

namespace tide {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Every buffer the kernels touch is HBM; pointers that arrive through a table would otherwise be
// generic (flat) pointers, so accesses go through global-address-space casts to get global_*
// instructions instead of flat_* ones.
#define TIDE_GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ float widen_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float widen_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float widen1(unsigned short b) {
  return __uint_as_float(static_cast<unsigned int>(b) << 16);
}

// Streaming (non-temporal) 16-byte accesses: every input byte is read once and every output byte
// written once, so nothing is worth keeping in the caches.
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
__device__ __forceinline__ u32x4 load16_stream(const void* p) { return load_hbm(static_cast<const u32x4*>(p)); }
__device__ __forceinline__ unsigned short load_u16(const unsigned short* p) { return *(const TIDE_GLOBAL unsigned short*)p; }
__device__ __forceinline__ void store16_stream(void* p, f32x4 v) { store_hbm(static_cast<f32x4*>(p), v); }
__device__ __forceinline__ void store_f32(float* p, float v) { store_hbm(p, v); }

// acc[0..7] = widen(x); element order inside a bf16x8 vector: x.x low half is element 0.
__device__ __forceinline__ void widen8(const u32x4 x, float acc[8]) {
  acc[0] = widen_lo(x.x); acc[1] = widen_hi(x.x);
  acc[2] = widen_lo(x.y); acc[3] = widen_hi(x.y);
  acc[4] = widen_lo(x.z); acc[5] = widen_hi(x.z);
  acc[6] = widen_lo(x.w); acc[7] = widen_hi(x.w);
}

__device__ __forceinline__ void add8(const u32x4 x, float acc[8]) {
  acc[0] += widen_lo(x.x); acc[1] += widen_hi(x.x);
  acc[2] += widen_lo(x.y); acc[3] += widen_hi(x.y);
  acc[4] += widen_lo(x.z); acc[5] += widen_hi(x.z);
  acc[6] += widen_lo(x.w); acc[7] += widen_hi(x.w);
}

__device__ __forceinline__ void store8(float* dst, const float acc[8], bool dst16) {
  if (dst16) {
    f32x4 a = {acc[0], acc[1], acc[2], acc[3]};
    f32x4 b = {acc[4], acc[5], acc[6], acc[7]};
    store16_stream(dst, a);
    store16_stream(dst + 4, b);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) store_f32(dst + k, acc[k]);
  }
}

// Fixed-order fp32 sum of one element over contributors (element path, head/tail, unaligned).
template <int CT>
__device__ __forceinline__ float sum1(const unsigned short* const* src, int C, int64_t i) {
  const int n = CT > 0 ? CT : C;
  float acc = widen1(load_u16(src[0] + i));
  for (int c = 1; c < n; ++c) acc += widen1(load_u16(src[c] + i));
  return acc;
}

// NV 8-output vectors per call, kThreads vectors apart: all NV*C loads are issued before the
// first add, so each thread keeps NV*C 16-byte loads in flight.
template <int CT, int NV>
__device__ __forceinline__ void sum_vecs(const unsigned short* const* src, int64_t i0, float* dst, bool dst16) {
  u32x4 x[NV][CT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int k = 0; k < NV; ++k) x[k][c] = load16_stream(src[c] + i0 + 8 * kThreads * k);
  float a[NV][8];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    widen8(x[k][0], a[k]);
#pragma unroll
    for (int c = 1; c < CT; ++c) add8(x[k][c], a[k]);
  }
#pragma unroll
  for (int k = 0; k < NV; ++k) store8(dst + i0 + 8 * kThreads * k, a[k], dst16);
}

template <int CT>
__device__ __forceinline__ void sum8(const unsigned short* const* src, int C, int64_t i, float* d,
                                     bool dst16) {
  float a[8];
  if constexpr (CT > 0) {
    u32x4 x[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) x[c] = load16_stream(src[c] + i);
    widen8(x[0], a);
#pragma unroll
    for (int c = 1; c < CT; ++c) add8(x[c], a);
  } else {
    widen8(load16_stream(src[0] + i), a);
    for (int c = 1; c < C; ++c) add8(load16_stream(src[c] + i), a);
  }
  store8(d, a, dst16);
}

constexpr int kMaxStaticC = 8;

// RS kernel.  CT > 0: contributor count fixed at compile time; CT == 0: runtime C (any C >= 1).
// VEC: all gradient and shard base pointers are 16-byte aligned (checked on the host), so the
// 16-byte phase of an element depends only on its offset.
template <int CT, bool VEC>
__global__ __launch_bounds__(kThreads) void rs_kernel(const RsChunk* __restrict__ chunks, int64_t first,
                                                      int64_t count, int items_per_wg,
                                                      void* const* __restrict__ ptrs, int32_t P,
                                                      int32_t C) {
  const int tid = threadIdx.x;
  const unsigned short* const* __restrict__ gptr = reinterpret_cast<const unsigned short* const*>(ptrs);
  float* const* __restrict__ sptr = reinterpret_cast<float* const*>(ptrs + static_cast<int64_t>(C) * P);
  const int nc = CT > 0 ? CT : C;

  for (int j = 0; j < items_per_wg; ++j) {
    const int64_t item = static_cast<int64_t>(blockIdx.x) + static_cast<int64_t>(j) * gridDim.x;
    if (item >= count) break;
    const RsChunk ch = chunks[first + item];

    // Source pointers of this item, one per contributor (wave-uniform).
    const unsigned short* src[CT > 0 ? CT : kMaxStaticC];
    const unsigned short* const* srcp;
    if constexpr (CT > 0) {
#pragma unroll
      for (int c = 0; c < CT; ++c) src[c] = gptr[static_cast<int64_t>(c) * P + ch.p] + ch.src;
      srcp = src;
    } else {
      srcp = nullptr;
    }
    float* dst = sptr[ch.r] + ch.dst;
    const int n = ch.nvalid;

    if constexpr (CT == 0) {
      // Runtime C: per-element pointer lookups through the table (scalar loads, cached).
      const int64_t base = ch.src;
      const int head = VEC ? min(n, static_cast<int>((-base) & 7)) : n;
      for (int i = tid; i < head; i += kThreads) {
        const int64_t e = base + i;
        float acc = widen1(load_u16(gptr[ch.p] + e));
        for (int c = 1; c < nc; ++c) acc += widen1(load_u16(gptr[static_cast<int64_t>(c) * P + ch.p] + e));
        store_f32(dst + i, acc);
      }
      if (VEC) {
        const int nb = (n - head) >> 3;
        const int tail = (n - head) & 7;
        const bool dst16 = ((ch.dst + head) & 3) == 0;
        for (int v = tid; v < nb; v += kThreads) {
          const int64_t e = base + head + 8 * static_cast<int64_t>(v);
          float a[8];
          widen8(load16_stream(gptr[ch.p] + e), a);
          for (int c = 1; c < nc; ++c) add8(load16_stream(gptr[static_cast<int64_t>(c) * P + ch.p] + e), a);
          store8(dst + head + 8 * v, a, dst16);
        }
        for (int i = tid; i < tail; i += kThreads) {
          const int64_t k = head + 8 * static_cast<int64_t>(nb) + i;
          float acc = widen1(load_u16(gptr[ch.p] + base + k));
          for (int c = 1; c < nc; ++c) acc += widen1(load_u16(gptr[static_cast<int64_t>(c) * P + ch.p] + base + k));
          store_f32(dst + k, acc);
        }
      }
    } else {
      if (VEC) {
        const int head = min(n, static_cast<int>((-ch.src) & 7));
        const int nb = (n - head) >> 3;
        const int tail = (n - head) & 7;
        const bool dst16 = ((ch.dst + head) & 3) == 0;
        if (tid < head) store_f32(dst + tid, sum1<CT>(srcp, nc, tid));
        constexpr int NV = TIDE_RS_VECS;
        int v = tid;
        for (; v + (NV - 1) * kThreads < nb; v += NV * kThreads)
          sum_vecs<CT, NV>(srcp, head + 8 * static_cast<int64_t>(v), dst, dst16);
        for (; v < nb; v += kThreads) {
          const int64_t i0 = head + 8 * static_cast<int64_t>(v);
          sum8<CT>(srcp, nc, i0, dst + i0, dst16);
        }
        if (tid < tail) {
          const int64_t k = head + 8 * static_cast<int64_t>(nb) + tid;
          store_f32(dst + k, sum1<CT>(srcp, nc, k));
        }
      } else {
        for (int i = tid; i < n; i += kThreads) store_f32(dst + i, sum1<CT>(srcp, nc, i));
      }
    }

    // Padding rows of this rank's slice: +0.0.
    for (int i = tid; i < ch.npad; i += kThreads) store_f32(dst + n + i, 0.0f);
  }
}

// AG kernel: bit copy of n bf16 elements per item.  VEC: stage and parameter bases are 16-byte
// aligned, so an item whose source and destination offsets agree mod 8 elements copies 16-byte
// vectors after a short head.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void ag_kernel(const AgChunk* __restrict__ chunks, int64_t first,
                                                      int64_t count, int items_per_wg,
                                                      const unsigned short* __restrict__ stage,
                                                      unsigned short* const* __restrict__ params) {
  const int tid = threadIdx.x;
  for (int j = 0; j < items_per_wg; ++j) {
    const int64_t item = static_cast<int64_t>(blockIdx.x) + static_cast<int64_t>(j) * gridDim.x;
    if (item >= count) break;
    const AgChunk ch = chunks[first + item];
    const unsigned short* src = stage + ch.src;
    unsigned short* dst = params[ch.p] + ch.dst;
    const int n = ch.n;
    if (VEC && ((ch.src - ch.dst) & 7) == 0) {
      const int head = min(n, static_cast<int>((-ch.src) & 7));
      const int nb = (n - head) >> 3;
      const int tail = (n - head) & 7;
      if (tid < head) store_hbm(dst + tid, load_hbm(src + tid));
      const u32x4* s = reinterpret_cast<const u32x4*>(src + head);
      u32x4* d = reinterpret_cast<u32x4*>(dst + head);
      constexpr int NV = TIDE_AG_VECS;
      int v = tid;
      for (; v + (NV - 1) * kThreads < nb; v += NV * kThreads) {
        u32x4 x[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) x[k] = load_hbm(s + v + k * kThreads);
#pragma unroll
        for (int k = 0; k < NV; ++k) store_hbm(d + v + k * kThreads, x[k]);
      }
      for (; v < nb; v += kThreads) store_hbm(d + v, load_hbm(s + v));
      if (tid < tail) {
        const int k = head + 8 * nb + tid;
        store_hbm(dst + k, load_hbm(src + k));
      }
    } else {
      for (int i = tid; i < n; i += kThreads) store_hbm(dst + i, load_hbm(src + i));
    }
  }
}

template <int CT>
hipError_t launch_rs_ct(const RsChunk* chunks, int64_t first, int64_t count, int grid, int items,
                        void* const* ptrs, int32_t P, int32_t C, bool vec, hipStream_t s) {
  if (vec)
    hipLaunchKernelGGL((rs_kernel<CT, true>), dim3(grid), dim3(kThreads), 0, s, chunks, first, count, items,
                       ptrs, P, C);
  else
    hipLaunchKernelGGL((rs_kernel<CT, false>), dim3(grid), dim3(kThreads), 0, s, chunks, first, count, items,
                       ptrs, P, C);
  return hipGetLastError();
}

}  // namespace

int launch_rs(const RsChunk* chunks, int64_t first, int64_t count, int grid, int items_per_wg,
              const void* const* dev_ptrs, int32_t P, int32_t C, bool vec, void* hip_stream) {
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  void* const* ptrs = const_cast<void* const*>(dev_ptrs);
  switch (C) {
    case 1: return launch_rs_ct<1>(chunks, first, count, grid, items_per_wg, ptrs, P, C, vec, s);
    case 2: return launch_rs_ct<2>(chunks, first, count, grid, items_per_wg, ptrs, P, C, vec, s);
    case 3: return launch_rs_ct<3>(chunks, first, count, grid, items_per_wg, ptrs, P, C, vec, s);
    case 4: return launch_rs_ct<4>(chunks, first, count, grid, items_per_wg, ptrs, P, C, vec, s);
    case 5: return launch_rs_ct<5>(chunks, first, count, grid, items_per_wg, ptrs, P, C, vec, s);
    case 6: return launch_rs_ct<6>(chunks, first, count, grid, items_per_wg, ptrs, P, C, vec, s);
    case 7: return launch_rs_ct<7>(chunks, first, count, grid, items_per_wg, ptrs, P, C, vec, s);
    case 8: return launch_rs_ct<8>(chunks, first, count, grid, items_per_wg, ptrs, P, C, vec, s);
    default: return launch_rs_ct<0>(chunks, first, count, grid, items_per_wg, ptrs, P, C, vec, s);
  }
}

int launch_ag(const AgChunk* chunks, int64_t first, int64_t count, int grid, int items_per_wg,
              const void* stage, const void* const* dev_params, bool vec, void* hip_stream) {
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const unsigned short* st = static_cast<const unsigned short*>(stage);
  unsigned short* const* pp = reinterpret_cast<unsigned short* const*>(const_cast<void* const*>(dev_params));
  if (vec)
    hipLaunchKernelGGL((ag_kernel<true>), dim3(grid), dim3(kThreads), 0, s, chunks, first, count, items_per_wg,
                       st, pp);
  else
    hipLaunchKernelGGL((ag_kernel<false>), dim3(grid), dim3(kThreads), 0, s, chunks, first, count, items_per_wg,
                       st, pp);
  return hipGetLastError();
}

}  // namespace tide
