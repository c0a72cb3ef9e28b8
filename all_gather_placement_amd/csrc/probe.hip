// Occupancy and interference probes for gfx950 (libtide_probe.so); see include/tide_probe.h.
#include <hip/hip_runtime.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <chrono>
#include <vector>

#include "../../include/tide_probe.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr unsigned long long kMaxPolls = 1ull << 26;

// s_getreg immediates: (size - 1) << 11 | offset << 6 | register id.
constexpr int kHwIdAll = (31 << 11) | (0 << 6) | 4;   // HW_ID, all 32 bits
constexpr int kXccIdAll = (3 << 11) | (0 << 6) | 20;  // XCC_ID bits 3:0

__device__ __forceinline__ void spin_until(unsigned long long t0, unsigned long long ticks) {
  unsigned long long polls = 0;
  while (static_cast<unsigned long long>(wall_clock64()) - t0 < ticks && ++polls < kMaxPolls)
    __builtin_amdgcn_s_sleep(2);
}

__device__ __forceinline__ void record(tide_probe_record* records, unsigned long long t0) {
  const unsigned long long t1 = static_cast<unsigned long long>(wall_clock64());
  if (records != nullptr && threadIdx.x == 0) {
    tide_probe_record r;
    r.start = t0;
    r.end = t1;
    r.hw_id = static_cast<uint32_t>(__builtin_amdgcn_s_getreg(kHwIdAll));
    r.xcc_id = static_cast<uint32_t>(__builtin_amdgcn_s_getreg(kXccIdAll));
    r.reserved = 0;
    records[blockIdx.x] = r;
  }
}

// GEMM-shaped: 64 KiB of LDS and the whole unified register file of a SIMD per wave -- 256
// architectural VGPRs and 256 accumulation registers (the clobbers of v255 and a255 make the
// allocation cover both), as a matrix-core GEMM holding its accumulators in AGPRs does -- so the
// workgroup needs the same CU resources as the victim GEMM's: one wave per SIMD, nothing beside it.
__global__ __launch_bounds__(kProbeThreads) void probe_gemm_shaped(tide_probe_record* records,
                                                                   unsigned long long ticks) {
  __shared__ unsigned int lds[16384];
  const unsigned long long t0 = static_cast<unsigned long long>(wall_clock64());
  asm volatile("" ::: "v255", "a255");
  lds[threadIdx.x * 64] = threadIdx.x;
  __syncthreads();
  spin_until(t0, ticks);
  if (lds[((threadIdx.x + 1) % kProbeThreads) * 64] == 0xFFFFFFFFu) records = nullptr;  // keep LDS live
  record(records, t0);
}

__global__ __launch_bounds__(kProbeThreads) void probe_small(tide_probe_record* records, unsigned long long ticks) {
  const unsigned long long t0 = static_cast<unsigned long long>(wall_clock64());
  spin_until(t0, ticks);
  record(records, t0);
}

// One wave that sleeps for `ticks` of the constant-rate wall clock and reads the shader cycle
// counter (s_memtime, which counts shader clocks) at both ends: cycles / wall time = the mean shader
// clock of the CU it ran on over that interval.
__global__ __launch_bounds__(64) void probe_clock(uint64_t* out, unsigned long long ticks) {
  const unsigned long long w0 = static_cast<unsigned long long>(wall_clock64());
  const unsigned long long c0 = static_cast<unsigned long long>(clock64());
  spin_until(w0, ticks);
  const unsigned long long c1 = static_cast<unsigned long long>(clock64());
  const unsigned long long w1 = static_cast<unsigned long long>(wall_clock64());
  if (threadIdx.x == 0) {
    out[0] = w0;
    out[1] = w1;
    out[2] = c0;
    out[3] = c1;
  }
}

// RS-shaped mix probe: the access shape of the reduce-scatter's full work items, with the reads or
// the writes left out.  One 128-thread workgroup per 1024-output item, items spread over the 8 XCDs
// in contiguous ranges; per lane one 16-byte non-temporal buffer load from each of the C
// contributors, 8 widen-and-add sums in ascending contributor order, an LDS exchange, and two
// 16-byte non-temporal stores of whole cache lines.  MODE 0: loads and stores; 1: loads only (the
// stores sit behind a test no sum can pass, which keeps the loads live); 2: stores only (a pattern).
constexpr int kMixThreads = 128;
constexpr int kMixItem = kMixThreads * 8;
typedef unsigned int mix_u32x4 __attribute__((ext_vector_type(4)));
typedef float mix_f32x4 __attribute__((ext_vector_type(4)));
constexpr int kRawBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kNtLoad = 2;                     // nt
constexpr int kNtStore = 18;                   // nt sc1

template <int CT, int MODE>
__global__ __launch_bounds__(kMixThreads) void probe_mix(const unsigned short* const* __restrict__ src,
                                                          float* __restrict__ dst, int64_t items) {
  __shared__ mix_f32x4 xfer[2 * kMixThreads];
  const int64_t b = blockIdx.x, x = b % 8, i = b / 8;
  const int64_t item = x * (items / 8) + (x < items % 8 ? x : items % 8) + i;
  const int tid = threadIdx.x;
  mix_f32x4 o0, o1;
  if (MODE == 2) {
    o0 = mix_f32x4{float(tid), 1.0f, 2.0f, 3.0f};
    o1 = mix_f32x4{float(tid), 4.0f, 5.0f, 6.0f};
  } else {
    mix_u32x4 v[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<unsigned short*>(src[c] + item * kMixItem), 0, 2 * kMixItem, kRawBufferWord3);
      v[c] = __builtin_bit_cast(mix_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * tid, 0, kNtLoad));
    }
    float a[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a[2 * k] = __uint_as_float(v[0][k] << 16);
      a[2 * k + 1] = __uint_as_float(v[0][k] & 0xffff0000u);
    }
#pragma unroll
    for (int c = 1; c < CT; ++c)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a[2 * k] += __uint_as_float(v[c][k] << 16);
        a[2 * k + 1] += __uint_as_float(v[c][k] & 0xffff0000u);
      }
    xfer[2 * tid] = mix_f32x4{a[0], a[1], a[2], a[3]};
    xfer[2 * tid + 1] = mix_f32x4{a[4], a[5], a[6], a[7]};
    __syncthreads();
    o0 = xfer[tid];
    o1 = xfer[tid + kMixThreads];
    // a NaN with payload 0x1234 in its low bits: sums of widened bf16 values never produce it
    if (MODE == 1 && __float_as_uint(o0.x) != 0x7fc01234u) return;
  }
  const __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc(dst + item * kMixItem, 0, 4 * kMixItem, kRawBufferWord3);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(mix_u32x4, o0), rd, 16 * tid, 0, kNtStore);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(mix_u32x4, o1), rd, 16 * (tid + kMixThreads), 0,
                                         kNtStore);
}

template <int CT, int MODE>
int launch_mix(const unsigned short* const* src, float* dst, int64_t items, int32_t lds_bytes, hipStream_t s) {
  hipFuncAttributes attr;
  hipError_t e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&probe_mix<CT, MODE>));
  if (e != hipSuccess) return e;
  const int dyn = lds_bytes > static_cast<int>(attr.sharedSizeBytes) ? lds_bytes - static_cast<int>(attr.sharedSizeBytes) : 0;
  hipLaunchKernelGGL((probe_mix<CT, MODE>), dim3(static_cast<unsigned>(items)), dim3(kMixThreads), dyn, s, src, dst,
                     items);
  return hipGetLastError();
}

template <int CT>
int launch_mix_c(int32_t mode, const unsigned short* const* src, float* dst, int64_t items, int32_t lds_bytes,
                 hipStream_t s) {
  switch (mode) {
    case TIDE_PROBE_MIX_BOTH: return launch_mix<CT, 0>(src, dst, items, lds_bytes, s);
    case TIDE_PROBE_MIX_READS: return launch_mix<CT, 1>(src, dst, items, lds_bytes, s);
    default: return launch_mix<CT, 2>(src, dst, items, lds_bytes, s);
  }
}

// The HSA agent of HIP device `dev`, matched by PCI domain, bus and device.
struct AgentMatch {
  uint32_t domain, bdf;
  hsa_agent_t agent;
  bool found;
};

hsa_status_t match_agent(hsa_agent_t a, void* data) {
  auto* m = static_cast<AgentMatch*>(data);
  hsa_device_type_t t;
  if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &t) != HSA_STATUS_SUCCESS || t != HSA_DEVICE_TYPE_GPU)
    return HSA_STATUS_SUCCESS;
  uint32_t domain = 0, bdf = 0;
  if (hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_DOMAIN), &domain) != HSA_STATUS_SUCCESS ||
      hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_BDFID), &bdf) != HSA_STATUS_SUCCESS)
    return HSA_STATUS_SUCCESS;
  if (domain == m->domain && (bdf & ~7u) == (m->bdf & ~7u)) {  // function bits ignored
    m->agent = a;
    m->found = true;
    return HSA_STATUS_INFO_BREAK;
  }
  return HSA_STATUS_SUCCESS;
}

bool current_gpu_agent(hsa_agent_t* out) {
  int dev = 0, bus = 0, device = 0, domain = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&bus, hipDeviceAttributePciBusId, dev) != hipSuccess ||
      hipDeviceGetAttribute(&device, hipDeviceAttributePciDeviceId, dev) != hipSuccess ||
      hipDeviceGetAttribute(&domain, hipDeviceAttributePciDomainID, dev) != hipSuccess)
    return false;
  if (hsa_init() != HSA_STATUS_SUCCESS) return false;  // reference counted: HIP holds the runtime open too
  AgentMatch m{static_cast<uint32_t>(domain), (static_cast<uint32_t>(bus) << 8) | (static_cast<uint32_t>(device) << 3),
               {0}, false};
  hsa_iterate_agents(match_agent, &m);
  if (m.found) *out = m.agent;
  return m.found;
}

}  // namespace

extern "C" {

int32_t tide_probe_dma_rect_copies(int32_t n, const tide_probe_rect* rects, int64_t timeout_ms, double* elapsed_us) {
  if (n < 1 || rects == nullptr || timeout_ms < 0) return -1;
  const int64_t u32max = 0xffffffffll;
  for (int32_t i = 0; i < n; ++i) {
    const tide_probe_rect& r = rects[i];
    if (r.dst == nullptr || r.src == nullptr || r.width <= 0 || r.rows <= 0 || r.width > u32max || r.rows > u32max ||
        r.width % 4 || r.dst_pitch % 4 || r.src_pitch % 4 || r.width > r.dst_pitch || r.width > r.src_pitch ||
        (reinterpret_cast<uintptr_t>(r.dst) & 3) || (reinterpret_cast<uintptr_t>(r.src) & 3))
      return -1;
  }
  hsa_agent_t gpu;
  if (!current_gpu_agent(&gpu)) return -2;
  std::vector<hsa_signal_t> sig;
  sig.reserve(n);
  int32_t rc = 0;
  const auto t0 = std::chrono::steady_clock::now();
  for (int32_t i = 0; i < n && rc == 0; ++i) {
    const tide_probe_rect& r = rects[i];
    hsa_signal_t s;
    if (hsa_signal_create(1, 0, nullptr, &s) != HSA_STATUS_SUCCESS) {
      rc = -1;
      break;
    }
    hsa_pitched_ptr_t dst{r.dst, static_cast<size_t>(r.dst_pitch), static_cast<size_t>(r.dst_pitch * r.rows)};
    hsa_pitched_ptr_t src{const_cast<void*>(r.src), static_cast<size_t>(r.src_pitch),
                          static_cast<size_t>(r.src_pitch * r.rows)};
    const hsa_dim3_t zero{0, 0, 0};
    const hsa_dim3_t range{static_cast<uint32_t>(r.width), static_cast<uint32_t>(r.rows), 1};
    const hsa_status_t st =
        hsa_amd_memory_async_copy_rect(&dst, &zero, &src, &zero, &range, gpu, hsaDeviceToDevice, 0, nullptr, s);
    if (st != HSA_STATUS_SUCCESS) {
      hsa_signal_destroy(s);
      rc = static_cast<int32_t>(st);
      break;
    }
    sig.push_back(s);
  }
  // wait for every issued copy, against one deadline
  const auto deadline = t0 + std::chrono::milliseconds(timeout_ms);
  for (hsa_signal_t s : sig) {
    while (hsa_signal_load_scacquire(s) != 0) {
      const auto now = std::chrono::steady_clock::now();
      if (now >= deadline) {
        rc = -3;
        break;
      }
      const uint64_t left_ns =
          static_cast<uint64_t>(std::chrono::duration_cast<std::chrono::nanoseconds>(deadline - now).count());
      hsa_signal_wait_scacquire(s, HSA_SIGNAL_CONDITION_LT, 1, left_ns, HSA_WAIT_STATE_BLOCKED);
    }
    if (rc == -3) break;
  }
  const auto t1 = std::chrono::steady_clock::now();
  if (elapsed_us) *elapsed_us = std::chrono::duration<double, std::micro>(t1 - t0).count();
  if (rc != -3)
    for (hsa_signal_t s : sig) hsa_signal_destroy(s);  // after a timeout they may still be signalled: kept
  return rc;
}

int32_t tide_probe_mix(int32_t C, int32_t mode, const void* const* src, float* dst, int64_t items, int32_t lds_bytes,
                       void* stream) {
  if ((C != 1 && C != 2 && C != 4 && C != 8) || mode < TIDE_PROBE_MIX_BOTH || mode > TIDE_PROBE_MIX_WRITES ||
      items < 1 || items > 0x7fffffff || lds_bytes < 0 || dst == nullptr ||
      (mode != TIDE_PROBE_MIX_WRITES && src == nullptr))
    return -1;
  const unsigned short* const* s = reinterpret_cast<const unsigned short* const*>(src);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  switch (C) {
    case 1: return launch_mix_c<1>(mode, s, dst, items, lds_bytes, hs);
    case 2: return launch_mix_c<2>(mode, s, dst, items, lds_bytes, hs);
    case 4: return launch_mix_c<4>(mode, s, dst, items, lds_bytes, hs);
    default: return launch_mix_c<8>(mode, s, dst, items, lds_bytes, hs);
  }
}

int32_t tide_probe_clock(int64_t spin_ticks, uint64_t* out, void* stream) {
  if (spin_ticks < 0 || out == nullptr) return -1;
  hipLaunchKernelGGL(probe_clock, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), out,
                     static_cast<unsigned long long>(spin_ticks));
  return static_cast<int32_t>(hipGetLastError());
}

int32_t tide_probe_launch(int32_t num_wgs, int32_t shape, int64_t spin_ticks, tide_probe_record* records,
                          void* stream) {
  if (num_wgs < 1 || spin_ticks < 0 || (shape != TIDE_PROBE_GEMM_SHAPED && shape != TIDE_PROBE_SMALL)) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned long long ticks = static_cast<unsigned long long>(spin_ticks);
  if (shape == TIDE_PROBE_GEMM_SHAPED)
    hipLaunchKernelGGL(probe_gemm_shaped, dim3(num_wgs), dim3(kProbeThreads), 0, s, records, ticks);
  else
    hipLaunchKernelGGL(probe_small, dim3(num_wgs), dim3(kProbeThreads), 0, s, records, ticks);
  return static_cast<int32_t>(hipGetLastError());
}

int32_t tide_probe_stream_create_cu_mask(int32_t first_cu, int32_t n_cus, void** stream) {
  int dev = 0, cus = 0;
  if (stream == nullptr || first_cu < 0 || n_cus < 1) return -1;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return -1;
  if (static_cast<int64_t>(first_cu) + n_cus > cus) return -1;
  std::vector<uint32_t> mask((cus + 31) / 32, 0u);
  for (int i = first_cu; i < first_cu + n_cus; ++i) mask[i / 32] |= 1u << (i % 32);
  hipStream_t s = nullptr;
  const hipError_t e = hipExtStreamCreateWithCUMask(&s, static_cast<uint32_t>(mask.size()), mask.data());
  if (e != hipSuccess) return static_cast<int32_t>(e);
  *stream = s;
  return 0;
}

int32_t tide_probe_stream_destroy(void* stream) {
  if (stream == nullptr) return -1;
  return static_cast<int32_t>(hipStreamDestroy(static_cast<hipStream_t>(stream)));
}

int64_t tide_probe_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -1;
  return khz;
}

#ifndef TIDE_BUILD_ID
#define TIDE_BUILD_ID "unknown"
#endif
const char* tide_probe_build_id(void) { return TIDE_BUILD_ID; }

}  // extern "C"
