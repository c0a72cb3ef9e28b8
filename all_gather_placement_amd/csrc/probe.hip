// Occupancy and interference probes for gfx950 (libtide_probe.so); see include/tide_probe.h.
#include <hip/hip_runtime.h>

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

}  // namespace

extern "C" {

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

int64_t tide_probe_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -1;
  return khz;
}

}  // extern "C"
