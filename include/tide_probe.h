/*
 * tide_probe.h -- occupancy and interference instruments for MI355X (gfx950), a separate library
 * (libtide_probe.so) used by the measurements, not by the reduce-scatter or placement path.
 *
 * They reproduce, on MI355X, the two instruments of "The Endgame of FSDP Communication:
 * Layout-Aware Collectives on Copy Engines, RDMA, and NVSwitch" ([Endgame]) that explain why
 * communication workgroups slow a concurrent GEMM:
 *   - Table 5's probe: workgroups shaped like a one-wave GEMM's, one per compute unit, each
 *     recording where it ran (XCC, shader engine, shader array, CU) and when it started and ended;
 *     probe workgroups that start after the first wave were displaced by resident workgroups;
 *   - Figure 4's spin kernels: k small workgroups that stay resident for a fixed time.
 * All waits are bounded by a deadline on the constant-rate wall clock and by an iteration cap, so
 * every wave exits.  Records are written with vector stores.
 */
#ifndef TIDE_PROBE_H
#define TIDE_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One record per probe workgroup (32 bytes): wall-clock start and end (ticks of the device wall
 * clock, see tide_probe_wall_clock_khz), the raw HW_ID register (CU_ID bits 11:8, SH_ID bit 12,
 * SE_ID bits 14:13) and the XCC_ID register (bits 3:0) of the workgroup's first wave. */
typedef struct tide_probe_record {
  uint64_t start;
  uint64_t end;
  uint32_t hw_id;
  uint32_t xcc_id;
  uint64_t reserved;
} tide_probe_record;

/* Shapes of probe workgroup. */
enum {
  TIDE_PROBE_GEMM_SHAPED = 0, /* 256 threads, 64 KiB LDS, 256 VGPRs + 256 AGPRs per wave (a whole
                                 SIMD register file): the footprint of a matrix-core GEMM workgroup
                                 such as the one-wave bf16 victim (one 256x256 tile per CU) */
  TIDE_PROBE_SMALL = 1        /* 256 threads, no LDS, few VGPRs: the footprint of a communication
                                 workgroup (spin kernel) */
};

/*
 * Launch `num_wgs` probe workgroups of `shape` on `stream` (a hipStream_t as void*).  Each
 * workgroup records its start time, spins until `spin_ticks` wall-clock ticks have passed since
 * its own start (at most 2^26 polls), records its end and location into records[blockIdx].
 *   records  device array of num_wgs tide_probe_record, or NULL (no records written).
 * Returns 0 or a hipError_t value; -1 for bad arguments (num_wgs < 1, bad shape, spin_ticks < 0).
 */
int32_t tide_probe_launch(int32_t num_wgs, int32_t shape, int64_t spin_ticks, tide_probe_record* records,
                          void* stream);

/*
 * Shader clock probe: one 64-thread workgroup on `stream` sleeps until `spin_ticks` wall-clock ticks
 * have passed (at most 2^26 polls) and writes out[0..3] = wall clock at start and end, shader cycle
 * counter (s_memtime) at start and end.  (out[3]-out[2]) / (out[1]-out[0]) * wall-clock kHz is the
 * mean shader clock of its CU over the interval; launched beside other work on another stream it
 * records the clock that work ran at ([Endgame] Table 4 fixes the SM clock; MI355X boxes without
 * that privilege record it instead).
 *   out  device array of 4 uint64_t, written with vector stores.
 * Returns 0 or a hipError_t value; -1 for spin_ticks < 0 or a NULL `out`.
 */
int32_t tide_probe_clock(int64_t spin_ticks, uint64_t* out, void* stream);

/* Modes of the mix probe. */
enum {
  TIDE_PROBE_MIX_BOTH = 0,   /* contributor loads, sums and stores: the reduce-scatter's full items */
  TIDE_PROBE_MIX_READS = 1,  /* the loads and sums only */
  TIDE_PROBE_MIX_WRITES = 2  /* the stores only (a fixed pattern) */
};

/*
 * Mix probe: the reduce-scatter's access shape for flat, 16-byte-aligned buffers, with its reads or
 * its writes left out, so that the memory system's read-only, write-only and mixed rates can be
 * measured in the shape the reduction uses ([Endgame] Figure 6a's node-local fp32 sums).  One
 * 128-thread workgroup per item of 1024 outputs; item k of contributor c is elements
 * [1024k, 1024k+1024) of src[c], its outputs are elements [1024k, 1024k+1024) of dst; items are
 * spread over the 8 XCDs in contiguous ranges.
 *   C          1, 2, 4 or 8.
 *   src        device array of C device pointers (NULL allowed for TIDE_PROBE_MIX_WRITES); each
 *              contributor holds 1024*items bf16, 16-byte aligned.
 *   dst        device, 1024*items fp32, 16-byte aligned.  TIDE_PROBE_MIX_BOTH writes the ordered
 *              sums (as the reduce-scatter would), TIDE_PROBE_MIX_WRITES a pattern,
 *              TIDE_PROBE_MIX_READS nothing.
 *   lds_bytes  local memory each workgroup requests (static + dynamic): sets how many workgroups
 *              fit in a CU; 0 = the kernel's own only.
 * Returns 0 or a hipError_t value; -1 for bad arguments (C, mode, items < 1 or > 2^31-1, NULL dst,
 * NULL src with loads, lds_bytes < 0).
 */
int32_t tide_probe_mix(int32_t C, int32_t mode, const void* const* src, float* dst, int64_t items, int32_t lds_bytes,
                       void* stream);

/*
 * A stream whose kernels may run only on the compute units selected by bits [first_cu, first_cu +
 * n_cus) of a CU mask (hipExtStreamCreateWithCUMask; the runtime maps mask bits onto the XCDs' CUs,
 * and tide_probe_launch's records show where they landed).  Instruments the alternative to a CU
 * budget -- confining communication to a fixed set of CUs -- beside [Endgame] Figure 3's account of
 * resident communication workgroups holding CUs a concurrent GEMM needs.  Default priority.
 *   first_cu, n_cus  0 <= first_cu, 1 <= n_cus, first_cu + n_cus <= the current device's CU count.
 *   stream           receives the hipStream_t (as void*); release it with tide_probe_stream_destroy
 *                    after the work on it has finished.
 * Returns 0 or a hipError_t value; -1 for bad arguments (ranges above, NULL stream) or when the
 * device's CU count cannot be read.
 */
int32_t tide_probe_stream_create_cu_mask(int32_t first_cu, int32_t n_cus, void** stream);

/* Destroy a stream made by tide_probe_stream_create_cu_mask.  Returns 0 or a hipError_t value; -1 for NULL. */
int32_t tide_probe_stream_destroy(void* stream);

/* One rectangular copy for tide_probe_dma_rect_copies: `rows` rows of `width` bytes, row i read from
 * src + i*src_pitch and written to dst + i*dst_pitch (device addresses; every address, pitch and
 * width a multiple of 4 bytes). */
typedef struct tide_probe_rect {
  void* dst;
  const void* src;
  int64_t dst_pitch;
  int64_t src_pitch;
  int64_t width;
  int64_t rows;
} tide_probe_rect;

/*
 * Rectangular copies on the DMA engines, the copy-engine form of [Endgame] Figure 5b's placement
 * (each parameter filled from the stage slots by one strided copy).  HIP's 2-D copies between device
 * buffers run as shader kernels on ROCm; the DMA engines' rectangular copy is reached through the HSA
 * runtime's provisional hsa_amd_memory_async_copy_rect on the current device's GPU agent.  All n
 * copies are issued before any is waited for, then the host waits for every one (at most timeout_ms
 * in all).  The copies are not ordered with any HIP stream: the caller synchronises the device
 * first and reads the results after the call returns.
 *   elapsed_us  may be NULL; receives the host time from the first issue to the last completion.
 * Returns 0; -1 for bad arguments (n < 1, NULL rects, a NULL pointer, a size or pitch not a
 * positive multiple of 4, width beyond a pitch, more than 2^32-1 rows or width bytes); -2 when the
 * current device's GPU agent is not found; -3 when the copies did not all finish within timeout_ms
 * (some may still be running); otherwise the hsa_status_t of the first copy the runtime refused
 * (the copies issued before it have finished when the call returns).
 */
int32_t tide_probe_dma_rect_copies(int32_t n, const tide_probe_rect* rects, int64_t timeout_ms, double* elapsed_us);

/* Device wall-clock rate in kHz (hipDeviceAttributeWallClockRate of the current device), or -1. */
int64_t tide_probe_wall_clock_khz(void);

/* Build id of this library (16 hex digits of the SHA-256 of its sources, headers and compile flags;
 * "unknown" if none was set): the binding refuses a library built from other sources.  Host only. */
const char* tide_probe_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* TIDE_PROBE_H */
