/*
 * tide.h -- C ABI of the MI355X (gfx950) layout-aware reduce-scatter and all-gather placement.
 *
 * Method: "The Endgame of FSDP Communication: Layout-Aware Collectives on Copy Engines, RDMA, and
 * NVSwitch" (arXiv 2610.38228; [Endgame] below).  FSDP2 keeps parameters and gradients as
 * per-parameter tensors while its collectives work on flat rank-major buffers; TIDE folds the
 * layout conversion into the collectives' addressing, so each piece of data is stored a single
 * time, directly in its destination ([Endgame] abstract; Figure 1).  This library implements, on one GPU, the
 * node-local level of that idea:
 *
 *   - reduce-scatter (RS): C contributors' per-parameter bf16 gradients are read in place (no
 *     full-group pack; the in-place input mode of [Endgame] Table 1), summed in fp32 (the mixed-precision mode
 *     of the abstract; Figure 6a's node-local fp32 partials) and written into R flat fp32 shards;
 *   - all-gather placement (AG): a rank-major bf16 stage buffer is landed directly into
 *     per-parameter storage ([Endgame] Figure 5b: each parameter filled by a single strided copy).
 *
 * Geometry ([Endgame] Table 2; symbols were lost in the text we have, names are ours):
 *   parameter p has shape (rows_p, d1, d2, ...); row length L_p = d1*d2*... (1 for 1-D);
 *   padded per-rank rows m_p = ceil(rows_p / R); per-rank shard elements e_p = m_p * L_p;
 *   prefix offset o_p = sum_{q<p} e_q; per-rank packed shard elements S = sum_p e_p.
 *   Rank r holds rows [r*m_p, r*m_p + v) of p with v = clamp(rows_p - r*m_p, 0, m_p); the other
 *   (m_p - v) rows of its slice are padding.  Offsets are in elements; the byte offset is x2 in a
 *   bf16 buffer and x4 in an fp32 buffer.
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device addresses on the current device; host arrays are read only
 *     during the call and may be freed as soon as it returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  RS and AG calls are
 *     stream-ordered and asynchronous: they return after enqueueing, results are valid once the
 *     stream reaches that point.  Inputs are never written.
 *   - Errors are returned as tide_status; nothing is printed and nothing is thrown.  On
 *     TIDE_ERR_INVALID or TIDE_ERR_NOMEM no work has been enqueued; on TIDE_ERR_HIP or
 *     TIDE_ERR_UNSUPPORTED part of the work may have been (the stream then holds an incomplete
 *     result, and TIDE_AG_SDMA still joins its copy streams back into `stream`).
 *     tide_last_hip_error() gives the HIP error code behind the calling thread's most recent
 *     TIDE_ERR_HIP or TIDE_ERR_UNSUPPORTED.
 *   - A layout is immutable after creation and may be used from several streams and threads at
 *     once.  The library owns it; the caller owns every buffer and stream.
 *   - The library reads no environment variables: every choice (engine, launch form) is an
 *     argument.
 */
#ifndef TIDE_H
#define TIDE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tide_layout tide_layout;

/*
 * Launch forms of the kernel paths (reduce-scatter, reduce-scatter from slots, placement kernel,
 * slot packing).  Each of those calls takes a pair (launch_form, launch_count).  The form decides
 * how many of the library's workgroups are resident at once and how long each one lives; it never
 * changes a result.  [Endgame] Figure 3: communication workgroups that stay resident push a
 * concurrent GEMM's workgroups into a second wave; Figure 4: the GEMM slows down as more
 * communication workgroups stay resident, so TIDE bounds their number and lifetime.  On MI355X a
 * GEMM workgroup that holds a whole SIMD register file waits until every library workgroup on its
 * compute unit (CU) has exited, so what matters is how soon a CU is empty again.
 */
typedef enum tide_launch_form {
  /* launch_count must be 0.  RS: one launch of CU-exclusive workgroups (below) whose width and
   * items per group the library picks for C (tuned on MI355X for throughput on its own), so no
   * workgroup outlives its few items and a CU is empty again within one workgroup lifetime.
   * Placement kernel and slot packing: one launch, one 128-thread workgroup per work item. */
  TIDE_LAUNCH_DEFAULT = 0,
  /* launch_count = B >= 1: at most 256*B threads of the library's workgroups resident at a time
   * (2B workgroups of 128 threads); each processes a few work items (RS 4 -- 80 KiB of traffic at
   * C = 8 --, placement and packing 8 -- 64 KiB) and exits, and the call issues as many launches as
   * needed, so a concurrent kernel finds free CUs within one short launch. */
  TIDE_LAUNCH_BOUNDED = 1,
  /* launch_count = N work items per workgroup: one launch of workgroups that each request the
   * largest local memory one workgroup may (a whole CU's on MI355X), so a CU holds one of them and
   * is empty whenever it exits; N items (N*C*2 KiB of RS loads) stay in flight per CU.
   * RS: N = 1..8 (128*N threads, one item per 128-thread group), or N = 16 for C <= 4 (1024
   * threads, each 128-thread group keeping 2 items' loads in flight at once).
   * Placement kernel and slot packing: N = 1..8. */
  TIDE_LAUNCH_CU_EXCLUSIVE = 2,
  /* RS only.  launch_count = N in 1..TIDE_MAX_WGS_PER_CU: one launch of single-item 128-thread
   * workgroups, at most N of them resident per CU (each requests 1/N of the CU's local memory; an N
   * at or above the hardware's own limit leaves that limit).  From N = 2 up a CU is never empty
   * during the call, so a kernel that waits for whole CUs waits for the whole call. */
  TIDE_LAUNCH_PER_CU_CAP = 3
} tide_launch_form;

#define TIDE_MAX_WGS_PER_CU 64          /* largest launch_count of TIDE_LAUNCH_PER_CU_CAP */
#define TIDE_CU_EXCLUSIVE_MAX_ITEMS 16  /* largest launch_count of TIDE_LAUNCH_CU_EXCLUSIVE (RS) */

typedef enum tide_status {
  TIDE_OK = 0,
  TIDE_ERR_INVALID = 1,     /* bad argument: null pointer, bad size, misalignment, overlap */
  TIDE_ERR_NOMEM = 2,       /* host or device allocation failed */
  TIDE_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed */
  TIDE_ERR_UNSUPPORTED = 4  /* valid request the runtime or device refused */
} tide_status;

/* Placement engines for tide_ag_place. */
enum {
  TIDE_AG_KERNEL = 0, /* hand-written gfx950 copy kernel: the bandwidth path (uses CUs) */
  TIDE_AG_SDMA = 1,   /* DMA (SDMA) engines: one 1-D no-compute-unit copy per (parameter, rank)
                         segment, spread over the library's internal copy streams (the runtime runs
                         only the tiniest segments as a small copy kernel).  On one MI355X a call
                         costs ~65 us before any byte moves and large copies stream 1.1-1.6 TB/s:
                         0.9-2 TB/s of traffic for large segments, 0.03-0.1 TB/s for thousands of
                         small ones.  For callers that must leave the CUs to compute.  (The DMA
                         engines' rectangular copy, which would fill each parameter in one copy,
                         streams 0.10-0.12 TB/s on MI355X and is not ordered with HIP streams, so it
                         is not used.) */
  TIDE_AG_COPY2D = 2  /* one runtime 2-D copy per parameter (row pitch = one stage slot) plus one
                         copy for the rank whose slice is part padding; the HIP runtime picks the
                         engine (on ROCm 7.2 a shader blit kernel, i.e. it uses CUs). */
};

/*
 * Build the layout of one parameter group ([Endgame] Table 2; Figure 1).
 *   num_params   P >= 1
 *   ndims        host [P]; ndims[p] >= 1 is the rank of parameter p's shape
 *   dims         host, the P shapes concatenated (sum of ndims entries), each entry >= 0
 *   num_ranks    R >= 1
 *   out          receives the new layout (unchanged on error)
 * Host-only: no HIP call is made.  Device tables are uploaded on first use per device, or by
 * tide_layout_prepare().  Errors: TIDE_ERR_INVALID (bad argument, or S or any offset beyond 2^62),
 * TIDE_ERR_NOMEM.
 */
tide_status tide_layout_create(int32_t num_params, const int32_t* ndims, const int64_t* dims,
                               int32_t num_ranks, tide_layout** out);

/* Free a layout and its device tables.  First waits for the work still queued that reads them --
 * the kernels of its immediate calls (each pointer-table slot's event), its DMA-engine copies (the
 * library's internal copy streams) and the launches of prepared calls not yet destroyed (as
 * tide_call_destroy) -- but not for other work on the device.  Prepared calls of the layout should
 * be destroyed first and must not be launched afterwards.  NULL is ignored. */
void tide_layout_destroy(tide_layout* layout);

/* Upload the layout's device tables to the current device (idempotent).  The library's device
 * memory (these tables, pointer-table slots, prepared calls' tables) comes from the device's
 * stream-ordered memory pool on an internal stream, so freeing it never waits for the whole device.
 * After this, RS and AG calls on that device allocate nothing except when a call passes more
 * pointers than any earlier one.  An immediate call writes its table of buffer addresses into one
 * of 8 slots per device with a small kernel on its stream; when all 8 hold tables of calls still in
 * flight, it waits on the host for the oldest to finish (prepared calls own their tables and never
 * wait).  Errors: TIDE_ERR_INVALID (null), TIDE_ERR_NOMEM, TIDE_ERR_HIP. */
tide_status tide_layout_prepare(const tide_layout* layout);

/* Geometry queries (host only).  Return -1 for a NULL layout. */
int32_t tide_layout_num_params(const tide_layout* layout);  /* P */
int32_t tide_layout_num_ranks(const tide_layout* layout);   /* R */
int64_t tide_layout_shard_numel(const tide_layout* layout); /* S */
int64_t tide_layout_num_rs_chunks(const tide_layout* layout); /* work items of one RS call */
int64_t tide_layout_num_ag_chunks(const tide_layout* layout); /* work items of one AG call */

/* Per-parameter geometry: rows_p, L_p, m_p, o_p (any output pointer may be NULL).
 * Errors: TIDE_ERR_INVALID (null layout or p out of range). */
tide_status tide_layout_param(const tide_layout* layout, int32_t p, int64_t* rows, int64_t* row_len,
                              int64_t* padded_rows, int64_t* offset);

/* Segment (p, r): rank r's slice of parameter p.
 *   src_offset  first element of the slice inside parameter p's storage (r * m_p * L_p)
 *   valid       elements that carry data (v * L_p)
 *   dst_offset  first element of the slice inside rank r's flat shard (o_p)
 *   pad         padding elements that follow the valid ones in the shard ((m_p - v) * L_p)
 * Errors: TIDE_ERR_INVALID. */
tide_status tide_layout_segment(const tide_layout* layout, int32_t p, int32_t r, int64_t* src_offset,
                                int64_t* valid, int64_t* dst_offset, int64_t* pad);

/* Work-item tables, for tests and tools (host only).  Copies items [first, first + n) into `out`:
 * RS items as 6 int64 each (p, r, src_offset, dst_offset, nvalid, npad) -- nvalid summed elements
 * of parameter p from src_offset land in shard r at dst_offset, then npad zeros; AG items as 4
 * int64 each (p, stage_offset, param_offset, n).  Errors: TIDE_ERR_INVALID (null, range). */
tide_status tide_layout_copy_rs_items(const tide_layout* layout, int64_t first, int64_t n, int64_t* out);
tide_status tide_layout_copy_ag_items(const tide_layout* layout, int64_t first, int64_t n, int64_t* out);
/* Padding ranges of a packed slot (tide_slot_pack zero-fills them): 2 int64 each (slot element
 * offset, count).  tide_layout_num_slot_pad_items gives their number (-1 for NULL). */
int64_t tide_layout_num_slot_pad_items(const tide_layout* layout);
tide_status tide_layout_copy_slot_pad_items(const tide_layout* layout, int64_t first, int64_t n, int64_t* out);

/*
 * Reduce-scatter, bf16 in, fp32 out ([Endgame] abstract: per-parameter bf16 gradients reduced
 * into fp32 shards; Figure 6a: node-local fp32 sums; Table 1: the in-place input mode; Figure 1:
 * every output stored once, in its destination).
 *   C          number of contributors, >= 1
 *   grads      host [C*P]: grads[c*P + p] is contributor c's gradient of parameter p, a contiguous
 *              row-major bf16 device tensor of rows_p * L_p elements, 2-byte aligned (NULL allowed
 *              only for empty parameters).  Read in place, never written.
 *   shards     host [R]: shards[r] is rank r's flat fp32 device shard of S elements, 4-byte aligned.
 *   launch_form, launch_count  see tide_launch_form.  TIDE_LAUNCH_DEFAULT picks, for C contributors,
 *              CU-exclusive workgroups of 1024 threads taking 8 items for C >= 4 and 16 for C <= 3
 *              (2 items' loads in flight per 128-thread group): the most items whose traffic stays
 *              within that of a C = 8 workgroup, so no workgroup outlives one at C = 8.  On MI355X
 *              that streams 5.9-6.34 TB/s at C = 1-8; single-item workgroups under a per-CU cap
 *              (TIDE_LAUNCH_PER_CU_CAP 12 for C <= 2, 8 for C = 3, 4) stream up to 6% more at C <= 4
 *              but never empty a CU, so a concurrent GEMM waits for the whole call.  Kernels are
 *              compiled for C = 1..16; larger C take a runtime-C form that loads contributors in
 *              blocks of 8.
 *   stream     hipStream_t as void*.
 * Result, for every r, p and element k of the slice: shards[r][o_p + k] =
 *   x_0 (+) x_1 (+) ... (+) x_{C-1}, x_c = grads[c*P+p][r*m_p*L_p + k] widened exactly to fp32,
 *   (+) an IEEE binary32 add with round-to-nearest-even, applied in ascending c, for k < v*L_p;
 *   +0.0 for the padding elements v*L_p <= k < e_p.  Every shard element is written exactly once,
 *   whatever the launch form; fp32 denormals are kept.
 * 16-byte-aligned grads and shards take the vector path; any other legal alignment takes a
 * slower element path with identical results.
 * Errors: TIDE_ERR_INVALID (null layout/arrays, C < 1, C*P > 2^24, an unknown launch form or a
 * launch_count outside its range for the form and C, null or misaligned pointer, any shard
 * overlapping another shard or any gradient), TIDE_ERR_NOMEM, TIDE_ERR_HIP.
 */
tide_status tide_rs_bf16_to_fp32(const tide_layout* layout, int32_t C, const void* const* grads,
                                 float* const* shards, int32_t launch_form, int32_t launch_count, void* stream);

/*
 * All-gather placement ([Endgame] Figure 5b: each parameter filled from the stage slots by a single
 * strided copy; abstract: shards land directly in parameter storage).
 *   stage      device, R*S bf16 elements, rank-major: rank r's shard starts at element r*S.
 *   params     host [P]: params[p] is parameter p's contiguous bf16 device storage of rows_p * L_p
 *              elements (NULL allowed only for empty parameters).
 *   mode       TIDE_AG_KERNEL, TIDE_AG_SDMA or TIDE_AG_COPY2D.
 *   launch_form, launch_count  see tide_launch_form (TIDE_AG_KERNEL only; the DMA modes take
 *              TIDE_LAUNCH_DEFAULT, 0).  Default: one 128-thread workgroup per work item.  Bounded:
 *              each workgroup copies 8 items; with at most 4 of them per CU, two items are loaded
 *              before either is stored.  CU-exclusive: workgroups of 128*N threads copying N items.
 *              TIDE_LAUNCH_PER_CU_CAP is not offered for the placement.
 * Result: params[p][r*m_p*L_p + k] = stage[r*S + o_p + k] for every r and k < v*L_p, copied as
 * bits; stage padding is never read into a parameter; every parameter element is written once.
 * All pointers must be 2-byte aligned; 16-byte alignment selects the vector path.
 * TIDE_AG_SDMA work is ordered after the caller's earlier work on `stream`, and later work on
 * `stream` waits for it (event fork/join with the internal copy streams).
 * Errors: TIDE_ERR_INVALID (null/misaligned pointer, bad mode, a launch form other than the default
 * with a DMA mode, an unknown or unsupported form or a launch_count outside its range, a parameter
 * overlapping the stage or another parameter), TIDE_ERR_UNSUPPORTED (the runtime refused a copy
 * kind), TIDE_ERR_NOMEM, TIDE_ERR_HIP.
 */
tide_status tide_ag_place(const tide_layout* layout, const void* stage, void* const* params, int32_t mode,
                          int32_t launch_form, int32_t launch_count, void* stream);

/*
 * Slot-Reuse, step 1: pack one contributor's per-parameter bf16 gradients into a rank-major
 * all-gather buffer that is no longer needed (the optional Slot-Reuse mode of the [Endgame] abstract;
 * Figure 7: the reduce-scatter then reads the buffer, which is reused only after that read).
 *   grads      host [P]: grads[p] is parameter p's contiguous bf16 gradient (rows_p * L_p elements,
 *              2-byte aligned; NULL allowed only for empty parameters).  Read, never written.
 *   slot       device, R*S bf16 elements in the stage layout (rank r's shard at element r*S).
 *   launch_form, launch_count  as for tide_ag_place with TIDE_AG_KERNEL.
 * Result: slot[r*S + o_p + k] = grads[p][r*m_p*L_p + k] for k < v*L_p (bit copy), and +0 (bits 0)
 * in every padding element; every slot element is written once.  The exact inverse of
 * tide_ag_place.  Errors: as tide_ag_place (the slot must not overlap any gradient).
 */
tide_status tide_slot_pack(const tide_layout* layout, const void* const* grads, void* slot, int32_t launch_form,
                           int32_t launch_count, void* stream);

/*
 * Slot-Reuse, step 2: reduce-scatter from C packed slots ([Endgame] Figure 7).
 *   slots      host [C]: slots[c] is contributor c's packed slot, R*S bf16 elements, 2-byte aligned
 *              (slots may alias each other; they are read, never written).
 *   shards, launch_form, launch_count, stream: as tide_rs_bf16_to_fp32.
 * Result: shards[r][k] = x_0 (+) ... (+) x_{C-1} with x_c = slots[c][r*S + k] widened, for every
 * valid element, and +0.0 for every padding element whatever the slots hold there.  Identical to
 * tide_rs_bf16_to_fp32 on the gradients the slots were packed from.
 * Errors: as tide_rs_bf16_to_fp32.
 */
tide_status tide_rs_slots_bf16_to_fp32(const tide_layout* layout, int32_t C, const void* const* slots,
                                       float* const* shards, int32_t launch_form, int32_t launch_count,
                                       void* stream);

/*
 * Allocation-free reduce-scatter, for callers that cannot allocate device memory: code running
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *   Arguments and result: exactly those of tide_rs_bf16_to_fp32 (same kernels, same launch forms,
 *   bit-identical shards).
 *   Scratch: the call's table of buffer addresses (C*P + R pointers) is written, by a small kernel
 *   on `stream`, into a fixed device array of TIDE_NOALLOC_MAX_PTRS pointers (512 KiB) that the
 *   library holds on each device it runs on until the process ends, instead of the layout's
 *   allocated ring of tables.  The call makes no hipMalloc, hipFree, hipHostMalloc or copy from host
 *   memory; it only launches kernels (host bookkeeping aside).  The table is rewritten in full by
 *   every call, so nothing needs clearing between calls.
 *   Concurrency: every call on a device shares that device's array, so calls that may overlap on one
 *   device (other streams, other threads) race on it; calls on one stream are ordered.
 *   Requirements: the layout has been prepared on the current device (tide_layout_prepare, which
 *   allocates its device tables); C*P + R <= TIDE_NOALLOC_MAX_PTRS.
 * Errors: those of tide_rs_bf16_to_fp32; TIDE_ERR_INVALID also when C*P + R exceeds
 * TIDE_NOALLOC_MAX_PTRS or the layout was not prepared on the current device (no work enqueued).
 */
#define TIDE_NOALLOC_MAX_PTRS 65536
tide_status tide_rs_bf16_to_fp32_noalloc(const tide_layout* layout, int32_t C, const void* const* grads,
                                         float* const* shards, int32_t launch_form, int32_t launch_count,
                                         void* stream);

/*
 * Prepared calls.  A training step issues the same collectives on the same buffers every step
 * (FSDP2 keeps its gradient, shard and stage buffers for the whole run), so the argument checks
 * and the device table of buffer addresses can be done once.  tide_*_prepare takes exactly the
 * arguments of the immediate call of the same name (minus the stream), applies the same checks,
 * and uploads a device table of the buffer addresses that the call owns; tide_call_launch then
 * enqueues the work on a stream with the result the immediate call would have given.
 *   - For the kernel paths (RS, RS from slots, slot packing, TIDE_AG_KERNEL placement),
 *     tide_call_launch launches kernels and, outside graph capture, records the call's completion
 *     event on the stream (created on the first launch on each stream): no device allocation, no
 *     copy, no check beyond the current device.  Such launches may be captured into a HIP graph and
 *     the graph replayed; each replay recomputes the result from the buffers' current contents.
 *   - TIDE_AG_COPY2D and TIDE_AG_SDMA calls enqueue runtime copies as the immediate call does
 *     (TIDE_AG_SDMA through the layout's internal copy streams).
 *   - The buffers named at prepare time must stay allocated while the call may launch; their
 *     contents may change freely between launches.  The layout must outlive its calls.
 *   - A call may be launched from several threads and streams at once (it is immutable); launches
 *     whose outputs overlap race, as immediate calls do.
 *   - The call belongs to the device that was current at prepare time; tide_call_launch returns
 *     TIDE_ERR_INVALID on any other device.
 * Errors of tide_*_prepare: those of the immediate call, plus TIDE_ERR_INVALID for a NULL `out`;
 * `*out` is set only on TIDE_OK.  Errors of tide_call_launch: TIDE_ERR_INVALID (NULL call, wrong
 * device), TIDE_ERR_UNSUPPORTED, TIDE_ERR_HIP.
 */
typedef struct tide_call tide_call;

tide_status tide_rs_prepare(const tide_layout* layout, int32_t C, const void* const* grads, float* const* shards,
                            int32_t launch_form, int32_t launch_count, tide_call** out);
tide_status tide_ag_prepare(const tide_layout* layout, const void* stage, void* const* params, int32_t mode,
                            int32_t launch_form, int32_t launch_count, tide_call** out);
tide_status tide_slot_pack_prepare(const tide_layout* layout, const void* const* grads, void* slot,
                                   int32_t launch_form, int32_t launch_count, tide_call** out);
tide_status tide_rs_slots_prepare(const tide_layout* layout, int32_t C, const void* const* slots,
                                  float* const* shards, int32_t launch_form, int32_t launch_count, tide_call** out);

/* Enqueue a prepared call on `stream` (hipStream_t as void*). */
tide_status tide_call_launch(const tide_call* call, void* stream);

/* Free a prepared call (its device table, on the call's device).  Waits first for the call's own
 * launches -- each kernel launch records an event on its stream, one event per stream -- so a call
 * destroyed with launches in flight is safe and work of other streams is not waited for.  Launches
 * captured into a graph carry no event; if the call was ever captured, destroy waits for the whole
 * device instead, and no graph holding its launches may be replayed afterwards.  NULL is ignored. */
void tide_call_destroy(tide_call* call);

/* Launch shape of RS calls with C contributors in a launch form on the current device: threads per
 * workgroup, work items per workgroup, outputs per full work item, and the local memory (static +
 * dynamic, bytes) each workgroup requests -- a CU holds as many RS workgroups as fit in its local
 * memory (one in the CU-exclusive forms, N with TIDE_LAUNCH_PER_CU_CAP).  Any output pointer may be
 * NULL.  Errors: TIDE_ERR_INVALID (C < 1, an unknown form or a launch_count outside its range),
 * TIDE_ERR_HIP. */
tide_status tide_rs_launch_shape(int32_t C, int32_t launch_form, int32_t launch_count, int32_t* threads,
                                 int32_t* items_per_workgroup, int32_t* item_outputs, int32_t* lds_bytes);

/* Static, NUL-terminated name of a status code ("TIDE_OK", ...; "unknown" otherwise). */
const char* tide_status_str(int32_t status);

/* HIP error code (hipError_t value) behind the calling thread's last TIDE_ERR_HIP or
 * TIDE_ERR_UNSUPPORTED (also set for TIDE_ERR_NOMEM from a device allocation), 0 if none. */
int32_t tide_last_hip_error(void);

/* Build id of this library: a static, NUL-terminated string of 16 hex digits, the first digits of
 * the SHA-256 of the sources, headers and compile flags it was built from ("unknown" for a build
 * that did not set one).  The Python binding compares it with the sources beside the library and
 * refuses a library built from other sources.  Host only; makes no HIP call. */
const char* tide_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* TIDE_H */
