// Layout creation and queries: geometry of one FSDP parameter group and its work-item tables.
//
// Geometry follows [Endgame] Table 2 (padded per-rank rows, row length, per-rank shard size,
// prefix offset, per-rank packed shard size) and Figure 1 (per-parameter storage on one side of
// FSDP2's contract boundary, flat rank-major shards on the other):
//   L_p = product of shape_p[1:], m_p = ceil(rows_p / R), e_p = m_p * L_p, o_p = sum_{q<p} e_q,
//   v(p, r) = clamp(rows_p - r * m_p, 0, m_p).
// The segment (p, r) is the contiguous run of v * L_p elements at element r * m_p * L_p of
// parameter p, whose home is element o_p of rank r's shard, followed there by (m_p - v) * L_p
// padding elements.  Segments are cut into work items whose interior boundaries sit on 16-byte
// source boundaries, so the kernels need no per-element lookup.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <new>

#include "../../include/tide.h"
#include "layout.h"

namespace tide {
namespace {

constexpr int64_t kMaxElems = int64_t(1) << 62;

inline int64_t clamp64(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Cut [0, n) of a segment whose first element sits at absolute source offset `src0` into pieces
// whose interior boundaries are at absolute offsets align_down(src0, 8) + k * chunk.
template <typename F>
void cut(int64_t src0, int64_t n, int64_t chunk, F&& emit) {
  const int64_t base = src0 & ~int64_t(7);
  int64_t pos = 0;
  while (pos < n) {
    const int64_t s = src0 + pos;
    const int64_t k = (s - base) / chunk + 1;
    const int64_t end = base + k * chunk;  // next boundary strictly after s
    const int64_t len = (end - s) < (n - pos) ? (end - s) : (n - pos);
    emit(pos, len);
    pos += len;
  }
}

thread_local int g_last_hip_error = 0;

// Copy a host table to new device memory (nothing for an empty table).
template <typename T>
hipError_t upload(hipStream_t aux, const std::vector<T>& v, T** out) {
  *out = nullptr;
  if (v.empty()) return hipSuccess;
  void* p = nullptr;
  const int e = dev_alloc_copy(aux, v.data(), v.size() * sizeof(T), &p);
  *out = static_cast<T*>(p);
  return static_cast<hipError_t>(e);
}

// Order in which workgroups take work items (before any XCD renumbering in the kernels):
//   0: parameter-major (p, r, position): each contributor tensor is read front to back;
//   1: rank-major (r, p, position): each shard is written front to back;
//   2: interleaved: the k-th item of every segment before the (k+1)-th of any.
template <typename Item, typename RankOf>
void order_one(std::vector<Item>& v, int order, RankOf rank_of) {
  if (order == 1) {
    std::stable_sort(v.begin(), v.end(), [&](const Item& a, const Item& b) { return rank_of(a) < rank_of(b); });
  } else if (order == 2) {
    std::vector<int64_t> k(v.size());
    for (size_t i = 0; i < v.size(); ++i) {
      const bool same = i > 0 && v[i].p == v[i - 1].p && rank_of(v[i]) == rank_of(v[i - 1]);
      k[i] = same ? k[i - 1] + 1 : 0;
    }
    std::vector<size_t> idx(v.size());
    for (size_t i = 0; i < idx.size(); ++i) idx[i] = i;
    std::stable_sort(idx.begin(), idx.end(), [&](size_t a, size_t b) { return k[a] < k[b]; });
    std::vector<Item> out(v.size());
    for (size_t i = 0; i < idx.size(); ++i) out[i] = v[idx[i]];
    v.swap(out);
  }
}

}  // namespace

void order_items(tide_layout* L) {
  order_one(L->rs_chunks, TIDE_RS_ITEM_ORDER, [](const RsChunk& c) { return c.r; });
  const int64_t S = L->S;
  order_one(L->ag_chunks, TIDE_AG_ITEM_ORDER, [S](const AgChunk& c) { return S > 0 ? c.src / S : 0; });
}

void set_last_hip_error(int err) { g_last_hip_error = err; }

int dev_alloc_copy(hipStream_t aux, const void* host, size_t bytes, void** out) {
  *out = nullptr;
  void* p = nullptr;
  hipError_t e = hipMallocAsync(&p, bytes, aux);
  if (e != hipSuccess) return e;
  if (host != nullptr) e = hipMemcpyAsync(p, host, bytes, hipMemcpyHostToDevice, aux);
  if (e == hipSuccess) e = hipStreamSynchronize(aux);
  if (e != hipSuccess) {
    (void)hipFreeAsync(p, aux);
    return e;
  }
  *out = p;
  return hipSuccess;
}

void dev_free(void* p, hipStream_t aux) {
  if (p != nullptr) (void)hipFreeAsync(p, aux);
}

int rs_device_info(int device, DeviceState* st) {
  hipError_t e = static_cast<hipError_t>(
      rs_lds_info(device, &st->lds_per_cu, &st->rs_static_lds_ct, &st->rs_static_lds_rt));
  if (e == hipSuccess) e = hipDeviceGetAttribute(&st->lds_per_wg, hipDeviceAttributeMaxSharedMemoryPerBlock, device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&st->cus, hipDeviceAttributeMultiprocessorCount, device);
  return e;
}

int device_state(const tide_layout* layout, DeviceState** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  auto it = layout->devices.find(dev);
  if (it != layout->devices.end()) {
    *out = &it->second;
    return hipSuccess;
  }
  DeviceState st;
  e = static_cast<hipError_t>(rs_device_info(dev, &st));
  if (e == hipSuccess) e = static_cast<hipError_t>(noalloc_scratch(dev, &st.scratch, &st.scratch_ptrs));
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&st.aux, hipStreamNonBlocking);
  if (e != hipSuccess) return e;
  e = upload(st.aux, layout->rs_chunks, &st.rs);
  if (e == hipSuccess) e = upload(st.aux, layout->ag_chunks, &st.ag);
  if (e == hipSuccess) e = upload(st.aux, layout->slot_pad_items, &st.slot_pad);
  if (e != hipSuccess) {
    dev_free(st.rs, st.aux);
    dev_free(st.ag, st.aux);
    dev_free(st.slot_pad, st.aux);
    (void)hipStreamSynchronize(st.aux);
    (void)hipStreamDestroy(st.aux);
    return e;
  }
  auto res = layout->devices.emplace(dev, st);
  *out = &res.first->second;
  return hipSuccess;
}

}  // namespace tide

using tide::AgChunk;
using tide::ParamGeom;
using tide::RsChunk;

extern "C" {

tide_status tide_layout_create(int32_t num_params, const int32_t* ndims, const int64_t* dims,
                               int32_t num_ranks, tide_layout** out) {
  if (out == nullptr || ndims == nullptr || dims == nullptr || num_params < 1 || num_ranks < 1)
    return TIDE_ERR_INVALID;
  tide_layout* L = new (std::nothrow) tide_layout();
  if (L == nullptr) return TIDE_ERR_NOMEM;
  try {
    L->P = num_params;
    L->R = num_ranks;
    L->params.resize(num_params);
    int64_t di = 0, o = 0;
    for (int32_t p = 0; p < num_params; ++p) {
      const int32_t nd = ndims[p];
      if (nd < 1 || nd > 64) {
        delete L;
        return TIDE_ERR_INVALID;
      }
      int64_t rows = dims[di];
      int64_t len = 1;
      bool bad = rows < 0;
      for (int32_t k = 1; k < nd; ++k) {
        const int64_t d = dims[di + k];
        if (d < 0) bad = true;
        else if (d > 0 && len > tide::kMaxElems / d) bad = true;
        else len *= d;
      }
      di += nd;
      if (bad) {
        delete L;
        return TIDE_ERR_INVALID;
      }
      ParamGeom g;
      g.rows = rows;
      g.L = len;
      g.m = (rows + num_ranks - 1) / num_ranks;
      if (g.L > 0 && g.m > tide::kMaxElems / g.L / num_ranks) {
        delete L;
        return TIDE_ERR_INVALID;
      }
      g.e = g.m * g.L;
      g.numel = rows * len;
      g.o = o;
      o += g.e;
      if (o > tide::kMaxElems / num_ranks) {
        delete L;
        return TIDE_ERR_INVALID;
      }
      L->params[p] = g;
    }
    L->S = o;

    // Work items, built parameter-major (p, r, position) and then put in kernel order.
    for (int32_t p = 0; p < num_params; ++p) {
      const ParamGeom& g = L->params[p];
      for (int32_t r = 0; r < num_ranks; ++r) {
        const int64_t v = tide::clamp64(g.rows - int64_t(r) * g.m, 0, g.m);
        const int64_t nvalid = v * g.L, npad = (g.m - v) * g.L;
        const int64_t src0 = int64_t(r) * g.m * g.L;
        tide::cut(src0, nvalid, tide::kRsChunk, [&](int64_t pos, int64_t len) {
          L->rs_chunks.push_back(RsChunk{src0 + pos, g.o + pos, p, r, int32_t(len), 0});
        });
        for (int64_t pos = 0; pos < npad; pos += tide::kRsChunk) {
          const int64_t len = (npad - pos) < tide::kRsChunk ? (npad - pos) : tide::kRsChunk;
          L->rs_chunks.push_back(RsChunk{0, g.o + nvalid + pos, p, r, 0, int32_t(len)});
        }
        const int64_t stage0 = int64_t(r) * L->S + g.o;
        tide::cut(stage0, nvalid, tide::kAgChunk, [&](int64_t pos, int64_t len) {
          L->ag_chunks.push_back(AgChunk{stage0 + pos, src0 + pos, p, int32_t(len), 0});
        });
        for (int64_t pos = 0; pos < npad; pos += tide::kAgChunk) {
          const int64_t len = (npad - pos) < tide::kAgChunk ? (npad - pos) : tide::kAgChunk;
          L->slot_pad_items.push_back(AgChunk{stage0 + nvalid + pos, 0, p, int32_t(len), 0});
        }
      }
    }
    tide::order_items(L);
  } catch (const std::bad_alloc&) {
    delete L;
    return TIDE_ERR_NOMEM;
  }
  *out = L;
  return TIDE_OK;
}

void tide_layout_destroy(tide_layout* layout) {
  if (layout == nullptr) return;
  int cur = 0;
  // No HIP call at all for a layout that never reached a device (host-only use).
  const bool have_dev = !layout->devices.empty() && hipGetDevice(&cur) == hipSuccess;
  if (have_dev) {
    // Prepared calls not destroyed yet (the contract asks for them to go first): their queued
    // launches read the tables below.
    std::lock_guard<std::mutex> lock(layout->mu);
    tide::wait_for_calls(layout);
  }
  for (auto& kv : layout->devices) {
    if (hipSetDevice(kv.first) != hipSuccess) continue;
    // What else may still read the tables: immediate calls' kernels (each ring slot's event is
    // recorded after the kernels that read it) and DMA copies (the internal streams).  Work of
    // other streams that never used the layout is not waited for.
    tide::DeviceState& st = kv.second;
    for (auto& s : st.slots) {
      if (s.done) {
        if (s.pending) (void)hipEventSynchronize(s.done);
        (void)hipEventDestroy(s.done);
      }
      tide::dev_free(s.dev, st.aux);
    }
    for (int k = 0; k < tide::kDmaStreams; ++k) {
      if (st.dma[k]) {
        (void)hipStreamSynchronize(st.dma[k]);
        (void)hipStreamDestroy(st.dma[k]);
      }
      if (st.dma_join[k]) (void)hipEventDestroy(st.dma_join[k]);
    }
    if (st.dma_fork) (void)hipEventDestroy(st.dma_fork);
    // stream-ordered frees on the internal stream: they wait for nothing but that stream
    tide::dev_free(st.rs, st.aux);
    tide::dev_free(st.ag, st.aux);
    tide::dev_free(st.slot_pad, st.aux);
    (void)hipStreamSynchronize(st.aux);
    (void)hipStreamDestroy(st.aux);
  }
  if (have_dev && !layout->devices.empty()) (void)hipSetDevice(cur);
  delete layout;
}

tide_status tide_layout_prepare(const tide_layout* layout) {
  if (layout == nullptr) return TIDE_ERR_INVALID;
  std::lock_guard<std::mutex> lock(layout->mu);
  tide::DeviceState* st = nullptr;
  const int e = tide::device_state(layout, &st);
  if (e == hipErrorOutOfMemory) return TIDE_ERR_NOMEM;
  if (e != hipSuccess) {
    tide::set_last_hip_error(e);
    return TIDE_ERR_HIP;
  }
  return TIDE_OK;
}

int32_t tide_layout_num_params(const tide_layout* layout) { return layout ? layout->P : -1; }
int32_t tide_layout_num_ranks(const tide_layout* layout) { return layout ? layout->R : -1; }
int64_t tide_layout_shard_numel(const tide_layout* layout) { return layout ? layout->S : -1; }
int64_t tide_layout_num_rs_chunks(const tide_layout* layout) {
  return layout ? int64_t(layout->rs_chunks.size()) : -1;
}
int64_t tide_layout_num_ag_chunks(const tide_layout* layout) {
  return layout ? int64_t(layout->ag_chunks.size()) : -1;
}

tide_status tide_layout_param(const tide_layout* layout, int32_t p, int64_t* rows, int64_t* row_len,
                              int64_t* padded_rows, int64_t* offset) {
  if (layout == nullptr || p < 0 || p >= layout->P) return TIDE_ERR_INVALID;
  const ParamGeom& g = layout->params[p];
  if (rows) *rows = g.rows;
  if (row_len) *row_len = g.L;
  if (padded_rows) *padded_rows = g.m;
  if (offset) *offset = g.o;
  return TIDE_OK;
}

tide_status tide_layout_segment(const tide_layout* layout, int32_t p, int32_t r, int64_t* src_offset,
                                int64_t* valid, int64_t* dst_offset, int64_t* pad) {
  if (layout == nullptr || p < 0 || p >= layout->P || r < 0 || r >= layout->R) return TIDE_ERR_INVALID;
  const ParamGeom& g = layout->params[p];
  const int64_t v = tide::clamp64(g.rows - int64_t(r) * g.m, 0, g.m);
  if (src_offset) *src_offset = int64_t(r) * g.m * g.L;
  if (valid) *valid = v * g.L;
  if (dst_offset) *dst_offset = g.o;
  if (pad) *pad = (g.m - v) * g.L;
  return TIDE_OK;
}

tide_status tide_layout_copy_rs_items(const tide_layout* layout, int64_t first, int64_t n, int64_t* out) {
  if (layout == nullptr || out == nullptr || first < 0 || n < 0 ||
      first + n > int64_t(layout->rs_chunks.size()))
    return TIDE_ERR_INVALID;
  for (int64_t i = 0; i < n; ++i) {
    const RsChunk& c = layout->rs_chunks[first + i];
    int64_t* o = out + 6 * i;
    o[0] = c.p; o[1] = c.r; o[2] = c.src; o[3] = c.dst; o[4] = c.nvalid; o[5] = c.npad;
  }
  return TIDE_OK;
}

tide_status tide_layout_copy_ag_items(const tide_layout* layout, int64_t first, int64_t n, int64_t* out) {
  if (layout == nullptr || out == nullptr || first < 0 || n < 0 ||
      first + n > int64_t(layout->ag_chunks.size()))
    return TIDE_ERR_INVALID;
  for (int64_t i = 0; i < n; ++i) {
    const AgChunk& c = layout->ag_chunks[first + i];
    int64_t* o = out + 4 * i;
    o[0] = c.p; o[1] = c.src; o[2] = c.dst; o[3] = c.n;
  }
  return TIDE_OK;
}

int64_t tide_layout_num_slot_pad_items(const tide_layout* layout) {
  return layout ? int64_t(layout->slot_pad_items.size()) : -1;
}

tide_status tide_layout_copy_slot_pad_items(const tide_layout* layout, int64_t first, int64_t n, int64_t* out) {
  if (layout == nullptr || out == nullptr || first < 0 || n < 0 ||
      first + n > int64_t(layout->slot_pad_items.size()))
    return TIDE_ERR_INVALID;
  for (int64_t i = 0; i < n; ++i) {
    const AgChunk& c = layout->slot_pad_items[first + i];
    out[2 * i] = c.src;
    out[2 * i + 1] = c.n;
  }
  return TIDE_OK;
}

const char* tide_status_str(int32_t status) {
  switch (status) {
    case TIDE_OK: return "TIDE_OK";
    case TIDE_ERR_INVALID: return "TIDE_ERR_INVALID";
    case TIDE_ERR_NOMEM: return "TIDE_ERR_NOMEM";
    case TIDE_ERR_HIP: return "TIDE_ERR_HIP";
    case TIDE_ERR_UNSUPPORTED: return "TIDE_ERR_UNSUPPORTED";
    default: return "unknown";
  }
}

int32_t tide_last_hip_error(void) { return tide::g_last_hip_error; }

#ifndef TIDE_BUILD_ID
#define TIDE_BUILD_ID "unknown"
#endif
const char* tide_build_id(void) { return TIDE_BUILD_ID; }

}  // extern "C"
