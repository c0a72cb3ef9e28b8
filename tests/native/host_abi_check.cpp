// Host-only exercise of libtide's layout and validation code under AddressSanitizer and UBSan.
// Built with g++ (no device code): the kernel launchers are stubs that abort, and every call made
// here returns before any HIP call (layouts never reach a device; invalid arguments are rejected
// first).  Exit status 0 = all checks passed.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../../all_gather_placement_amd/csrc/tide_internal.h"
#include "tide.h"

namespace tide {
int launch_rs(const RsChunk*, int64_t, int64_t, int, int, const void* const*, int32_t, int32_t, int64_t, bool, bool,
              int, void*) {
  std::fprintf(stderr, "launch_rs reached in a host-only check\n");
  std::abort();
}
int rs_lds_info(int, int*, int*, int*) {
  std::fprintf(stderr, "rs_lds_info reached in a host-only check\n");
  std::abort();
}
int launch_ag(const AgChunk*, int64_t, int64_t, int, int, int, void*, const void* const*, bool, bool, void*) {
  std::fprintf(stderr, "launch_ag reached in a host-only check\n");
  std::abort();
}
int launch_fill_zero(const AgChunk*, int64_t, void*, void*) {
  std::fprintf(stderr, "launch_fill_zero reached in a host-only check\n");
  std::abort();
}
int launch_rs_cu(const RsChunk*, int64_t, int, int, const void* const*, int32_t, int32_t, int64_t, bool, bool, int,
                 void*) {
  std::fprintf(stderr, "launch_rs_cu reached in a host-only check\n");
  std::abort();
}
int launch_ag_cu(const AgChunk*, int64_t, int, void*, const void* const*, bool, bool, int, void*) {
  std::fprintf(stderr, "launch_ag_cu reached in a host-only check\n");
  std::abort();
}
int noalloc_scratch(int, void**, int64_t*) {
  std::fprintf(stderr, "noalloc_scratch reached in a host-only check\n");
  std::abort();
}
int launch_put_ptrs(void*, void* const*, int64_t, void*) {
  std::fprintf(stderr, "launch_put_ptrs reached in a host-only check\n");
  std::abort();
}
}  // namespace tide

static int failures = 0;
#define CHECK(cond)                                                       \
  do {                                                                    \
    if (!(cond)) {                                                        \
      std::fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

int main() {
  std::mt19937_64 rng(12345);
  int64_t groups = 0;
  for (int it = 0; it < 400; ++it) {
    const int32_t R = 1 + int32_t(rng() % 70);
    const int32_t P = 1 + int32_t(rng() % 7);
    std::vector<int32_t> nd(P);
    std::vector<int64_t> dims;
    std::vector<int64_t> rows(P), len(P);
    for (int32_t p = 0; p < P; ++p) {
      nd[p] = 1 + int32_t(rng() % 4);
      rows[p] = int64_t(rng() % 3000);
      len[p] = 1;
      dims.push_back(rows[p]);
      for (int k = 1; k < nd[p]; ++k) {
        const int64_t d = int64_t(rng() % 9);
        dims.push_back(d);
        len[p] *= d;
      }
    }
    tide_layout* L = nullptr;
    CHECK(tide_layout_create(P, nd.data(), dims.data(), R, &L) == TIDE_OK);
    if (!L) continue;
    ++groups;
    // geometry against the closed forms; every output element covered exactly once
    int64_t S = 0;
    for (int32_t p = 0; p < P; ++p) {
      int64_t r0, l0, m0, o0;
      CHECK(tide_layout_param(L, p, &r0, &l0, &m0, &o0) == TIDE_OK);
      CHECK(r0 == rows[p] && l0 == len[p] && m0 == (rows[p] + R - 1) / R && o0 == S);
      S += m0 * l0;
    }
    CHECK(tide_layout_shard_numel(L) == S);
    const int64_t nrs = tide_layout_num_rs_chunks(L), nag = tide_layout_num_ag_chunks(L);
    const int64_t npad = tide_layout_num_slot_pad_items(L);
    std::vector<int64_t> rs(6 * (nrs + 1)), ag(4 * (nag + 1)), pad(2 * (npad + 1));
    CHECK(tide_layout_copy_rs_items(L, 0, nrs, rs.data()) == TIDE_OK);
    CHECK(tide_layout_copy_ag_items(L, 0, nag, ag.data()) == TIDE_OK);
    CHECK(tide_layout_copy_slot_pad_items(L, 0, npad, pad.data()) == TIDE_OK);
    CHECK(tide_layout_copy_rs_items(L, nrs, 1, rs.data()) == TIDE_ERR_INVALID);
    std::vector<uint8_t> cover(size_t(R) * size_t(S), 0), slot(size_t(R) * size_t(S), 0);
    for (int64_t i = 0; i < nrs; ++i) {
      const int64_t* c = &rs[6 * i];
      for (int64_t k = 0; k < c[4] + c[5]; ++k) ++cover[size_t(c[1]) * S + c[3] + k];
    }
    for (int64_t i = 0; i < nag; ++i)
      for (int64_t k = 0; k < ag[4 * i + 3]; ++k) ++slot[ag[4 * i + 1] + k];
    for (int64_t i = 0; i < npad; ++i)
      for (int64_t k = 0; k < pad[2 * i + 1]; ++k) ++slot[pad[2 * i] + k];
    for (size_t i = 0; i < cover.size(); ++i) {
      CHECK(cover[i] == 1);
      CHECK(slot[i] == 1);
      if (failures > 20) return 1;
    }
    tide_layout_destroy(L);
  }
  // invalid arguments, each rejected before any HIP call
  int32_t nd1[1] = {2};
  int64_t d1[2] = {4, 4};
  tide_layout* L = nullptr;
  CHECK(tide_layout_create(0, nd1, d1, 4, &L) == TIDE_ERR_INVALID);
  CHECK(tide_layout_create(1, nd1, d1, 0, &L) == TIDE_ERR_INVALID);
  int64_t huge[2] = {int64_t(1) << 40, int64_t(1) << 40};
  CHECK(tide_layout_create(1, nd1, huge, 4, &L) == TIDE_ERR_INVALID);
  CHECK(tide_layout_create(1, nd1, d1, 4, &L) == TIDE_OK);
  const uintptr_t base = uintptr_t(1) << 40;
  const void* g[1] = {reinterpret_cast<void*>(base)};
  float* sh[4];
  for (int r = 0; r < 4; ++r) sh[r] = reinterpret_cast<float*>(base + (uintptr_t(1) << 20) * (r + 1));
  const int D = TIDE_LAUNCH_DEFAULT;
  CHECK(tide_rs_bf16_to_fp32(L, 0, g, sh, D, 0, nullptr) == TIDE_ERR_INVALID);
  sh[2] = sh[1];
  CHECK(tide_rs_bf16_to_fp32(L, 1, g, sh, D, 0, nullptr) == TIDE_ERR_INVALID);  // shards overlap
  sh[2] = reinterpret_cast<float*>(base + 8);
  CHECK(tide_rs_bf16_to_fp32(L, 1, g, sh, D, 0, nullptr) == TIDE_ERR_INVALID);  // shard inside a gradient
  void* pp[1] = {reinterpret_cast<void*>(base + 2)};
  CHECK(tide_ag_place(L, reinterpret_cast<void*>(base), pp, TIDE_AG_KERNEL, D, 0, nullptr) == TIDE_ERR_INVALID);
  CHECK(tide_ag_place(L, reinterpret_cast<void*>(base), pp, 7, D, 0, nullptr) == TIDE_ERR_INVALID);
  CHECK(tide_slot_pack(L, const_cast<const void* const*>(pp), reinterpret_cast<void*>(base), D, 0, nullptr) ==
        TIDE_ERR_INVALID);
  const void* sl[2] = {reinterpret_cast<void*>(base), reinterpret_cast<void*>(base + 1)};
  float* sh2[4];
  for (int r = 0; r < 4; ++r) sh2[r] = reinterpret_cast<float*>(base + (uintptr_t(1) << 20) * (r + 1));
  CHECK(tide_rs_slots_bf16_to_fp32(L, 2, sl, sh2, D, 0, nullptr) == TIDE_ERR_INVALID);  // odd slot address
  // launch forms out of range are refused before anything else (the rest of these calls is valid)
  {
    const int bad_rs[][3] = {  // {C, form, count}
        {1, 9, 0}, {1, -1, 0}, {1, TIDE_LAUNCH_DEFAULT, 1}, {1, TIDE_LAUNCH_BOUNDED, 0},
        {1, TIDE_LAUNCH_BOUNDED, -3}, {1, TIDE_LAUNCH_CU_EXCLUSIVE, 0}, {1, TIDE_LAUNCH_CU_EXCLUSIVE, 9},
        {1, TIDE_LAUNCH_CU_EXCLUSIVE, 24}, {1, TIDE_LAUNCH_CU_EXCLUSIVE, 64}, {3, TIDE_LAUNCH_CU_EXCLUSIVE, 32},
        {5, TIDE_LAUNCH_CU_EXCLUSIVE, 16}, {1, TIDE_LAUNCH_PER_CU_CAP, 0},
        {1, TIDE_LAUNCH_PER_CU_CAP, TIDE_MAX_WGS_PER_CU + 1}};
    for (const auto& b : bad_rs) {
      std::vector<const void*> gg(size_t(b[0]), g[0]);
      CHECK(tide_rs_bf16_to_fp32(L, b[0], gg.data(), sh2, b[1], b[2], nullptr) == TIDE_ERR_INVALID);
      CHECK(tide_rs_slots_bf16_to_fp32(L, b[0], gg.data(), sh2, b[1], b[2], nullptr) == TIDE_ERR_INVALID);
      CHECK(tide_rs_launch_shape(b[0], b[1], b[2], nullptr, nullptr, nullptr, nullptr) == TIDE_ERR_INVALID);
    }
    void* qq[1] = {reinterpret_cast<void*>(base + (uintptr_t(1) << 30))};
    const int bad_ag[][3] = {  // {mode, form, count}
        {TIDE_AG_KERNEL, TIDE_LAUNCH_PER_CU_CAP, 4}, {TIDE_AG_KERNEL, TIDE_LAUNCH_CU_EXCLUSIVE, 9},
        {TIDE_AG_KERNEL, TIDE_LAUNCH_CU_EXCLUSIVE, 0}, {TIDE_AG_KERNEL, TIDE_LAUNCH_BOUNDED, 0},
        {TIDE_AG_KERNEL, TIDE_LAUNCH_DEFAULT, 2}, {TIDE_AG_SDMA, TIDE_LAUNCH_CU_EXCLUSIVE, 4},
        {TIDE_AG_SDMA, TIDE_LAUNCH_BOUNDED, 8}, {TIDE_AG_COPY2D, TIDE_LAUNCH_BOUNDED, 8}};
    for (const auto& b : bad_ag)
      CHECK(tide_ag_place(L, reinterpret_cast<void*>(base), qq, b[0], b[1], b[2], nullptr) == TIDE_ERR_INVALID);
    CHECK(tide_slot_pack(L, const_cast<const void* const*>(qq), reinterpret_cast<void*>(base), TIDE_LAUNCH_PER_CU_CAP,
                         2, nullptr) == TIDE_ERR_INVALID);
  }
  // the allocation-free RS applies the same checks, and refuses a pointer table beyond its scratch
  CHECK(tide_rs_bf16_to_fp32_noalloc(L, 1, g, sh, D, 0, nullptr) == TIDE_ERR_INVALID);  // shard inside a gradient
  CHECK(tide_rs_bf16_to_fp32_noalloc(L, 0, g, sh2, D, 0, nullptr) == TIDE_ERR_INVALID);
  CHECK(tide_rs_bf16_to_fp32_noalloc(L, 1, g, sh2, TIDE_LAUNCH_CU_EXCLUSIVE, 9, nullptr) == TIDE_ERR_INVALID);
  {
    // C = TIDE_NOALLOC_MAX_PTRS contributors (all aliasing one valid gradient) + R shards: one too many
    std::vector<const void*> many(TIDE_NOALLOC_MAX_PTRS, g[0]);
    CHECK(tide_rs_bf16_to_fp32_noalloc(L, TIDE_NOALLOC_MAX_PTRS, many.data(), sh2, D, 0, nullptr) == TIDE_ERR_INVALID);
  }
  // prepared calls apply the same checks, and leave *out untouched
  tide_call* call = nullptr;
  CHECK(tide_rs_prepare(L, 1, g, sh, D, 0, &call) == TIDE_ERR_INVALID && call == nullptr);
  CHECK(tide_rs_prepare(L, 0, g, sh2, D, 0, &call) == TIDE_ERR_INVALID && call == nullptr);
  CHECK(tide_rs_prepare(L, 1, g, sh2, TIDE_LAUNCH_CU_EXCLUSIVE, 9, &call) == TIDE_ERR_INVALID && call == nullptr);
  CHECK(tide_ag_prepare(L, reinterpret_cast<void*>(base), pp, TIDE_AG_KERNEL, TIDE_LAUNCH_PER_CU_CAP, 1, &call) ==
        TIDE_ERR_INVALID);
  CHECK(tide_ag_prepare(L, reinterpret_cast<void*>(base), pp, TIDE_AG_SDMA, TIDE_LAUNCH_CU_EXCLUSIVE, 4, &call) ==
        TIDE_ERR_INVALID);
  CHECK(tide_ag_prepare(L, reinterpret_cast<void*>(base), pp, TIDE_AG_KERNEL, TIDE_LAUNCH_CU_EXCLUSIVE, 9, &call) ==
        TIDE_ERR_INVALID);
  CHECK(tide_ag_prepare(L, reinterpret_cast<void*>(base), pp, TIDE_AG_KERNEL, D, 0, &call) == TIDE_ERR_INVALID);
  CHECK(tide_ag_prepare(L, reinterpret_cast<void*>(base), pp, 7, D, 0, &call) == TIDE_ERR_INVALID);
  CHECK(tide_slot_pack_prepare(L, const_cast<const void* const*>(pp), reinterpret_cast<void*>(base), D, 0, &call) ==
        TIDE_ERR_INVALID);
  CHECK(tide_rs_slots_prepare(L, 2, sl, sh2, D, 0, &call) == TIDE_ERR_INVALID && call == nullptr);
  CHECK(tide_rs_prepare(L, 1, g, sh2, D, 0, nullptr) == TIDE_ERR_INVALID);  // no output handle
  CHECK(tide_call_launch(nullptr, nullptr) == TIDE_ERR_INVALID);
  int32_t th = 0, it = 0, out = 0, lds = 0;
  CHECK(tide_rs_launch_shape(0, D, 0, &th, &it, &out, &lds) == TIDE_ERR_INVALID);
  // Every work item is taken exactly once by the kernels' own index maps (item_index, xcd_slot) under
  // every launch plan the entry points make: single-item launches, bounded launches (RS 4 and
  // placement 8 items per workgroup, budgets of 2B workgroups), with and without the XCD remap, and
  // CU-exclusive workgroups of W groups taking KI items each.
  {
    std::vector<int> seen;
    int64_t bad_plans = 0;
    auto check_plan = [&](int64_t count, bool bounded, int64_t max_wgs, int items, bool remap) {
      seen.assign(size_t(count), 0);
      const tide::Plan plan = tide::plan_for(count, bounded, max_wgs, items);
      for (int64_t first = 0; first < count; first += plan.per_launch) {
        const int64_t n = std::min<int64_t>(plan.per_launch, count - first);
        const int64_t grid = std::min<int64_t>(plan.grid, n);
        for (int64_t b = 0; b < grid; ++b)
          for (int j = 0; j < plan.items; ++j) {
            const int64_t it = tide::item_index(remap, grid, b, j, n);
            if (it >= n) break;  // the kernels' loops end at the first item past their launch
            ++seen[size_t(first + it)];
          }
      }
      for (int64_t i = 0; i < count; ++i) bad_plans += seen[size_t(i)] != 1;
    };
    auto check_cu = [&](int64_t count, int W, int KI) {
      seen.assign(size_t(count), 0);
      const int64_t grid = (count + int64_t(W) * KI - 1) / (int64_t(W) * KI);
      for (int64_t b = 0; b < grid; ++b)
        for (int g = 0; g < W; ++g)
          for (int k = 0; k < KI; ++k) {
            const int64_t it = (tide::xcd_slot(grid, b) * W + g) * KI + k;
            if (it < count) ++seen[size_t(it)];
          }
      for (int64_t i = 0; i < count; ++i) bad_plans += seen[size_t(i)] != 1;
    };
    const int64_t counts[] = {1, 2, 3, 7, 8, 9, 15, 16, 17, 63, 100, 1023, 1024, 1025, 4097, 70001};
    for (int64_t count : counts) {
      for (bool remap : {false, true}) {
        check_plan(count, false, 0, 0, remap);
        for (int64_t B : {1, 2, 3, 7, 64, 512, 5000}) {
          check_plan(count, true, B * tide::kBudgetThreads / tide::kThreads, tide::kRsBoundedItems, remap);
          check_plan(count, true, B * tide::kBudgetThreads / tide::kAgThreads, tide::kAgBoundedItems, remap);
        }
      }
      for (int W = 1; W <= tide::kRsCuMaxGroups; ++W)
        for (int KI : {1, 2}) check_cu(count, W, KI);
    }
    CHECK(bad_plans == 0);
  }
  tide_call_destroy(nullptr);
  CHECK(tide_last_hip_error() == 0);
  tide_layout_destroy(L);
  tide_layout_destroy(nullptr);
  std::printf("host checks: %lld groups, %d failures\n", static_cast<long long>(groups), failures);
  return failures == 0 ? 0 : 1;
}
