"""The allocation-free reduce-scatter (tide_rs_bf16_to_fp32_noalloc) against the allocating entry point
(tide_rs_bf16_to_fp32), both called through the C ABI.

Two calls in a row on one stream, with no synchronisation between them: a larger group first, then a
smaller one (fewer parameters, ranks and contributors), so the second call's address table overwrites
the front of the first's in the library's shared scratch array while stream order keeps the first
call's kernels ahead of it.  Each call's shards must equal, bit for bit, what the allocating call
gives on the same inputs (and what the oracle gives), in the default launch, bounded launches, the
CU-exclusive form and a per-CU cap.  The refusals (layout not prepared on the device, table beyond the scratch)
are checked before any work is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from all_gather_placement_amd import (TIDE_NOALLOC_MAX_PTRS, Launch, Layout, TideError, load_library,
                                      tide_rs_bf16_to_fp32_noalloc)
from workloads import normal_bf16_bits
from tests.test_gpu_parity import dev_bf16, host_bits_f32, poisoned_shards, say

pytestmark = pytest.mark.gpu

TIDE_OK, TIDE_ERR_INVALID = 0, 1

# (shapes, R, C): the second group is smaller in every respect (P, R, C and S).
FIRST = ([(4096, 512), (2048,), (1500, 300), (7, 5), (33, 17, 3)], 8, 8)
SECOND = ([(257, 33), (3,)], 4, 3)


def _c_call(name, L, grads, shards, launch, stream):
    """One C-ABI call: `name` with the layout handle, C, the host pointer arrays, the launch form and
    count, and the stream."""
    lib = load_library()
    flat = [g.data_ptr() for row in grads for g in row]
    g_arr = (ctypes.c_void_p * len(flat))(*flat)
    s_arr = (ctypes.c_void_p * len(shards))(*[s.data_ptr() for s in shards])
    return getattr(lib, name)(L.handle, len(grads), g_arr, s_arr, launch.form, launch.count, stream.cuda_stream)


def _inputs(shapes, C, seed):
    bits = [[normal_bf16_bits(s, 1.0, seed, c, p) for p, s in enumerate(shapes)] for c in range(C)]
    return bits, [[dev_bf16(b) for b in row] for row in bits]


@pytest.mark.parametrize("launch", [Launch(), Launch.bounded(3), Launch.cu_exclusive(4), Launch.per_cu_cap(6)], ids=str)
def test_noalloc_matches_the_allocating_call_on_two_calls_in_a_row(gpu_available, launch):
    stream = torch.cuda.Stream()
    groups = []
    for k, (shapes, R, C) in enumerate((FIRST, SECOND)):
        bits, grads = _inputs(shapes, C, 300 + k)
        L = Layout(shapes, R)
        L.prepare()
        groups.append((shapes, R, bits, grads, L, poisoned_shards(R, L.S), poisoned_shards(R, L.S)))
    torch.cuda.synchronize()
    say(f"allocation-free RS, launch {launch}: two calls in a row on one stream")
    for shapes, R, bits, grads, L, out_noalloc, _ in groups:
        assert _c_call("tide_rs_bf16_to_fp32_noalloc", L, grads, out_noalloc, launch, stream) == TIDE_OK
    for shapes, R, bits, grads, L, _, out_ref in groups:
        assert _c_call("tide_rs_bf16_to_fp32", L, grads, out_ref, launch, stream) == TIDE_OK
    stream.synchronize()
    for k, (shapes, R, bits, grads, L, out_noalloc, out_ref) in enumerate(groups):
        got = np.stack([host_bits_f32(s) for s in out_noalloc])
        ref = np.stack([host_bits_f32(s) for s in out_ref])
        assert np.array_equal(got, ref), f"call {k}: {int((got != ref).sum())} elements differ from the allocating call"
        assert np.array_equal(got, oracle.reduce_scatter(bits, shapes, R).view(np.uint32)), f"call {k} vs the oracle"
        L.close()


def test_noalloc_refusals(gpu_available):
    shapes, R, C = SECOND
    bits, grads = _inputs(shapes, C, 310)
    stream = torch.cuda.Stream()
    with Layout(shapes, R) as L:
        shards = poisoned_shards(R, L.S)
        # not prepared on this device: the device tables would have to be allocated
        assert _c_call("tide_rs_bf16_to_fp32_noalloc", L, grads, shards, Launch(), stream) == TIDE_ERR_INVALID
        L.prepare()
        # a table beyond the scratch array: C*P + R > TIDE_NOALLOC_MAX_PTRS (aliased contributors)
        many = [grads[0]] * (TIDE_NOALLOC_MAX_PTRS // len(shapes) + 1)
        assert _c_call("tide_rs_bf16_to_fp32_noalloc", L, many, shards, Launch(), stream) == TIDE_ERR_INVALID
        with pytest.raises(TideError, match="exceed"):
            tide_rs_bf16_to_fp32_noalloc(L.handle, many, shards, Launch(), stream)
        stream.synchronize()
        assert all(bool((s.view(torch.int32) == s.view(torch.int32)[0]).all()) for s in shards)  # untouched
        assert _c_call("tide_rs_bf16_to_fp32_noalloc", L, grads, shards, Launch(), stream) == TIDE_OK
        stream.synchronize()
        got = np.stack([host_bits_f32(s) for s in shards])
        assert np.array_equal(got, oracle.reduce_scatter(bits, shapes, R).view(np.uint32))
