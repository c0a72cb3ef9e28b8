"""ctypes binding of libtide.so (include/tide.h).  Argument marshalling only.

Every entry point of the C ABI is exposed under its own name; :class:`Layout` wraps a layout
handle for convenience.  Tensors are torch tensors on the current HIP device (torch provides the
device memory and the stream); the binding passes their data pointers and the stream handle and
raises :class:`TideError` on any non-OK status.  There is no fallback: if the library is missing,
every call raises.
"""
from __future__ import annotations

import ctypes
import os
import weakref
from typing import NamedTuple, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libtide.so"

TIDE_OK = 0
TIDE_ERR_INVALID = 1
TIDE_ERR_NOMEM = 2
TIDE_ERR_HIP = 3
TIDE_ERR_UNSUPPORTED = 4
TIDE_AG_KERNEL = 0
TIDE_AG_SDMA = 1
TIDE_AG_COPY2D = 2
TIDE_LAUNCH_DEFAULT = 0
TIDE_LAUNCH_BOUNDED = 1
TIDE_LAUNCH_CU_EXCLUSIVE = 2
TIDE_LAUNCH_PER_CU_CAP = 3
TIDE_MAX_WGS_PER_CU = 64
TIDE_CU_EXCLUSIVE_MAX_ITEMS = 16
TIDE_NOALLOC_MAX_PTRS = 65536


class Launch(NamedTuple):
    """A launch form and its count (include/tide.h tide_launch_form): how many of the library's
    workgroups are resident at once and how long each lives.  Never changes a result."""

    form: int = TIDE_LAUNCH_DEFAULT
    count: int = 0

    @staticmethod
    def default() -> "Launch":
        """The library's choice (RS: CU-exclusive workgroups shaped for C)."""
        return Launch(TIDE_LAUNCH_DEFAULT, 0)

    @staticmethod
    def bounded(budget: int) -> "Launch":
        """Launches of at most 256*budget resident threads, short-lived workgroups."""
        if int(budget) < 1:
            raise ValueError(f"a bounded launch needs a budget >= 1, got {budget}")
        return Launch(TIDE_LAUNCH_BOUNDED, int(budget))

    @staticmethod
    def cu_exclusive(items: int) -> "Launch":
        """One launch of workgroups that hold a whole CU each and take `items` work items."""
        n = int(items)
        if not (1 <= n <= 8 or n == 16):
            raise ValueError(f"CU-exclusive workgroups take 1..8 or 16 items, got {n}")
        return Launch(TIDE_LAUNCH_CU_EXCLUSIVE, n)

    @staticmethod
    def per_cu_cap(n: int) -> "Launch":
        """RS only: one launch of single-item workgroups, at most n of them per CU."""
        if not 1 <= int(n) <= TIDE_MAX_WGS_PER_CU:
            raise ValueError(f"a per-CU cap must be 1..{TIDE_MAX_WGS_PER_CU}, got {n}")
        return Launch(TIDE_LAUNCH_PER_CU_CAP, int(n))

    def __str__(self):
        names = {TIDE_LAUNCH_DEFAULT: "default", TIDE_LAUNCH_BOUNDED: "bounded",
                 TIDE_LAUNCH_CU_EXCLUSIVE: "cu_exclusive", TIDE_LAUNCH_PER_CU_CAP: "per_cu_cap"}
        name = names.get(self.form, f"form{self.form}")
        return name if self.form == TIDE_LAUNCH_DEFAULT else f"{name}({self.count})"


DEFAULT = Launch()


def _launch(launch) -> Launch:
    if launch is None:
        return DEFAULT
    if not isinstance(launch, tuple) or len(launch) != 2:
        raise TypeError(f"launch must be a Launch (form, count), got {launch!r}")
    return Launch(int(launch[0]), int(launch[1]))


_lib = None


class TideError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0, detail: str = ""):
        self.status = status
        self.hip_error = hip_error
        name = _lib.tide_status_str(status).decode() if _lib is not None else str(status)
        extra = f" (hipError {hip_error})" if hip_error else ""
        extra += f": {detail}" if detail else ""
        super().__init__(f"{where}: {name}{extra}")


def library_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load_library(path: str | None = None):
    """Load libtide.so (once).  Raises if it is not built: there is no other implementation."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m all_gather_placement_amd.build`")
    lib = ctypes.CDLL(path)
    if path == library_path():
        # a library built from other sources than the ones beside it is refused, never run
        from .build import LIB, check_current

        check_current(LIB, loaded=lib)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    P_i32, P_i64 = ctypes.POINTER(i32), ctypes.POINTER(i64)
    sig = {
        "tide_layout_create": (i32, [i32, P_i32, P_i64, i32, ctypes.POINTER(vp)]),
        "tide_layout_destroy": (None, [vp]),
        "tide_layout_prepare": (i32, [vp]),
        "tide_layout_num_params": (i32, [vp]),
        "tide_layout_num_ranks": (i32, [vp]),
        "tide_layout_shard_numel": (i64, [vp]),
        "tide_layout_num_rs_chunks": (i64, [vp]),
        "tide_layout_num_ag_chunks": (i64, [vp]),
        "tide_layout_param": (i32, [vp, i32, P_i64, P_i64, P_i64, P_i64]),
        "tide_layout_segment": (i32, [vp, i32, i32, P_i64, P_i64, P_i64, P_i64]),
        "tide_rs_bf16_to_fp32": (i32, [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32, vp]),
        "tide_rs_bf16_to_fp32_noalloc": (i32, [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32, vp]),
        "tide_ag_place": (i32, [vp, vp, ctypes.POINTER(vp), i32, i32, i32, vp]),
        "tide_layout_copy_rs_items": (i32, [vp, i64, i64, P_i64]),
        "tide_layout_copy_ag_items": (i32, [vp, i64, i64, P_i64]),
        "tide_slot_pack": (i32, [vp, ctypes.POINTER(vp), vp, i32, i32, vp]),
        "tide_rs_slots_bf16_to_fp32": (i32, [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32, vp]),
        "tide_layout_num_slot_pad_items": (i64, [vp]),
        "tide_layout_copy_slot_pad_items": (i32, [vp, i64, i64, P_i64]),
        "tide_rs_prepare": (i32, [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32, ctypes.POINTER(vp)]),
        "tide_ag_prepare": (i32, [vp, vp, ctypes.POINTER(vp), i32, i32, i32, ctypes.POINTER(vp)]),
        "tide_slot_pack_prepare": (i32, [vp, ctypes.POINTER(vp), vp, i32, i32, ctypes.POINTER(vp)]),
        "tide_rs_slots_prepare": (i32, [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32,
                                        ctypes.POINTER(vp)]),
        "tide_call_launch": (i32, [vp, vp]),
        "tide_call_destroy": (None, [vp]),
        "tide_rs_launch_shape": (i32, [i32, i32, i32, P_i32, P_i32, P_i32, P_i32]),
        "tide_status_str": (ctypes.c_char_p, [i32]),
        "tide_last_hip_error": (i32, []),
        "tide_build_id": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == library_path():
        _lib = lib
    return lib


def _check(status: int, where: str):
    if status != TIDE_OK:
        hip = _lib.tide_last_hip_error() if status in (TIDE_ERR_HIP, TIDE_ERR_UNSUPPORTED) else 0
        raise TideError(status, where, hip)


def _ptr(x) -> int | None:
    """Device address of a torch tensor (or a raw int address); None for None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _expect_counts(layout: int, where: str, rows=None, per_param=None, per_rank=None):
    """The C entry points read host pointer arrays of exactly the sizes the layout implies (C*P, P,
    R); check the Python sequences before handing them over, so no array is read past its end."""
    lib = load_library()
    P, R = lib.tide_layout_num_params(layout), lib.tide_layout_num_ranks(layout)
    bad = []
    if rows is not None:
        if len(rows) < 1:
            bad.append("no contributors")
        bad += [f"contributor {c} has {len(r)} tensors, the layout has {P} parameters"
                for c, r in enumerate(rows) if len(r) != P]
    if per_param is not None and len(per_param) != P:
        bad.append(f"{len(per_param)} tensors for {P} parameters")
    if per_rank is not None and len(per_rank) != R:
        bad.append(f"{len(per_rank)} shards for {R} ranks")
    if bad:
        raise TideError(TIDE_ERR_INVALID, where, 0, "; ".join(bad[:3]))


def _stream_handle(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------------------------------------
# Entry points under their C names
# ------------------------------------------------------------------------------------------------

def tide_layout_create(shapes: Sequence[Sequence[int]], R: int) -> int:
    """Create a layout for parameter shapes over R ranks; returns the raw handle."""
    lib = load_library()
    shapes = [tuple(int(d) for d in s) for s in shapes]
    P = len(shapes)
    ndims = (ctypes.c_int32 * max(P, 1))(*[len(s) for s in shapes])
    flat = [d for s in shapes for d in s]
    dims = (ctypes.c_int64 * max(len(flat), 1))(*flat)
    out = ctypes.c_void_p()
    _check(lib.tide_layout_create(P, ndims, dims, int(R), ctypes.byref(out)), "tide_layout_create")
    return out.value


def tide_rs_bf16_to_fp32(layout: int, grads, shards, launch: Launch = DEFAULT, stream=None):
    """grads: C lists of P bf16 tensors (or addresses); shards: R fp32 tensors (or addresses)."""
    lib = load_library()
    _expect_counts(layout, "tide_rs_bf16_to_fp32", rows=grads, per_rank=shards)
    C = len(grads)
    flat = [_ptr(g) for row in grads for g in row]
    g_arr = (ctypes.c_void_p * max(len(flat), 1))(*flat)
    s_list = [_ptr(s) for s in shards]
    s_arr = (ctypes.c_void_p * max(len(s_list), 1))(*s_list)
    _check(lib.tide_rs_bf16_to_fp32(layout, C, g_arr, s_arr, *_launch(launch), _stream_handle(stream)),
           "tide_rs_bf16_to_fp32")


def tide_rs_bf16_to_fp32_noalloc(layout: int, grads, shards, launch: Launch = DEFAULT, stream=None):
    """As tide_rs_bf16_to_fp32, allocating nothing: the address table goes into the library's fixed
    per-device scratch array (at most TIDE_NOALLOC_MAX_PTRS = C*P + R pointers); the layout must have
    been prepared on the current device.  Calls that overlap on one device race on that array."""
    lib = load_library()
    _expect_counts(layout, "tide_rs_bf16_to_fp32_noalloc", rows=grads, per_rank=shards)
    C = len(grads)
    flat = [_ptr(g) for row in grads for g in row]
    n = len(flat) + len(shards)
    if n > TIDE_NOALLOC_MAX_PTRS:
        raise TideError(TIDE_ERR_INVALID, "tide_rs_bf16_to_fp32_noalloc", 0,
                        f"C*P + R = {n} pointers exceed the scratch table's {TIDE_NOALLOC_MAX_PTRS}")
    g_arr = (ctypes.c_void_p * max(len(flat), 1))(*flat)
    s_list = [_ptr(s) for s in shards]
    s_arr = (ctypes.c_void_p * max(len(s_list), 1))(*s_list)
    _check(lib.tide_rs_bf16_to_fp32_noalloc(layout, C, g_arr, s_arr, *_launch(launch), _stream_handle(stream)),
           "tide_rs_bf16_to_fp32_noalloc")


def tide_ag_place(layout: int, stage, params, mode: int = TIDE_AG_KERNEL, launch: Launch = DEFAULT, stream=None):
    """stage: R*S bf16 tensor (or address); params: P bf16 tensors (or addresses)."""
    lib = load_library()
    _expect_counts(layout, "tide_ag_place", per_param=params)
    p_list = [_ptr(p) for p in params]
    p_arr = (ctypes.c_void_p * max(len(p_list), 1))(*p_list)
    _check(lib.tide_ag_place(layout, _ptr(stage), p_arr, int(mode), *_launch(launch), _stream_handle(stream)),
           "tide_ag_place")


def tide_slot_pack(layout: int, grads, slot, launch: Launch = DEFAULT, stream=None):
    """grads: P bf16 tensors of one contributor (or addresses); slot: R*S bf16 tensor (or address)."""
    lib = load_library()
    _expect_counts(layout, "tide_slot_pack", per_param=grads)
    g_list = [_ptr(g) for g in grads]
    g_arr = (ctypes.c_void_p * max(len(g_list), 1))(*g_list)
    _check(lib.tide_slot_pack(layout, g_arr, _ptr(slot), *_launch(launch), _stream_handle(stream)), "tide_slot_pack")


def tide_rs_slots_bf16_to_fp32(layout: int, slots, shards, launch: Launch = DEFAULT, stream=None):
    """slots: C packed R*S bf16 tensors (or addresses); shards: R fp32 tensors (or addresses)."""
    lib = load_library()
    _expect_counts(layout, "tide_rs_slots_bf16_to_fp32", per_rank=shards)
    sl = [_ptr(x) for x in slots]
    sl_arr = (ctypes.c_void_p * max(len(sl), 1))(*sl)
    sh = [_ptr(x) for x in shards]
    sh_arr = (ctypes.c_void_p * max(len(sh), 1))(*sh)
    _check(lib.tide_rs_slots_bf16_to_fp32(layout, len(sl), sl_arr, sh_arr, *_launch(launch), _stream_handle(stream)),
           "tide_rs_slots_bf16_to_fp32")


def _ptr_array(xs):
    xs = [_ptr(x) for x in xs]
    return (ctypes.c_void_p * max(len(xs), 1))(*xs)


def tide_rs_prepare(layout: int, grads, shards, launch: Launch = DEFAULT) -> int:
    """Prepared RS call (see tide_call_launch); returns the raw tide_call handle."""
    lib = load_library()
    _expect_counts(layout, "tide_rs_prepare", rows=grads, per_rank=shards)
    out = ctypes.c_void_p()
    _check(lib.tide_rs_prepare(layout, len(grads), _ptr_array([g for row in grads for g in row]),
                               _ptr_array(shards), *_launch(launch), ctypes.byref(out)), "tide_rs_prepare")
    return out.value


def tide_ag_prepare(layout: int, stage, params, mode: int = TIDE_AG_KERNEL, launch: Launch = DEFAULT) -> int:
    lib = load_library()
    _expect_counts(layout, "tide_ag_prepare", per_param=params)
    out = ctypes.c_void_p()
    _check(lib.tide_ag_prepare(layout, _ptr(stage), _ptr_array(params), int(mode), *_launch(launch), ctypes.byref(out)),
           "tide_ag_prepare")
    return out.value


def tide_slot_pack_prepare(layout: int, grads, slot, launch: Launch = DEFAULT) -> int:
    lib = load_library()
    _expect_counts(layout, "tide_slot_pack_prepare", per_param=grads)
    out = ctypes.c_void_p()
    _check(lib.tide_slot_pack_prepare(layout, _ptr_array(grads), _ptr(slot), *_launch(launch), ctypes.byref(out)),
           "tide_slot_pack_prepare")
    return out.value


def tide_rs_slots_prepare(layout: int, slots, shards, launch: Launch = DEFAULT) -> int:
    lib = load_library()
    _expect_counts(layout, "tide_rs_slots_prepare", per_rank=shards)
    out = ctypes.c_void_p()
    _check(lib.tide_rs_slots_prepare(layout, len(slots), _ptr_array(slots), _ptr_array(shards), *_launch(launch),
                                     ctypes.byref(out)), "tide_rs_slots_prepare")
    return out.value


def tide_call_launch(call: int, stream=None):
    _check(load_library().tide_call_launch(call, _stream_handle(stream)), "tide_call_launch")


def tide_call_destroy(call: int):
    load_library().tide_call_destroy(call)


def tide_rs_launch_shape(C: int = 8, launch: Launch = DEFAULT) -> dict:
    """RS launch shape for C contributors in a launch form on the current device: threads,
    items_per_workgroup, item_outputs, lds_bytes."""
    v = [ctypes.c_int32() for _ in range(4)]
    _check(load_library().tide_rs_launch_shape(int(C), *_launch(launch), *[ctypes.byref(x) for x in v]),
           "tide_rs_launch_shape")
    return dict(zip(("threads", "items_per_workgroup", "item_outputs", "lds_bytes"), (x.value for x in v)))


class Layout:
    """Owning wrapper of a tide_layout handle for one parameter group over R ranks."""

    def __init__(self, shapes: Sequence[Sequence[int]], R: int):
        self._lib = load_library()
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        self.R = int(R)
        self.handle = tide_layout_create(self.shapes, self.R)
        self.P = self._lib.tide_layout_num_params(self.handle)
        self.S = self._lib.tide_layout_shard_numel(self.handle)
        self._calls = weakref.WeakSet()  # prepared calls made from this layout

    def close(self):
        """Free the layout.  Prepared calls made from it are closed first (they address its
        tables), so launching one afterwards raises instead of touching freed memory."""
        if getattr(self, "handle", None):
            for call in list(getattr(self, "_calls", ())):
                call.close()
            self._lib.tide_layout_destroy(self.handle)
            self.handle = None

    def _bound(self, handle: int, keep) -> "BoundCall":
        call = BoundCall(handle, keep)
        self._calls.add(call)
        return call

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # geometry --------------------------------------------------------------------------------
    def param(self, p: int):
        """(rows_p, L_p, m_p, o_p)."""
        v = [ctypes.c_int64() for _ in range(4)]
        _check(self._lib.tide_layout_param(self.handle, int(p), *[ctypes.byref(x) for x in v]), "tide_layout_param")
        return tuple(x.value for x in v)

    def segment(self, p: int, r: int):
        """(src_offset, valid, dst_offset, pad) of rank r's slice of parameter p."""
        v = [ctypes.c_int64() for _ in range(4)]
        _check(self._lib.tide_layout_segment(self.handle, int(p), int(r), *[ctypes.byref(x) for x in v]),
               "tide_layout_segment")
        return tuple(x.value for x in v)

    @property
    def num_rs_chunks(self) -> int:
        return self._lib.tide_layout_num_rs_chunks(self.handle)

    @property
    def num_ag_chunks(self) -> int:
        return self._lib.tide_layout_num_ag_chunks(self.handle)

    def rs_items(self):
        """RS work items as an (n, 6) int64 array: p, r, src_offset, dst_offset, nvalid, npad."""
        import numpy as np

        n = self.num_rs_chunks
        out = np.zeros((max(n, 1), 6), dtype=np.int64)
        _check(self._lib.tide_layout_copy_rs_items(self.handle, 0, n, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
               "tide_layout_copy_rs_items")
        return out[:n]

    def ag_items(self):
        """AG work items as an (n, 4) int64 array: p, stage_offset, param_offset, n."""
        import numpy as np

        n = self.num_ag_chunks
        out = np.zeros((max(n, 1), 4), dtype=np.int64)
        _check(self._lib.tide_layout_copy_ag_items(self.handle, 0, n, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
               "tide_layout_copy_ag_items")
        return out[:n]

    def slot_pad_items(self):
        """Padding ranges of a packed slot as an (n, 2) int64 array: slot offset, count."""
        import numpy as np

        n = self._lib.tide_layout_num_slot_pad_items(self.handle)
        out = np.zeros((max(n, 1), 2), dtype=np.int64)
        _check(self._lib.tide_layout_copy_slot_pad_items(self.handle, 0, n,
                                                         out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
               "tide_layout_copy_slot_pad_items")
        return out[:n]

    def prepare(self):
        _check(self._lib.tide_layout_prepare(self.handle), "tide_layout_prepare")

    # collectives -----------------------------------------------------------------------------
    def rs_bf16_to_fp32(self, grads, shards, launch: Launch = DEFAULT, stream=None):
        _check_shapes_rs(self, grads, shards)
        tide_rs_bf16_to_fp32(self.handle, grads, shards, launch, stream)

    def ag_place(self, stage, params, mode: int = TIDE_AG_KERNEL, launch: Launch = DEFAULT, stream=None):
        _check_shapes_ag(self, stage, params)
        tide_ag_place(self.handle, stage, params, mode, launch, stream)

    # prepared calls (validate once, launch many times; graph-capturable kernel paths) ---------
    def bind_rs(self, grads, shards, launch: Launch = DEFAULT) -> BoundCall:
        _check_shapes_rs(self, grads, shards)
        return self._bound(tide_rs_prepare(self.handle, grads, shards, launch), (grads, shards, self))

    def bind_ag(self, stage, params, mode: int = TIDE_AG_KERNEL, launch: Launch = DEFAULT) -> BoundCall:
        _check_shapes_ag(self, stage, params)
        return self._bound(tide_ag_prepare(self.handle, stage, params, mode, launch), (stage, params, self))

    def bind_slot_pack(self, grads, slot, launch: Launch = DEFAULT) -> BoundCall:
        _check_shapes_ag(self, slot, grads)
        return self._bound(tide_slot_pack_prepare(self.handle, grads, slot, launch), (grads, slot, self))

    def bind_rs_slots(self, slots, shards, launch: Launch = DEFAULT) -> BoundCall:
        _check_shapes_rs(self, [], shards)
        for sl in slots:
            _check_stage(self, sl)
        return self._bound(tide_rs_slots_prepare(self.handle, slots, shards, launch), (slots, shards, self))

    def slot_pack(self, grads, slot, launch: Launch = DEFAULT, stream=None):
        _check_shapes_ag(self, slot, grads)
        tide_slot_pack(self.handle, grads, slot, launch, stream)

    def rs_slots_bf16_to_fp32(self, slots, shards, launch: Launch = DEFAULT, stream=None):
        _check_shapes_rs(self, [], shards)
        for sl in slots:
            _check_stage(self, sl)
        tide_rs_slots_bf16_to_fp32(self.handle, slots, shards, launch, stream)


class BoundCall:
    """Owner of a prepared call (tide_call): checked and uploaded once, each launch() is one ctypes
    call that only enqueues work.  Keeps references to the tensors and the layout so that their
    memory outlives the call."""

    def __init__(self, handle: int, keep):
        self._lib = load_library()
        self.handle = handle
        self._keep = keep

    def launch(self, stream=None):
        if not self.handle:
            raise TideError(TIDE_ERR_INVALID, "tide_call_launch", 0, "the call or its layout was closed")
        _check(self._lib.tide_call_launch(self.handle, _stream_handle(stream)), "tide_call_launch")

    def close(self):
        """Free the call (the library waits for the device's queued work first)."""
        if getattr(self, "handle", None):
            self._lib.tide_call_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _is_tensor(x) -> bool:
    return hasattr(x, "data_ptr") and hasattr(x, "dtype")


def _check_device(tensors):
    """Every tensor argument on the current device: the library launches there, so an address on
    another device would reach its kernels as a foreign pointer."""
    import torch

    devs = {t.device.index for t in tensors if _is_tensor(t)}
    if not devs:
        return
    cur = torch.cuda.current_device() if torch.cuda.is_available() else None
    if len(devs) > 1 or (cur is not None and devs != {cur}):
        raise ValueError(f"all tensors must be on the current device (cuda:{cur}); got devices {sorted(devs)}")


def _check_shapes_rs(L: Layout, grads, shards):
    """Host-side shape/dtype/device checks of torch arguments (the C ABI sees only addresses)."""
    import torch

    _check_device([g for row in grads for g in row] + list(shards))

    if len(shards) != L.R:
        raise ValueError(f"expected {L.R} shards, got {len(shards)}")
    for row in grads:
        if len(row) != L.P:
            raise ValueError(f"each contributor needs {L.P} gradients, got {len(row)}")
        for g, shape in zip(row, L.shapes):
            if _is_tensor(g):
                if g.dtype != torch.bfloat16 or not g.is_cuda or not g.is_contiguous() or tuple(g.shape) != shape:
                    raise ValueError(f"gradient must be a contiguous cuda bf16 tensor of shape {shape}")
    for s in shards:
        if _is_tensor(s):
            if s.dtype != torch.float32 or not s.is_cuda or not s.is_contiguous() or s.numel() != L.S:
                raise ValueError(f"shard must be a contiguous cuda fp32 tensor of {L.S} elements")


def _check_stage(L: Layout, stage):
    import torch

    _check_device([stage])

    if _is_tensor(stage):
        if stage.dtype != torch.bfloat16 or not stage.is_cuda or not stage.is_contiguous() or stage.numel() != L.R * L.S:
            raise ValueError(f"stage/slot must be a contiguous cuda bf16 tensor of R*S = {L.R * L.S} elements")


def _check_shapes_ag(L: Layout, stage, params):
    import torch

    if len(params) != L.P:
        raise ValueError(f"expected {L.P} parameters, got {len(params)}")
    _check_device([stage] + list(params))
    _check_stage(L, stage)
    for q, shape in zip(params, L.shapes):
        if _is_tensor(q):
            if q.dtype != torch.bfloat16 or not q.is_cuda or not q.is_contiguous() or tuple(q.shape) != shape:
                raise ValueError(f"parameter must be a contiguous cuda bf16 tensor of shape {shape}")
