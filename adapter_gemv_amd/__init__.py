"""Python binding of ``liblora_gemv.so``, the gfx950 heterogeneous-adapter LoRA delta.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in ``include/lora_gemv.h``.  PyTorch provides device memory and the
stream (the current torch stream unless one is given).  There is no CPU path:
if the library is not built, importing the binding's functions raises.

The calls follow "m07 -- Multi-Adapter (LoRA) Serving", "6. Deep Dive A:
Batching Heterogeneous Adapters": the batch, an index vector mapping each row
to an adapter slot, and an adapter table read on the device.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "LoraError", "Segments", "segment_bound", "ModuleIO", "MODULES", "TABLE_ENTRY_DTYPE", "lib", "workspace_bytes",
    "build_segments", "shrink", "expand", "apply_layer", "apply_layer_noalloc", "decode_layer",
    "decode_layer_launches", "layer_shrink", "layer_expand", "pack_table", "STATIC_SCRATCH_BYTES",
    "status_string", "MAX_RANK", "host_lib", "LinearIO", "LinearQ4IO", "Q4_GROUP", "MASK_INT8_ITEMS", "module_mask",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblora_gemv.so")
MAX_RANK = 64
STATIC_SCRATCH_BYTES = 16 << 20  # LORA_STATIC_SCRATCH_BYTES
MODULES = ("q", "k", "v", "o", "gate", "up", "down")

# lora_adapter_entry_t, 32 bytes
TABLE_ENTRY_DTYPE = np.dtype([("A", "<u8"), ("B", "<u8"), ("rank", "<i4"), ("scale", "<f4"), ("format", "<i4"),
                              ("reserved", "<i4")])
FORMAT_BF16, FORMAT_INT8_ROWS = 0, 1  # lora_factor_format_t
assert TABLE_ENTRY_DTYPE.itemsize == 32


class LoraError(RuntimeError):
    pass


class _Seg(ctypes.Structure):
    _fields_ = [("perm", ctypes.c_void_p), ("seg_offsets", ctypes.c_void_p), ("seg_adapter", ctypes.c_void_p),
                ("num_segments", ctypes.c_void_p), ("tile_counts", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("max_segments", ctypes.c_int32)]


class _IO(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("ldx", ctypes.c_int64), ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64),
                ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32)]


class _LinIO(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("ldx", ctypes.c_int64), ("W", ctypes.c_void_p), ("ldw", ctypes.c_int64),
                ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64), ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32)]


class _LinQ4IO(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("ldx", ctypes.c_int64), ("Wq", ctypes.c_void_p), ("ldwq", ctypes.c_int64),
                ("Ws", ctypes.c_void_p), ("lds", ctypes.c_int64), ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64),
                ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LoraError(f"{LIB_PATH} is missing: build it with `python -m adapter_gemv_amd.build` "
                            "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        st, i32, i64, u32, vp, sz = (ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                     ctypes.c_void_p, ctypes.c_size_t)
        L.lora_workspace_bytes.restype = sz
        L.lora_workspace_bytes.argtypes = [i32, i32, i32, i64]
        L.lora_status_string.restype = ctypes.c_char_p
        L.lora_status_string.argtypes = [st]
        L.lora_build_segments.restype = st
        L.lora_build_segments.argtypes = [vp, i32, i32, _Seg, vp, sz, vp]
        L.lora_shrink.restype = st
        L.lora_shrink.argtypes = [vp, i64, i32, i32, vp, i32, i32, i32, _Seg, i32, vp, i64, vp, sz, vp]
        L.lora_expand.restype = st
        L.lora_expand.argtypes = [vp, i64, i32, i32, vp, i32, i32, i32, _Seg, i32, vp, i64, vp, sz, vp]
        for name in ("lora_apply_layer", "lora_layer_shrink", "lora_layer_expand"):
            f = getattr(L, name)
            f.restype = st
            f.argtypes = [ctypes.POINTER(_IO), u32, i32, vp, i32, _Seg, i32, vp, sz, vp]
        L.lora_decode_layer.restype = st
        L.lora_decode_layer.argtypes = [ctypes.POINTER(_IO), u32, i32, vp, vp, i32, _Seg, i32, vp, sz, vp]
        L.lora_decode_layer_launches.restype = i32
        L.lora_decode_layer_launches.argtypes = [ctypes.POINTER(_IO), u32, i32, i32, _Seg, i32]
        L.lora_apply_layer_noalloc.restype = st
        L.lora_apply_layer_noalloc.argtypes = [ctypes.POINTER(_IO), u32, i32, vp, i32, _Seg, i32, vp]
        L.lora_apply_layer_stacked.restype = st
        L.lora_apply_layer_stacked.argtypes = [ctypes.POINTER(_IO), u32, i32, vp, i32, vp, vp, i32, _Seg, i32, vp, sz,
                                               vp]
        L.lora_linear_workspace_bytes.restype = sz
        L.lora_linear_workspace_bytes.argtypes = [i32, i32, i32, i64, i32]
        for name in ("lora_linear_layer", "lora_linear_shrink", "lora_linear_expand"):
            f = getattr(L, name)
            f.restype = st
            f.argtypes = [ctypes.POINTER(_LinIO), u32, i32, vp, vp, i32, _Seg, i32, vp, sz, vp]
        for name in ("lora_linear_layer_q4", "lora_linear_shrink_q4", "lora_linear_expand_q4"):
            f = getattr(L, name)
            f.restype = st
            f.argtypes = [ctypes.POINTER(_LinQ4IO), u32, i32, vp, vp, i32, _Seg, i32, vp, sz, vp]
        L.lora_form_batch.restype = st
        L.lora_form_batch.argtypes = [vp, i32, vp, ctypes.c_float, i32, i32, i32, i32, vp, vp]
        _lib = L
    return _lib


_host = None


def host_lib() -> ctypes.CDLL:
    """The library of the host-only calls (lora_form_batch, lora_status_string):
    liblora_gemv.so, or with LORA_SANITIZE=1 in the environment their
    AddressSanitizer + UndefinedBehaviorSanitizer build liblora_host_san.so
    (``python -m adapter_gemv_amd.build --sanitize``; the process must have
    the sanitizer runtime preloaded)."""
    global _host
    if _host is None:
        if os.environ.get("LORA_SANITIZE") != "1":
            return lib()
        path = os.path.join(HERE, "liblora_host_san.so")
        if not os.path.exists(path):
            raise LoraError(f"{path} is missing: build it with `python -m adapter_gemv_amd.build --sanitize`")
        L = ctypes.CDLL(path)
        L.lora_status_string.restype = ctypes.c_char_p
        L.lora_status_string.argtypes = [ctypes.c_int]
        L.lora_form_batch.restype = ctypes.c_int
        L.lora_form_batch.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p]
        _host = L
    return _host


def status_string(code: int) -> str:
    return host_lib().lora_status_string(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise LoraError(f"{what}: {status_string(code)}")


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, what, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{what} must be on the GPU")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{what} must have {ndim} dims")
    if t.dim() >= 1 and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{what} must have unit stride in its last dim")


class Segments:
    """Device buffers of lora_segments_t for batches of up to ``num_rows`` rows.

    ``max_segments`` (host, 0 = none) bounds the segments of a build: the
    number of distinct valid adapter ids of the batch, which the host that
    formed the batch knows (see ``segment_bound``).  The calls size their
    work items for it; a build with more segments drops those of the highest
    slots and counts their rows into the status word."""

    def __init__(self, num_rows: int, device="cuda", max_segments: int = 0):
        import torch
        n = max(int(num_rows), 1)
        i32 = dict(dtype=torch.int32, device=device)
        self.num_rows = int(num_rows)
        self.max_segments = int(max_segments)
        self.perm = torch.zeros(n, **i32)
        self.seg_offsets = torch.zeros(n + 1, **i32)
        self.seg_adapter = torch.zeros(n, **i32)
        self.num_segments = torch.zeros(1, **i32)
        self.tile_counts = torch.zeros(2, **i32)
        self.status = torch.zeros(1, **i32)

    def c(self) -> _Seg:
        if self.max_segments < 0:
            raise ValueError("max_segments must be >= 0")
        return _Seg(self.perm.data_ptr(), self.seg_offsets.data_ptr(), self.seg_adapter.data_ptr(),
                    self.num_segments.data_ptr(), self.tile_counts.data_ptr(), self.status.data_ptr(),
                    self.max_segments)

    def host(self):
        """(perm, seg_offsets, seg_adapter, status) copied to the host (synchronises)."""
        ns = int(self.num_segments.item())
        offs = self.seg_offsets[:ns + 1].cpu().numpy()
        return (self.perm[:int(offs[-1])].cpu().numpy(), offs, self.seg_adapter[:ns].cpu().numpy(),
                int(self.status.item()))


def segment_bound(row_adapter, num_slots: int) -> int:
    """Host ids (any int array, one per row; for several adapters per row, a
    [rows, depth] array: the most over the columns) -> the distinct valid
    slots, the tightest ``Segments.max_segments`` for a batch (0 when it has
    none)."""
    import numpy as np
    ids = np.asarray(row_adapter)
    if ids.size == 0:
        return 0
    cols = ids.reshape(ids.shape[0], -1).T if ids.ndim > 1 else ids[None]
    return max((int(np.unique(c[(c >= 0) & (c < num_slots)]).size) for c in cols), default=0)


class ModuleIO:
    """One projection for the layer calls: x [rows, >= d_in], y [rows, >= d_out], bf16."""

    def __init__(self, x, y, d_in=None, d_out=None):
        self.x, self.y = x, y
        self.d_in = int(x.shape[1] if d_in is None else d_in)
        self.d_out = int(y.shape[1] if d_out is None else d_out)


def workspace_bytes(num_rows: int, num_slots: int, max_rank: int, sum_d_in: int) -> int:
    return int(lib().lora_workspace_bytes(num_rows, num_slots, max_rank, sum_d_in))


class LinearIO:
    """One projection for linear_layer: x [rows, >= d_in], W [d_out, >= d_in]
    (the base weight), y [rows, >= d_out] (written), bf16."""

    def __init__(self, x, W, y, d_in=None, d_out=None):
        self.x, self.W, self.y = x, W, y
        self.d_in = int(x.shape[1] if d_in is None else d_in)
        self.d_out = int(W.shape[0] if d_out is None else d_out)


Q4_GROUP = 128  # LORA_Q4_GROUP


class LinearQ4IO:
    """One projection for linear_layer_q4: x [rows, >= d_in] bf16, Wq uint8
    [d_out, >= d_in / 2] (packed signed 4-bit weights, the even input in the
    low nibble), Ws float32 [d_out, >= d_in / Q4_GROUP] (group scales), y
    [rows, >= d_out] bf16 (written)."""

    def __init__(self, x, Wq, Ws, y, d_in=None, d_out=None):
        self.x, self.Wq, self.Ws, self.y = x, Wq, Ws, y
        self.d_in = int(x.shape[1] if d_in is None else d_in)
        self.d_out = int(Wq.shape[0] if d_out is None else d_out)


def linear_workspace_bytes(num_rows: int, num_slots: int, max_rank: int, sum_d_in: int, n_modules: int) -> int:
    return int(lib().lora_linear_workspace_bytes(num_rows, num_slots, max_rank, sum_d_in, n_modules))


def linear_layer(ios, num_rows, row_adapter, table, num_slots, seg, max_rank, ws, stream=None, module_mask=None,
                 _fn="lora_linear_layer"):
    """Base projection + delta of every projection in ``ios`` ({name:
    LinearIO}, or {name: LinearQ4IO} for 4-bit base weights); see
    lora_linear_layer and lora_linear_layer_q4."""
    import torch
    _need(row_adapter, torch.int32, "row_adapter", 1)
    q4 = any(isinstance(io, LinearQ4IO) for io in ios.values())
    arr = ((_LinQ4IO if q4 else _LinIO) * 7)()
    mask = 0
    for i, name in enumerate(MODULES):
        io = ios.get(name)
        if io is None:
            continue
        if isinstance(io, LinearQ4IO) != q4:
            raise TypeError("linear_layer: every projection LinearIO, or every projection LinearQ4IO")
        for t, what in ((io.x, "x"), (io.y, "y")) + (() if q4 else ((io.W, "W"),)):
            _need(t, torch.bfloat16, f"{name}.{what}", 2)
        if io.x.shape[0] < num_rows or io.y.shape[0] < num_rows:
            raise ValueError(f"{name}: fewer rows than num_rows")
        if q4:
            _need(io.Wq, torch.uint8, f"{name}.Wq", 2)
            _need(io.Ws, torch.float32, f"{name}.Ws", 2)
            arr[i] = _LinQ4IO(io.x.data_ptr(), io.x.stride(0), io.Wq.data_ptr(), io.Wq.stride(0), io.Ws.data_ptr(),
                              io.Ws.stride(0), io.y.data_ptr(), io.y.stride(0), io.d_in, io.d_out)
        else:
            arr[i] = _LinIO(io.x.data_ptr(), io.x.stride(0), io.W.data_ptr(), io.W.stride(0), io.y.data_ptr(),
                            io.y.stride(0), io.d_in, io.d_out)
        mask |= 1 << i
    if q4:
        _fn += "_q4"
    _check(getattr(lib(), _fn)(arr, mask if module_mask is None else module_mask, num_rows, _ptr(row_adapter),
                               _ptr(table), num_slots, seg.c(), max_rank, _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)), _fn)


def linear_shrink(*args, **kw):
    """The shrink part of linear_layer (v per row and projection into ws)."""
    linear_layer(*args, _fn="lora_linear_shrink", **kw)


def linear_expand(*args, **kw):
    """The fused part of linear_layer (W.x + delta into y), after linear_shrink."""
    linear_layer(*args, _fn="lora_linear_expand", **kw)


def pack_table(A_ptrs, B_ptrs, ranks, scales, formats=None) -> np.ndarray:
    """Host bytes of a table of lora_adapter_entry_t; arrays of shape [num_slots, n_mod]
    (formats: FORMAT_BF16 where omitted)."""
    ranks = np.asarray(ranks)
    t = np.zeros(ranks.shape, TABLE_ENTRY_DTYPE)
    t["A"] = np.asarray(A_ptrs, np.uint64)
    t["B"] = np.asarray(B_ptrs, np.uint64)
    t["rank"] = ranks.astype(np.int32)
    t["scale"] = np.asarray(scales, np.float32)
    if formats is not None:
        t["format"] = np.asarray(formats, np.int32)
    return t


def build_segments(row_adapter, num_slots: int, seg: Segments, ws, stream=None):
    """Group rows by adapter slot (stable); see lora_build_segments."""
    import torch
    _need(row_adapter, torch.int32, "row_adapter", 1)
    n = row_adapter.shape[0]
    if n > seg.num_rows:
        raise ValueError("Segments buffers too small for this batch")
    _check(lib().lora_build_segments(_ptr(row_adapter), n, num_slots, seg.c(), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)), "lora_build_segments")


def shrink(x, table, num_slots: int, n_mod: int, module: int, seg: Segments, max_rank: int, v, ws, stream=None):
    """v[b, :rank] = A . x[b] for rows in a segment; see lora_shrink."""
    import torch
    _need(x, torch.bfloat16, "x", 2)
    _need(v, torch.float32, "v", 2)
    _check(lib().lora_shrink(_ptr(x), x.stride(0), x.shape[0], x.shape[1], _ptr(table), num_slots, n_mod, module,
                             seg.c(), max_rank, _ptr(v), v.stride(0), _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(stream)), "lora_shrink")


def expand(v, table, num_slots: int, n_mod: int, module: int, seg: Segments, max_rank: int, y, ws, stream=None):
    """y[b] = bf16(y[b] + scale * B . v[b]) for rows in a segment; see lora_expand."""
    import torch
    _need(v, torch.float32, "v", 2)
    _need(y, torch.bfloat16, "y", 2)
    _check(lib().lora_expand(_ptr(v), v.stride(0), y.shape[0], y.shape[1], _ptr(table), num_slots, n_mod, module,
                             seg.c(), max_rank, _ptr(y), y.stride(0), _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(stream)), "lora_expand")


def _ios(ios, num_rows):
    import torch
    arr = (_IO * 7)()
    mask = 0
    for i, name in enumerate(MODULES):
        io = ios.get(name) if isinstance(ios, dict) else (ios[i] if i < len(ios) else None)
        if io is None:
            continue
        _need(io.x, torch.bfloat16, f"{name}.x", 2)
        _need(io.y, torch.bfloat16, f"{name}.y", 2)
        if io.x.shape[0] < num_rows or io.y.shape[0] < num_rows:
            raise ValueError(f"{name}: fewer rows than num_rows")
        arr[i] = _IO(io.x.data_ptr(), io.x.stride(0), io.y.data_ptr(), io.y.stride(0), io.d_in, io.d_out)
        mask |= 1 << i
    return arr, mask


MASK_INT8_ITEMS = 1 << 16  # LORA_MASK_INT8_ITEMS


def module_mask(ios, int8_items: bool = False) -> int:
    """The module_mask of the projections in ``ios`` ({name: io}); with
    int8_items, LORA_MASK_INT8_ITEMS too (the table's entries are int8: the
    shrink's items are sized for one-byte factors)."""
    mask = 0
    for i, name in enumerate(MODULES):
        if name in ios:
            mask |= 1 << i
    return mask | (MASK_INT8_ITEMS if int8_items else 0)


def _layer(fn, what, ios, num_rows, table, num_slots, seg, max_rank, ws, stream, module_mask):
    arr, mask = _ios(ios, num_rows)
    if module_mask is None:
        module_mask = mask
    _check(fn(arr, module_mask, num_rows, _ptr(table), num_slots, seg.c(), max_rank, _ptr(ws),
              ws.numel() * ws.element_size(), _stream(stream)), what)


def apply_layer(ios, num_rows, table, num_slots, seg, max_rank, ws, stream=None, module_mask=None):
    """Delta of every projection given in ``ios`` ({name: ModuleIO}); see lora_apply_layer."""
    _layer(lib().lora_apply_layer, "lora_apply_layer", ios, num_rows, table, num_slots, seg, max_rank, ws, stream,
           module_mask)


def decode_layer(ios, num_rows, row_adapter, table, num_slots, seg, max_rank, ws, stream=None, module_mask=None):
    """Segments and the layer delta of a decode batch (one launch for a batch
    of distinct adapters); see lora_decode_layer."""
    import torch
    _need(row_adapter, torch.int32, "row_adapter", 1)
    if row_adapter.shape[0] < num_rows:
        raise ValueError("row_adapter: fewer ids than num_rows")
    arr, mask = _ios(ios, num_rows)
    if module_mask is None:
        module_mask = mask
    _check(lib().lora_decode_layer(arr, module_mask, num_rows, _ptr(row_adapter), _ptr(table), num_slots, seg.c(),
                                   max_rank, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "lora_decode_layer")


def decode_layer_launches(ios, num_rows, num_slots, seg, max_rank, module_mask=None) -> int:
    """Kernel launches lora_decode_layer makes for these arguments (1 or 3; 0 if it would reject them)."""
    arr, mask = _ios(ios, num_rows)
    return int(lib().lora_decode_layer_launches(arr, mask if module_mask is None else module_mask, num_rows,
                                                num_slots, seg.c(), max_rank))


def apply_layer_noalloc(ios, num_rows, table, num_slots, seg, max_rank, stream=None, module_mask=None):
    """apply_layer with the library's static device scratch instead of a
    workspace (allocates nothing); see lora_apply_layer_noalloc."""
    arr, mask = _ios(ios, num_rows)
    if module_mask is None:
        module_mask = mask
    _check(lib().lora_apply_layer_noalloc(arr, module_mask, num_rows, _ptr(table), num_slots, seg.c(), max_rank,
                                          _stream(stream)), "lora_apply_layer_noalloc")


def layer_shrink(ios, num_rows, table, num_slots, seg, max_rank, ws, stream=None, module_mask=None):
    _layer(lib().lora_layer_shrink, "lora_layer_shrink", ios, num_rows, table, num_slots, seg, max_rank, ws, stream,
           module_mask)


def layer_expand(ios, num_rows, table, num_slots, seg, max_rank, ws, stream=None, module_mask=None):
    _layer(lib().lora_layer_expand, "lora_layer_expand", ios, num_rows, table, num_slots, seg, max_rank, ws, stream,
           module_mask)


def apply_layer_stacked(ios, num_rows, row_adapters, table, num_slots, seg, max_rank, ws, stream=None,
                        module_mask=None, pass_max_rank=None):
    """Several adapters per row (``row_adapters``: device int32 [num_rows, depth],
    -1 pads; ``pass_max_rank``: optional largest rank of each column); see
    lora_apply_layer_stacked."""
    import torch
    _need(row_adapters, torch.int32, "row_adapters", 2)
    if row_adapters.shape[0] < num_rows or not row_adapters.is_contiguous():
        raise ValueError("row_adapters: a contiguous [num_rows, depth] tensor")
    depth = row_adapters.shape[1]
    pr = None
    if pass_max_rank is not None:
        pr = np.ascontiguousarray(pass_max_rank, dtype=np.int32)
        if pr.shape != (depth,):
            raise ValueError("pass_max_rank: one rank per column")
    arr, mask = _ios(ios, num_rows)
    if module_mask is None:
        module_mask = mask
    _check(lib().lora_apply_layer_stacked(arr, module_mask, num_rows, _ptr(row_adapters), depth,
                                          None if pr is None else pr.ctypes.data_as(ctypes.c_void_p),
                                          _ptr(table), num_slots, seg.c(), max_rank, _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)),
           "lora_apply_layer_stacked")


def form_batch(adapters, max_batch: int, max_distinct: int, min_batch: int = 0, reserved_tail: int = 0,
               waited_ms=None, max_wait_ms: float = 0.0) -> np.ndarray:
    """lora_form_batch on host arrays: queue positions of the chosen requests,
    in batch order.  ``adapters``: int32 adapter slot per waiting request,
    oldest first (negative = base only); ``waited_ms``: optional float ages."""
    a = np.ascontiguousarray(adapters, dtype=np.int32)
    w = None if waited_ms is None else np.ascontiguousarray(waited_ms, dtype=np.float32)
    if w is not None and w.shape != a.shape:
        raise LoraError("form_batch: waited_ms must match adapters")
    out = np.empty(max(1, min(int(max_batch), a.size)), np.int32)
    count = ctypes.c_int32(0)
    code = host_lib().lora_form_batch(a.ctypes.data_as(ctypes.c_void_p), a.size,
                                 None if w is None else w.ctypes.data_as(ctypes.c_void_p), float(max_wait_ms),
                                 int(max_batch), int(max_distinct), int(min_batch), int(reserved_tail),
                                 out.ctypes.data_as(ctypes.c_void_p), ctypes.byref(count))
    _check(code, "form_batch")
    return out[:count.value].copy()
