"""CPU oracle for the heterogeneous-adapter LoRA delta -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and has
no fallback to it.  It shares no code with ``adapter_gemv_amd``; the two meet
only at the seeded inputs from ``workloads`` and at the comparison.

The arithmetic lives in ``lora_oracle.c`` (plain C, fp64, one thread); this
module builds it with gcc and marshals numpy arrays through ctypes.  The
pages' analytic byte and FLOP accounting lives in ``oracle.costmodel``.

Functions and the passages they follow:

* ``build_segments`` -- group rows by adapter ("6. Deep Dive A: Batching
  Heterogeneous Adapters" on "m07 -- Multi-Adapter (LoRA) Serving": an index
  vector maps each sequence to an adapter slot; "One weight read, many
  adapters" on "LoRA, quotas and noisy neighbours": tag each row with its
  adapter and group).
* ``lora_module`` -- v = A.x, delta = scale * B.v, y = y0 + delta for one
  projection ("2. Scale Numbers" for the shapes of A and B; "6. Deep Dive A"
  for y = Wx + (B.A)x(alpha/r)).
* ``lora_layer`` -- the same for every projection in a module mask.
* int8 factors ("9. Bottlenecks and Evolution" on "m07", item 3: quantised
  adapters) -- dequantised exactly (one fp32 scale per row), then the same
  sums.
* ``lora_layer_stacked`` -- several adapters on one row (same section, item
  5: multi-adapter composition): each projection's delta is the sum of the
  single-adapter deltas of the row's list, y = y0 + that sum.
* ``batch_former.form_batch`` -- the adapter-aware batch former ("6. Deep
  Dive A", "The adapter-aware scheduler"; "The Revision", R1).
* ``linear_layer`` -- base projection and adapter delta together, y = W.x +
  delta (same page, "6. Deep Dive A": y = Wx + (BA)x(alpha/r)), the result
  a fused base + delta kernel produces.  W.x is a numpy matmul over the
  exactly decoded bf16 values, in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")
_LIB = os.path.join(_HERE, "liblora_oracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build, loaded instead when
# LORA_SANITIZE=1 (the process must have the sanitizer runtime preloaded)
_SAN_LIB = os.path.join(_HERE, "liblora_oracle_san.so")
_SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

_i32p = ctypes.POINTER(ctypes.c_int32)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_f32p = ctypes.POINTER(ctypes.c_float)
_vpp = ctypes.POINTER(ctypes.c_void_p)

_lib = None


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with the host C compiler (no fast-math, -O2); with
    sanitize, its ASan + UBSan build liblora_oracle_san.so instead."""
    out = _SAN_LIB if sanitize else _LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.run(
            ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off",
             "-fPIC", "-shared", "-Wall", "-Wextra", *(_SANITIZE_FLAGS if sanitize else []), "-o", tmp, _SRC],
            check=True)
        os.replace(tmp, out)
    return out


def library_path() -> str:
    """The oracle library this process loads: the sanitizer build when
    LORA_SANITIZE=1, else the plain one."""
    return _SAN_LIB if os.environ.get("LORA_SANITIZE") == "1" else _LIB


def _load():
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build(force=True, sanitize=path == _SAN_LIB)
        _lib = _configure(ctypes.CDLL(path))
    return _lib


def _configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    lib.oracle_build_segments.restype = ctypes.c_int32
    lib.oracle_build_segments.argtypes = [
        _i32p, ctypes.c_int32, ctypes.c_int32, _i32p, _i32p, _i32p, _i32p]
    lib.oracle_lora_module.restype = ctypes.c_int32
    lib.oracle_lora_module.argtypes = [
        _u16p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
        _u16p, ctypes.c_int64, ctypes.c_int32,
        _i32p, ctypes.c_int32, _vpp, _vpp, _i32p, _f32p, _i32p, ctypes.c_int32,
        _i32p, ctypes.c_int32, _f64p, _f64p, _f64p, _f64p]
    lib.oracle_base_bf16.restype = None
    lib.oracle_base_bf16.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _u16p, ctypes.c_int64,
                                     _i32p, ctypes.c_int32, _f64p]
    lib.oracle_base_q4.restype = None
    lib.oracle_base_q4.argtypes = [ctypes.POINTER(ctypes.c_uint8), ctypes.c_int64, _f32p, ctypes.c_int64,
                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _u16p, ctypes.c_int64,
                                   _i32p, ctypes.c_int32, _f64p]
    return lib


def _ptr(a: np.ndarray, typ):
    return a.ctypes.data_as(typ)


@dataclass
class Segments:
    perm: np.ndarray          # int32 [n_valid]  original row of each sorted position
    seg_offsets: np.ndarray   # int32 [nseg + 1]
    seg_adapter: np.ndarray   # int32 [nseg]
    num_segments: int
    num_bad_ids: int          # rows with id >= num_slots


def build_segments(ids: np.ndarray, num_slots: int) -> Segments:
    """Stable grouping of rows by adapter id (ids < 0: base-only, skipped)."""
    lib = _load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n = ids.shape[0]
    perm = np.full(max(n, 1), -1, np.int32)
    offs = np.zeros(max(n, 1) + 1, np.int32)
    adap = np.full(max(n, 1), -1, np.int32)
    nseg = np.zeros(1, np.int32)
    bad = lib.oracle_build_segments(_ptr(ids, _i32p), n, num_slots, _ptr(perm, _i32p),
                                    _ptr(offs, _i32p), _ptr(adap, _i32p), _ptr(nseg, _i32p))
    ns = int(nseg[0])
    nvalid = int(offs[ns])
    return Segments(perm[:nvalid].copy(), offs[:ns + 1].copy(), adap[:ns].copy(), ns, int(bad))


@dataclass
class ModuleResult:
    v: np.ndarray       # float64 [n_sel, max_rank]
    delta: np.ndarray   # float64 [n_sel, d_out]
    y: np.ndarray       # float64 [n_sel, d_out]
    num_bad_rank: int


FMT_BF16, FMT_INT8_ROWS = 0, 1


def lora_module(x: np.ndarray, y0: np.ndarray, ids: np.ndarray,
                A_ptrs: np.ndarray, B_ptrs: np.ndarray, ranks: np.ndarray,
                scales: np.ndarray, max_rank: int, rows=None,
                keep_alive=(), fmts=None) -> ModuleResult:
    """The delta of one projection for the selected rows.

    x   uint16 (bf16 bits) [num_rows, >= d_in]; y0 uint16 [num_rows, >= d_out]
    A_ptrs / B_ptrs: uint64 host addresses, one per slot, of the factors:
    bf16 A [rank, d_in] and B [d_out, round_up(rank, 8)] (row-major), or,
    where ``fmts`` says FMT_INT8_ROWS, the int8 blocks described in
    ``lora_oracle.c``; ranks int32, scales float32, fmts int32 (default all
    bf16), one per slot.  ``keep_alive`` holds the arrays those addresses
    point into.  ``rows``: row indices to compute (default: all).
    """
    lib = _load()
    assert x.dtype == np.uint16 and y0.dtype == np.uint16
    assert x.ndim == 2 and y0.ndim == 2 and x.strides[1] == 2 and y0.strides[1] == 2
    num_rows = x.shape[0]
    assert y0.shape[0] == num_rows
    d_in, d_out = x.shape[1], y0.shape[1]
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    assert ids.shape[0] == num_rows
    if rows is None:
        rows = np.arange(num_rows, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < num_rows)
    num_slots = ranks.shape[0]
    A_ptrs = np.ascontiguousarray(A_ptrs, dtype=np.uint64)
    B_ptrs = np.ascontiguousarray(B_ptrs, dtype=np.uint64)
    ranks = np.ascontiguousarray(ranks, dtype=np.int32)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    fmts = None if fmts is None else np.ascontiguousarray(fmts, dtype=np.int32)
    n_sel = rows.shape[0]
    v = np.zeros((n_sel, max_rank), np.float64)
    delta = np.zeros((n_sel, d_out), np.float64)
    y = np.zeros((n_sel, d_out), np.float64)
    scratch = np.zeros(max_rank + d_out, np.float64)
    bad = lib.oracle_lora_module(
        _ptr(x, _u16p), x.strides[0] // 2, num_rows, d_in,
        _ptr(y0, _u16p), y0.strides[0] // 2, d_out,
        _ptr(ids, _i32p), num_slots,
        A_ptrs.ctypes.data_as(_vpp), B_ptrs.ctypes.data_as(_vpp),
        _ptr(ranks, _i32p), _ptr(scales, _f32p), None if fmts is None else _ptr(fmts, _i32p), max_rank,
        _ptr(rows, _i32p), n_sel, _ptr(v, _f64p), _ptr(delta, _f64p), _ptr(y, _f64p),
        _ptr(scratch, _f64p))
    return ModuleResult(v, delta, y, int(bad))


def lora_layer(workload, rows=None, modules=None) -> dict:
    """Every projection of a layer-shaped workload (see ``workloads``).

    Returns {module_name: ModuleResult}.  ``modules`` restricts the set.
    """
    out = {}
    for m in workload.modules:
        if modules is not None and m.name not in modules:
            continue
        A_ptrs, B_ptrs, ranks, scales = workload.host_table(m.index)
        out[m.name] = lora_module(workload.x[m.x_name], workload.y0[m.name], workload.ids,
                                  A_ptrs, B_ptrs, ranks, scales, workload.max_rank, rows=rows,
                                  fmts=workload.fmt[:, m.index])
    return out


def lora_layer_stacked(workload, row_adapters, rows=None, modules=None, pass_max_rank=None) -> dict:
    """Several adapters per row: ``row_adapters`` int32 [num_rows, depth]
    (negative entries add nothing).  For every projection, delta = sum over t
    of the single-adapter delta of column t, in fp64; y = y0 + delta.
    ``pass_max_rank`` [depth]: the largest rank column t admits (entries above
    it are skipped as bad); default the workload's max_rank.

    Returns {module_name: ModuleResult}; ``v`` is [depth, n_sel, max_rank]
    and ``num_bad_rank`` the sum over the passes.
    """
    ra = np.ascontiguousarray(row_adapters, dtype=np.int32)
    assert ra.ndim == 2 and ra.shape[0] == workload.num_rows
    out = {}
    for m in workload.modules:
        if modules is not None and m.name not in modules:
            continue
        A_ptrs, B_ptrs, ranks, scales = workload.host_table(m.index)
        mr = [workload.max_rank] * ra.shape[1] if pass_max_rank is None else [int(r) for r in pass_max_rank]
        passes = [lora_module(workload.x[m.x_name], workload.y0[m.name], ra[:, t], A_ptrs, B_ptrs, ranks, scales,
                              mr[t], rows=rows, fmts=workload.fmt[:, m.index])
                  for t in range(ra.shape[1])]
        delta = passes[0].delta.copy()
        for p in passes[1:]:
            delta += p.delta
        sel = np.arange(workload.num_rows) if rows is None else np.asarray(rows)
        y0 = workload.y0[m.name][sel, :m.d_out]
        y0 = (y0.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # bf16 bits, decoded exactly
        v = np.zeros((len(passes), delta.shape[0], max([workload.max_rank] + mr)), np.float64)
        for t, p in enumerate(passes):
            v[t, :, :p.v.shape[1]] = p.v  # each pass's v is as wide as its own max rank
        out[m.name] = ModuleResult(v, delta, y0 + delta, sum(p.num_bad_rank for p in passes))
    return out


def base_projection(W, x: np.ndarray, rows=None) -> np.ndarray:
    """W.x for the selected rows in fp64 (oracle_base_bf16 / oracle_base_q4:
    plain loops, ascending k): W uint16 (bf16) [d_out, d_in], or a 4-bit
    weight (an object with q uint8 [d_out, ldwq], two signed 4-bit values per
    byte with the lower input index in the low nibble; scales fp32
    [d_out, lds], one per `group` consecutive inputs of a row; d_in, d_out);
    x uint16 [num_rows, >= d_in]."""
    lib = _load()
    x = np.ascontiguousarray(x)
    sel = np.arange(x.shape[0], dtype=np.int32) if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    if hasattr(W, "scales"):
        d_out, d_in = W.d_out, W.d_in
        out = np.empty((sel.size, d_out), np.float64)
        q, s = np.ascontiguousarray(W.q), np.ascontiguousarray(W.scales)
        lib.oracle_base_q4(q.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), q.shape[1], _ptr(s, _f32p), s.shape[1],
                           W.group, d_out, d_in, _ptr(x, _u16p), x.shape[1], _ptr(sel, _i32p), sel.size,
                           _ptr(out, _f64p))
        return out
    W = np.ascontiguousarray(W)
    d_out, d_in = W.shape
    out = np.empty((sel.size, d_out), np.float64)
    lib.oracle_base_bf16(_ptr(W, _u16p), W.shape[1], d_out, d_in, _ptr(x, _u16p), x.shape[1], _ptr(sel, _i32p),
                         sel.size, _ptr(out, _f64p))
    return out



def linear_layer(workload, rows=None, modules=None) -> dict:
    """Base projection plus adapter delta for every projection of a workload
    with base weights: {module_name: ModuleResult} with y = W.x + delta (the
    base output replaces y0)."""
    out = {}
    for m in workload.modules:
        if modules is not None and m.name not in modules:
            continue
        A_ptrs, B_ptrs, ranks, scales = workload.host_table(m.index)
        r = lora_module(workload.x[m.x_name], workload.y0[m.name], workload.ids, A_ptrs, B_ptrs, ranks, scales,
                        workload.max_rank, rows=rows, fmts=workload.fmt[:, m.index])
        base = base_projection(workload.W[m.name], workload.x[m.x_name], rows)
        out[m.name] = ModuleResult(r.v, r.delta, base + r.delta, r.num_bad_rank)
    return out
