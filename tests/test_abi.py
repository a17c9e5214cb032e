"""The C-ABI library loads, exports every function include/lora_gemv.h declares,
and rejects bad host arguments with the documented status codes.

Every call here fails validation, which runs before the first HIP call, so no
device is touched (the pointers are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

import adapter_gemv_amd as lg

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lora_gemv.h")
OK, NULL, SHAPE, RANK, ALIGN, WS, MODULE, LAUNCH, SCRATCH = range(9)
P = 0x10000          # an aligned fake device address (never dereferenced)
BIG = 1 << 40


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared()
    assert {"lora_build_segments", "lora_shrink", "lora_expand", "lora_apply_layer"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", lg.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lora_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    L = lg.lib()
    for n in names:
        getattr(L, n)


def test_read_ceiling_library_is_separate():
    # the benchmark's read-ceiling kernel lives in a library of its own: the C ABI exports no such symbol
    here = os.path.dirname(lg.LIB_PATH)
    path = os.path.join(here, "libread_ceiling.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    assert {"read_ceiling_launch", "read_ceiling_blocks"} <= set(re.findall(r"\bT (\w+)", out))
    main = subprocess.run(["nm", "-D", "--defined-only", lg.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "read_ceiling" not in main
    L = ctypes.CDLL(path)
    L.read_ceiling_blocks.argtypes = [ctypes.c_uint64]
    assert [L.read_ceiling_blocks(n) for n in (1, 65536, 65537, 1 << 30)] == [1, 1, 2, 16384]
    L.read_ceiling_launch.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    assert L.read_ceiling_launch(None, 64, P, None) != 0  # rejected before any HIP call
    assert L.read_ceiling_launch(P, 0, P, None) != 0


def seg(**kw):
    d = dict(perm=P, seg_offsets=P, seg_adapter=P, num_segments=P, tile_counts=P, status=P)
    d.update(kw)
    return lg._Seg(**d)


def test_status_strings():
    for c in range(9):
        s = lg.status_string(c)
        assert s.startswith("LORA_")
    assert "unknown" in lg.status_string(99)


def test_workspace_query():
    L = lg.lib()
    assert L.lora_workspace_bytes(128, 128, 64, 8192) > 0
    assert L.lora_workspace_bytes(-1, 128, 64, 0) == 0
    assert L.lora_workspace_bytes(128, 0, 64, 0) == 0
    assert L.lora_workspace_bytes(128, 128, 0, 0) == 0
    assert L.lora_workspace_bytes(128, 128, 65, 0) == 0
    # grows with rows, rank and the projections' input sizes
    assert L.lora_workspace_bytes(256, 128, 64, 8192) > L.lora_workspace_bytes(128, 128, 64, 8192)
    assert L.lora_workspace_bytes(128, 128, 64, 65536) > L.lora_workspace_bytes(128, 128, 64, 8192)


@pytest.mark.parametrize("args,code", [
    (dict(seg=seg(perm=None)), NULL),
    (dict(seg=seg(status=None)), NULL),
    (dict(seg=seg(tile_counts=None)), NULL),
    (dict(n=-1), SHAPE),
    (dict(slots=0), SHAPE),
    (dict(ids=None), NULL),
    (dict(n=5000, ws=None), NULL),           # long batches need workspace
    (dict(n=5000, ws_bytes=0), WS),          # long batches need workspace
    (dict(seg=seg(max_segments=-1)), SHAPE),
])
def test_build_segments_rejects(args, code):
    a = dict(ids=P, n=128, slots=16, seg=seg(), ws=P, ws_bytes=BIG)
    a.update(args)
    assert lg.lib().lora_build_segments(a["ids"], a["n"], a["slots"], a["seg"], a["ws"], a["ws_bytes"], None) == code


SHRINK = dict(x=P, ldx=1024, n=64, d=1024, table=P, slots=8, n_mod=7, module=0, seg=seg(), max_rank=16, v=P, ldv=16,
              ws=P, ws_bytes=BIG)


@pytest.mark.parametrize("fn", ["lora_shrink", "lora_expand"])
@pytest.mark.parametrize("args,code", [
    (dict(x=None), NULL), (dict(table=None), NULL), (dict(v=None), NULL),
    (dict(seg=seg(seg_adapter=None)), NULL), (dict(seg=seg(max_segments=-3)), SHAPE),
    (dict(n_mod=0), MODULE), (dict(n_mod=8), MODULE), (dict(module=7), MODULE), (dict(module=-1), MODULE),
    (dict(max_rank=0), RANK), (dict(max_rank=65), RANK),
    (dict(n=-1), SHAPE), (dict(slots=0), SHAPE), (dict(d=0), SHAPE), (dict(ldx=1016), SHAPE), (dict(ldv=8), SHAPE),
    (dict(d=1020, ldx=1024), ALIGN), (dict(ldx=1028), ALIGN), (dict(x=P + 8), ALIGN), (dict(v=P + 4), ALIGN),
    (dict(ldv=18), ALIGN),
])
def test_shrink_expand_reject(fn, args, code):
    a = dict(SHRINK)
    a.update(args)
    L = lg.lib()
    if fn == "lora_shrink":
        r = L.lora_shrink(a["x"], a["ldx"], a["n"], a["d"], a["table"], a["slots"], a["n_mod"], a["module"], a["seg"],
                          a["max_rank"], a["v"], a["ldv"], a["ws"], a["ws_bytes"], None)
    else:  # same roles: v in, x plays y
        r = L.lora_expand(a["v"], a["ldv"], a["n"], a["d"], a["table"], a["slots"], a["n_mod"], a["module"], a["seg"],
                          a["max_rank"], a["x"], a["ldx"], a["ws"], a["ws_bytes"], None)
    assert r == code


@pytest.mark.parametrize("args,code", [(dict(ws=None), NULL), (dict(ws_bytes=16), WS), (dict(ws=P + 8), ALIGN)])
def test_shrink_workspace(args, code):
    a = dict(SHRINK)
    a.update(args)
    r = lg.lib().lora_shrink(a["x"], a["ldx"], a["n"], a["d"], a["table"], a["slots"], a["n_mod"], a["module"],
                             a["seg"], a["max_rank"], a["v"], a["ldv"], a["ws"], a["ws_bytes"], None)
    assert r == code


def ios(**over):
    arr = (lg._IO * 7)()
    for i in range(7):
        arr[i] = lg._IO(P, 8192, P, 8192, 8192, 8192)
    for k, v in over.items():
        i, field = k.split("_", 1)
        setattr(arr[int(i)], field, v)
    return arr


@pytest.mark.parametrize("fn", ["lora_apply_layer", "lora_layer_shrink", "lora_layer_expand"])
@pytest.mark.parametrize("args,code", [
    (dict(io=None), NULL), (dict(table=None), NULL), (dict(ws=None), NULL), (dict(seg=seg(num_segments=None)), NULL),
    (dict(seg=seg(max_segments=-1)), SHAPE),
    (dict(mask=0), MODULE), (dict(mask=0x80), MODULE),
    (dict(mask=1 << 16), MODULE), (dict(mask=0x7F | 1 << 17), MODULE),   # the int8-items flag alone; an unknown bit
    (dict(mask=0x7F | 1 << 16, n=-1), SHAPE),                             # the flag with the modules is accepted
    (dict(n=-1), SHAPE), (dict(slots=0), SHAPE),
    (dict(max_rank=0), RANK), (dict(max_rank=100), RANK),
    (dict(io=ios(**{"3_x": None})), NULL), (dict(io=ios(**{"0_y": None})), NULL),
    (dict(io=ios(**{"2_d_out": 0})), SHAPE), (dict(io=ios(**{"1_ldy": 4096})), SHAPE),
    (dict(io=ios(**{"6_d_in": 1004, "6_ldx": 1008})), ALIGN), (dict(io=ios(**{"4_y": P + 2})), ALIGN),
    (dict(ws_bytes=1024), WS), (dict(ws=P + 4), ALIGN),
])
def test_layer_rejects(fn, args, code):
    a = dict(io=ios(), mask=0x7F, n=128, table=P, slots=128, seg=seg(), max_rank=64, ws=P, ws_bytes=BIG)
    a.update(args)
    f = getattr(lg.lib(), fn)
    assert f(a["io"], a["mask"], a["n"], a["table"], a["slots"], a["seg"], a["max_rank"], a["ws"], a["ws_bytes"],
             None) == code


@pytest.mark.parametrize("args,code", [
    (dict(io=None), NULL), (dict(table=None), NULL), (dict(seg=seg(status=None)), NULL),
    (dict(mask=0), MODULE), (dict(n=-1), SHAPE), (dict(max_rank=65), RANK),
    (dict(io=ios(**{"4_y": P + 2})), ALIGN),
    # the partials of 128 rows at rank 64 over all seven 70B projections fit the static scratch;
    # 2048 rows do not (LORA_ERR_SCRATCH before any device work)
    (dict(n=2048), SCRATCH),
])
def test_noalloc_rejects(args, code):
    a = dict(io=ios(), mask=0x7F, n=128, table=P, slots=128, seg=seg(), max_rank=64)
    a.update(args)
    L = lg.lib()
    assert L.lora_workspace_bytes(128, 128, 64, 7 * 8192) <= lg.STATIC_SCRATCH_BYTES
    assert L.lora_workspace_bytes(2048, 128, 64, 7 * 8192) > lg.STATIC_SCRATCH_BYTES
    assert L.lora_apply_layer_noalloc(a["io"], a["mask"], a["n"], a["table"], a["slots"], a["seg"], a["max_rank"],
                                      None) == code


def test_masked_out_modules_are_not_checked():
    # an invalid projection outside the mask is ignored; the call then fails
    # only at the (too small) workspace check
    a = ios(**{"5_x": None, "5_d_in": 3})
    r = lg.lib().lora_apply_layer(a, 0x01, 128, P, 128, seg(), 64, P, 16, None)
    assert r == WS


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    s = lg.Segments.__new__(lg.Segments)
    with pytest.raises((TypeError, ValueError)):
        lg.build_segments(torch.zeros(4, dtype=torch.int32), 4, s, torch.zeros(16, dtype=torch.uint8))


def test_segment_bound_counts_distinct_valid_slots():
    import numpy as np
    assert lg.segment_bound(np.array([3, 3, -1, 7, 9, 2, 3]), 8) == 3          # 9 >= slots, -1 base only
    assert lg.segment_bound(np.zeros(0, np.int32), 8) == 0
    assert lg.segment_bound(np.array([-1, -2]), 8) == 0
    # several adapters per row: the most over the columns (one build per column)
    assert lg.segment_bound(np.array([[0, 1], [0, 2], [0, 3], [5, -1]]), 8) == 3
    s = lg.Segments.__new__(lg.Segments)  # no buffers: the bound is checked first
    s.max_segments = -1
    with pytest.raises(ValueError):
        s.c()


def lin_ios(q4=False, **over):
    if q4:
        arr = (lg._LinQ4IO * 7)()
        for i in range(7):
            arr[i] = lg._LinQ4IO(P, 8192, P, 4096, P, 64, P, 8192, 8192, 8192)
    else:
        arr = (lg._LinIO * 7)()
        for i in range(7):
            arr[i] = lg._LinIO(P, 8192, P, 8192, P, 8192, 8192, 8192)
    for k, v in over.items():
        i, field = k.split("_", 1)
        setattr(arr[int(i)], field, v)
    return arr


LIN_BAD = [
    (dict(io=None), NULL), (dict(table=None), NULL), (dict(ws=None), NULL), (dict(row_adapter=None), NULL),
    (dict(mask=0), MODULE), (dict(n=-1), SHAPE), (dict(max_rank=0), RANK), (dict(ws_bytes=1024), WS),
]


@pytest.mark.parametrize("fn", ["lora_linear_layer", "lora_linear_shrink", "lora_linear_expand"])
@pytest.mark.parametrize("args,code", LIN_BAD + [
    (dict(io=lin_ios(**{"2_W": None})), NULL), (dict(io=lin_ios(**{"0_ldw": 4096})), SHAPE),
    (dict(io=lin_ios(**{"3_W": P + 2})), ALIGN), (dict(io=lin_ios(**{"1_d_in": 1004, "1_ldx": 1008})), ALIGN),
])
def test_linear_rejects(fn, args, code):
    a = dict(io=lin_ios(), mask=0x7F, n=128, row_adapter=P, table=P, slots=128, seg=seg(), max_rank=64, ws=P,
             ws_bytes=1 << 40)
    a.update(args)
    assert getattr(lg.lib(), fn)(a["io"], a["mask"], a["n"], a["row_adapter"], a["table"], a["slots"], a["seg"],
                                 a["max_rank"], a["ws"], a["ws_bytes"], None) == code


@pytest.mark.parametrize("fn", ["lora_linear_layer_q4", "lora_linear_shrink_q4", "lora_linear_expand_q4"])
@pytest.mark.parametrize("args,code", LIN_BAD + [
    (dict(io=lin_ios(True, **{"2_Wq": None})), NULL), (dict(io=lin_ios(True, **{"5_Ws": None})), NULL),
    (dict(io=lin_ios(True, **{"0_d_in": 8000, "0_ldx": 8000})), ALIGN),   # not a multiple of 128
    (dict(io=lin_ios(True, **{"1_ldwq": 4088})), ALIGN),                  # not a multiple of 16
    (dict(io=lin_ios(True, **{"1_ldwq": 4080})), SHAPE),                  # < d_in / 2
    (dict(io=lin_ios(True, **{"4_lds": 63})), SHAPE),                     # < d_in / 128
    (dict(io=lin_ios(True, **{"6_Ws": P + 2})), ALIGN), (dict(io=lin_ios(True, **{"3_Wq": P + 8})), ALIGN),
    (dict(io=lin_ios(True, **{"2_ldwq": 1 << 20})), SHAPE),               # W of 8 GiB
])
def test_linear_q4_rejects(fn, args, code):
    a = dict(io=lin_ios(True), mask=0x7F, n=128, row_adapter=P, table=P, slots=128, seg=seg(), max_rank=64, ws=P,
             ws_bytes=1 << 40)
    a.update(args)
    assert getattr(lg.lib(), fn)(a["io"], a["mask"], a["n"], a["row_adapter"], a["table"], a["slots"], a["seg"],
                                 a["max_rank"], a["ws"], a["ws_bytes"], None) == code
