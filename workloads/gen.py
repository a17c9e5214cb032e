"""Seeded synthetic workloads shaped like the pages' 70B serving examples.

Inputs only: this module draws random numbers, rounds them to bf16 and lays
them out in host memory.  It computes nothing of the LoRA delta.  Both the GPU
tests/bench and the CPU oracle take their inputs from here.

Every draw has its own ``numpy.random.SeedSequence(seed, spawn_key=...)``
keyed by its role, so the values do not depend on draw order or on how many
threads fill them.  Values are drawn in float32 and rounded to bf16 with
round-to-nearest-even.

Shapes follow "m07 -- Multi-Adapter (LoRA) Serving", "2. Scale Numbers" (70B:
hidden 8192, GQA kv-dim 1024, FFN 28672); adapter popularity for the skewed
workload is a finite Zipf law as on "12. Adapter Serving and Multi-Tenant
Customization", "Power-law traffic and placement strategy" (exponent 1.1 here).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# Column order of the adapter table: one entry per (slot, projection).
MODULE_NAMES = ("q", "k", "v", "o", "gate", "up", "down")
MODULE_INDEX = {n: i for i, n in enumerate(MODULE_NAMES)}
N_MOD = len(MODULE_NAMES)

D_MODEL, KV_DIM, FFN_DIM = 8192, 1024, 28672
SHAPES_70B = {
    "q": (D_MODEL, D_MODEL), "k": (D_MODEL, KV_DIM), "v": (D_MODEL, KV_DIM),
    "o": (D_MODEL, D_MODEL), "gate": (D_MODEL, FFN_DIM), "up": (D_MODEL, FFN_DIM),
    "down": (FFN_DIM, D_MODEL),
}
# Which activation tensor feeds each projection in a transformer layer.
X_OF_70B = {"q": "x_qkv", "k": "x_qkv", "v": "x_qkv", "o": "x_o",
            "gate": "x_gateup", "up": "x_gateup", "down": "x_down"}

_CHUNK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))

# Roles of the independent draws.
_R_IDS, _R_RANK, _R_PLACE, _R_X, _R_Y, _R_A, _R_B, _R_LEN, _R_PAD, _R_W = range(10)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(int(k) for k in key)))


def normal_bf16(seed: int, key: tuple, n: int, std: float, out: np.ndarray | None = None) -> np.ndarray:
    """n draws of N(0, std^2) (std is the standard deviation), as bf16 bits."""
    if out is None:
        out = np.empty(n, np.uint16)
    nch = (n + _CHUNK - 1) // _CHUNK

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        t = _rng(seed, *key, c).standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            t *= np.float32(std)
        out[lo:hi] = bf16_bits(t)

    if nch <= 1:
        for c in range(nch):
            fill(c)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(nch)))
    return out


@dataclass
class ModuleSpec:
    name: str
    index: int      # column in the adapter table
    d_in: int
    d_out: int
    x_name: str     # activation tensor that feeds this projection


@dataclass
class Workload:
    """One batch of rows, their adapters and the tensors of every projection.

    Every A and B lives in one flat bf16 ``pool``; ``a_off``/``b_off`` give the
    element offset of entry (slot, column) (-1 where the rank is 0).  A is
    [rank, d_in] row-major and compact; B is [d_out, rank] row-major with its
    rows ``ldb(rank)`` (rank rounded up to a multiple of 8) elements apart.
    The padding columns hold random values that no computation may use.
    """
    name: str
    seed: int
    num_rows: int
    num_slots: int
    max_rank: int
    ids: np.ndarray                  # int32 [num_rows], -1 = base only
    modules: list                    # [ModuleSpec]
    x: dict                          # name -> uint16 [num_rows, d_in]
    y0: dict                         # module name -> uint16 [num_rows, d_out]
    pool: np.ndarray                 # uint16 flat
    a_off: np.ndarray                # int64 [num_slots, N_MOD]
    b_off: np.ndarray                # int64 [num_slots, N_MOD]
    ranks: np.ndarray                # int32 [num_slots, N_MOD]
    scales: np.ndarray               # float32 [num_slots, N_MOD]
    seq_lens: np.ndarray | None = None
    notes: dict = field(default_factory=dict)
    fmt: np.ndarray | None = None    # int32 [num_slots, N_MOD]: FMT_BF16 or FMT_INT8_ROWS
    stack: np.ndarray | None = None  # int32 [num_rows, depth]: several adapters per row (ids = column 0)
    W: dict | None = None            # module name -> base weight (fused workloads): uint16 [d_out, d_in]
                                     # bf16, or a Q4Weight

    def __post_init__(self):
        if self.fmt is None:
            self.fmt = np.zeros((self.num_slots, N_MOD), np.int32)

    @property
    def module_mask(self) -> int:
        m = 0
        for s in self.modules:
            m |= 1 << s.index
        return m

    def module(self, name: str) -> ModuleSpec:
        for s in self.modules:
            if s.name == name:
                return s
        raise KeyError(name)

    def A(self, slot: int, col: int) -> np.ndarray:
        assert self.fmt[slot, col] == FMT_BF16
        r = int(self.ranks[slot, col])
        d_in = self._spec_col(col).d_in
        o = int(self.a_off[slot, col])
        return self.pool[o:o + r * d_in].reshape(r, d_in)

    def B(self, slot: int, col: int) -> np.ndarray:
        """[d_out, rank] view (rows ldb(rank) apart in the pool)."""
        assert self.fmt[slot, col] == FMT_BF16
        r = int(self.ranks[slot, col])
        d_out = self._spec_col(col).d_out
        o = int(self.b_off[slot, col])
        return self.pool[o:o + d_out * ldb(r)].reshape(d_out, ldb(r))[:, :r]

    def A_q8(self, slot: int, col: int):
        """int8 A: (row scales float32 [rank], values int8 [rank, d_in] view;
        rows lda8(d_in) bytes apart)."""
        assert self.fmt[slot, col] == FMT_INT8_ROWS
        r = int(self.ranks[slot, col])
        d_in = self._spec_col(col).d_in
        raw = self.pool.view(np.uint8)[2 * int(self.a_off[slot, col]):]
        sa = raw[:4 * r].view(np.float32)
        o = 4 * _align(r, 4)
        q = raw[o:o + r * lda8(d_in)].view(np.int8).reshape(r, lda8(d_in))[:, :d_in]
        return sa, q

    def B_q8(self, slot: int, col: int):
        """int8 B: (row scales float32 [d_out], values int8 [d_out, rank] view;
        rows ldb8(rank) bytes apart)."""
        assert self.fmt[slot, col] == FMT_INT8_ROWS
        r = int(self.ranks[slot, col])
        d_out = self._spec_col(col).d_out
        raw = self.pool.view(np.uint8)[2 * int(self.b_off[slot, col]):]
        sb = raw[:4 * d_out].view(np.float32)
        o = 4 * _align(d_out, 4)
        q = raw[o:o + d_out * ldb8(r)].view(np.int8).reshape(d_out, ldb8(r))[:, :r]
        return sb, q

    def _spec_col(self, col):
        for s in self.modules:
            if s.index == col:
                return s
        raise KeyError(col)

    def host_table(self, col: int):
        """Host addresses of each slot's A and B for one table column."""
        base = self.pool.ctypes.data
        a = np.where(self.a_off[:, col] >= 0, base + 2 * self.a_off[:, col], 0).astype(np.uint64)
        b = np.where(self.b_off[:, col] >= 0, base + 2 * self.b_off[:, col], 0).astype(np.uint64)
        return a, b, self.ranks[:, col].copy(), self.scales[:, col].copy()

    def adapter_bytes_used(self) -> int:
        """Bytes of A and B at their ranks and formats (padding not counted)."""
        return int(sum(entry_bytes(int(self.ranks[a, s.index]), s.d_in, s.d_out, int(self.fmt[a, s.index]))
                       for s in self.modules for a in range(self.num_slots)))


def ldb(rank: int) -> int:
    """Row stride of B: the rank rounded up to a multiple of 8."""
    return (int(rank) + 7) // 8 * 8


# Factor formats of a table entry.  FMT_INT8_ROWS: symmetric int8 with one
# fp32 scale per row ("9. Bottlenecks and Evolution" on "m07 -- Multi-Adapter
# (LoRA) Serving", item 3, fixes no scheme; this is the reading taken).  A
# block: float scales[round_up(rank, 4)], then int8 A[rank][lda8(d_in)]; B
# block: float scales[round_up(d_out, 4)], then int8 B[d_out][ldb8(rank)].
FMT_BF16, FMT_INT8_ROWS = 0, 1


def ldb8(rank: int) -> int:
    """Row stride (bytes) of an int8 B: the rank rounded up to a multiple of 16."""
    return (int(rank) + 15) // 16 * 16


def lda8(d_in: int) -> int:
    """Row stride (bytes) of an int8 A: d_in rounded up to a multiple of 16."""
    return (int(d_in) + 15) // 16 * 16


def entry_bytes(rank: int, d_in: int, d_out: int, fmt: int) -> int:
    """Bytes the method reads for one (adapter, projection) at its rank."""
    if rank <= 0:
        return 0
    if fmt == FMT_INT8_ROWS:
        return rank * (d_in + d_out) + 4 * (rank + d_out)
    return 2 * rank * (d_in + d_out)


def _block_elems(rank: int, d_in: int, d_out: int, fmt: int):
    """(A, B) block sizes in uint16 pool elements."""
    if fmt == FMT_INT8_ROWS:
        a = 4 * _align(rank, 4) + rank * lda8(d_in)
        b = 4 * _align(d_out, 4) + d_out * ldb8(rank)
        return (a + 1) // 2, (b + 1) // 2
    return rank * d_in, d_out * ldb(rank)


def quantize_rows(v: np.ndarray):
    """Symmetric int8 per row: scale = max|row| / 127 (float32), q = round(v /
    scale) (ties to even), clamped to [-127, 127]; rows of zeros get scale 0."""
    v = np.asarray(v, np.float32)
    m = np.abs(v).max(axis=1)
    scale = (m / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0))
    q = np.clip(np.rint(v / safe[:, None]), -127, 127).astype(np.int8)
    return scale, q


def _fill_adapters(seed, pool, modules, ranks, a_off, b_off, ab_std, slots, fmt=None):
    jobs = []
    for a in slots:
        for s in modules:
            r = int(ranks[a, s.index])
            if r > 0:
                jobs.append((a, s, r))
    raw = pool.view(np.uint8)

    def fill_q8(a, s, r, oa, ob):
        # the same draws as the bf16 factors, quantised per row
        av = bf16_to_f32(normal_bf16(seed, (_R_A, a, s.index), r * s.d_in, ab_std)).reshape(r, s.d_in)
        bv = bf16_to_f32(normal_bf16(seed, (_R_B, a, s.index), s.d_out * r, ab_std)).reshape(s.d_out, r)
        sa, qa = quantize_rows(av)
        sb, qb = quantize_rows(bv)
        o = 2 * oa
        raw[o:o + 4 * r] = sa.view(np.uint8)
        o += 4 * _align(r, 4)
        la = lda8(s.d_in)
        fa = raw[o:o + r * la].reshape(r, la)
        fa[:, :s.d_in] = qa.view(np.uint8)
        if la > s.d_in:  # padding: random bytes that no computation may use
            fa[:, s.d_in:] = _rng(seed, _R_PAD, a, s.index, 1).integers(0, 256, size=(r, la - s.d_in), dtype=np.uint8)
        o = 2 * ob
        raw[o:o + 4 * s.d_out] = sb.view(np.uint8)
        o += 4 * _align(s.d_out, 4)
        lb = ldb8(r)
        full = raw[o:o + s.d_out * lb].reshape(s.d_out, lb)
        full[:, :r] = qb.view(np.uint8)
        if lb > r:  # padding: random bytes that no computation may use
            full[:, r:] = _rng(seed, _R_PAD, a, s.index).integers(0, 256, size=(s.d_out, lb - r), dtype=np.uint8)

    def fill(job):
        a, s, r = job
        oa, ob = int(a_off[a, s.index]), int(b_off[a, s.index])
        if fmt is not None and fmt[a, s.index] == FMT_INT8_ROWS:
            return fill_q8(a, s, r, oa, ob)
        normal_bf16(seed, (_R_A, a, s.index), r * s.d_in, ab_std, out=pool[oa:oa + r * s.d_in])
        lb = ldb(r)
        if lb == r:
            normal_bf16(seed, (_R_B, a, s.index), s.d_out * r, ab_std, out=pool[ob:ob + s.d_out * r])
        else:
            full = pool[ob:ob + s.d_out * lb].reshape(s.d_out, lb)
            full[:, :r] = normal_bf16(seed, (_R_B, a, s.index), s.d_out * r, ab_std).reshape(s.d_out, r)
            full[:, r:] = normal_bf16(seed, (_R_PAD, a, s.index), s.d_out * (lb - r), 1.0).reshape(s.d_out, lb - r)

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fill, jobs))


def _align(n, a=64):
    return (n + a - 1) // a * a


def build_workload(name, seed, num_rows, num_slots, shapes: dict, ids, ranks,
                   x_of=None, x_std=1.0, ab_std=0.02, y_std=1.0, scales=None,
                   paged_capacity_rank=None, placement=None, seq_lens=None,
                   ab_fill=None, max_rank=None, fmt=None):
    """Assemble a workload.

    shapes: {module name: (d_in, d_out)}; ranks: int array [num_slots, N_MOD]
    (columns of modules not in ``shapes`` must be 0); ids: int32 [num_rows].
    With ``paged_capacity_rank`` every slot is a fixed-size page sized for that
    rank and adapter a lives in page ``placement[a]``.
    ``ab_fill``: optional callable(workload) replacing the random A/B values.
    ``fmt``: factor format per (slot, column), or one code for all
    (FMT_BF16 default; FMT_INT8_ROWS quantises the same draws per row).
    """
    modules = [ModuleSpec(n, MODULE_INDEX[n], shapes[n][0], shapes[n][1],
                          (x_of or {}).get(n, "x_" + n)) for n in MODULE_NAMES if n in shapes]
    ranks = np.asarray(ranks, dtype=np.int32)
    assert ranks.shape == (num_slots, N_MOD)
    if max_rank is None:
        max_rank = max(1, int(ranks.max()))
    if scales is None:
        scales = np.ones((num_slots, N_MOD), np.float32)
    fmt = np.broadcast_to(np.asarray(FMT_BF16 if fmt is None else fmt, np.int32), (num_slots, N_MOD)).copy()
    a_off = np.full((num_slots, N_MOD), -1, np.int64)
    b_off = np.full((num_slots, N_MOD), -1, np.int64)
    if paged_capacity_rank is None:
        pos = 0
        for a in range(num_slots):
            for s in modules:
                r = int(ranks[a, s.index])
                if r > 0:
                    ea, eb = _block_elems(r, s.d_in, s.d_out, int(fmt[a, s.index]))
                    a_off[a, s.index] = pos
                    pos = _align(pos + ea)
                    b_off[a, s.index] = pos
                    pos = _align(pos + eb)
        pool = np.zeros(max(pos, 64), np.uint16)
    else:
        cap = int(paged_capacity_rank)
        region = {}
        page = 0
        for s in modules:
            ea = max(_block_elems(cap, s.d_in, s.d_out, f)[0] for f in (FMT_BF16, FMT_INT8_ROWS))
            eb = max(_block_elems(cap, s.d_in, s.d_out, f)[1] for f in (FMT_BF16, FMT_INT8_ROWS))
            region[s.name] = (page, _align(page + ea))
            page = _align(region[s.name][1] + eb)
        page_elems = page
        pool = np.zeros(page_elems * num_slots, np.uint16)
        for a in range(num_slots):
            base = int(placement[a]) * page_elems
            for s in modules:
                if ranks[a, s.index] > 0:
                    a_off[a, s.index] = base + region[s.name][0]
                    b_off[a, s.index] = base + region[s.name][1]
    w = Workload(name=name, seed=seed, num_rows=num_rows, num_slots=num_slots, max_rank=max_rank,
                 ids=np.asarray(ids, dtype=np.int32), modules=modules, x={}, y0={}, pool=pool,
                 a_off=a_off, b_off=b_off, ranks=ranks, scales=np.asarray(scales, np.float32),
                 seq_lens=seq_lens, fmt=fmt)
    xd = {}
    for s in modules:
        xd.setdefault(s.x_name, s.d_in)
        assert xd[s.x_name] == s.d_in
    for i, (xn, d_in) in enumerate(sorted(xd.items())):
        w.x[xn] = normal_bf16(seed, (_R_X, i), num_rows * d_in, x_std).reshape(num_rows, d_in)
    for s in modules:
        w.y0[s.name] = normal_bf16(seed, (_R_Y, s.index), num_rows * s.d_out, y_std).reshape(num_rows, s.d_out)
    if ab_fill is None:
        _fill_adapters(seed, pool, modules, ranks, a_off, b_off, ab_std, range(num_slots), fmt)
    else:
        ab_fill(w)
    return w


# --------------------------------------------------------------------------
# The five workloads.  Standard deviations: N(0, 0.02) means std 0.02.

def tiny(seed=1, x_std=0.02):
    """d_in = d_out = 256, rank 8, 4 adapters, 16 decode rows, ids uniform."""
    n, slots = 16, 4
    ids = _rng(seed, _R_IDS).integers(0, slots, size=n)
    ranks = np.zeros((slots, N_MOD), np.int32)
    ranks[:, MODULE_INDEX["q"]] = 8
    return build_workload("tiny_decode", seed, n, slots, {"q": (256, 256)}, ids, ranks,
                          x_of={"q": "x"}, x_std=x_std, ab_std=0.02, y_std=1.0)


def q_proj(seed=2, rank=16, rows=128):
    """70B q_proj decode: 8192 -> 8192, one distinct adapter per row."""
    ids = _rng(seed, _R_IDS).permutation(rows)
    ranks = np.zeros((rows, N_MOD), np.int32)
    ranks[:, MODULE_INDEX["q"]] = rank
    return build_workload(f"q_proj_r{rank}_b{rows}", seed, rows, rows, {"q": SHAPES_70B["q"]}, ids,
                          ranks, x_of={"q": "x"}, x_std=1.0, ab_std=0.02, y_std=1.0)


def full_layer(seed=3, rank=64, rows=128, fmt=FMT_BF16):
    """70B layer, all seven projections at one rank, one distinct adapter per row
    (fmt=FMT_INT8_ROWS: the same draws quantised to int8 per row)."""
    ids = _rng(seed, _R_IDS).permutation(rows)
    ranks = np.full((rows, N_MOD), rank, np.int32)
    tag = "_int8" if fmt == FMT_INT8_ROWS else ""
    return build_workload(f"full_layer_r{rank}_b{rows}{tag}", seed, rows, rows, SHAPES_70B, ids, ranks,
                          x_of=X_OF_70B, x_std=1.0, ab_std=0.02, y_std=1.0, fmt=fmt)


def stacked_layer(seed=7, rows=128, n_domain=4, domain_rank=64, style_rank=16):
    """70B layer, all seven projections, two adapters per row: one of
    ``n_domain`` shared domain adapters (rank 64) and a style adapter of its own
    (rank 16), the "domain + style" composition of "9. Bottlenecks and
    Evolution", item 5, on "m07 -- Multi-Adapter (LoRA) Serving".  Slots
    [0, n_domain) hold the domain adapters, the next ``rows`` the styles."""
    g = _rng(seed, _R_IDS)
    stack = np.stack([g.integers(0, n_domain, size=rows), n_domain + g.permutation(rows)], 1).astype(np.int32)
    slots = n_domain + rows
    ranks = np.full((slots, N_MOD), style_rank, np.int32)
    ranks[:n_domain] = domain_rank
    w = build_workload(f"stacked_layer_{n_domain}x{domain_rank}_{rows}x{style_rank}", seed, rows, slots, SHAPES_70B,
                       stack[:, 0], ranks, x_of=X_OF_70B, x_std=1.0, ab_std=0.02, y_std=1.0)
    w.stack = stack
    return w


def add_base_weights(w: Workload) -> Workload:
    """Base weights W [d_out, d_in] (bf16, row-major like a linear layer's
    weight) for every projection, N(0, 1/d_in), so W.x has unit variance like
    the y0 of the other workloads."""
    w.W = {}
    for s in w.modules:
        w.W[s.name] = normal_bf16(w.seed, (_R_W, s.index), s.d_out * s.d_in,
                                  1.0 / np.sqrt(s.d_in)).reshape(s.d_out, s.d_in)
    return w


Q4_GROUP = 128  # inputs per scale of a 4-bit base weight (LORA_Q4_GROUP)


@dataclass
class Q4Weight:
    """A 4-bit base weight: q uint8 [d_out, d_in / 2] (two signed 4-bit
    values per byte, the lower input index in the low nibble), scales fp32
    [d_out, d_in / group]: W[n][k] = scales[n][k // group] * value k of row n."""
    q: np.ndarray
    scales: np.ndarray
    group: int
    d_in: int
    d_out: int


def quantize_q4(Wbits: np.ndarray, group: int = Q4_GROUP) -> Q4Weight:
    """Symmetric 4-bit quantisation of a bf16 weight [d_out, d_in], one scale
    per `group` inputs of a row: scale = max|w| / 7 over the group (1 for an
    all-zero group), q = round-half-even(w / scale) clamped to [-8, 7]."""
    d_out, d_in = Wbits.shape
    assert d_in % group == 0 and d_in % 2 == 0
    wf = bf16_to_f32(Wbits).astype(np.float64).reshape(d_out, d_in // group, group)
    scales = (np.abs(wf).max(axis=2) / 7.0).astype(np.float32)
    scales[scales == 0] = 1.0
    q = np.clip(np.rint(wf / scales[:, :, None].astype(np.float64)), -8, 7).astype(np.int8).reshape(d_out, d_in)
    nib = (q & 0xF).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return Q4Weight(packed, scales, group, d_in, d_out)


def add_base_weights_q4(w: Workload, group: int = Q4_GROUP) -> Workload:
    """4-bit base weights for every projection: the bf16 draws of
    add_base_weights quantised by quantize_q4."""
    add_base_weights(w)
    w.W = {name: quantize_q4(W, group) for name, W in w.W.items()}
    return w


def fused_layer_q4(seed=8, rank=64, rows=128):
    """fused_layer with 4-bit base weights (0.43 GB of weights and scales):
    the pages' INT4 base with BF16 adapters, 8 of the 128 rows base-only."""
    w = full_layer(seed, rank, rows)
    w.ids[::16] = -1  # base-only rows in the same batch
    w.name = f"fused_layer_q4_r{rank}_b{rows}"
    return add_base_weights_q4(w)


def fused_layer(seed=8, rank=64, rows=128):
    """The full 70B layer of full_layer_r64 with its base weights: base
    projection and adapter delta together (1.63 GB of W and 2.65 GB of
    adapters per step)."""
    w = full_layer(seed, rank, rows)
    w.name = f"fused_layer_r{rank}_b{rows}"
    return add_base_weights(w)


def zipf_ids(seed, num_rows, num_slots, s=1.1):
    """Finite Zipf(s) over num_slots popularity ranks by inverse CDF, mapped to
    slot ids through a seeded permutation."""
    k = np.arange(1, num_slots + 1, dtype=np.float64)
    p = k ** (-s)
    cdf = np.cumsum(p / p.sum())
    g = _rng(seed, _R_IDS)
    u = g.random(num_rows)
    rank_idx = np.minimum(np.searchsorted(cdf, u, side="right"), num_slots - 1)
    to_slot = g.permutation(num_slots)
    return to_slot[rank_idx].astype(np.int32)


def zipf_paged(seed=4, num_slots=512, rows=256, s=1.1, ids=None, name=None):
    """512 adapters in fixed pages sized for rank 64, ranks drawn from
    {8,16,32,64}, 256 rows with Zipf(1.1) ids, attention q/k/v/o shapes.
    ``ids`` replaces the drawn row ids (a batch chosen from a queue)."""
    ids = zipf_ids(seed, rows, num_slots, s) if ids is None else np.asarray(ids, np.int32)
    rows = int(ids.size)
    rk = _rng(seed, _R_RANK).choice(np.array([8, 16, 32, 64]), size=num_slots)
    ranks = np.zeros((num_slots, N_MOD), np.int32)
    for n in ("q", "k", "v", "o"):
        ranks[:, MODULE_INDEX[n]] = rk
    placement = _rng(seed, _R_PLACE).permutation(num_slots)
    shapes = {n: SHAPES_70B[n] for n in ("q", "k", "v", "o")}
    return build_workload(name or f"zipf_paged_{num_slots}x{rows}", seed, rows, num_slots, shapes, ids, ranks,
                          x_of=X_OF_70B, x_std=1.0, ab_std=0.02, y_std=1.0,
                          paged_capacity_rank=64, placement=placement)


# The waiting queue the batch former chooses from: requests in arrival order,
# Zipf(1.1) over the same 512 paged adapters, twice the batch.
ZIPF_QUEUE = dict(seed=6, num_rows=512, num_slots=512, s=1.1)
# The former's settings for it ("6. Deep Dive A": cap 32; "The Revision", R1:
# 4 of the 32 held for the tail): a batch of 256 rows, at least 128.
ZIPF_FORMER = dict(max_batch=256, max_distinct=32, min_batch=128, reserved_tail=4)


def zipf_queue():
    """Adapter slot of each waiting request, oldest first."""
    return zipf_ids(**ZIPF_QUEUE)


def prefill(seed=5, rank=16, num_seqs=32, lo=128, hi=2048):
    """32 prefill sequences with lengths uniform in [128, 2048], adapter s for
    sequence s, q and o projections 8192 -> 8192."""
    lens = _rng(seed, _R_LEN).integers(lo, hi + 1, size=num_seqs)
    ids = np.repeat(np.arange(num_seqs, dtype=np.int32), lens)
    ranks = np.zeros((num_seqs, N_MOD), np.int32)
    for n in ("q", "o"):
        ranks[:, MODULE_INDEX[n]] = rank
    shapes = {n: SHAPES_70B[n] for n in ("q", "o")}
    return build_workload(f"prefill_r{rank}_{num_seqs}seq", seed, int(lens.sum()), num_seqs, shapes, ids,
                          ranks, x_of=X_OF_70B, x_std=1.0, ab_std=0.02, y_std=1.0, seq_lens=lens)


def build_workload_for_tests(seed, rows, slots, d_in, d_out, rank, ids, ranks=None, scales=None,
                             x_std=0.02, ab_fill=None, ab_fill_after=None, max_rank=None, fmt=None):
    """A single-projection ("q", table column 0) workload of any small shape.

    ``rank`` gives every slot the same rank unless ``ranks`` [slots, 7] is
    passed.  ``ab_fill(w)`` replaces the random A/B draw; ``ab_fill_after(w)``
    edits A/B after it.
    """
    if ranks is None:
        ranks = np.zeros((slots, N_MOD), np.int32)
        ranks[:, 0] = rank
    w = build_workload(f"test_{rows}x{d_in}x{d_out}", seed, rows, slots, {"q": (d_in, d_out)},
                       np.asarray(ids), ranks, x_of={"q": "x"}, x_std=x_std, ab_std=0.02, y_std=1.0,
                       scales=scales, ab_fill=ab_fill, max_rank=max_rank, fmt=fmt)
    if ab_fill_after is not None:
        ab_fill_after(w)
    return w


WORKLOADS = {
    "tiny": tiny,
    "q_proj_r16": q_proj,
    "full_layer_r64": full_layer,
    "zipf_paged": zipf_paged,
    "prefill_r16": lambda seed=5: prefill(seed, rank=16),
    "prefill_r64": lambda seed=5: prefill(seed, rank=64),
    "full_layer_r64_int8": lambda seed=3: full_layer(seed, fmt=FMT_INT8_ROWS),
    "stacked_layer": stacked_layer,
    "fused_layer_r64": fused_layer,
    "fused_layer_q4_r64": fused_layer_q4,
}


def make_workload(name: str, **kw) -> Workload:
    return WORKLOADS[name](**kw)
