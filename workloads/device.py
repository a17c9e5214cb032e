"""Copy a seeded ``Workload`` to GPU memory for the HIP library.

Only memory placement and the packing of the adapter table (device addresses
of each slot's factors) happen here; no arithmetic of the method.  Not
imported by ``workloads/__init__`` so that the CPU side never loads torch's
GPU state or the HIP library.
"""
from __future__ import annotations

import numpy as np
import torch

import adapter_gemv_amd as lg

from .gen import FMT_INT8_ROWS, Workload


def bf16_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on ``device``."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def to_bits(t: torch.Tensor) -> np.ndarray:
    """torch.bfloat16 tensor -> uint16 numpy bit patterns (host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


class DeviceWorkload:
    """Device copies of a workload: ids, x, pristine y0, working y, the factor
    pool, the adapter table, segment buffers and a workspace."""

    def __init__(self, w: Workload, device="cuda", ws_extra_rows: int = 0, bound_segments: bool = False):
        """bound_segments: give the calls the batch's distinct adapter count
        (of each column of ``w.stack`` when set), as a host that formed the
        batch would."""
        self.w = w
        self.device = device
        self.ids = torch.from_numpy(np.ascontiguousarray(w.ids, dtype=np.int32)).to(device)
        self.x = {k: bf16_tensor(v, device) for k, v in w.x.items()}
        self.y0 = {k: bf16_tensor(v, device) for k, v in w.y0.items()}
        self.y = {k: v.clone() for k, v in self.y0.items()}
        self.pool = bf16_tensor(w.pool, device)
        self.table_host = self.pack(self.pool.data_ptr())
        self.table = torch.from_numpy(self.table_host.view(np.uint8).reshape(-1).copy()).to(device)
        bound = lg.segment_bound(w.ids if w.stack is None else w.stack, w.num_slots) if bound_segments else 0
        self.seg = lg.Segments(w.num_rows + ws_extra_rows, device, max_segments=bound)
        sum_d_in = sum(m.d_in for m in w.modules)
        self.ws_bytes = lg.workspace_bytes(w.num_rows + ws_extra_rows, w.num_slots, w.max_rank, sum_d_in)
        self.ws = torch.zeros(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.ios = {m.name: lg.ModuleIO(self.x[m.x_name], self.y[m.name]) for m in w.modules}
        # every targeted entry int8: the layer calls size their items for one-byte factors
        cols = [m.index for m in w.modules]
        used = w.ranks[:, cols] > 0
        self.int8_items = bool(used.any() and (w.fmt[:, cols][used] == FMT_INT8_ROWS).all())
        self.mask = lg.module_mask(self.ios, int8_items=self.int8_items)
        self.W = self.lin_ios = None
        if w.W is not None:  # base weights: the fused calls, and a workspace for them
            self.W, self.lin_ios = {}, {}
            for m in w.modules:
                W = w.W[m.name]
                if hasattr(W, "scales"):  # 4-bit weights and their group scales
                    q = torch.from_numpy(np.ascontiguousarray(W.q)).to(device)
                    sc = torch.from_numpy(np.ascontiguousarray(W.scales, dtype=np.float32)).to(device)
                    self.W[m.name] = (q, sc)
                    self.lin_ios[m.name] = lg.LinearQ4IO(self.x[m.x_name], q, sc, self.y[m.name], d_in=m.d_in)
                else:
                    self.W[m.name] = bf16_tensor(W, device)
                    self.lin_ios[m.name] = lg.LinearIO(self.x[m.x_name], self.W[m.name], self.y[m.name])
            nb = lg.linear_workspace_bytes(w.num_rows + ws_extra_rows, w.num_slots, w.max_rank, sum_d_in,
                                           len(w.modules))
            if nb > self.ws_bytes:
                self.ws_bytes = nb
                self.ws = torch.zeros(nb, dtype=torch.uint8, device=device)

    def pack(self, base: int, ranks=None, scales=None) -> np.ndarray:
        w = self.w
        A = np.where(w.a_off >= 0, base + 2 * w.a_off, 0).astype(np.uint64)
        B = np.where(w.b_off >= 0, base + 2 * w.b_off, 0).astype(np.uint64)
        return lg.pack_table(A, B, w.ranks if ranks is None else ranks, w.scales if scales is None else scales,
                             w.fmt)

    def upload_table(self, table_host: np.ndarray):
        self.table.copy_(torch.from_numpy(table_host.view(np.uint8).reshape(-1).copy()).to(self.device))

    def reset_y(self, zero: bool = False):
        for k in self.y:
            if zero:
                self.y[k].zero_()
            else:
                self.y[k].copy_(self.y0[k])

    # ---- the library calls on this workload
    def build_segments(self, stream=None):
        lg.build_segments(self.ids, self.w.num_slots, self.seg, self.ws, stream)

    def apply_layer(self, stream=None):
        lg.apply_layer(self.ios, self.w.num_rows, self.table, self.w.num_slots, self.seg, self.w.max_rank, self.ws,
                       stream, module_mask=self.mask)

    def decode_layer(self, stream=None):
        """Segments and every projection through lora_decode_layer."""
        lg.decode_layer(self.ios, self.w.num_rows, self.ids, self.table, self.w.num_slots, self.seg, self.w.max_rank,
                        self.ws, stream, module_mask=self.mask)

    def decode_launches(self) -> int:
        return lg.decode_layer_launches(self.ios, self.w.num_rows, self.w.num_slots, self.seg, self.w.max_rank,
                                        module_mask=self.mask)

    def step(self, stream=None):
        """One pass of the decode path: segments, then every projection."""
        self.build_segments(stream)
        self.apply_layer(stream)
