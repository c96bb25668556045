"""Run a synthetic workload through libpa.so on the GPU.

Uploads a :class:`~paged_kv_cache_87_amd.workloads.Workload` to device
memory and drives one step through the C-ABI binding: slot mapping of the
step's new tokens, the K/V write into the pools, then decode (with the
partition merge when partitioned) or causal prefill -- the fused read of the
nanoserve Day 19 page (write this step's K/V, then attend over the whole
history through the block table).  torch only holds device memory and
supplies the stream; every step runs in the library's kernels.
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding as pa
from .workloads import BF16, F32, BF16_NAN_BITS, Workload


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Stored values (float32, or bf16 bit patterns in uint16) -> GPU tensor."""
    if dtype == F32:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return t.view(torch.bfloat16)


def to_host_stored(t: torch.Tensor) -> np.ndarray:
    """GPU tensor -> stored values (float32, or bf16 bit patterns as uint16)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def i32(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


# Pool layouts a step can run on: the block layout and how the K and V pools
# are held (separate arrays; K and V of a block side by side; one layer of a
# [2, layers, N, block] pool; one layer of per-layer K and V arrays).
POOL_LAYOUTS = {
    "token": ("token", "separate"),
    "head": ("head", "separate"),
    "unified_token": ("token", "unified"),
    "unified_head": ("head", "unified"),
    "layers_token": ("token", "layers"),
    "layers_head": ("head", "per_layer"),
}
POOL_LAYERS, POOL_LAYER = 3, 1


class GpuStep:
    """Device-resident copy of a workload, ready to run its step."""

    def __init__(self, w: Workload, device="cuda", partition_size=None, layout="token"):
        self.w = w
        self.device = device
        self.partition_size = w.partition_size if partition_size is None else partition_size
        self.layout = layout
        tdt = torch.float32 if w.dtype == F32 else torch.bfloat16
        self.storage = [self._filled(shape, tdt) for shape in self._storage_shapes(layout)]
        self.k_cache, self.v_cache = self._views(layout, self.storage)
        self.pool = pa.KVPool(self.k_cache, self.v_cache, POOL_LAYOUTS[layout][0])
        self.block_tables = i32(w.block_tables, device)
        self.context_lens = i32(w.context_lens, device)
        self.seqs = pa.SeqDesc(self.block_tables, self.context_lens, w.max_context_len)
        self.q = to_device(w.q, w.dtype, device)
        # NaN until a kernel writes it, so a row the kernels skip cannot pass
        # for a result left in reused memory
        self.out = torch.full_like(self.q, float("nan"))
        self.new_k = to_device(w.new_k, w.dtype, device)
        self.new_v = to_device(w.new_v, w.dtype, device)
        self.slots = torch.full((w.new_k.shape[0],), -7, dtype=torch.int64, device=device)
        self.q_start_loc = None if w.q_start_loc is None else i32(w.q_start_loc, device)
        self.max_q_len = 0
        if w.q_start_loc is not None:
            self.max_q_len = int(np.diff(w.q_start_loc).max()) if w.num_seqs else 0
        self.workspace = pa.decode_workspace(self.pool, self.seqs, w.num_q_heads,
                                             self.partition_size,
                                             device) if w.kind == "decode" else None

    def _filled(self, shape, tdt):
        w = self.w
        if w.pool_fill != "nan":
            return torch.zeros(shape, dtype=tdt, device=self.device)
        if w.dtype == F32:
            return torch.full(shape, float("nan"), dtype=tdt, device=self.device)
        return torch.full(shape, BF16_NAN_BITS, dtype=torch.int16,
                          device=self.device).view(torch.bfloat16)

    def _storage_shapes(self, layout):
        w = self.w
        N, B, H, D = w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim
        blk = (B, H, D) if POOL_LAYOUTS[layout][0] == "token" else (H, B, D)
        kind = POOL_LAYOUTS[layout][1]
        if kind == "separate":          # one [N, block] array each for K and V
            return [(N, *blk), (N, *blk)]
        if kind == "unified":           # K and V of a block side by side
            return [(N, 2, *blk)]
        if kind == "layers":            # [2, layers, N, block], one layer used
            return [(2, POOL_LAYERS, N, *blk)]
        return [(POOL_LAYERS, N, *blk), (POOL_LAYERS, N, *blk)]   # per-layer K and V arrays

    @staticmethod
    def _views(layout, st):
        kind = POOL_LAYOUTS[layout][1]
        if kind == "separate":
            return st[0], st[1]
        if kind == "unified":
            return st[0][:, 0], st[0][:, 1]
        if kind == "layers":
            return st[0][0, POOL_LAYER], st[0][1, POOL_LAYER]
        return st[0][POOL_LAYER], st[1][POOL_LAYER]

    # -- setup: history written before the step ------------------------------
    def write_history(self):
        w = self.w
        n = int(w.hist_k.shape[0])
        if n == 0:
            return
        hist_end = i32(w.hist_end, self.device)
        hist_qsl = i32(w.hist_q_start_loc, self.device)
        seqs = pa.SeqDesc(self.block_tables, hist_end, int(w.hist_end.max()))
        slots = torch.empty(n, dtype=torch.int64, device=self.device)
        pa.pa_slot_mapping(self.pool, seqs, slots, q_start_loc=hist_qsl)
        # write in chunks so the host->device copies of very long histories stay bounded
        chunk = 1 << 18
        for a in range(0, n, chunk):
            b = min(n, a + chunk)
            k = to_device(w.hist_k[a:b], w.dtype, self.device)
            v = to_device(w.hist_v[a:b], w.dtype, self.device)
            pa.pa_write_kv(self.pool, k, v, slots[a:b])
        torch.cuda.synchronize()

    # -- the step ------------------------------------------------------------
    def slot_mapping(self):
        if self.w.kind == "decode":
            return pa.pa_slot_mapping(self.pool, self.seqs, self.slots)
        return pa.pa_slot_mapping(self.pool, self.seqs, self.slots, q_start_loc=self.q_start_loc)

    def write(self):
        pa.pa_write_kv(self.pool, self.new_k, self.new_v, self.slots)

    def append(self):
        """Decode step's slot mapping and write in one launch."""
        pa.pa_append_kv(self.pool, self.seqs, self.new_k, self.new_v, self.slots)

    def decode_step(self):
        """Decode step in one launch: the write of the new token's K/V and the
        decode (pa_decode_step)."""
        w = self.w
        return pa.pa_decode_step(self.pool, self.seqs, self.new_k, self.new_v, self.q, self.out,
                                 w.scale, self.partition_size, self.workspace, self.slots)

    def attend(self, partition_size=None):
        w = self.w
        if w.kind == "decode":
            ps = self.partition_size if partition_size is None else partition_size
            ws = self.workspace
            if partition_size is not None and partition_size != self.partition_size:
                ws = pa.decode_workspace(self.pool, self.seqs, w.num_q_heads, ps, self.device)
            return pa.pa_decode(self.pool, self.seqs, self.q, self.out, w.scale, ps, ws)
        return pa.pa_prefill(self.pool, self.seqs, self.q, self.out, self.q_start_loc,
                             self.max_q_len, w.scale)

    def step(self):
        self.slot_mapping()
        self.write()
        return self.attend()

    # -- results on the host -----------------------------------------------------
    def out_f64(self) -> np.ndarray:
        return self.out.float().cpu().numpy().astype(np.float64)

    def pools_stored(self):
        """K and V pools as stored values, [num_blocks, block_size, Hkv, D]
        whatever the layout."""
        k, v = to_host_stored(self.k_cache), to_host_stored(self.v_cache)
        if POOL_LAYOUTS[self.layout][0] == "head":
            k, v = k.transpose(0, 2, 1, 3), v.transpose(0, 2, 1, 3)
        return np.ascontiguousarray(k), np.ascontiguousarray(v)


def run_workload(w: Workload, partition_size=None, layout="token") -> GpuStep:
    g = GpuStep(w, partition_size=partition_size, layout=layout)
    g.write_history()
    g.step()
    torch.cuda.synchronize()
    return g


__all__ = ["GpuStep", "run_workload", "POOL_LAYOUTS", "to_device", "to_host_stored", "i32", "BF16", "F32"]
