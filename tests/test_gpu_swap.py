"""GPU parity of the block swap between the device pool and a pinned host
pool, through the C ABI: the tiered oracle decides which blocks move where,
the library moves them, and both pools are compared with the oracle's numpy
mirror bit for bit after every call; then a decode over blocks that went
out to the host and came back matches the decode before, bit for bit.
Needs an MI355X and the built libpa.so."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import announce, need_gpu
from oracle.offload import CPU, GPU, NONE, OffloadError, TieredBlockManager, swap_copy
from paged_kv_cache_87_amd import binding as pa
from paged_kv_cache_87_amd import runner
from paged_kv_cache_87_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _pinned(a: np.ndarray, dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if dtype == wl.BF16
                         else np.ascontiguousarray(a, dtype=np.float32))
    t = t.pin_memory()
    return t.view(torch.bfloat16) if dtype == wl.BF16 else t


def _stored(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.mark.parametrize("dtype,hkv,d", [(wl.BF16, 8, 128), (wl.F32, 2, 64), (wl.BF16, 1, 64)])
def test_swap_stream_bit_exact(dtype, hkv, d):
    n_gpu, n_cpu, shape = 40, 24, (16, hkv, d)
    rng = np.random.Generator(np.random.PCG64(4242 + hkv))
    announce(f"swap stream {dtype} {hkv}x{d}")
    m = TieredBlockManager(n_gpu, n_cpu)
    poison = wl.poison_value(dtype)
    sdt = wl.storage_np_dtype(dtype)
    mirror = {GPU: [np.full((n_gpu, *shape), poison, dtype=sdt) for _ in range(2)],
              CPU: [np.full((n_cpu, *shape), poison, dtype=sdt) for _ in range(2)]}
    dev = [runner.to_device(a, dtype) for a in mirror[GPU]]
    host = [_pinned(a, dtype) for a in mirror[CPU]]
    pool = pa.KVPool(*dev)
    seed = 0
    moves = 0
    for step in range(60):
        live = [i for i, (t, _) in enumerate(m.mapping) if t != NONE]
        on = {t: [i for i in live if m.mapping[i][0] == t] for t in (GPU, CPU)}
        r = int(rng.integers(0, 4))
        try:
            if r == 0:
                # new blocks get fresh data on whichever tier backs them
                for lid in m.allocate(int(rng.integers(1, 6))):
                    t, p = m.mapping[lid]
                    seed += 1
                    for j in range(2):
                        val = wl.normal_values(900 + seed, j, shape, dtype)
                        mirror[t][j][p] = val
                        if t == GPU:
                            dev[j][p] = runner.to_device(val, dtype)
                        else:
                            host[j][p] = _pinned(val, dtype)
            elif r == 1 and live:
                ids = rng.choice(live, size=int(rng.integers(1, max(2, len(live) // 3))),
                                 replace=False)
                m.free_blocks([int(i) for i in ids])
            elif r in (2, 3):
                src, dst = (GPU, CPU) if r == 2 else (CPU, GPU)
                if not on[src]:
                    continue
                ids = [int(i) for i in rng.choice(on[src], size=int(rng.integers(
                    1, len(on[src]) + 1)), replace=False)]
                pairs = m.swap_out(ids) if r == 2 else m.swap_in(ids)
                swap_copy(*mirror[src], *mirror[dst], pairs)
                gpu_ids = [p[0] if r == 2 else p[1] for p in pairs]
                cpu_ids = [p[1] if r == 2 else p[0] for p in pairs]
                pa.pa_swap_blocks(pool, host[0], host[1], runner.i32(gpu_ids),
                                  runner.i32(cpu_ids), pa.PA_SWAP_OUT if r == 2 else pa.PA_SWAP_IN)
                torch.cuda.synchronize()
                moves += len(pairs)
        except OffloadError as e:
            assert e.kind == "no_blocks"
        for j in range(2):
            assert runner.to_host_stored(dev[j]).tobytes() == mirror[GPU][j].tobytes(), step
            assert _stored(host[j]).tobytes() == mirror[CPU][j].tobytes(), step
    assert moves > 40


def test_out_of_pool_ids_are_skipped():
    dtype, shape = wl.BF16, (16, 2, 64)
    announce("swap skips out-of-pool ids")
    k = wl.normal_values(77, 1, (8, *shape), dtype)
    v = wl.normal_values(77, 2, (8, *shape), dtype)
    hk = np.zeros((4, *shape), dtype=k.dtype)
    hv = hk.copy()
    dev = pa.KVPool(runner.to_device(k, dtype), runner.to_device(v, dtype))
    host = [_pinned(hk, dtype), _pinned(hv, dtype)]
    pa.pa_swap_blocks(dev, *host, runner.i32([5, -1, 8, 2]), runner.i32([0, 1, 2, 4]),
                      pa.PA_SWAP_OUT)
    torch.cuda.synchronize()
    hk[0], hv[0] = k[5], v[5]                   # only the first pair is inside both pools
    assert _stored(host[0]).tobytes() == hk.tobytes()
    assert _stored(host[1]).tobytes() == hv.tobytes()


def test_pageable_host_pool_is_refused():
    dtype, shape = wl.BF16, (16, 2, 64)
    announce("swap refuses pageable memory")
    dev = pa.KVPool(torch.zeros((8, *shape), dtype=torch.bfloat16, device="cuda"),
                    torch.zeros((8, *shape), dtype=torch.bfloat16, device="cuda"))
    pageable = torch.zeros((4, *shape), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pa.pa_swap_blocks(dev, pageable, pageable, runner.i32([0]), runner.i32([0]),
                          pa.PA_SWAP_OUT)
    # past the binding's check: the library itself refuses, before any launch
    import ctypes
    hp = pa.PaKVPool(pageable.data_ptr(), pageable.data_ptr(), 4, 16, 2, 64, pa.PA_BF16)
    cp = dev.c()
    ids = runner.i32([0])
    st = pa.load_library().pa_swap_blocks(ctypes.byref(cp), ctypes.byref(hp), ids.data_ptr(),
                                          ids.data_ptr(), 1, pa.PA_SWAP_OUT, None)
    assert st == pa.PA_ERR_INVALID_ARG
    assert "pinned" in pa.load_library().pa_last_error().decode()
    # device memory passed as the host pool is refused too
    hp = dev.c()
    st = pa.load_library().pa_swap_blocks(ctypes.byref(cp), ctypes.byref(hp), ids.data_ptr(),
                                          ids.data_ptr(), 1, pa.PA_SWAP_IN, None)
    assert st == pa.PA_ERR_INVALID_ARG


@pytest.mark.parametrize("partition_size", [0, 256])
def test_decode_after_swap_round_trip_is_bitwise_equal(partition_size):
    """Sequences 1 and 3 go out to the host; their device blocks are
    overwritten with NaN by other data; they come back into other device
    blocks (the FIFO order of the tiered manager), the block table follows,
    and the decode gives the same bits as before."""
    w = wl.decode_workload("swap_decode", 78, dtype=wl.BF16, num_q_heads=32, num_kv_heads=8,
                           head_dim=128, block_size=16, num_blocks=512,
                           context_lens=[300, 1000, 17, 777, 2048], width=160,
                           partition_size=partition_size)
    announce(f"{w.name} partition={partition_size}")
    g = runner.run_workload(w)
    before = g.out.clone()
    tab = g.block_tables.cpu().numpy().copy()
    # the tiered manager tracks every pool block: logical id == device block id
    # at the start; blocks no table entry names go back to the free deque
    m = TieredBlockManager(w.num_blocks, 256)
    m.allocate(w.num_blocks)
    m.free_blocks(sorted(set(range(w.num_blocks)) - set(int(b) for b in tab.ravel())))
    nblk = [(int(c) + 15) // 16 for c in w.context_lens]
    moved = {s: [int(b) for b in tab[s, :nblk[s]]] for s in (1, 3)}
    hk = torch.empty((256, 16, 8, 128), dtype=torch.bfloat16).pin_memory()
    hv = torch.empty_like(hk).pin_memory()
    for s, lids in moved.items():
        pairs = m.swap_out(lids)
        pa.pa_swap_blocks(g.pool, hk, hv, runner.i32([p[0] for p in pairs]),
                          runner.i32([p[1] for p in pairs]), pa.PA_SWAP_OUT)
    torch.cuda.synchronize()
    assert all(m.mapping[lid][0] == CPU for lids in moved.values() for lid in lids)
    # the device blocks they left are scribbled over, as a reuse would
    gone = [b for lids in moved.values() for b in lids]
    g.pool.k_cache[gone] = float("nan")
    g.pool.v_cache[gone] = float("nan")
    # the first free device blocks go to someone else, so the swap in lands elsewhere
    m.allocate(7)
    for s, lids in moved.items():
        pairs = m.swap_in(lids)
        pa.pa_swap_blocks(g.pool, hk, hv, runner.i32([p[1] for p in pairs]),
                          runner.i32([p[0] for p in pairs]), pa.PA_SWAP_IN)
        tab[s, :nblk[s]] = [m.mapping[lid][1] for lid in lids]
    torch.cuda.synchronize()
    assert all(tab[s, i] != moved[s][i] for s in moved for i in range(nblk[s]))
    g.seqs = pa.SeqDesc(runner.i32(tab), g.context_lens, int(max(w.context_lens)))
    g.out.zero_()
    pa.pa_decode(g.pool, g.seqs, g.q, g.out, w.scale, partition_size, g.workspace)
    torch.cuda.synchronize()
    assert torch.equal(g.out.view(torch.int16), before.view(torch.int16))
