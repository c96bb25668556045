"""GPU parity of the copy-on-write write path through the C ABI: the block
copy bit for bit, and a decode step of sequences that share a prefix whose
last block is partly filled, driven by the library's allocator, against the
oracle (oracle allocator, numpy block copy, write, decode).  Needs an MI355X
and the built libpa.so."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.paged_attention as orc
from gpu_common import announce, assert_close, need_gpu
from oracle.allocator import Allocator, copy_blocks
from paged_kv_cache_87_amd import binding as pa
from paged_kv_cache_87_amd import runner
from paged_kv_cache_87_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _pool_pair(num_blocks, hkv, d, dtype, seed):
    k = wl.normal_values(seed, 1, (num_blocks, 16, hkv, d), dtype)
    v = wl.normal_values(seed, 2, (num_blocks, 16, hkv, d), dtype)
    return k, v


@pytest.mark.parametrize("dtype,hkv,d", [(wl.F32, 2, 128), (wl.BF16, 8, 128), (wl.BF16, 1, 64)])
def test_copy_blocks_bit_exact(dtype, hkv, d):
    announce(f"copy_blocks {dtype} {hkv}x{d}")
    k, v = _pool_pair(96, hkv, d, dtype, 71)
    # disjoint pairs (a destination that is also a source races, by contract)
    pairs = [(3, 40), (7, 41), (0, 95), (50, 2), (63, 64)]
    bad = [(-1, 5), (5, 96), (96, 1)]                           # skipped: outside the pool
    kg, vg = runner.to_device(k, dtype), runner.to_device(v, dtype)
    pool = pa.KVPool(kg, vg)
    src = runner.i32([p[0] for p in pairs + bad])
    dst = runner.i32([p[1] for p in pairs + bad])
    pa.pa_copy_blocks(pool, src, dst)
    torch.cuda.synchronize()
    ko, vo = k.copy(), v.copy()
    copy_blocks(ko, vo, pairs)
    assert runner.to_host_stored(kg).tobytes() == ko.tobytes()
    assert runner.to_host_stored(vg).tobytes() == vo.tobytes()


def test_copy_on_write_decode_step():
    """Four sequences share a 100-token prefix (7 blocks, the last holding 4
    tokens).  Each appends one token at position 100: the first three
    writers get copies of the shared partial block, the last one owns it by
    then and writes in place; the full blocks stay shared."""
    dtype, hq, hkv, d, bs = wl.BF16, 8, 2, 128, 16
    nb, width, S, P = 64, 16, 4, 100
    announce("cow decode step")
    lib_alloc, ora = pa.BlockAllocator(nb), Allocator(nb)
    base = lib_alloc.allocate(7)
    assert base == ora.allocate(7)
    for _ in range(S - 1):
        lib_alloc.fork(base)
        ora.fork(base)
    tables = [list(base) + [-1] * (width - 7) for _ in range(S)]
    used = [7] * S
    copies = []
    for s in range(S):
        got = lib_alloc.prepare_write(tables[s], used[s], bs, P, 1, width=width)
        assert got == ora.prepare_write(tables[s], used[s], bs, P, 1, width)
        tables[s], used[s], c = got
        copies += c
    assert [c[0] for c in copies] == [base[6]] * (S - 1)       # three copies of the partial block
    assert tables[S - 1][:7] == base                            # the last writer kept it
    assert all(t[:6] == base[:6] for t in tables)               # full blocks stay shared
    assert [lib_alloc.refcount(b) for b in base] == [S] * 6 + [1]

    pk = wl.normal_values(72, 1, (P, hkv, d), dtype)
    pv = wl.normal_values(72, 2, (P, hkv, d), dtype)
    nk = wl.normal_values(72, 3, (S, hkv, d), dtype)
    nv = wl.normal_values(72, 4, (S, hkv, d), dtype)
    q = wl.normal_values(72, 5, (S, hq, d), dtype)
    prefix_slots = np.array([base[p // bs] * bs + p % bs for p in range(P)], dtype=np.int64)
    lens = np.full(S, P + 1, dtype=np.int32)
    tab = np.array(tables, dtype=np.int32)
    scale = 1.0 / np.sqrt(d)

    # oracle: prefix write, copies, this step's write, decode
    ko = np.full((nb, bs, hkv, d), wl.poison_value(dtype), dtype=wl.storage_np_dtype(dtype))
    vo = ko.copy()
    orc.write_kv_cache(ko, vo, pk, pv, prefix_slots)
    copy_blocks(ko, vo, copies)
    slots_ref = orc.slot_mapping(tab, lens, bs)
    orc.write_kv_cache(ko, vo, nk, nv, slots_ref)
    out_ref = orc.decode(q, ko, vo, tab, lens, scale, dtype)
    for s in range(S):   # each sequence reads the prefix and then its own token
        hist = orc.gather_history(ko, tab[s], P + 1)
        assert hist[:P].tobytes() == pk.tobytes() and hist[P].tobytes() == nk[s].tobytes()

    # library: the same steps on the GPU
    tdt = torch.bfloat16
    kg = torch.empty((nb, bs, hkv, d), dtype=tdt, device="cuda")
    vg = torch.empty_like(kg)
    poison = int(np.array(wl.poison_value(dtype)).view(np.int16))
    kg.view(torch.int16).fill_(poison)
    vg.view(torch.int16).fill_(poison)
    pool = pa.KVPool(kg, vg)
    pa.pa_write_kv(pool, runner.to_device(pk, dtype), runner.to_device(pv, dtype),
                   torch.from_numpy(prefix_slots).cuda())
    pa.pa_copy_blocks(pool, runner.i32([c[0] for c in copies]), runner.i32([c[1] for c in copies]))
    seqs = pa.SeqDesc(runner.i32(tab), runner.i32(lens), P + 1)
    slots = torch.full((S,), -7, dtype=torch.int64, device="cuda")
    pa.pa_slot_mapping(pool, seqs, slots)
    pa.pa_write_kv(pool, runner.to_device(nk, dtype), runner.to_device(nv, dtype), slots)
    qg = runner.to_device(q, dtype)
    out = torch.full_like(qg, float("nan"))   # a skipped row stays NaN
    pa.pa_decode(pool, seqs, qg, out, scale, 0, None)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(), slots_ref)
    assert runner.to_host_stored(kg).tobytes() == ko.tobytes()
    assert runner.to_host_stored(vg).tobytes() == vo.tobytes()
    assert_close(out.float().cpu().numpy().astype(np.float64), out_ref, dtype, "cow decode")
