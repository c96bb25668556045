"""Block sizes other than 16 (JuliaPagedAttn README, "API Reference":
PagedEngine's block_size; Pico-vLLM #5 Paged Attention, BlockManager's
block_size): slot mapping, the K/V write, decode (whole pairs and split),
bf16 and fp32 prefill, in both block layouts, against the CPU oracle through
the C ABI.  The kernels walk 16-token units: a block of 16 tokens or more
holds whole units, a block of 8 holds half of one."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import announce, assert_close, assert_pools_equal, need_gpu, oracle_step
from paged_kv_cache_87_amd import binding as pa
from paged_kv_cache_87_amd import runner
from paged_kv_cache_87_amd import workloads as wl

pytestmark = pytest.mark.gpu

BLOCK_SIZES = (8, 32, 64, 128, 256)


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _check(w, layout="token", partition_size=None, append=False):
    announce(f"{w.name} layout={layout} partition={partition_size}")
    g = runner.GpuStep(w, layout=layout, partition_size=partition_size)
    g.write_history()
    if append:
        g.append()
    else:
        g.slot_mapping()
        g.write()
    g.attend()
    torch.cuda.synchronize()
    k_ref, v_ref, slots_ref, out_ref = oracle_step(w)
    assert np.array_equal(g.slots.cpu().numpy(), slots_ref), "slot mapping differs"
    assert_pools_equal(g, k_ref, v_ref)
    return assert_close(g.out_f64(), out_ref, w.dtype, f"{w.name} {layout} p={partition_size}")


@pytest.mark.parametrize("block_size", BLOCK_SIZES)
@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("partition_size", [0, 16, 64])
def test_decode_block_sizes(block_size, layout, partition_size):
    lens = [1, 7, 8, 9, 15, 16, 17, 33, 100, 257, 700, 1500]
    nb = sum(-(-L // block_size) for L in lens) + 4
    w = wl.decode_workload(f"decode_b{block_size}", 800 + block_size, dtype=wl.BF16,
                           num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=block_size,
                           num_blocks=nb, context_lens=lens, partition_size=partition_size)
    _check(w, layout=layout, append=partition_size == 16)


@pytest.mark.parametrize("block_size", (8, 32, 128))
def test_decode_block_sizes_f32_gpt2(block_size):
    """fp32, 12 heads of 64 (the GPT-2 shape), contexts ending 7 tokens into a block."""
    lens = [119, 503, 1015, 2039]
    nb = sum(-(-L // block_size) for L in lens) + 4
    w = wl.decode_workload(f"decode_f32_b{block_size}", 820 + block_size, dtype=wl.F32,
                           num_q_heads=12, num_kv_heads=12, head_dim=64, block_size=block_size,
                           num_blocks=nb, context_lens=lens, partition_size=256)
    _check(w)


@pytest.mark.parametrize("block_size", BLOCK_SIZES)
@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_prefill_block_sizes(block_size, dtype):
    lens = [1, 7, 8, 9, 31, 33, 64, 100, 300, 41]
    q_lens = [1, 7, 8, 9, 31, 33, 64, 60, 300, 50]
    nb = sum(-(-L // block_size) for L in lens) + 4
    w = wl.prefill_workload(f"prefill_b{block_size}_{dtype}", 840 + block_size, dtype=dtype,
                            num_q_heads=8, num_kv_heads=2, head_dim=128 if dtype == wl.BF16 else 64,
                            block_size=block_size, num_blocks=nb, context_lens=lens,
                            q_lens=q_lens)
    _check(w)
    _check(w, layout="head")


def test_noalloc_block_size_8():
    lens = [5, 300, 1025, 16]
    w = wl.decode_workload("noalloc_b8", 860, dtype=wl.BF16, num_q_heads=32, num_kv_heads=8,
                           head_dim=128, block_size=8, num_blocks=400, context_lens=lens,
                           partition_size=64)
    announce(w.name)
    g = runner.run_workload(w)
    out = torch.full_like(g.q, float("nan"))
    pa.pa_decode_noalloc(g.pool, g.seqs, g.q, out, w.scale, 64)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), g.out.view(torch.uint8))
