"""pa_decode_noalloc -- the decode without a caller workspace, its split
results in the library's own per-GPU device array -- against pa_decode with
a workspace of the caller's (the same kernels: bit for bit) and against the
CPU oracle (within tolerance), through the C ABI.  Two calls in a row, the
second on a smaller batch, so the array's contents from the first call must
not leak into the second."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import announce, assert_close, need_gpu, oracle_step
from paged_kv_cache_87_amd import binding as pa
from paged_kv_cache_87_amd import runner
from paged_kv_cache_87_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _against_workspace_decode(w):
    announce(f"{w.name} noalloc partition={w.partition_size}")
    g = runner.run_workload(w)                  # pa_decode with its own zeroed workspace
    want = g.out.clone()
    out = torch.full_like(g.q, float("nan"))
    pa.pa_decode_noalloc(g.pool, g.seqs, g.q, out, w.scale, w.partition_size)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), want.view(torch.uint8)), w.name
    _, _, _, out_ref = oracle_step(w)
    assert_close(out.float().cpu().numpy().astype(np.float64), out_ref, w.dtype,
                 w.name + " noalloc")
    return g


def test_noalloc_two_calls_second_smaller():
    rng = np.random.default_rng(760)
    lens = [int(x) for x in rng.integers(1, 2500, size=48)]
    big = wl.decode_workload("noalloc_big", 760, dtype=wl.BF16, num_q_heads=32, num_kv_heads=8,
                             head_dim=128, block_size=16, num_blocks=8192, context_lens=lens,
                             partition_size=64)
    small = wl.decode_workload("noalloc_small", 761, dtype=wl.F32, num_q_heads=8, num_kv_heads=2,
                               head_dim=64, block_size=16, num_blocks=256,
                               context_lens=[3, 100, 700, 17], partition_size=32)
    _against_workspace_decode(big)
    _against_workspace_decode(small)


def test_noalloc_unsplit_and_headline_size():
    """partition 0 (no split: the array is not used) and the 64-sequence
    random-length batch at partition 1024 (the bench's decode)."""
    w = wl.decode_workload("noalloc_unsplit", 762, dtype=wl.BF16, num_q_heads=16, num_kv_heads=4,
                           head_dim=128, block_size=16, num_blocks=512,
                           context_lens=[1, 40, 900, 2000], partition_size=0)
    _against_workspace_decode(w)
    _against_workspace_decode(wl.llama_gqa_decode(partition_size=1024))


def test_noalloc_array_size():
    assert pa.load_library().pa_decode_noalloc_max_bytes() == (256 + 16 * 1024 + 256) * 1024
