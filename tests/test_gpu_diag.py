"""The read-bandwidth probe pa_read_checksum (include/pa.h): every output word
is the XOR of the little-endian 32-bit words of its share of the buffer,
checked here against numpy on random bytes, including shares of unequal
length and words whose share is empty."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import announce, need_gpu
from paged_kv_cache_87_amd import binding as pa

pytestmark = pytest.mark.gpu


def expected(host: np.ndarray, num_words: int) -> np.ndarray:
    w = host.view("<u4")
    chunks = host.size // 16
    per = -(-chunks // num_words)
    out = np.zeros(num_words, np.uint32)
    for i in range(num_words):
        lo, hi = min(i * per, chunks) * 4, min((i + 1) * per, chunks) * 4
        if hi > lo:
            out[i] = np.bitwise_xor.reduce(w[lo:hi])
    return out


@pytest.mark.parametrize("nbytes,num_words",
                         [(16 << 20, 1000), ((1 << 20) + 48, 7), (4096, 300), (64 << 20, 8192)])
def test_read_checksum(nbytes, num_words):
    need_gpu()
    announce(f"read_checksum bytes={nbytes} words={num_words}")
    host = np.random.default_rng(nbytes + num_words).integers(0, 256, size=nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    words = torch.full((num_words,), -1, dtype=torch.int32, device="cuda")
    pa.pa_read_checksum(buf, words)
    torch.cuda.synchronize()
    assert np.array_equal(words.cpu().numpy().view(np.uint32), expected(host, num_words))
