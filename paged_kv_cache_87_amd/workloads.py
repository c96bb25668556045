"""Seeded synthetic inputs for paged attention.

This module only draws inputs: values, block tables, context lengths and the
list of positions written before and during a step.  It holds none of the
method's arithmetic (no slot computation, no attention), so both the HIP
library and the CPU oracle can be fed from it without sharing any code.

Values are N(0, 1) draws (numpy PCG64, seeded), rounded to bf16 by
round-to-nearest-even for bf16 workloads and stored as ``uint16`` bit
patterns; fp32 workloads store ``float32``.  Block tables are slices of one
random permutation of the pool's block ids, taken in sequence order (a shared
prefix first, when there is one).  Unused table entries point at a block that
no sequence owns, so a read past a sequence's last block lands on poison.
"""

from __future__ import annotations

import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"
BF16_NAN_BITS = 0x7FC0


def make_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (torch's CPU cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


_CHUNK = 1 << 22


def _fill_normal(out: np.ndarray, seed: int, tag: int) -> None:
    """N(0,1) float32 draws into ``out`` (1-D), chunk c drawn from its own
    PCG64 stream keyed by (seed, tag, c): the result does not depend on how
    many threads fill it."""
    n = out.shape[0]

    def one(c):
        ss = np.random.SeedSequence(entropy=seed, spawn_key=(tag, c))
        g = np.random.Generator(np.random.PCG64(ss))
        a = c * _CHUNK
        g.standard_normal(size=min(_CHUNK, n - a), dtype=np.float32, out=out[a:a + _CHUNK])

    chunks = range((n + _CHUNK - 1) // _CHUNK)
    if n <= _CHUNK:
        for c in chunks:
            one(c)
        return
    import concurrent.futures as cf
    workers = min(16, len(os.sched_getaffinity(0)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, chunks))


def normal_values(seed: int, tag: int, shape, dtype: str) -> np.ndarray:
    """N(0,1) values of ``shape``: float32, or bf16 bit patterns (RNE)."""
    x = np.empty(int(np.prod(shape)), dtype=np.float32)
    _fill_normal(x, seed, tag)
    x = x.reshape(shape)
    if dtype == F32:
        return x
    if dtype == BF16:
        return round_to_bf16_bits(x)
    raise ValueError(dtype)


def storage_np_dtype(dtype: str):
    return np.float32 if dtype == F32 else np.uint16


def poison_value(dtype: str):
    return np.float32(np.nan) if dtype == F32 else np.uint16(BF16_NAN_BITS)


@dataclass
class Workload:
    """One synthetic paged-attention problem.

    Pools are ``[num_blocks, block_size, num_kv_heads, head_dim]`` per K and
    V.  Before the step, sequence ``s`` has positions ``hist_start[s] ..
    hist_end[s]-1`` written with ``hist_k``/``hist_v`` (packed in sequence
    order).  The step writes ``new_k``/``new_v``: for decode one token per
    sequence at position ``context_lens[s]-1``; for prefill the tokens listed
    by ``q_start_loc`` (the newest ``q_len`` positions of each sequence).
    """

    name: str
    kind: str                      # "decode" | "prefill"
    dtype: str                     # "f32" | "bf16"
    num_blocks: int
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    block_tables: np.ndarray       # int32 [S, max_blocks_per_seq]
    context_lens: np.ndarray       # int32 [S]
    hist_start: np.ndarray         # int32 [S]
    hist_end: np.ndarray           # int32 [S]
    hist_k: np.ndarray             # storage [sum(hist_end-hist_start), Hkv, D]
    hist_v: np.ndarray
    new_k: np.ndarray              # storage [T, Hkv, D]
    new_v: np.ndarray
    q: np.ndarray                  # storage [S (decode) or T (prefill), Hq, D]
    q_start_loc: Optional[np.ndarray] = None   # int32 [S+1] for prefill
    partition_size: int = 0
    pool_fill: str = "nan"         # "nan" (tests) or "zero" (bench)
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def hist_q_start_loc(self) -> np.ndarray:
        """``[S+1]`` offsets of each sequence's history rows in ``hist_k``."""
        lens = (self.hist_end - self.hist_start).astype(np.int64)
        return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)

    def empty_pool(self) -> np.ndarray:
        shape = (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
        fill = poison_value(self.dtype) if self.pool_fill == "nan" else 0
        pool = np.empty(shape, dtype=storage_np_dtype(self.dtype))
        pool.fill(fill)
        return pool

    def kv_bytes_read(self) -> int:
        """K and V bytes that one pass over every context reads."""
        elt = 4 if self.dtype == F32 else 2
        return int(2 * self.num_kv_heads * self.head_dim * elt * int(self.context_lens.astype(np.int64).sum()))


def _tables(rng, blocks_per_seq, num_blocks, width, shared_prefix_blocks=0):
    """Slices of one permutation of the pool's block ids; the first
    ``shared_prefix_blocks`` ids are shared by every sequence.  One id is kept
    back as the pad entry for unused table slots."""
    perm = rng.permutation(num_blocks).astype(np.int32)
    pad = perm[-1]
    S = len(blocks_per_seq)
    tables = np.full((S, width), pad, dtype=np.int32)
    cursor = shared_prefix_blocks
    prefix = perm[:shared_prefix_blocks]
    for s, nb in enumerate(blocks_per_seq):
        own = nb - shared_prefix_blocks
        if own < 0:
            raise ValueError("sequence shorter than the shared prefix")
        if cursor + own > num_blocks - 1:
            raise ValueError("pool too small for the requested contexts")
        tables[s, :shared_prefix_blocks] = prefix
        tables[s, shared_prefix_blocks:nb] = perm[cursor:cursor + own]
        cursor += own
    return tables


def _ceil_div(a, b):
    return -(-a // b)


def _drawer(seed, dtype, with_values):
    """Value source: successive N(0,1) arrays (tags 1, 2, ...), or (with
    ``with_values=False``, for checks of the tables alone) zero-stride
    placeholders of the right shape that cost no memory."""
    if with_values:
        tags = iter(range(1, 1 << 30))
        return lambda shape: normal_values(seed, next(tags), shape, dtype)
    z = np.zeros((), dtype=storage_np_dtype(dtype))
    return lambda shape: np.broadcast_to(z, shape)


def decode_workload(name, seed, *, dtype, num_q_heads, num_kv_heads, head_dim,
                    block_size, num_blocks, context_lens, width=None,
                    shared_prefix_tokens=0, partition_size=0, pool_fill="nan",
                    scale=None, with_values=True):
    """A decode step: histories of ``context_lens[s]-1`` tokens already in the
    pool, one new token per sequence written in the step, one query row per
    (sequence, query head).  With ``shared_prefix_tokens`` (a multiple of the
    block size) every sequence's first blocks are the same physical blocks,
    written once (by sequence 0)."""
    rng = make_rng(seed)
    context_lens = np.asarray(context_lens, dtype=np.int32)
    S = context_lens.shape[0]
    if shared_prefix_tokens % block_size:
        raise ValueError("shared prefix must be whole blocks")
    if shared_prefix_tokens and int(context_lens.min()) <= shared_prefix_tokens:
        # the step's token would land in a shared block (a copy-on-write write)
        raise ValueError("every context must extend past the shared prefix")
    nblk = [_ceil_div(int(L), block_size) for L in context_lens]
    if width is None:
        width = max(max(nblk), 1) if nblk else 1
    tables = _tables(rng, nblk, num_blocks, width, shared_prefix_tokens // block_size)
    hist_start = np.zeros(S, dtype=np.int32)
    if shared_prefix_tokens:
        hist_start[1:] = shared_prefix_tokens
    hist_end = np.maximum(context_lens - 1, 0).astype(np.int32)
    hist_start = np.minimum(hist_start, hist_end)
    n_hist = int((hist_end - hist_start).astype(np.int64).sum())
    Hkv, D = num_kv_heads, head_dim
    draw = _drawer(seed, dtype, with_values)
    hist_k = draw((n_hist, Hkv, D))
    hist_v = draw((n_hist, Hkv, D))
    new_k = draw((S, Hkv, D))
    new_v = draw((S, Hkv, D))
    q = draw((S, num_q_heads, D))
    return Workload(
        name=name, kind="decode", dtype=dtype, num_blocks=num_blocks,
        block_size=block_size, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, scale=float(scale if scale is not None else 1.0 / np.sqrt(head_dim)),
        block_tables=tables, context_lens=context_lens, hist_start=hist_start,
        hist_end=hist_end, hist_k=hist_k, hist_v=hist_v, new_k=new_k, new_v=new_v,
        q=q, q_start_loc=None, partition_size=partition_size, pool_fill=pool_fill,
        meta={"seed": seed, "shared_prefix_tokens": shared_prefix_tokens},
    )


def prefill_workload(name, seed, *, dtype, num_q_heads, num_kv_heads, head_dim,
                     block_size, num_blocks, context_lens, q_lens=None, width=None,
                     pool_fill="nan", scale=None, with_values=True):
    """A prefill step: sequence ``s`` has ``context_lens[s] - q_lens[s]``
    tokens already in the pool and ``q_lens[s]`` new tokens (default: the
    whole prompt), all written in the step and all attending causally."""
    rng = make_rng(seed)
    context_lens = np.asarray(context_lens, dtype=np.int32)
    S = context_lens.shape[0]
    q_lens = context_lens.copy() if q_lens is None else np.asarray(q_lens, dtype=np.int32)
    nblk = [_ceil_div(int(L), block_size) for L in context_lens]
    if width is None:
        width = max(max(nblk), 1) if nblk else 1
    tables = _tables(rng, nblk, num_blocks, width)
    hist_start = np.zeros(S, dtype=np.int32)
    # more new tokens than the context holds: nothing was written before
    hist_end = np.maximum(context_lens - q_lens, 0).astype(np.int32)
    n_hist = int(hist_end.astype(np.int64).sum())
    T = int(q_lens.astype(np.int64).sum())
    Hkv, D = num_kv_heads, head_dim
    draw = _drawer(seed, dtype, with_values)
    hist_k = draw((n_hist, Hkv, D))
    hist_v = draw((n_hist, Hkv, D))
    new_k = draw((T, Hkv, D))
    new_v = draw((T, Hkv, D))
    q = draw((T, num_q_heads, D))
    q_start_loc = np.concatenate([[0], np.cumsum(q_lens.astype(np.int64))]).astype(np.int32)
    return Workload(
        name=name, kind="prefill", dtype=dtype, num_blocks=num_blocks,
        block_size=block_size, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, scale=float(scale if scale is not None else 1.0 / np.sqrt(head_dim)),
        block_tables=tables, context_lens=context_lens, hist_start=hist_start,
        hist_end=hist_end, hist_k=hist_k, hist_v=hist_v, new_k=new_k, new_v=new_v,
        q=q, q_start_loc=q_start_loc, partition_size=0, pool_fill=pool_fill,
        meta={"seed": seed},
    )


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------

SEED_BASE = 87000


def tiny_decode(pool_fill="nan", with_values=True):
    """Batch 1, 8 query heads over 2 KV heads, head_dim 64, block 16, context
    128 (8 blocks drawn from a shuffled 64-block pool), fp32, scale 1/8."""
    return decode_workload("tiny_decode", SEED_BASE + 1, dtype=F32, num_q_heads=8,
                           num_kv_heads=2, head_dim=64, block_size=16, num_blocks=64,
                           context_lens=[128], scale=0.125, pool_fill=pool_fill,
                           with_values=with_values)


GPT2_BATCHES = (1, 2, 4, 8)
GPT2_CONTEXTS = (119, 503, 1015, 2039)   # nominal 128/512/1024/2048 minus 9: last block holds 7


def gpt2_decode(batch, context, dtype, pool_fill="nan", partition_size=0):
    """GPT-2-small-shaped decode: 12 heads (MHA), head_dim 64, block 16,
    4096-block pool, every sequence at the same context."""
    idx = GPT2_BATCHES.index(batch) * len(GPT2_CONTEXTS) + GPT2_CONTEXTS.index(context)
    seed = SEED_BASE + 200 + idx + (100 if dtype == BF16 else 0)
    return decode_workload(f"gpt2_decode_b{batch}_c{context}_{dtype}", seed, dtype=dtype,
                           num_q_heads=12, num_kv_heads=12, head_dim=64, block_size=16,
                           num_blocks=4096, context_lens=[context] * batch,
                           partition_size=partition_size, pool_fill=pool_fill)


def llama_gqa_decode(pool_fill="nan", partition_size=512, batch=64, max_context=8192,
                     fixed_context=None, with_values=True):
    """Llama-style GQA decode: 32 query / 8 KV heads, head_dim 128, bf16,
    block 16, batch 64, contexts uniform in [1, 8192], 40000-block pool,
    table width 512."""
    rng = make_rng(SEED_BASE + 3)
    if fixed_context is None:
        lens = rng.integers(1, max_context + 1, size=batch).astype(np.int32)
    else:
        lens = np.full(batch, fixed_context, dtype=np.int32)
    name = "llama_gqa_decode" if fixed_context is None else f"llama_gqa_decode_ctx{fixed_context}"
    return decode_workload(name, SEED_BASE + 30, dtype=BF16, num_q_heads=32,
                           num_kv_heads=8, head_dim=128, block_size=16, num_blocks=40000,
                           context_lens=lens, width=max_context // 16,
                           partition_size=partition_size, pool_fill=pool_fill,
                           with_values=with_values)


def batched_prefill(pool_fill="nan", batch=16, lo=256, hi=2048, with_values=True):
    """Batched causal prefill: 32 query / 8 KV heads, head_dim 128, bf16,
    16 prompts with lengths uniform in [256, 2048], block 16, 4096-block
    pool; every prompt token is new in the step."""
    rng = make_rng(SEED_BASE + 4)
    lens = rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    return prefill_workload("batched_prefill", SEED_BASE + 40, dtype=BF16, num_q_heads=32,
                            num_kv_heads=8, head_dim=128, block_size=16, num_blocks=4096,
                            context_lens=lens, pool_fill=pool_fill, with_values=with_values)


def long_context_cow(pool_fill="nan", batch=16, context=32768, prefix=4096,
                     partition_size=512, with_values=True):
    """Long-context split-partition decode with a shared prefix: 32/8 GQA
    heads, head_dim 128, bf16, batch 16, context 32768 of which the first 4096
    tokens (256 blocks) are the same physical blocks in every table; partition
    size 512."""
    return decode_workload("long_context_cow", SEED_BASE + 5, dtype=BF16, num_q_heads=32,
                           num_kv_heads=8, head_dim=128, block_size=16,
                           num_blocks=32768, context_lens=[context] * batch,
                           shared_prefix_tokens=prefix, partition_size=partition_size,
                           pool_fill=pool_fill, with_values=with_values)


__all__ = [
    "F32", "BF16", "BF16_NAN_BITS", "Workload", "make_rng", "round_to_bf16_bits",
    "normal_values", "storage_np_dtype", "poison_value", "decode_workload",
    "prefill_workload", "tiny_decode", "GPT2_BATCHES", "GPT2_CONTEXTS", "gpt2_decode",
    "llama_gqa_decode", "batched_prefill", "long_context_cow",
]
