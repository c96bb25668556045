"""CPU oracle for paged attention (numpy, float64).

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously correct
statement of what the paged-attention path computes.  Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP library and imports nothing from
the ``paged_kv_cache_87_amd`` package; the two meet only on inputs produced by
the seeded generators in ``paged_kv_cache_87_amd.workloads``.

Sources (three web pages on paged KV caches):

* "JuliaPagedAttn" README: sections "Block Layout", "Online Softmax",
  "Copy-on-Write", "API Reference" (``write_kv_cache!``,
  ``paged_attention_cpu!``), "Running Tests" and "Project Structure"
  (``cache_layout.jl``: slot mapping).
* "Pico-vLLM 开发日志 #5 Paged Attention": the block-manager listing (pool
  tensor ``[2, num_layers, num_blocks, block_size, num_kv_heads, head_dim]``),
  ``get_block_table`` (int32 physical ids) and the note on the +1 context
  length (the current token's K/V already exist when attending).
* "nanoserve Day 19: the fused paged read wired into attention": "What I
  added today" (write this step's K/V to its slots, then attend over the
  whole history through the block table), "Why it matters" (the paged read
  equals gather-then-normal-SDPA), "What I learned" item 4 (GQA: the cache
  stores the compact KV heads, the repeat to query heads happens at read
  time) and "Diagram" (``slot_mapping``).

Conventions (readings where the pages are silent; each is pinned by a test):

* Pool: one array per K and V, row-major ``[num_blocks, block_size,
  num_kv_heads, head_dim]`` (the Pico-vLLM pool with the leading ``[2,
  num_layers]`` indices fixed).  bf16 storage is held as ``uint16`` bit
  patterns; fp32 storage as ``float32``.
* Slot: ``slot = block_table[s][pos // block_size] * block_size +
  pos % block_size`` -- the flat index of the token row in the pool viewed
  as ``[num_blocks * block_size, num_kv_heads, head_dim]`` (0-based).
* GQA: query head ``h`` reads KV head ``h // n_rep`` with ``n_rep =
  num_q_heads // num_kv_heads`` (repeat-interleave of the compact heads).
* ``context_lens[s]`` counts every token already in the pool, including the
  one written this step.  A context length of 0 gives an all-zero output.
* Prefill query ``i`` of a sequence with ``q_len`` new tokens sits at
  position ``context_len - q_len + i`` and attends to positions
  ``0 .. context_len - q_len + i`` (causal, diagonal included); a query
  whose position is negative (more new tokens than the context holds) sees
  no key and gives zeros.

Arithmetic: stored values are upcast exactly to float64 and every sum,
exponential and division is done in float64.  The softmax is the plain
two-pass form (maximum first, then exponentials and their sum); the method on
the pages (running max / running sum) reaches the same value in exact
arithmetic.
"""

from __future__ import annotations

import numpy as np

F32 = "f32"
BF16 = "bf16"


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: a bf16 is the high half of an IEEE
    binary32, so shifting the 16 bits up by 16 gives the binary32 with the
    same value."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored array (float32 array or bf16 bits)."""
    if dtype == F32:
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f64(stored)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# slot mapping and the K/V write
# --------------------------------------------------------------------------

def token_positions(context_lens, q_start_loc=None):
    """(sequence, position) of each new token.

    Without ``q_start_loc`` there is one new token per sequence, the last one
    of its context (decode).  With ``q_start_loc`` (``[S+1]`` prefix offsets
    into the token list) sequence ``s`` owns tokens ``q_start_loc[s] ..
    q_start_loc[s+1]-1``; they are its newest ``q_len`` positions.
    """
    context_lens = [int(x) for x in np.asarray(context_lens).reshape(-1)]
    out = []
    if q_start_loc is None:
        for s, L in enumerate(context_lens):
            out.append((s, L - 1))
        return out
    q_start_loc = [int(x) for x in np.asarray(q_start_loc).reshape(-1)]
    for s, L in enumerate(context_lens):
        q_len = q_start_loc[s + 1] - q_start_loc[s]
        for i in range(q_len):
            out.append((s, L - q_len + i))
    return out


def slot_mapping(block_tables, context_lens, block_size, q_start_loc=None):
    """Flat pool slot of every new token (int64); -1 where the position has
    no block (negative position, or past the table's width).

    A position ``pos`` of sequence ``s`` lives in logical block
    ``pos // block_size`` at offset ``pos % block_size``; the block table maps
    the logical block to a physical block id, and the slot is that physical
    block's first row plus the offset (JuliaPagedAttn "Project Structure":
    slot mapping in the cache layout; nanoserve Day 19 "Diagram":
    ``slot_mapping``).
    """
    block_tables = np.asarray(block_tables)
    width = block_tables.shape[1] if block_tables.ndim == 2 else 0
    slots = []
    for s, pos in token_positions(context_lens, q_start_loc):
        if pos < 0:
            slots.append(-1)
            continue
        logical_block = pos // block_size
        offset = pos % block_size
        if logical_block >= width:
            slots.append(-1)
            continue
        physical_block = int(block_tables[s, logical_block])
        slots.append(physical_block * block_size + offset)
    return np.asarray(slots, dtype=np.int64)


def write_kv_cache(k_cache, v_cache, k_new, v_new, slots):
    """Scatter each new token's K and V rows ``[num_kv_heads, head_dim]``
    into its slot, in place, copying the stored values unchanged (JuliaPagedAttn
    "API Reference", ``write_kv_cache!``; nanoserve Day 19 "What I added
    today": the write scatters this step's K/V to its slots).  Slots below 0
    are padding and are skipped."""
    block_size = k_cache.shape[1]
    for t, slot in enumerate(np.asarray(slots).reshape(-1)):
        slot = int(slot)
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        k_cache[block, offset] = k_new[t]
        v_cache[block, offset] = v_new[t]


# --------------------------------------------------------------------------
# reading the history
# --------------------------------------------------------------------------

def gather_history(cache, block_table_row, context_len):
    """Contiguous history ``[context_len, num_kv_heads, head_dim]`` of one
    sequence, block by block through its table (the gather read that
    nanoserve Day 19 "Why it matters" compares the paged read against)."""
    block_size = cache.shape[1]
    n_blocks = -(-int(context_len) // block_size)
    parts = [cache[int(block_table_row[j])] for j in range(n_blocks)]
    if not parts:
        return cache[:0, 0]
    return np.concatenate(parts, axis=0)[: int(context_len)]


def read_through_table(cache, block_table_row, context_len):
    """Same history as ``gather_history`` but read token by token: token ``t``
    is row ``t % block_size`` of physical block ``block_table[t //
    block_size]``.  It materialises nothing block-wise; it is the independent
    second read path that must agree byte for byte with the gather."""
    block_size = cache.shape[1]
    out = np.empty((int(context_len),) + cache.shape[2:], dtype=cache.dtype)
    for t in range(int(context_len)):
        out[t] = cache[int(block_table_row[t // block_size]), t % block_size]
    return out


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def sdpa_two_pass(q, keys, values, scale):
    """Softmax attention of one query row over a contiguous history, float64.

    ``q`` is ``[head_dim]``, ``keys``/``values`` are ``[n, head_dim]``.
    First pass: the maximum score.  Second pass: ``exp(score - max)``, their
    sum, and the weighted sum of value rows.  An empty history gives zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(q.shape[-1], dtype=np.float64)
    scores = scale * (keys @ q)
    m = scores.max()
    p = np.exp(scores - m)
    return (p @ values) / p.sum()


def kv_head_of(q_head, num_q_heads, num_kv_heads):
    """GQA: query heads are grouped ``n_rep`` at a time onto one KV head (the
    compact KV heads are repeated to the query heads at read time)."""
    n_rep = num_q_heads // num_kv_heads
    return q_head // n_rep


def _check_heads(num_q_heads, num_kv_heads):
    if num_kv_heads <= 0 or num_q_heads % num_kv_heads != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype):
    """Decode attention: one query row per (sequence, query head) over that
    sequence's whole history, read through the block table (JuliaPagedAttn
    "API Reference", ``paged_attention_cpu!(O, Q, K_cache, V_cache,
    block_table, context_lengths, layer, scale)``; nanoserve Day 19).

    ``q`` is ``[S, Hq, D]`` in storage format, pools ``[N, B, Hkv, D]``.
    Returns float64 ``[S, Hq, D]``.
    """
    S, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    _check_heads(Hq, Hkv)
    qf = to_f64(q, dtype)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        L = int(context_lens[s])
        keys = to_f64(gather_history(k_cache, block_tables[s], L), dtype)
        vals = to_f64(gather_history(v_cache, block_tables[s], L), dtype)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[s, h] = sdpa_two_pass(qf[s, h], keys[:, g, :], vals[:, g, :], scale)
    return out


def prefill(q, k_cache, v_cache, block_tables, context_lens, q_start_loc, scale, dtype):
    """Causal attention for every new token of every sequence (JuliaPagedAttn
    "Features": batched prefill, all prompt positions in one call).

    ``q`` is ``[T, Hq, D]`` (tokens of sequence ``s`` at ``q_start_loc[s] ..
    q_start_loc[s+1]-1``).  Query ``i`` of sequence ``s`` sits at position
    ``p = context_lens[s] - q_len + i`` and attends to positions ``0..p``
    (causal, its own position included).  A query whose position is negative
    (more new tokens than the context holds) sees no key and gives zeros.
    Returns float64 ``[T, Hq, D]``.

    Per sequence and query head, the scores of all its queries against all
    its keys are one matrix product; keys after a query's position are left
    out of that query's row; then each row takes the same two-pass softmax as
    ``sdpa_two_pass`` (row maximum over the visible keys, exponentials and
    their sum, the weighted sum of value rows).
    """
    T, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    _check_heads(Hq, Hkv)
    qf = to_f64(q, dtype)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    positions = token_positions(context_lens, q_start_loc)
    q_start_loc = np.asarray(q_start_loc)
    for s in range(len(context_lens)):
        lo, hi = int(q_start_loc[s]), int(q_start_loc[s + 1])
        if hi == lo:
            continue
        L = int(context_lens[s])
        keys = to_f64(gather_history(k_cache, block_tables[s], L), dtype)
        vals = to_f64(gather_history(v_cache, block_tables[s], L), dtype)
        pos = np.array([positions[t][1] for t in range(lo, hi)], dtype=np.int64)
        # key t is visible to a query at position p when t <= p
        visible = np.arange(L)[None, :] <= pos[:, None]
        rows = np.nonzero(visible.any(axis=1))[0]       # queries that see a key
        if rows.size == 0:
            continue
        visible = visible[rows]
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            scores = scale * (qf[lo + rows, h] @ keys[:, g, :].T)
            m = np.where(visible, scores, -np.inf).max(axis=1, keepdims=True)
            p = np.exp(np.where(visible, scores - m, -np.inf))
            out[lo + rows, h] = (p @ vals[:, g, :]) / p.sum(axis=1, keepdims=True)
    return out


# --------------------------------------------------------------------------
# split-context decode: per-partition statistics and their log-sum-exp merge
# --------------------------------------------------------------------------

def partition_stats(q, keys, values, scale, partition_size):
    """Split a history into consecutive partitions of ``partition_size``
    tokens and return, per partition ``j``, the maximum score ``m_j``, the sum
    ``l_j = sum exp(score - m_j)`` and the partition's normalised output
    ``o_j = sum exp(score - m_j) v / l_j`` (float64 arrays ``[P]``, ``[P]``,
    ``[P, D]``).  The running max / running sum of the online softmax on the
    JuliaPagedAttn page ("Online Softmax") are exactly these quantities for a
    prefix; a partition is a prefix of its own slice."""
    q = np.asarray(q, dtype=np.float64)
    n = keys.shape[0]
    ms, ls, os_ = [], [], []
    for start in range(0, n, partition_size):
        k = keys[start:start + partition_size]
        v = values[start:start + partition_size]
        scores = scale * (k @ q)
        m = scores.max()
        p = np.exp(scores - m)
        ms.append(m)
        ls.append(p.sum())
        os_.append((p @ v) / p.sum())
    D = values.shape[-1]
    return (np.asarray(ms, dtype=np.float64), np.asarray(ls, dtype=np.float64),
            np.asarray(os_, dtype=np.float64).reshape(-1, D))


def lse_merge(m, l, o):
    """Merge per-partition softmax statistics: with ``M = max_j m_j`` and
    weights ``w_j = l_j * exp(m_j - M)``, the output is ``sum_j w_j o_j /
    sum_j w_j``.  No partitions gives zeros."""
    m = np.asarray(m, dtype=np.float64)
    if m.size == 0:
        return np.zeros(np.asarray(o).shape[-1], dtype=np.float64)
    M = m.max()
    w = np.asarray(l, dtype=np.float64) * np.exp(m - M)
    return (w @ np.asarray(o, dtype=np.float64)) / w.sum()


# --------------------------------------------------------------------------
# tolerance used by parity tests
# --------------------------------------------------------------------------

def tolerance(dtype: str) -> float:
    """Maximum absolute error allowed between a GPU result and this oracle:
    1e-5 for fp32 inputs, 2e-2 for bf16 inputs accumulated in fp32."""
    return 1e-5 if dtype == F32 else 2e-2


def max_abs_err(gpu_f64: np.ndarray, ref_f64: np.ndarray) -> float:
    if gpu_f64.size == 0:
        return 0.0
    return float(np.max(np.abs(np.asarray(gpu_f64, np.float64) - ref_f64)))


__all__ = [
    "F32", "BF16", "bf16_bits_to_f64", "to_f64", "token_positions", "slot_mapping",
    "write_kv_cache", "gather_history", "read_through_table", "sdpa_two_pass",
    "kv_head_of", "decode", "prefill", "partition_stats", "lse_merge",
    "tolerance", "max_abs_err",
]
