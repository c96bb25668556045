"""Drive one synthetic workload through the CPU oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/paged_attention.py``).  The workload
object is read by attribute only (``block_tables``, ``context_lens``,
``hist_*``, ``new_*``, ``q`` ...); nothing from the HIP package is imported.

A step is: slot mapping of the step's new tokens, the K/V write into the
pools, then decode attention (one query row per sequence) or causal prefill
(all new tokens), in that order -- the fused read of the nanoserve Day 19
page ("What I added today": write this step's K/V, then attend over the whole
history through the block table).
"""

from __future__ import annotations

import numpy as np

from . import paged_attention as pa


def build_pools(w):
    """Fresh K and V pools (poison- or zero-filled) with every sequence's
    pre-step history written through the oracle's own slot mapping."""
    k_cache = w.empty_pool()
    v_cache = w.empty_pool()
    if w.hist_k.shape[0]:
        slots = pa.slot_mapping(w.block_tables, w.hist_end, w.block_size,
                                q_start_loc=w.hist_q_start_loc)
        pa.write_kv_cache(k_cache, v_cache, w.hist_k, w.hist_v, slots)
    return k_cache, v_cache


def step_slots(w):
    if w.kind == "decode":
        return pa.slot_mapping(w.block_tables, w.context_lens, w.block_size)
    return pa.slot_mapping(w.block_tables, w.context_lens, w.block_size,
                           q_start_loc=w.q_start_loc)


def write_step(w, k_cache, v_cache):
    slots = step_slots(w)
    pa.write_kv_cache(k_cache, v_cache, w.new_k, w.new_v, slots)
    return slots


def attend(w, k_cache, v_cache):
    """Attention output (float64) after the step's write."""
    if w.kind == "decode":
        return pa.decode(w.q, k_cache, v_cache, w.block_tables, w.context_lens, w.scale, w.dtype)
    return pa.prefill(w.q, k_cache, v_cache, w.block_tables, w.context_lens, w.q_start_loc,
                      w.scale, w.dtype)


def run_step(w):
    """Pools, slots and attention output for one step of ``w``."""
    k_cache, v_cache = build_pools(w)
    slots = write_step(w, k_cache, v_cache)
    out = attend(w, k_cache, v_cache)
    return k_cache, v_cache, slots, out


__all__ = ["build_pools", "step_slots", "write_step", "attend", "run_step", "np"]
