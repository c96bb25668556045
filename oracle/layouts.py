"""CPU oracle for the block layouts of a K/V pool (numpy).

TEST INFRASTRUCTURE ONLY.  Only the test suite may import it.  It shares no
code with the library and imports nothing from the ``paged_kv_cache_87_amd``
package.

The oracle's pools are logical arrays ``[num_blocks, block_size,
num_kv_heads, head_dim]`` (the Pico-vLLM pool tensor with its K/V and layer
indices fixed, "核心数据结构和设计模式").  The layouts below say where each
element of a block sits in memory:

* token-major: the same order, ``[block_size, num_kv_heads, head_dim]``;
* head-major: JuliaPagedAttn "Block Layout" stores a block's K (and V) as
  ``[head_dim, block_size, num_kv_heads]`` in Julia's column-major order,
  i.e. element (d, t, h) at offset d + D (t + B h), which is the row-major
  array ``[num_kv_heads, block_size, head_dim]``.
"""

from __future__ import annotations

import numpy as np


def block_offset(t: int, h: int, d: int, B: int, H: int, D: int, layout: str) -> int:
    """Element offset of (token t, KV head h, element d) inside one block."""
    if layout == "token":
        return (t * H + h) * D + d
    if layout == "head":
        return d + D * (t + B * h)          # column-major [D, B, H]
    raise ValueError(layout)


def to_layout(pool: np.ndarray, layout: str) -> np.ndarray:
    """Physical array of a logical pool ``[N, B, H, D]`` in ``layout``:
    ``[N, B, H, D]`` (token) or ``[N, H, B, D]`` (head)."""
    if layout == "token":
        return pool.copy()
    if layout == "head":
        return np.ascontiguousarray(pool.transpose(0, 2, 1, 3))
    raise ValueError(layout)


def from_layout(phys: np.ndarray, layout: str) -> np.ndarray:
    """Inverse of ``to_layout``."""
    if layout == "token":
        return phys.copy()
    if layout == "head":
        return np.ascontiguousarray(phys.transpose(0, 2, 1, 3))
    raise ValueError(layout)
