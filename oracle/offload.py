"""CPU oracle for the GPU <-> pinned-host offload tier (plain Python).

TEST INFRASTRUCTURE ONLY.  Only the test suite may import it.  It shares no
code with the library and imports nothing from the ``paged_kv_cache_87_amd``
package.

Source: "Pico-vLLM 开发日志 #5 Paged Attention", the BlockManager listing and
its optional offload methods:

* two physical pools, GPU and CPU (the CPU one in pinned memory), each with
  a deque of free physical ids filled with ``range(n)``;
* logical blocks, also drawn from a deque, each mapped to a pair
  (tier, physical id); an unmapped logical block is (NONE, -1);
* ``allocate`` hands out logical blocks backed by the GPU while GPU blocks
  are free, then by the CPU; it refuses (changing nothing) when the two
  tiers together hold fewer free blocks than asked;
* ``free`` returns the physical block to its tier's deque (right end) and
  the logical id to the logical deque; an unmapped block is an error;
* ``swap_out`` moves each listed logical block that lives on the GPU to a
  CPU block taken from the left of the CPU deque: the block's K and V are
  copied, the GPU block goes back to the GPU deque and the mapping is
  updated; ``swap_in`` is the mirror image.  A listed block on the wrong
  tier is an error.

Readings where the page is silent (each pinned by a test):

* a refused swap changes nothing: the whole list is checked (tier, and
  enough free blocks on the target tier, which the page's ``popleft`` would
  otherwise fail on halfway) before any block moves;
* a logical id outside the range, or listed twice, is refused like a block
  on the wrong tier;
* the data move of one call is a list of (source physical, destination
  physical) pairs in listing order, which ``swap_copy`` applies.
"""

from __future__ import annotations

from collections import deque

GPU, CPU, NONE = "GPU", "CPU", "NONE"


class OffloadError(Exception):
    """A refused request; ``kind`` is "no_blocks" or "invalid"."""

    def __init__(self, kind: str, msg: str):
        super().__init__(msg)
        self.kind = kind


class TieredBlockManager:
    def __init__(self, num_gpu_blocks: int, num_cpu_blocks: int):
        self.free = {GPU: deque(range(num_gpu_blocks)), CPU: deque(range(num_cpu_blocks))}
        self.num_total = num_gpu_blocks + num_cpu_blocks
        self.mapping = [(NONE, -1)] * self.num_total
        self.logical_free = deque(range(self.num_total))

    @property
    def num_free_blocks(self) -> int:
        return len(self.free[GPU]) + len(self.free[CPU])

    def allocate(self, n: int) -> list[int]:
        if n > self.num_free_blocks:
            raise OffloadError("no_blocks", f"{n} blocks asked, {self.num_free_blocks} free")
        out = []
        for _ in range(n):
            tier = GPU if self.free[GPU] else CPU
            phys = self.free[tier].popleft()
            lid = self.logical_free.popleft()
            self.mapping[lid] = (tier, phys)
            out.append(lid)
        return out

    def _tier(self, lid: int) -> str:
        return self.mapping[lid][0] if 0 <= lid < self.num_total else NONE

    def free_blocks(self, ids: list[int]) -> None:
        if len(set(ids)) != len(ids):
            raise OffloadError("invalid", "a block is listed twice")
        for lid in ids:
            if self._tier(lid) == NONE:
                raise OffloadError("invalid", f"logical block {lid} is not allocated")
        for lid in ids:
            tier, phys = self.mapping[lid]
            self.free[tier].append(phys)
            self.logical_free.append(lid)
            self.mapping[lid] = (NONE, -1)

    def _swap(self, ids: list[int], src: str, dst: str) -> list[tuple[int, int]]:
        for lid in ids:
            if self._tier(lid) != src:
                raise OffloadError("invalid", f"logical block {lid} is not on the {src}")
        if len(set(ids)) != len(ids):
            raise OffloadError("invalid", "a block is listed twice")
        if len(ids) > len(self.free[dst]):
            raise OffloadError("no_blocks", f"{len(ids)} blocks to move, {len(self.free[dst])} "
                               f"free on the {dst}")
        pairs = []
        for lid in ids:
            _, old = self.mapping[lid]
            new = self.free[dst].popleft()
            pairs.append((old, new))            # data: old (src tier) -> new (dst tier)
            self.free[src].append(old)
            self.mapping[lid] = (dst, new)
        return pairs

    def swap_out(self, ids: list[int]) -> list[tuple[int, int]]:
        """(gpu block, cpu block) pairs, K and V of each copied GPU -> CPU."""
        return self._swap(ids, GPU, CPU)

    def swap_in(self, ids: list[int]) -> list[tuple[int, int]]:
        """(cpu block, gpu block) pairs, K and V of each copied CPU -> GPU."""
        return self._swap(ids, CPU, GPU)


def swap_copy(src_k, src_v, dst_k, dst_v, pairs) -> None:
    """Apply one call's data move: block ``s`` of the source pools to block
    ``d`` of the destination pools, for each (s, d) (numpy arrays
    ``[num_blocks, ...]``)."""
    for s, d in pairs:
        dst_k[d] = src_k[s]
        dst_v[d] = src_v[s]
