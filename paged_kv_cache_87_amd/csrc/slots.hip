// Slot mapping and the slot-mapped K/V write (gfx950).
//
// A token at position `pos` of sequence `s` lives in logical block
// pos / B at offset pos % B (B = block_size); the block table maps the
// logical block to a physical block, and the token's slot is the flat row
// physical * B + offset of the pool viewed as [num_blocks * B, Hkv, D]
// (JuliaPagedAttn README, "Project Structure": slot mapping in the cache
// layout; nanoserve Day 19, "Diagram": slot_mapping).  The write copies each
// new token's [Hkv, D] row into its slot bit for bit (JuliaPagedAttn "API
// Reference": write_kv_cache!; nanoserve Day 19 "What I added today"), in
// whichever block layout the pool has (token-major as the Pico-vLLM pool, or
// head-major as JuliaPagedAttn's "Block Layout").

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kSlotThreads = 256;
constexpr int kWriteThreads = 256;

// Slot of position `pos` of sequence `s` whose context is `L` tokens: the
// table's block for pos / block_size, offset pos % block_size (block_size =
// 2^shift); -1 when the position is not in the context or the table entry is
// not a block of the pool.
__device__ __forceinline__ int64_t slot_of(const int32_t* block_tables, int max_blocks_per_seq,
                                           int num_blocks, uint32_t shift, int s, int L,
                                           int pos) {
  if (pos < 0 || pos >= L) return -1;
  const int logical = pos >> shift;
  if (logical >= max_blocks_per_seq) return -1;
  const int phys = block_tables[static_cast<int64_t>(s) * max_blocks_per_seq + logical];
  if (phys < 0 || phys >= num_blocks) return -1;
  return (static_cast<int64_t>(phys) << shift) + (pos & ((1 << shift) - 1));
}

__global__ __launch_bounds__(kSlotThreads) void slot_mapping_kernel(SlotMappingArgs a) {
  const int i = blockIdx.x * kSlotThreads + threadIdx.x;
  if (i >= a.num_tokens) return;
  int s, q_len, idx;
  if (a.q_start_loc == nullptr) {
    s = i;
    q_len = 1;
    idx = 0;
  } else {
    // Last sequence whose first token is <= i (empty sequences share their
    // start with the next one, so the last such sequence is the owner).
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.q_start_loc[mid] <= i) lo = mid; else hi = mid - 1;
    }
    s = lo;
    q_len = a.q_start_loc[s + 1] - a.q_start_loc[s];
    idx = i - a.q_start_loc[s];
  }
  const int L = a.context_lens[s];
  a.slot_mapping[i] = idx >= 0 && idx < q_len
                          ? slot_of(a.block_tables, a.max_blocks_per_seq, a.num_blocks,
                                    a.block_shift, s, L, L - q_len + idx)
                          : -1;
}

// One 16-byte chunk per thread; blockIdx.y selects K (0) or V (1).  The
// source row of a token is [Hkv, D]; chunk `part` of it belongs to KV head
// part / (chunks per head row) and lands where the pool's layout puts that
// head's row of the slot's block.
__global__ __launch_bounds__(kWriteThreads) void write_kv_kernel(WriteKVArgs a) {
  const int chunks_per_row = a.row_bytes >> 4;
  const int chunks_per_head = a.head_bytes >> 4;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kWriteThreads + threadIdx.x;
  const int64_t total = static_cast<int64_t>(a.num_tokens) * chunks_per_row;
  if (c >= total) return;
  const int t = static_cast<int>(c / chunks_per_row);
  const int part = static_cast<int>(c - static_cast<int64_t>(t) * chunks_per_row);
  // the source chunk does not depend on the slot: its load overlaps the slot's
  const uint4* src = static_cast<const uint4*>(blockIdx.y == 0 ? a.k_new : a.v_new);
  const uint4 val = src[static_cast<int64_t>(t) * chunks_per_row + part];
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.num_slots) return;
  const int h = part / chunks_per_head;
  const int q = part - h * chunks_per_head;
  const int64_t blk = slot >> a.geom.block_shift;
  const int in_blk = static_cast<int>(slot - (blk << a.geom.block_shift));
  const int64_t dst_off = blk * a.geom.block_stride +
                          static_cast<int64_t>(in_blk) * a.geom.token_stride +
                          static_cast<int64_t>(h) * a.geom.head_stride + 16 * q;
  char* dst = static_cast<char*>(blockIdx.y == 0 ? a.k_cache : a.v_cache);
  *reinterpret_cast<uint4*>(dst + dst_off) = val;
}

// The decode step's write in one launch: each thread finds the slot of its
// sequence's newest position (context_lens[s] - 1) itself and copies one
// 16-byte chunk of that token's K (blockIdx.y 0) or V (1) row; the first
// chunk's thread of the K pass records the slot.
__global__ __launch_bounds__(kWriteThreads) void append_kv_kernel(AppendKVArgs a) {
  const int chunks_per_row = a.row_bytes >> 4;
  const int chunks_per_head = a.head_bytes >> 4;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kWriteThreads + threadIdx.x;
  if (c >= static_cast<int64_t>(a.num_seqs) * chunks_per_row) return;
  const int t = static_cast<int>(c / chunks_per_row);
  const int part = static_cast<int>(c - static_cast<int64_t>(t) * chunks_per_row);
  // the source chunk does not depend on the slot: its load overlaps the two
  // dependent loads (context length, table entry) that find the slot
  const uint4* src = static_cast<const uint4*>(blockIdx.y == 0 ? a.k_new : a.v_new);
  const uint4 val = src[static_cast<int64_t>(t) * chunks_per_row + part];
  const int L = a.context_lens[t];
  const int64_t slot = slot_of(a.block_tables, a.max_blocks_per_seq, a.num_blocks,
                               a.geom.block_shift, t, L, L - 1);
  if (part == 0 && blockIdx.y == 0 && a.slot_mapping != nullptr) a.slot_mapping[t] = slot;
  if (slot < 0) return;
  const int h = part / chunks_per_head;
  const int q = part - h * chunks_per_head;
  const int64_t blk = slot >> a.geom.block_shift;
  const int in_blk = static_cast<int>(slot - (blk << a.geom.block_shift));
  const int64_t dst_off = blk * a.geom.block_stride +
                          static_cast<int64_t>(in_blk) * a.geom.token_stride +
                          static_cast<int64_t>(h) * a.geom.head_stride + 16 * q;
  char* dst = static_cast<char*>(blockIdx.y == 0 ? a.k_cache : a.v_cache);
  *reinterpret_cast<uint4*>(dst + dst_off) = val;
}

}  // namespace

hipError_t launch_append_kv(const AppendKVArgs& a, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.num_seqs) * (a.row_bytes >> 4);
  const int64_t grid = (total + kWriteThreads - 1) / kWriteThreads;
  return launch_kernel(append_kv_kernel, dim3(static_cast<unsigned>(grid), 2), dim3(kWriteThreads), 0,
                       stream, a);
}

hipError_t launch_slot_mapping(const SlotMappingArgs& a, hipStream_t stream) {
  const int grid = (a.num_tokens + kSlotThreads - 1) / kSlotThreads;
  return launch_kernel(slot_mapping_kernel, dim3(grid), dim3(kSlotThreads), 0, stream, a);
}

hipError_t launch_write_kv(const WriteKVArgs& a, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.num_tokens) * (a.row_bytes >> 4);
  const int64_t grid = (total + kWriteThreads - 1) / kWriteThreads;
  return launch_kernel(write_kv_kernel, dim3(static_cast<unsigned>(grid), 2), dim3(kWriteThreads), 0,
                       stream, a);
}

}  // namespace pa
