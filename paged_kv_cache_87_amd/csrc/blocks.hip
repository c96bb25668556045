// Whole-block copies inside the K and V pools: the data move of a
// copy-on-write (JuliaPagedAttn README, "Copy-on-Write": when a sequence
// writes into a block that other sequences still share, the block is copied
// to a fresh one before the write).  Every listed (src, dst) pair copies one
// block of the K pool and the same block of the V pool, bit for bit.
//
// grid (pair, pool, quarter of the block), 256 threads; each thread moves
// 16-byte chunks with a stride of one workgroup.  A block's rows fill one
// contiguous span in every supported layout, so a block is copied as bytes;
// blocks may sit further apart than their span (K and V of a block stored
// together).  Pairs whose ids are outside the pool are skipped.
//
// The same kernel moves blocks between the device pool and a pool in pinned
// host memory (Pico-vLLM #5 Paged Attention, BlockManager swap_out /
// swap_in: a GPU block is copied into a CPU block of the pinned CPU pool and
// back): the device reads or writes the host pool directly through its
// mapping, so a whole batch of blocks is one launch.

#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopySplit = 4;        // workgroups per block and pool

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int p = blockIdx.x;
  const int src = a.src[p];
  const int dst = a.dst[p];
  if (src < 0 || src >= a.src_blocks || dst < 0 || dst >= a.dst_blocks) return;
  const char* base = static_cast<const char*>(blockIdx.y == 0 ? a.src_k : a.src_v);
  char* out = static_cast<char*>(blockIdx.y == 0 ? a.dst_k : a.dst_v);
  const int64_t chunks = a.block_bytes >> 4;          // 16-byte chunks per block
  const int64_t per = chunks / kCopySplit;
  const int64_t c0 = per * blockIdx.z;
  const uint4* s = reinterpret_cast<const uint4*>(base + static_cast<int64_t>(src) * a.src_stride);
  uint4* d = reinterpret_cast<uint4*>(out + static_cast<int64_t>(dst) * a.dst_stride);
  for (int64_t c = c0 + threadIdx.x; c < c0 + per; c += kCopyThreads) d[c] = s[c];
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  return launch_kernel(copy_blocks_kernel, dim3(a.num_pairs, 2, kCopySplit), dim3(kCopyThreads), 0,
                       stream, a);
}

}  // namespace pa
