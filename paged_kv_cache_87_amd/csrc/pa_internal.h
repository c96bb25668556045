// Internal interface between the C-ABI entry points (pa_api.cpp) and the
// kernel launchers.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Launch kernel(a) and return this launch's own status.  hipLaunchKernel
// reports only its own error; hipGetLastError after a hipLaunchKernelGGL
// would also return an earlier failure of some unrelated HIP call the caller
// made and did not clear, and blame it on the launch.
template <typename A>
inline hipError_t launch_kernel(void (*kernel)(A), dim3 grid, dim3 block, size_t lds,
                                hipStream_t stream, const A& a) {
  void* args[] = {const_cast<A*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, lds, stream);
}

// Thread-local error text behind pa_last_error(): clear at entry, set with
// the failing status (returned unchanged).
void clear_report();
pa_status report(pa_status status, const char* fmt, ...);

// The kernels walk a sequence's history in units of 16 tokens: unit j holds
// positions 16 j .. 16 j + 15.  A block of 16 or more tokens (a power of
// two) holds whole units; a block of 8 tokens holds half of one.
constexpr int kUnit = 16;

// Where a (block, token, KV head) row of head_dim elements sits in a pool, in
// bytes: block * block_stride + token * token_stride + head * head_stride.
// A block's rows fill one span of `span` bytes in every supported layout.
struct PoolGeom {
  int64_t block_stride;
  uint32_t token_stride;   // token-major: num_kv_heads * head row; head-major: one head row
  uint32_t head_stride;    // token-major: one head row; head-major: block_size head rows
  uint32_t span;           // block_size * num_kv_heads * head_dim * element size
  uint32_t block_shift;    // log2(block_size), 3 .. 8
};

struct SlotMappingArgs {
  uint32_t block_shift;        // log2(block_size)
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* q_start_loc;  // may be null (one token per sequence)
  int64_t* slot_mapping;
  int32_t num_seqs;
  int32_t max_blocks_per_seq;
  int32_t num_tokens;
  int32_t num_blocks;
};
hipError_t launch_slot_mapping(const SlotMappingArgs& a, hipStream_t stream);

struct WriteKVArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int64_t* slot_mapping;
  int32_t num_tokens;
  int32_t row_bytes;       // num_kv_heads * head_dim * element size (multiple of 16)
  int32_t head_bytes;      // head_dim * element size (multiple of 16)
  int64_t num_slots;       // num_blocks * block_size
  PoolGeom geom;
};
hipError_t launch_write_kv(const WriteKVArgs& a, hipStream_t stream);

struct AppendKVArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int64_t* slot_mapping;   // may be null
  int32_t num_seqs;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t row_bytes;       // num_kv_heads * head_dim * element size
  int32_t head_bytes;      // head_dim * element size
  PoolGeom geom;
};
hipError_t launch_append_kv(const AppendKVArgs& a, hipStream_t stream);

struct CopyBlocksArgs {
  const void* src_k;       // source pools (device or pinned host)
  const void* src_v;
  void* dst_k;             // destination pools (device or pinned host)
  void* dst_v;
  const int32_t* src;      // [num_pairs] source block ids
  const int32_t* dst;      // [num_pairs] destination block ids
  int32_t num_pairs;
  int32_t src_blocks;      // blocks of the source / destination pools
  int32_t dst_blocks;
  int64_t block_bytes;     // block span, block_size * num_kv_heads * head_dim * element size
                           // (multiple of 64)
  int64_t src_stride;      // bytes from one block to the next in the source / destination
  int64_t dst_stride;
};
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

struct ReadChecksumArgs {
  const void* buf;            // device buffer, 16-byte aligned
  uint64_t chunks;            // its 16-byte chunks
  uint64_t chunks_per_word;   // chunks XORed into one output word (the last share may be shorter)
  uint32_t* words;            // [num_words] device output
};
hipError_t launch_read_checksum(const ReadChecksumArgs& a, int num_words, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  void* out;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* part_o;           // [2 * max_slices, n_rep, head_dim] partial outputs
  float* part_ml;          // [2 * max_slices, n_rep, 2] their (max, sum)
  int32_t* counters;       // [num_seqs * num_kv_heads] arrivals, zero between calls
  const void* k_new;       // decode step only (else null): [num_seqs, num_kv_heads, head_dim]
  const void* v_new;       //   new K / V rows, written to their slots and attended from here
  int64_t* slot_mapping;   //   their slots, written (may be null)
  int32_t num_seqs;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t dtype;           // 0 = f32, 1 = bf16
  int32_t max_blocks_per_seq;
  int32_t context_cap;     // min(max_context_len, max_blocks_per_seq * block_size)
  int32_t min_slice_blocks;  // 0: every (sequence, KV head) in one pass; else split
  int32_t max_slices;      // split: upper bound of the grid (partial slots = 2x)
  int32_t seg_cost;        // split: price of a segment's fixed cost, in blocks
  float scale_log2;        // softmax scale * log2(e)
  PoolGeom geom;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// Workgroups launch_decode(a) uses on the current device (nothing launched).
hipError_t decode_grid(const DecodeArgs& a, int* grid);

struct PrefillArgs {
  const void* q;
  void* out;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* q_start_loc;
  int32_t num_seqs;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t context_cap;
  int32_t max_q_len;
  int32_t total_q_tokens;
  int32_t dtype;           // 0 = f32, 1 = bf16
  float scale_log2;
  PoolGeom geom;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Decode work plan kept in LDS by every workgroup: clamped context lengths and
// the prefix sum of blocks per KV head over the batch.
constexpr int kMaxDecodeSeqs = 4096;
inline size_t plan_lds_bytes(int num_seqs) {
  return (2 * static_cast<size_t>(num_seqs) + 1) * sizeof(int32_t);
}

// Workgroups of kernel `fn` (block size `threads`, `lds` bytes of dynamic
// LDS) that the current device holds at once; cached per (kernel, device,
// LDS size).
hipError_t resident_workgroups(const void* fn, int threads, size_t lds, int* out);

// Split decodes keep one arrival counter per (sequence, KV head) at the
// start of the workspace, in a header of fixed size so that it stays in place
// whatever the batch shape of the next call.  Its last kControlSlots words are
// the hand-out and exit counters of the units given out at run time.
constexpr int kCounterSlots = 65536;
constexpr int kControlSlots = 64;
constexpr int kPairSlots = kCounterSlots - kControlSlots;
constexpr size_t kCounterHeaderBytes = kCounterSlots * sizeof(int32_t);
// At most this many slices (workgroups) share a split decode.
constexpr int kMaxSlices = 2048;
// A split decode prices each (sequence, KV head) segment at this many blocks
// on top of its blocks when it cuts the work into equal slices.
constexpr int kSegCost = 24;

// Units of a split decode.  The work range [0, B) (blocks, each segment priced
// as kSegCost more) is cut into G static slices of Q1, one per workgroup, and
// after them into chunks of Q2 that the workgroups take one at a time as they
// finish (a counter in the workspace header hands them out): workgroups that
// run slower take fewer.  The static slices cover B - floor(B / 10), nine
// tenths of the work.  When every non-empty pair has the same length the
// slices alone cover it (equal work per workgroup, and the slices usually cut
// no pair), as they do when the chunks would not fit the partial slots
// (kMaxSlices units).  Unit u's pieces go to partial slots 2u (its first
// segment) and 2u + 1 (its last).  Shared by the kernel and the host's
// description of the split.
constexpr int kStaticTenths = 9;     // tenths of the work the static slices cover
constexpr int kChunkDiv = 16;        // chunk = static slice / kChunkDiv (at least min_slice)
struct UnitPlan {
  int32_t G, Q1, Q2, Bs, B, U;
  __host__ __device__ int32_t start(int32_t u) const {
    return u < G ? static_cast<int32_t>(static_cast<uint32_t>(u) * Q1 < static_cast<uint32_t>(Bs)
                                            ? static_cast<uint32_t>(u) * Q1
                                            : static_cast<uint32_t>(Bs))
                 : Bs + (u - G) * Q2;
  }
  __host__ __device__ int32_t end(int32_t u) const {
    return u < G ? start(u + 1)
                 : (static_cast<uint32_t>(u - G + 1) * Q2 < static_cast<uint32_t>(B - Bs)
                        ? Bs + (u - G + 1) * Q2
                        : B);
  }
  __host__ __device__ int32_t of(int32_t pos) const {
    return pos < Bs ? pos / Q1 : G + (pos - Bs) / Q2;
  }
};
// All in 32-bit unsigned arithmetic (B < 2^31, G <= 2048, so no sum below
// overflows), the same on the host and the device.
__host__ __device__ inline UnitPlan unit_plan(int32_t B, int32_t G, int32_t min_slice,
                                              int32_t max_units, bool equal_pairs) {
  const uint32_t b = static_cast<uint32_t>(B), g = static_cast<uint32_t>(G);
  const uint32_t ms = static_cast<uint32_t>(min_slice > 1 ? min_slice : 1);
  UnitPlan p;
  p.B = B;
  p.G = G;
  uint32_t q = (b + g - 1) / g;
  q = q > ms ? q : ms;
  const uint32_t stat = b - (b / 10) * (10 - kStaticTenths);   // work of the static slices
  uint32_t q1 = (stat + g - 1) / g;
  q1 = q1 > ms ? q1 : ms;
  const uint32_t bs = static_cast<uint64_t>(q1) * g < b ? q1 * g : b;
  uint32_t q2 = q1 / kChunkDiv;
  q2 = q2 > ms ? q2 : ms;
  const uint32_t chunks = (b - bs + q2 - 1) / q2;
  if (equal_pairs || chunks == 0 || g + chunks > static_cast<uint32_t>(max_units)) {
    p.Q1 = static_cast<int32_t>(q);
    p.Bs = static_cast<int32_t>(static_cast<uint64_t>(q) * g < b ? q * g : b);
    p.Q2 = p.Q1;
    p.U = G;
  } else {
    p.Q1 = static_cast<int32_t>(q1);
    p.Bs = static_cast<int32_t>(bs);
    p.Q2 = static_cast<int32_t>(q2);
    p.U = static_cast<int32_t>(g + chunks);
  }
  return p;
}

// Split plan shared by the workspace query and pa_decode.
struct DecodePlan {
  int32_t context_cap;
  int32_t min_slice_blocks;  // 0: no split
  int32_t max_slices;
  size_t workspace_bytes;
  size_t part_o_offset;      // byte offsets inside the workspace
  size_t part_ml_offset;
  int64_t max_blocks;        // num_kv_heads * num_seqs * (ceil(context_cap / block size) + segment price)
};
DecodePlan plan_decode(int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                       int32_t max_context_len, int32_t num_kv_heads, int32_t num_q_heads,
                       int32_t head_dim, int32_t partition_size);

}  // namespace pa
