// C-ABI entry points of libpa.so: host-side argument checks, the decode
// split plan and the mapping of HIP errors to status codes.  Every
// check runs before anything is enqueued; no entry point allocates.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "pa.h"
#include "pa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

void clear_error() { g_last_error[0] = '\0'; }

pa_status fail(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

pa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PA_OK;
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elt_size(int32_t dtype) { return dtype == PA_BF16 ? 2 : 4; }

pa_status check_pool(const pa_kv_pool* pool) {
  if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "pool descriptor is null");
  if (pool->k_cache == nullptr || pool->v_cache == nullptr)
    return fail(PA_ERR_INVALID_ARG, "k_cache or v_cache is null");
  if (!aligned16(pool->k_cache) || !aligned16(pool->v_cache))
    return fail(PA_ERR_INVALID_ARG, "k_cache and v_cache must be 16-byte aligned");
  if (pool->num_blocks <= 0 || pool->num_kv_heads <= 0 || pool->head_dim <= 0 ||
      pool->block_size <= 0)
    return fail(PA_ERR_INVALID_ARG, "pool sizes must be positive (num_blocks=%d block_size=%d "
                "num_kv_heads=%d head_dim=%d)", pool->num_blocks, pool->block_size,
                pool->num_kv_heads, pool->head_dim);
  if (pool->dtype != PA_F32 && pool->dtype != PA_BF16)
    return fail(PA_ERR_INVALID_ARG, "unknown dtype %d", pool->dtype);
  if (pool->block_size < 8 || pool->block_size > 256 ||
      (pool->block_size & (pool->block_size - 1)) != 0)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d (supported: 8, 16, 32, 64, 128, 256)",
                pool->block_size);
  if (pool->head_dim != 64 && pool->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", pool->head_dim);
  if (pool->num_kv_heads > 4096)
    return fail(PA_ERR_UNSUPPORTED, "num_kv_heads %d (at most 4096)", pool->num_kv_heads);
  if (pool->layout != PA_LAYOUT_TOKEN_MAJOR && pool->layout != PA_LAYOUT_HEAD_MAJOR)
    return fail(PA_ERR_INVALID_ARG, "unknown layout %d", pool->layout);
  const int64_t dense = static_cast<int64_t>(pool->block_size) * pool->num_kv_heads *
                        pool->head_dim;
  if (pool->block_stride != 0) {
    if (pool->block_stride < dense)
      return fail(PA_ERR_INVALID_ARG, "block_stride %lld is below the block's %lld elements",
                  static_cast<long long>(pool->block_stride), static_cast<long long>(dense));
    if ((pool->block_stride * elt_size(pool->dtype)) % 16 != 0)
      return fail(PA_ERR_INVALID_ARG, "block_stride %lld is not a multiple of 16 bytes",
                  static_cast<long long>(pool->block_stride));
    if (pool->block_stride > (int64_t(1) << 40) / pool->num_blocks)
      return fail(PA_ERR_UNSUPPORTED, "block_stride %lld x num_blocks %d is too large",
                  static_cast<long long>(pool->block_stride), pool->num_blocks);
  }
  return PA_OK;
}

// Byte geometry of a checked pool.
pa::PoolGeom geom_of(const pa_kv_pool* p) {
  const int e = elt_size(p->dtype);
  const uint32_t row = static_cast<uint32_t>(p->head_dim * e);
  pa::PoolGeom g{};
  g.span = static_cast<uint32_t>(p->block_size) * p->num_kv_heads * row;
  g.block_stride = p->block_stride != 0 ? p->block_stride * e : static_cast<int64_t>(g.span);
  if (p->layout == PA_LAYOUT_TOKEN_MAJOR) {
    g.token_stride = static_cast<uint32_t>(p->num_kv_heads) * row;
    g.head_stride = row;
  } else {
    g.token_stride = row;
    g.head_stride = static_cast<uint32_t>(p->block_size) * row;
  }
  g.block_shift = 0;
  while ((1 << g.block_shift) < p->block_size) ++g.block_shift;
  return g;
}

// Bytes from a pool's base pointer to the end of its last block.
size_t extent_bytes(const pa_kv_pool* p) {
  const pa::PoolGeom g = geom_of(p);
  return static_cast<size_t>(g.block_stride) * (p->num_blocks - 1) + g.span;
}

pa_status check_seqs(const pa_seq_desc* seqs, int32_t block_size) {
  if (seqs == nullptr) return fail(PA_ERR_INVALID_ARG, "sequence descriptor is null");
  if (seqs->num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs %d < 0", seqs->num_seqs);
  if (seqs->num_seqs > 0 && (seqs->block_tables == nullptr || seqs->context_lens == nullptr))
    return fail(PA_ERR_INVALID_ARG, "block_tables or context_lens is null");
  if (seqs->max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d must be positive",
                seqs->max_blocks_per_seq);
  if (seqs->max_context_len < 0)
    return fail(PA_ERR_INVALID_ARG, "max_context_len %d < 0", seqs->max_context_len);
  if (static_cast<int64_t>(seqs->max_blocks_per_seq) * block_size > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "max_blocks_per_seq too large");
  return PA_OK;
}

pa_status check_heads(const pa_kv_pool* pool, int32_t num_q_heads) {
  if (num_q_heads <= 0) return fail(PA_ERR_INVALID_ARG, "num_q_heads %d", num_q_heads);
  if (num_q_heads % pool->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, pool->num_kv_heads);
  const int n_rep = num_q_heads / pool->num_kv_heads;
  if (n_rep != 1 && n_rep != 2 && n_rep != 4 && n_rep != 8)
    return fail(PA_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads = %d (supported: 1, 2, 4, 8)",
                n_rep);
  return PA_OK;
}

// True when [p, p + bytes) starts and ends in memory the current device can
// address at the same pointer: pinned host memory (hipHostMalloc) when
// `host`, device memory otherwise.  A kernel that touched pageable or
// unmapped memory would fault, so the swap checks its arguments with this
// before anything is enqueued.
bool device_addressable(const void* p, size_t bytes, bool host) {
  const char* c = static_cast<const char*>(p);
  for (const char* q : {c, c + bytes - 1}) {
    hipPointerAttribute_t at{};
    if (hipPointerGetAttributes(&at, q) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    if (at.type != (host ? hipMemoryTypeHost : hipMemoryTypeDevice)) return false;
    if (at.devicePointer != q) return false;
  }
  return true;
}

int32_t context_cap(const pa_seq_desc* seqs, int32_t block_size) {
  const int64_t by_table = static_cast<int64_t>(seqs->max_blocks_per_seq) * block_size;
  return static_cast<int32_t>(seqs->max_context_len < by_table ? seqs->max_context_len : by_table);
}

}  // namespace

namespace pa {
void clear_report() { clear_error(); }
pa_status report(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}
}  // namespace pa

namespace pa {

hipError_t resident_workgroups(const void* fn, int threads, size_t lds, int* out) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, size_t>, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const auto key = std::make_tuple(fn, dev, lds);
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) {
      *out = it->second;
      return hipSuccess;
    }
  }
  int per_cu = 0, cus = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int n = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  {
    std::lock_guard<std::mutex> lock(mu);
    cache[key] = n;
  }
  *out = n;
  return hipSuccess;
}

DecodePlan plan_decode(int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                       int32_t max_context_len, int32_t num_kv_heads, int32_t num_q_heads,
                       int32_t head_dim, int32_t partition_size) {
  DecodePlan p{};
  const int64_t by_table = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  p.context_cap = static_cast<int32_t>(max_context_len < by_table ? max_context_len : by_table);
  // the kernel walks 16-token units
  const int64_t cap_blocks = (static_cast<int64_t>(p.context_cap) + kUnit - 1) / kUnit;
  p.max_blocks = static_cast<int64_t>(num_kv_heads) * num_seqs * cap_blocks;
  const int64_t cover = (cap_blocks > 0 ? cap_blocks : 1) * kUnit;
  if (partition_size <= 0 || partition_size >= cover) return p;   // no split
  p.min_slice_blocks = partition_size / kUnit;
  const int64_t slices = (p.max_blocks + p.min_slice_blocks - 1) / p.min_slice_blocks;
  p.max_blocks += static_cast<int64_t>(num_kv_heads) * num_seqs * kSegCost;   // work range
  p.max_slices = static_cast<int32_t>(slices < kMaxSlices ? (slices > 0 ? slices : 1)
                                                          : kMaxSlices);
  const size_t rows = static_cast<size_t>(2) * p.max_slices * (num_q_heads / num_kv_heads);
  p.part_o_offset = kCounterHeaderBytes;
  p.part_ml_offset = p.part_o_offset + (rows * head_dim * sizeof(float) + 255) / 256 * 256;
  p.workspace_bytes = p.part_ml_offset + rows * 2 * sizeof(float);
  return p;
}

}  // namespace pa

extern "C" {

const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS";
    default: return "PA_ERR_UNKNOWN";
  }
}

const char* pa_last_error(void) { return g_last_error; }

int32_t pa_version(void) { return (1 << 16) | 1; }

pa_status pa_slot_mapping(const pa_kv_pool* pool, const pa_seq_desc* seqs,
                          const int32_t* q_start_loc, int32_t num_tokens,
                          int64_t* slot_mapping, hipStream_t stream) {
  clear_error();
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if ((st = check_seqs(seqs, pool->block_size)) != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (slot_mapping == nullptr) return fail(PA_ERR_INVALID_ARG, "slot_mapping is null");
  if (seqs->num_seqs == 0) return fail(PA_ERR_INVALID_ARG, "tokens given but num_seqs is 0");
  if (q_start_loc == nullptr && num_tokens != seqs->num_seqs)
    return fail(PA_ERR_INVALID_ARG, "without q_start_loc num_tokens (%d) must equal num_seqs (%d)",
                num_tokens, seqs->num_seqs);
  pa::SlotMappingArgs a{geom_of(pool).block_shift, seqs->block_tables, seqs->context_lens,
                        q_start_loc, slot_mapping, seqs->num_seqs, seqs->max_blocks_per_seq,
                        num_tokens, pool->num_blocks};
  return hip_status(pa::launch_slot_mapping(a, stream), "slot_mapping launch");
}

pa_status pa_write_kv(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                      const int64_t* slot_mapping, int32_t num_tokens, hipStream_t stream) {
  clear_error();
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr)
    return fail(PA_ERR_INVALID_ARG, "k_new, v_new or slot_mapping is null");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PA_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  pa::WriteKVArgs a{k_new, v_new, pool->k_cache, pool->v_cache, slot_mapping, num_tokens,
                    pool->num_kv_heads * pool->head_dim * elt_size(pool->dtype),
                    pool->head_dim * elt_size(pool->dtype),
                    static_cast<int64_t>(pool->num_blocks) * pool->block_size, geom_of(pool)};
  return hip_status(pa::launch_write_kv(a, stream), "write_kv launch");
}

pa_status pa_append_kv(const pa_kv_pool* pool, const pa_seq_desc* seqs, const void* k_new,
                       const void* v_new, int64_t* slot_mapping, hipStream_t stream) {
  clear_error();
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if ((st = check_seqs(seqs, pool->block_size)) != PA_OK) return st;
  if (seqs->num_seqs == 0) return PA_OK;
  if (k_new == nullptr || v_new == nullptr)
    return fail(PA_ERR_INVALID_ARG, "k_new or v_new is null");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PA_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  pa::AppendKVArgs a{k_new, v_new, pool->k_cache, pool->v_cache, seqs->block_tables,
                     seqs->context_lens, slot_mapping, seqs->num_seqs, seqs->max_blocks_per_seq,
                     pool->num_blocks, pool->num_kv_heads * pool->head_dim * elt_size(pool->dtype),
                     pool->head_dim * elt_size(pool->dtype), geom_of(pool)};
  return hip_status(pa::launch_append_kv(a, stream), "append_kv launch");
}

pa_status pa_copy_blocks(const pa_kv_pool* pool, const int32_t* src_blocks,
                         const int32_t* dst_blocks, int32_t num_pairs, hipStream_t stream) {
  clear_error();
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs %d", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (src_blocks == nullptr || dst_blocks == nullptr)
    return fail(PA_ERR_INVALID_ARG, "src_blocks or dst_blocks is null");
  if (num_pairs > 65535)
    return fail(PA_ERR_UNSUPPORTED, "num_pairs %d (at most 65535 a call)", num_pairs);
  const pa::PoolGeom g = geom_of(pool);
  pa::CopyBlocksArgs a{pool->k_cache, pool->v_cache, pool->k_cache, pool->v_cache,
                       src_blocks, dst_blocks, num_pairs, pool->num_blocks, pool->num_blocks,
                       g.span, g.block_stride, g.block_stride};
  return hip_status(pa::launch_copy_blocks(a, stream), "copy_blocks launch");
}

pa_status pa_swap_blocks(const pa_kv_pool* device_pool, const pa_kv_pool* host_pool,
                         const int32_t* device_blocks, const int32_t* host_blocks,
                         int32_t num_pairs, int32_t direction, hipStream_t stream) {
  clear_error();
  pa_status st = check_pool(device_pool);
  if (st != PA_OK) return st;
  if ((st = check_pool(host_pool)) != PA_OK) return st;
  if (host_pool->block_size != device_pool->block_size ||
      host_pool->num_kv_heads != device_pool->num_kv_heads ||
      host_pool->head_dim != device_pool->head_dim || host_pool->dtype != device_pool->dtype ||
      host_pool->layout != device_pool->layout)
    return fail(PA_ERR_INVALID_ARG,
                "host and device pools differ in block shape, dtype or layout");
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
    return fail(PA_ERR_INVALID_ARG, "direction %d", direction);
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs %d", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (device_blocks == nullptr || host_blocks == nullptr)
    return fail(PA_ERR_INVALID_ARG, "device_blocks or host_blocks is null");
  if (num_pairs > 65535)
    return fail(PA_ERR_UNSUPPORTED, "num_pairs %d (at most 65535 a call)", num_pairs);
  const size_t ids = sizeof(int32_t) * static_cast<size_t>(num_pairs);
  for (const void* p : {device_pool->k_cache, device_pool->v_cache})
    if (!device_addressable(p, extent_bytes(device_pool), false))
      return fail(PA_ERR_INVALID_ARG, "device pool is not device memory of the current device");
  for (const void* p : {host_pool->k_cache, host_pool->v_cache})
    if (!device_addressable(p, extent_bytes(host_pool), true))
      return fail(PA_ERR_INVALID_ARG,
                  "host pool is not pinned host memory mapped at the same address");
  for (const void* p : {static_cast<const void*>(device_blocks),
                        static_cast<const void*>(host_blocks)})
    if (!device_addressable(p, ids, false) && !device_addressable(p, ids, true))
      return fail(PA_ERR_INVALID_ARG, "block id arrays must be device or pinned host memory");
  const bool out = direction == PA_SWAP_OUT;
  const pa_kv_pool* s = out ? device_pool : host_pool;
  const pa_kv_pool* d = out ? host_pool : device_pool;
  const pa::PoolGeom gs = geom_of(s), gd = geom_of(d);
  pa::CopyBlocksArgs a{s->k_cache, s->v_cache, d->k_cache, d->v_cache,
                       out ? device_blocks : host_blocks, out ? host_blocks : device_blocks,
                       num_pairs, s->num_blocks, d->num_blocks, gs.span, gs.block_stride,
                       gd.block_stride};
  return hip_status(pa::launch_copy_blocks(a, stream), "swap_blocks launch");
}

pa_status pa_read_checksum(const void* buf, size_t bytes, uint32_t* words, int32_t num_words,
                           hipStream_t stream) {
  clear_error();
  if (buf == nullptr || words == nullptr) return fail(PA_ERR_INVALID_ARG, "buf or words is null");
  if (bytes % 16 != 0) return fail(PA_ERR_INVALID_ARG, "bytes %zu is not a multiple of 16", bytes);
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(PA_ERR_INVALID_ARG, "buf is not 16-byte aligned");
  if (num_words < 1 || num_words > 65535)
    return fail(PA_ERR_INVALID_ARG, "num_words %d (1 .. 65535)", num_words);
  const uint64_t chunks = bytes / 16;
  const uint64_t per = (chunks + num_words - 1) / num_words;
  if (per > (uint64_t{1} << 27))
    return fail(PA_ERR_UNSUPPORTED, "%llu bytes per word (at most 2 GiB)",
                static_cast<unsigned long long>(per * 16));
  pa::ReadChecksumArgs a{buf, chunks, per, words};
  return hip_status(pa::launch_read_checksum(a, num_words, stream), "read_checksum launch");
}

size_t pa_decode_workspace_bytes(const pa_kv_pool* pool, const pa_seq_desc* seqs,
                                 int32_t num_q_heads, int32_t partition_size) {
  if (pool == nullptr || seqs == nullptr || seqs->num_seqs < 0 ||
      seqs->max_blocks_per_seq <= 0 || seqs->max_context_len < 0 || pool->num_kv_heads <= 0 ||
      pool->head_dim <= 0 || pool->block_size < 8 || pool->block_size > 256 ||
      (pool->block_size & (pool->block_size - 1)) != 0 || num_q_heads <= 0 ||
      num_q_heads % pool->num_kv_heads != 0 || partition_size < 0 ||
      partition_size % pa::kUnit != 0)
    return 0;
  return pa::plan_decode(seqs->num_seqs, seqs->max_blocks_per_seq, pool->block_size,
                         seqs->max_context_len, pool->num_kv_heads, num_q_heads, pool->head_dim,
                         partition_size)
      .workspace_bytes;
}

}  // extern "C"

namespace {

// Checks of a decode request shared by pa_decode and pa_decode_split_info,
// and its kernel arguments (workspace pointers left null).  With io, q and
// out are checked too.
pa_status prepare_decode(const pa_kv_pool* pool, const pa_seq_desc* seqs, const void* q,
                         void* out, int32_t num_q_heads, float scale, int32_t partition_size,
                         bool io, pa::DecodeArgs* a, pa::DecodePlan* plan) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if ((st = check_seqs(seqs, pool->block_size)) != PA_OK) return st;
  if ((st = check_heads(pool, num_q_heads)) != PA_OK) return st;
  if (partition_size < 0 || partition_size % pa::kUnit != 0)
    return fail(PA_ERR_INVALID_ARG, "partition_size %d must be 0 or a multiple of %d",
                partition_size, pa::kUnit);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  if (io && seqs->num_seqs > 0) {
    if (q == nullptr || out == nullptr) return fail(PA_ERR_INVALID_ARG, "q or out is null");
    if (!aligned16(q) || !aligned16(out))
      return fail(PA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  }
  *plan = pa::plan_decode(seqs->num_seqs, seqs->max_blocks_per_seq, pool->block_size,
                          seqs->max_context_len, pool->num_kv_heads, num_q_heads, pool->head_dim,
                          partition_size);
  if (plan->max_blocks >= (int64_t(1) << 31))
    return fail(PA_ERR_UNSUPPORTED, "num_kv_heads * num_seqs * context blocks = %lld (below 2^31)",
                static_cast<long long>(plan->max_blocks));
  if (seqs->num_seqs > pa::kMaxDecodeSeqs)
    return fail(PA_ERR_UNSUPPORTED, "num_seqs %d (at most %d)", seqs->num_seqs,
                pa::kMaxDecodeSeqs);
  if (plan->workspace_bytes > 0 &&
      static_cast<int64_t>(seqs->num_seqs) * pool->num_kv_heads > pa::kPairSlots)
    return fail(PA_ERR_UNSUPPORTED, "num_seqs * num_kv_heads = %lld (at most %d when split)",
                static_cast<long long>(seqs->num_seqs) * pool->num_kv_heads, pa::kPairSlots);
  *a = pa::DecodeArgs{};
  a->q = q;
  a->out = out;
  a->k_cache = pool->k_cache;
  a->v_cache = pool->v_cache;
  a->block_tables = seqs->block_tables;
  a->context_lens = seqs->context_lens;
  a->num_seqs = seqs->num_seqs;
  a->num_blocks = pool->num_blocks;
  a->num_kv_heads = pool->num_kv_heads;
  a->num_q_heads = num_q_heads;
  a->head_dim = pool->head_dim;
  a->dtype = pool->dtype;
  a->max_blocks_per_seq = seqs->max_blocks_per_seq;
  a->context_cap = plan->context_cap;
  a->min_slice_blocks = plan->min_slice_blocks;
  a->max_slices = plan->max_slices;
  a->seg_cost = plan->min_slice_blocks > 0 ? pa::kSegCost : 0;
  a->scale_log2 = scale * 1.4426950408889634f;
  a->geom = geom_of(pool);
  return PA_OK;
}

// pa_decode and pa_decode_step: the caller's workspace, then the launch
pa_status decode_with_workspace(pa::DecodeArgs& a, const pa::DecodePlan& plan, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (plan.workspace_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
                  plan.workspace_bytes, workspace == nullptr ? size_t(0) : workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    a.counters = static_cast<int32_t*>(workspace);
    a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.part_o_offset);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.part_ml_offset);
  }
  return hip_status(pa::launch_decode(a, stream), "decode launch");
}

}  // namespace

extern "C" {

pa_status pa_decode(const pa_kv_pool* pool, const pa_seq_desc* seqs, const void* q, void* out,
                    int32_t num_q_heads, float scale, int32_t partition_size, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  pa::DecodeArgs a;
  pa::DecodePlan plan;
  const pa_status st = prepare_decode(pool, seqs, q, out, num_q_heads, scale, partition_size,
                                      true, &a, &plan);
  if (st != PA_OK) return st;
  if (seqs->num_seqs == 0) return PA_OK;
  return decode_with_workspace(a, plan, workspace, workspace_bytes, stream);
}

pa_status pa_decode_step(const pa_kv_pool* pool, const pa_seq_desc* seqs, const void* k_new,
                         const void* v_new, int64_t* slot_mapping, const void* q, void* out,
                         int32_t num_q_heads, float scale, int32_t partition_size,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  pa::DecodeArgs a;
  pa::DecodePlan plan;
  const pa_status st = prepare_decode(pool, seqs, q, out, num_q_heads, scale, partition_size,
                                      true, &a, &plan);
  if (st != PA_OK) return st;
  if (seqs->num_seqs == 0) return PA_OK;
  if (k_new == nullptr || v_new == nullptr)
    return fail(PA_ERR_INVALID_ARG, "k_new or v_new is null");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PA_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot_mapping = slot_mapping;
  return decode_with_workspace(a, plan, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// pa_decode_noalloc: the split decode's counters and partial results in a
// device array of the library's own, for callers that cannot allocate.
// ---------------------------------------------------------------------------
namespace {

// Largest split decode workspace: the counter header, then partial outputs
// and (max, sum) pairs of 2 * kMaxSlices slots of 8 query heads x head_dim
// 128 (see plan_decode).
constexpr size_t kScratchBytes = pa::kCounterHeaderBytes +
                                 size_t(2) * pa::kMaxSlices * 8 * 128 * sizeof(float) +
                                 size_t(2) * pa::kMaxSlices * 8 * 2 * sizeof(float);

// Each GPU the library runs on holds its own copy until the process ends.
// In host code this name is only a handle for hipGetSymbolAddress, never a
// device address.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

struct ZeroArgs {
  uint32_t* p;
  uint32_t n;     // words
};

__global__ __launch_bounds__(256) void zero_words_kernel(ZeroArgs z) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < z.n; i += gridDim.x * 256u) z.p[i] = 0u;
}

// The current device's copy of `scratch`, looked up once per device; the
// first lookup also zeroes its counter header on `stream` (a fill kernel,
// so that a caller capturing the stream into a graph records no memset).
pa_status scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                        "hipGetSymbolAddress(scratch)");
    const ZeroArgs z{static_cast<uint32_t*>(ptr),
                     static_cast<uint32_t>(pa::kCounterHeaderBytes / sizeof(uint32_t))};
    e = pa::launch_kernel(zero_words_kernel, dim3(64), dim3(256), 0, stream, z);
    if (e != hipSuccess) return hip_status(e, "scratch counter clear");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_decode_noalloc_max_bytes(void) { return kScratchBytes; }

pa_status pa_decode_noalloc(const pa_kv_pool* pool, const pa_seq_desc* seqs, const void* q,
                            void* out, int32_t num_q_heads, float scale, int32_t partition_size,
                            hipStream_t stream) {
  clear_error();
  pa::DecodeArgs a;
  pa::DecodePlan plan;
  const pa_status st = prepare_decode(pool, seqs, q, out, num_q_heads, scale, partition_size,
                                      true, &a, &plan);
  if (st != PA_OK) return st;
  if (seqs->num_seqs == 0) return PA_OK;
  if (plan.workspace_bytes > kScratchBytes)
    return fail(PA_ERR_UNSUPPORTED,
                "this split needs %zu bytes of scratch; pa_decode_noalloc holds %zu",
                plan.workspace_bytes, kScratchBytes);
  if (plan.workspace_bytes > 0) {
    void* ptr = nullptr;
    const pa_status ss = scratch_for_current_device(stream, &ptr);
    if (ss != PA_OK) return ss;
    a.counters = static_cast<int32_t*>(ptr);
    a.part_o = reinterpret_cast<float*>(static_cast<char*>(ptr) + plan.part_o_offset);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ptr) + plan.part_ml_offset);
  }
  return hip_status(pa::launch_decode(a, stream), "decode launch");
}

pa_status pa_decode_split_info(const pa_kv_pool* pool, const pa_seq_desc* seqs,
                               const int32_t* host_context_lens, int32_t num_q_heads,
                               int32_t partition_size, pa_decode_split* info) {
  clear_error();
  if (info == nullptr) return fail(PA_ERR_INVALID_ARG, "info is null");
  pa::DecodeArgs a;
  pa::DecodePlan plan;
  const pa_status st = prepare_decode(pool, seqs, nullptr, nullptr, num_q_heads, 1.f,
                                      partition_size, false, &a, &plan);
  if (st != PA_OK) return st;
  if (seqs->num_seqs > 0 && host_context_lens == nullptr)
    return fail(PA_ERR_INVALID_ARG, "host_context_lens is null");
  *info = pa_decode_split{};
  if (seqs->num_seqs == 0) return PA_OK;
  int grid = 0;
  const pa_status hs = hip_status(pa::decode_grid(a, &grid), "decode grid query");
  if (hs != PA_OK) return hs;
  info->workgroups = grid;
  // the kernel's plan, from the host copy of the lengths: pair (s, g) owns
  // nb_s blocks priced nb_s + seg_cost, laid end to end; split, the work is cut
  // into the static slices and handed-out chunks of pa::unit_plan
  const int H = pool->num_kv_heads;
  const int C = a.seg_cost;
  int64_t B = 0;
  int nb_lo = 0x7fffffff, nb_hi = 0;
  for (int s = 0; s < seqs->num_seqs; ++s) {
    int L = host_context_lens[s];
    L = L < 0 ? 0 : (L > a.context_cap ? a.context_cap : L);
    if (L == 0) continue;
    const int nb = (L + pa::kUnit - 1) / pa::kUnit;
    B += static_cast<int64_t>(H) * (nb + C);
    nb_lo = nb < nb_lo ? nb : nb_lo;
    nb_hi = nb > nb_hi ? nb : nb_hi;
  }
  pa::UnitPlan up{};
  if (a.min_slice_blocks > 0) {
    up = pa::unit_plan(static_cast<int32_t>(B), grid, a.min_slice_blocks, a.max_slices,
                       nb_lo >= nb_hi);
    info->slice_blocks = up.Q1;
    info->chunk_blocks = up.U > up.G ? up.Q2 : 0;
    info->units = up.U;
  }
  int64_t pairs = 0, pieces = 0, pre = 0;
  int32_t most = 0;
  for (int s = 0; s < seqs->num_seqs; ++s) {
    int L = host_context_lens[s];
    L = L < 0 ? 0 : (L > a.context_cap ? a.context_cap : L);
    if (L == 0) continue;
    const int64_t nb = (L + pa::kUnit - 1) / pa::kUnit;
    for (int g = 0; g < H; ++g) {
      const int64_t A = H * pre + g * (nb + C) + C;   // work position of the pair's block 0
      const int64_t n = a.min_slice_blocks > 0
                            ? up.of(static_cast<int32_t>(A + nb - 1)) - up.of(static_cast<int32_t>(A)) + 1
                            : 1;
      ++pairs;
      pieces += n;
      if (n > most) most = static_cast<int32_t>(n);
    }
    pre += nb + C;
  }
  info->pairs = static_cast<int32_t>(pairs);
  info->max_pieces = most;
  info->mean_pieces = pairs > 0 ? static_cast<float>(static_cast<double>(pieces) / pairs) : 0.f;
  return PA_OK;
}

pa_status pa_prefill(const pa_kv_pool* pool, const pa_seq_desc* seqs, const void* q, void* out,
                     const int32_t* q_start_loc, int32_t total_q_tokens, int32_t max_q_len,
                     int32_t num_q_heads, float scale, hipStream_t stream) {
  clear_error();
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if ((st = check_seqs(seqs, pool->block_size)) != PA_OK) return st;
  if ((st = check_heads(pool, num_q_heads)) != PA_OK) return st;
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  if (total_q_tokens < 0 || max_q_len < 0)
    return fail(PA_ERR_INVALID_ARG, "total_q_tokens %d / max_q_len %d < 0", total_q_tokens,
                max_q_len);
  if (seqs->num_seqs == 0 || total_q_tokens == 0 || max_q_len == 0) return PA_OK;
  if (q == nullptr || out == nullptr || q_start_loc == nullptr)
    return fail(PA_ERR_INVALID_ARG, "q, out or q_start_loc is null");
  if (!aligned16(q) || !aligned16(out))
    return fail(PA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  pa::PrefillArgs a{};
  a.q = q;
  a.out = out;
  a.k_cache = pool->k_cache;
  a.v_cache = pool->v_cache;
  a.block_tables = seqs->block_tables;
  a.context_lens = seqs->context_lens;
  a.q_start_loc = q_start_loc;
  a.num_seqs = seqs->num_seqs;
  a.num_blocks = pool->num_blocks;
  a.num_kv_heads = pool->num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.head_dim = pool->head_dim;
  a.max_blocks_per_seq = seqs->max_blocks_per_seq;
  a.context_cap = context_cap(seqs, pool->block_size);
  a.max_q_len = max_q_len;
  a.total_q_tokens = total_q_tokens;
  a.dtype = pool->dtype;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.geom = geom_of(pool);
  return hip_status(pa::launch_prefill(a, stream), "prefill launch");
}

}  // extern "C"
