// Host-side physical block allocator with reference counts, the bookkeeping
// half of copy-on-write paging.
//
// Free blocks are handed out first-in first-out: ids 0 .. num_blocks-1 in
// order at first, released blocks appended at the back (Pico-vLLM #5 Paged
// Attention, "核心数据结构和设计模式", BlockManager: a deque of free ids,
// popleft to allocate, append to free).  A block named by several block
// tables carries a reference count above one; writing into such a block
// first moves the writer to a fresh copy and drops one reference from the
// shared block (JuliaPagedAttn README, "Copy-on-Write").
//
// Every operation checks its whole request before changing anything, so a
// failed call leaves the allocator as it was.

#include <cstdint>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

struct pa_block_allocator {
  int32_t num_blocks = 0;
  std::vector<int32_t> ring;       // free ids, FIFO, capacity num_blocks
  int32_t head = 0, count = 0;     // ring[head .. head+count) mod num_blocks
  std::vector<int32_t> refs;       // reference count per block, 0 = free

  int32_t pop() {
    const int32_t id = ring[head];
    head = head + 1 == num_blocks ? 0 : head + 1;
    --count;
    refs[id] = 1;
    return id;
  }
  void push(int32_t id) {
    int32_t tail = head + count;
    if (tail >= num_blocks) tail -= num_blocks;
    ring[tail] = id;
    ++count;
  }
};

extern "C" {

using pa::report;

pa_status pa_allocator_create(int32_t num_blocks, pa_block_allocator** out) {
  pa::clear_report();
  if (out == nullptr || num_blocks <= 0)
    return report(PA_ERR_INVALID_ARG, "allocator needs num_blocks > 0 and an out pointer");
  auto* a = new pa_block_allocator;
  a->num_blocks = num_blocks;
  a->ring.resize(num_blocks);
  a->refs.assign(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) a->ring[i] = i;
  a->count = num_blocks;
  *out = a;
  return PA_OK;
}

void pa_allocator_destroy(pa_block_allocator* a) { delete a; }

int32_t pa_allocator_num_free(const pa_block_allocator* a) { return a ? a->count : -1; }

int32_t pa_allocator_refcount(const pa_block_allocator* a, int32_t block) {
  if (a == nullptr || block < 0 || block >= a->num_blocks) return -1;
  return a->refs[block];
}

pa_status pa_allocator_allocate(pa_block_allocator* a, int32_t n, int32_t* blocks) {
  pa::clear_report();
  if (a == nullptr || n < 0 || (n > 0 && blocks == nullptr))
    return report(PA_ERR_INVALID_ARG, "allocate: null allocator or blocks, or n < 0");
  if (n > a->count)
    return report(PA_ERR_NO_BLOCKS, "allocate: %d blocks asked, %d free", n, a->count);
  for (int32_t i = 0; i < n; ++i) blocks[i] = a->pop();
  return PA_OK;
}

// blocks listed k times need k references (release) or one (fork)
static bool all_held(const pa_block_allocator* a, const int32_t* blocks, int32_t n,
                     bool count_repeats) {
  std::vector<int32_t> need;
  if (count_repeats) need.assign(a->num_blocks, 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    if (b < 0 || b >= a->num_blocks || a->refs[b] == 0) return false;
    if (count_repeats && ++need[b] > a->refs[b]) return false;
  }
  return true;
}

pa_status pa_allocator_fork(pa_block_allocator* a, const int32_t* blocks, int32_t n) {
  pa::clear_report();
  if (a == nullptr || n < 0 || (n > 0 && blocks == nullptr))
    return report(PA_ERR_INVALID_ARG, "fork: null allocator or blocks, or n < 0");
  if (!all_held(a, blocks, n, false))
    return report(PA_ERR_INVALID_ARG, "fork: a listed block is out of range or not allocated");
  for (int32_t i = 0; i < n; ++i) ++a->refs[blocks[i]];
  return PA_OK;
}

pa_status pa_allocator_release(pa_block_allocator* a, const int32_t* blocks, int32_t n) {
  pa::clear_report();
  if (a == nullptr || n < 0 || (n > 0 && blocks == nullptr))
    return report(PA_ERR_INVALID_ARG, "release: null allocator or blocks, or n < 0");
  if (!all_held(a, blocks, n, true))
    return report(PA_ERR_INVALID_ARG,
                  "release: a listed block is out of range or has fewer references than listed");
  for (int32_t i = 0; i < n; ++i)
    if (--a->refs[blocks[i]] == 0) a->push(blocks[i]);
  return PA_OK;
}

pa_status pa_allocator_prepare_write(pa_block_allocator* a, int32_t* table, int32_t width,
                                     int32_t* num_used, int32_t block_size, int32_t start,
                                     int32_t count, int32_t* copy_src, int32_t* copy_dst,
                                     int32_t copy_cap, int32_t* num_copies) {
  pa::clear_report();
  if (a == nullptr || table == nullptr || num_used == nullptr || num_copies == nullptr ||
      width <= 0 || block_size <= 0 || start < 0 || count < 0 || copy_cap < 0 ||
      (copy_cap > 0 && (copy_src == nullptr || copy_dst == nullptr)))
    return report(PA_ERR_INVALID_ARG, "prepare_write: null pointer or negative size");
  const int32_t used = *num_used;
  *num_copies = 0;
  if (used < 0 || used > width)
    return report(PA_ERR_INVALID_ARG, "prepare_write: num_used %d outside [0, %d]", used, width);
  if (count == 0) return PA_OK;
  const int64_t end = static_cast<int64_t>(start) + count;          // positions [start, end)
  const int64_t j0 = start / block_size;
  const int64_t j1 = (end - 1) / block_size;                        // last block touched
  if (j0 > used)
    return report(PA_ERR_INVALID_ARG, "prepare_write: position %d leaves a gap after %d blocks",
                  start, used);
  if (j1 >= width)
    return report(PA_ERR_INVALID_ARG, "prepare_write: block %lld past the table width %d",
                  static_cast<long long>(j1), width);
  // the request: shared blocks among the touched ones, then the appended blocks
  int32_t shared = 0;
  for (int64_t j = j0; j < used && j <= j1; ++j) {
    const int32_t b = table[j];
    if (b < 0 || b >= a->num_blocks || a->refs[b] == 0)
      return report(PA_ERR_INVALID_ARG, "prepare_write: table entry %lld names block %d, not held",
                    static_cast<long long>(j), b);
    if (a->refs[b] > 1) ++shared;
  }
  const int64_t appended = j1 + 1 > used ? j1 + 1 - used : 0;
  if (shared > copy_cap)
    return report(PA_ERR_INVALID_ARG, "prepare_write: %d copies needed, room for %d", shared,
                  copy_cap);
  if (shared + appended > a->count)
    return report(PA_ERR_NO_BLOCKS, "prepare_write: %lld blocks needed, %d free",
                  static_cast<long long>(shared + appended), a->count);
  int32_t nc = 0;
  for (int64_t j = j0; j < used && j <= j1; ++j) {
    const int32_t b = table[j];
    if (a->refs[b] > 1) {
      const int32_t fresh = a->pop();
      --a->refs[b];
      copy_src[nc] = b;
      copy_dst[nc] = fresh;
      ++nc;
      table[j] = fresh;
    }
  }
  for (int64_t j = used; j <= j1; ++j) table[j] = a->pop();
  *num_used = static_cast<int32_t>(j1 + 1 > used ? j1 + 1 : used);
  *num_copies = nc;
  return PA_OK;
}

}  // extern "C"
