// Host half of libpa: status messages, closed forms, the block allocator
// (free_block_queue) and the token -> slot mapping.  Plain C++17, no HIP:
// it also builds with g++ alone for host sanitizer runs.
//
// "Inside vLLM: Anatomy of a High-Throughput LLM Inference System",
// section "LLM Engine & Engine Core": the KV-cache manager keeps a
// free_block_queue; blocks map a sequence's tokens to where their keys and
// values live.  Section "LLM Engine constructor": the block-bytes formula.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace pa {

namespace {
thread_local char g_err[512] = "";
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

}  // namespace pa

using pa::fail;

extern "C" const char* pa_last_error(void) { return pa::g_err; }

extern "C" int pa_version(void) { return 100; }  // 0.1.0

extern "C" size_t pa_kv_block_bytes(int32_t block_size, int32_t num_kv_heads,
                                    int32_t head_size, int32_t dtype_bytes) {
  if (block_size <= 0 || num_kv_heads <= 0 || head_size <= 0 || dtype_bytes <= 0)
    return 0;
  return size_t(2) * size_t(block_size) * size_t(num_kv_heads) *
         size_t(head_size) * size_t(dtype_bytes);
}

extern "C" int64_t pa_num_blocks_for_budget(uint64_t budget_bytes,
                                            size_t block_bytes,
                                            int32_t num_layers) {
  if (block_bytes == 0 || num_layers <= 0) return -1;
  const unsigned __int128 per_id =
      (unsigned __int128)block_bytes * (unsigned __int128)num_layers;
  return (int64_t)((unsigned __int128)budget_bytes / per_id);
}

// ---------------------------------------------------------------------------
// Allocator: a ring buffer holds the free queue (head..tail), a refcount per
// block id.  Every operation is O(n) in its argument count; capacity is the
// pool size, so a block can never be queued twice.
// ---------------------------------------------------------------------------
struct pa_allocator {
  int32_t n = 0;
  std::vector<int32_t> ring;      // capacity n
  int32_t head = 0, count = 0;    // queue = ring[head .. head+count) mod n
  std::vector<int32_t> refcount;  // n
  void push_tail(int32_t id) { ring[(head + count) % n] = id; ++count; }
  int32_t pop_head() {
    int32_t id = ring[head];
    head = (head + 1) % n;
    --count;
    return id;
  }
};

extern "C" int pa_allocator_create(int32_t num_blocks,
                                   const int32_t* initial_order,
                                   pa_allocator** out) {
  if (!out) return fail(PA_EINVAL, "pa_allocator_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 0) return fail(PA_EINVAL, "pa_allocator_create: num_blocks < 0");
  pa_allocator* a = new (std::nothrow) pa_allocator();
  if (!a) return fail(PA_EINVAL, "pa_allocator_create: out of host memory");
  try {
    a->n = num_blocks;
    a->ring.assign(num_blocks > 0 ? num_blocks : 1, 0);
    a->refcount.assign(num_blocks, 0);
  } catch (...) {
    delete a;
    return fail(PA_EINVAL, "pa_allocator_create: out of host memory");
  }
  if (initial_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t id = initial_order[i];
      if (id < 0 || id >= num_blocks || seen[id]) {
        delete a;
        return fail(PA_EINVAL,
                    "pa_allocator_create: initial_order is not a permutation "
                    "(entry %d = %d)", i, id);
      }
      seen[id] = 1;
    }
  }
  for (int32_t i = 0; i < num_blocks; ++i)
    a->push_tail(initial_order ? initial_order[i] : i);
  *out = a;
  return PA_OK;
}

extern "C" void pa_allocator_destroy(pa_allocator* a) { delete a; }

extern "C" int pa_allocator_allocate(pa_allocator* a, int32_t n, int32_t* out_ids) {
  if (!a) return fail(PA_EINVAL, "pa_allocator_allocate: NULL handle");
  if (n < 0) return fail(PA_EINVAL, "pa_allocator_allocate: n = %d < 0", n);
  if (n == 0) return PA_OK;
  if (!out_ids) return fail(PA_EINVAL, "pa_allocator_allocate: out_ids is NULL");
  if (n > a->count)
    return fail(PA_ENOBLOCKS, "pa_allocator_allocate: need %d blocks, %d free", n, a->count);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = a->pop_head();
    a->refcount[id] = 1;
    out_ids[i] = id;
  }
  return PA_OK;
}

extern "C" int pa_allocator_share(pa_allocator* a, const int32_t* ids, int32_t n) {
  if (!a) return fail(PA_EINVAL, "pa_allocator_share: NULL handle");
  if (n < 0 || (n > 0 && !ids)) return fail(PA_EINVAL, "pa_allocator_share: bad id list");
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= a->n)
      return fail(PA_EINVAL, "pa_allocator_share: block %d out of range", id);
    if (a->refcount[id] == 0)
      return fail(PA_EINVAL, "pa_allocator_share: block %d is free", id);
  }
  for (int32_t i = 0; i < n; ++i) ++a->refcount[ids[i]];
  return PA_OK;
}

extern "C" int pa_allocator_free(pa_allocator* a, const int32_t* ids, int32_t n) {
  if (!a) return fail(PA_EINVAL, "pa_allocator_free: NULL handle");
  if (n < 0 || (n > 0 && !ids)) return fail(PA_EINVAL, "pa_allocator_free: bad id list");
  // validate the whole request first: multiplicity of each id <= refcount
  std::unordered_map<int32_t, int32_t> want;
  want.reserve(size_t(n) * 2);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= a->n)
      return fail(PA_EINVAL, "pa_allocator_free: block %d out of range", id);
    if (++want[id] > a->refcount[id])
      return fail(PA_EINVAL, "pa_allocator_free: block %d freed more often than it is held", id);
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (--a->refcount[id] == 0) a->push_tail(id);
  }
  return PA_OK;
}

extern "C" int32_t pa_allocator_num_free(const pa_allocator* a) { return a ? a->count : -1; }
extern "C" int32_t pa_allocator_num_blocks(const pa_allocator* a) { return a ? a->n : -1; }

extern "C" int pa_allocator_export(const pa_allocator* a, int32_t* queue_out,
                                   int32_t* refcount_out) {
  if (!a) return fail(PA_EINVAL, "pa_allocator_export: NULL handle");
  if (queue_out)
    for (int32_t i = 0; i < a->count; ++i) queue_out[i] = a->ring[(a->head + i) % a->n];
  if (refcount_out && a->n > 0)
    std::memcpy(refcount_out, a->refcount.data(), sizeof(int32_t) * size_t(a->n));
  return PA_OK;
}

extern "C" int pa_allocator_stats(const pa_allocator* a, const int32_t* seq_lens,
                                  int32_t B, int32_t block_size,
                                  int64_t* used_blocks, int64_t* tail_waste_tokens) {
  if (!a) return fail(PA_EINVAL, "pa_allocator_stats: NULL handle");
  if (B < 0 || (B > 0 && !seq_lens) || block_size <= 0)
    return fail(PA_EINVAL, "pa_allocator_stats: bad arguments");
  if (used_blocks) *used_blocks = int64_t(a->n) - a->count;
  if (tail_waste_tokens) {
    int64_t w = 0;
    for (int32_t b = 0; b < B; ++b) {
      const int64_t L = seq_lens[b];
      if (L < 0) return fail(PA_EINVAL, "pa_allocator_stats: seq_lens[%d] < 0", b);
      w += (L + block_size - 1) / block_size * block_size - L;
    }
    *tail_waste_tokens = w;
  }
  return PA_OK;
}

// ---------------------------------------------------------------------------
// slots
// ---------------------------------------------------------------------------
extern "C" int pa_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* start_pos, const int32_t* num_tokens,
                               int32_t B, int32_t block_size, int64_t* out,
                               int64_t* total) {
  if (B < 0 || block_size <= 0 || max_blocks_per_seq < 0)
    return fail(PA_EINVAL, "pa_slot_mapping: bad sizes");
  if (B > 0 && (!block_tables || !start_pos || !num_tokens))
    return fail(PA_EINVAL, "pa_slot_mapping: NULL array");
  int64_t k = 0;
  // validate everything before writing anything
  for (int32_t b = 0; b < B; ++b) {
    if (start_pos[b] < 0 || num_tokens[b] < 0)
      return fail(PA_EINVAL, "pa_slot_mapping: negative position/count for sequence %d", b);
    const int64_t last = int64_t(start_pos[b]) + num_tokens[b] - 1;
    if (num_tokens[b] > 0 && last / block_size >= max_blocks_per_seq)
      return fail(PA_EINVAL, "pa_slot_mapping: sequence %d position %lld beyond its table",
                  b, (long long)last);
    for (int64_t p = start_pos[b]; p <= last; p += block_size - (p % block_size)) {
      if (block_tables[int64_t(b) * max_blocks_per_seq + p / block_size] < 0)
        return fail(PA_EINVAL, "pa_slot_mapping: sequence %d position %lld has no block",
                    b, (long long)p);
    }
    k += num_tokens[b];
  }
  if (k > 0 && !out) return fail(PA_EINVAL, "pa_slot_mapping: out is NULL");
  k = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t* row = block_tables + int64_t(b) * max_blocks_per_seq;
    for (int32_t i = 0; i < num_tokens[b]; ++i) {
      const int64_t p = int64_t(start_pos[b]) + i;
      out[k++] = int64_t(row[p / block_size]) * block_size + p % block_size;
    }
  }
  if (total) *total = k;
  return PA_OK;
}
