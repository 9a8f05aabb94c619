// Host half of libpa: status messages, closed forms, the block allocator
// (free_block_queue), the token -> slot mapping, the decode work plan and
// the host half of a decode step.  Plain C++17, no HIP:
// it also builds with g++ alone for host sanitizer runs.
//
// "Inside vLLM: Anatomy of a High-Throughput LLM Inference System",
// section "LLM Engine & Engine Core": the KV-cache manager keeps a
// free_block_queue; blocks map a sequence's tokens to where their keys and
// values live.  Section "LLM Engine constructor": the block-bytes formula.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <utility>
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
// Allocator.  The free queue is a doubly linked list threaded through the
// block ids (push at the tail, pop at the head, and unlink of a cached free
// block that a prefix lookup takes back), a refcount per block id.  Every
// operation is O(n) in its argument count; a block is queued at most once.
//
// Prefix cache ("Im Inneren von vLLM", section "Fortgeschrittene
// Funktionen": KV caches of common prompt prefixes are kept and reused).  A
// full block's keys and values are a function of every token up to its end,
// so a cached block is identified by that whole token prefix.  The prefixes
// form a trie: a node is one full block of tokens under its parent node (the
// root is -1), so node identity is prefix identity and needs no hash that
// could collide.  A node holds the block that caches it, or -1 once that
// block has been evicted; a node with neither a block nor children is
// deleted, so node ids are never stale in a child's key.
// ---------------------------------------------------------------------------
namespace {

struct NodeKey {
  int32_t parent;
  std::vector<int32_t> tokens;
  bool operator==(const NodeKey& o) const {
    return parent == o.parent && tokens == o.tokens;
  }
};

// FNV-1a, 64-bit (Fowler, Noll, Vo): offset basis 14695981039346656037,
// prime 1099511628211, over the key's bytes.  Only the bucket choice depends
// on it; equality above is exact.
struct NodeKeyHash {
  size_t operator()(const NodeKey& k) const {
    uint64_t h = 14695981039346656037ull;
    auto mix = [&h](int32_t v) {
      uint32_t u = uint32_t(v);
      for (int i = 0; i < 4; ++i) {
        h ^= (u >> (8 * i)) & 0xFFu;
        h *= 1099511628211ull;
      }
    };
    mix(k.parent);
    for (int32_t t : k.tokens) mix(t);
    return size_t(h);
  }
};

struct Node {
  int32_t parent = -1;
  int32_t block = -1;     // block caching this prefix, -1: evicted
  int32_t children = 0;   // live child nodes
  std::vector<int32_t> tokens;
};

}  // namespace

struct pa_allocator {
  int32_t n = 0;
  std::vector<int32_t> prev, next;  // queue links, -1 at the ends
  std::vector<char> queued;
  int32_t head = -1, tail = -1, count = 0;
  std::vector<int32_t> refcount;  // n

  // prefix cache (block_size 0: not enabled)
  int32_t cache_bs = 0;
  std::vector<int32_t> block_node;  // node a block caches, or -1
  std::vector<Node> nodes;
  std::vector<int32_t> spare_nodes;
  std::unordered_map<NodeKey, int32_t, NodeKeyHash> index;
  int64_t cached = 0, hits = 0, evictions = 0;

  void push_tail(int32_t id) {
    prev[id] = tail;
    next[id] = -1;
    if (tail >= 0) next[tail] = id; else head = id;
    tail = id;
    queued[id] = 1;
    ++count;
  }
  void unlink(int32_t id) {
    if (prev[id] >= 0) next[prev[id]] = next[id]; else head = next[id];
    if (next[id] >= 0) prev[next[id]] = prev[id]; else tail = prev[id];
    prev[id] = next[id] = -1;
    queued[id] = 0;
    --count;
  }
  int32_t pop_head() {
    const int32_t id = head;
    unlink(id);
    return id;
  }

  int32_t find_child(int32_t parent, const int32_t* toks) const {
    NodeKey k{parent, std::vector<int32_t>(toks, toks + cache_bs)};
    auto it = index.find(k);
    return it == index.end() ? -1 : it->second;
  }
  int32_t child_or_new(int32_t parent, const int32_t* toks) {
    NodeKey k{parent, std::vector<int32_t>(toks, toks + cache_bs)};
    auto it = index.find(k);
    if (it != index.end()) return it->second;
    int32_t id;
    if (!spare_nodes.empty()) {
      id = spare_nodes.back();
      spare_nodes.pop_back();
    } else {
      id = int32_t(nodes.size());
      nodes.emplace_back();
    }
    Node& nd = nodes[id];
    nd.parent = parent;
    nd.block = -1;
    nd.children = 0;
    nd.tokens = k.tokens;
    if (parent >= 0) ++nodes[parent].children;
    index.emplace(std::move(k), id);
    return id;
  }
  // deletes nodes that cache nothing and have no children, walking up
  void prune(int32_t id) {
    while (id >= 0 && nodes[id].block < 0 && nodes[id].children == 0) {
      Node& nd = nodes[id];
      index.erase(NodeKey{nd.parent, nd.tokens});
      const int32_t parent = nd.parent;
      if (parent >= 0) --nodes[parent].children;
      nd.tokens.clear();
      spare_nodes.push_back(id);
      id = parent;
    }
  }
  // a cached block leaves the cache (it is about to hold other contents)
  void evict(int32_t id) {
    const int32_t nd = block_node[id];
    nodes[nd].block = -1;
    block_node[id] = -1;
    --cached;
    ++evictions;
    prune(nd);
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
    a->prev.assign(num_blocks, -1);
    a->next.assign(num_blocks, -1);
    a->queued.assign(num_blocks, 0);
    a->refcount.assign(num_blocks, 0);
    a->block_node.assign(num_blocks, -1);
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
    if (a->block_node[id] >= 0) a->evict(id);
    a->refcount[id] = 1;
    out_ids[i] = id;
  }
  return PA_OK;
}

extern "C" int pa_allocator_build_tables(pa_allocator* a, const int32_t* seq_lens, int32_t B,
                                         int32_t block_size, int32_t width,
                                         int32_t* block_tables) {
  if (!a) return fail(PA_EINVAL, "pa_allocator_build_tables: NULL handle");
  if (B < 0 || block_size <= 0 || width < 0 || (B > 0 && (!seq_lens || !block_tables)))
    return fail(PA_EINVAL, "pa_allocator_build_tables: bad arguments");
  int64_t total = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (seq_lens[b] < 0)
      return fail(PA_EINVAL, "pa_allocator_build_tables: seq_lens[%d] = %d", b, seq_lens[b]);
    const int64_t n = (int64_t(seq_lens[b]) + block_size - 1) / block_size;
    if (n > width)
      return fail(PA_EINVAL, "pa_allocator_build_tables: sequence %d needs %lld blocks, "
                  "rows hold %d", b, (long long)n, width);
    total += n;
  }
  if (total > a->count)
    return fail(PA_ENOBLOCKS, "pa_allocator_build_tables: need %lld blocks, %d free",
                (long long)total, a->count);
  for (int32_t b = 0; b < B; ++b) {
    const int32_t n = (seq_lens[b] + block_size - 1) / block_size;
    int32_t* row = block_tables + int64_t(b) * width;
    for (int32_t j = 0; j < n; ++j) {
      const int32_t id = a->pop_head();
      if (a->block_node[id] >= 0) a->evict(id);
      a->refcount[id] = 1;
      row[j] = id;
    }
    for (int32_t j = n; j < width; ++j) row[j] = -1;
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
  if (queue_out) {
    int32_t i = 0;
    for (int32_t id = a->head; id >= 0; id = a->next[id]) queue_out[i++] = id;
  }
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
// prefix cache
// ---------------------------------------------------------------------------
extern "C" int pa_prefix_cache_enable(pa_allocator* a, int32_t block_size) {
  if (!a) return fail(PA_EINVAL, "pa_prefix_cache_enable: NULL handle");
  if (block_size <= 0)
    return fail(PA_EINVAL, "pa_prefix_cache_enable: block_size = %d", block_size);
  if (a->cache_bs != 0 && a->cache_bs != block_size)
    return fail(PA_EINVAL, "pa_prefix_cache_enable: already enabled with block_size %d",
                a->cache_bs);
  a->cache_bs = block_size;
  return PA_OK;
}

extern "C" int pa_prefix_cache_acquire(pa_allocator* a, const int32_t* tokens,
                                       int32_t num_tokens, int32_t* out_ids,
                                       int32_t* num_hit) {
  if (!a) return fail(PA_EINVAL, "pa_prefix_cache_acquire: NULL handle");
  if (a->cache_bs == 0) return fail(PA_EINVAL, "pa_prefix_cache_acquire: cache not enabled");
  if (!num_hit) return fail(PA_EINVAL, "pa_prefix_cache_acquire: num_hit is NULL");
  if (num_tokens < 0 || (num_tokens > 0 && !tokens))
    return fail(PA_EINVAL, "pa_prefix_cache_acquire: bad token list");
  const int32_t full = num_tokens / a->cache_bs;
  if (full > 0 && !out_ids) return fail(PA_EINVAL, "pa_prefix_cache_acquire: out_ids is NULL");
  int32_t node = -1, h = 0;
  for (int32_t j = 0; j < full; ++j) {
    const int32_t child = a->find_child(node, tokens + int64_t(j) * a->cache_bs);
    if (child < 0 || a->nodes[child].block < 0) break;
    const int32_t id = a->nodes[child].block;
    if (a->refcount[id] == 0) a->unlink(id);  // a cached free block is taken back
    ++a->refcount[id];
    out_ids[h++] = id;
    node = child;
  }
  a->hits += h;
  *num_hit = h;
  return PA_OK;
}

extern "C" int pa_prefix_cache_insert(pa_allocator* a, const int32_t* tokens,
                                      int32_t num_tokens, const int32_t* block_ids,
                                      int32_t num_blocks) {
  if (!a) return fail(PA_EINVAL, "pa_prefix_cache_insert: NULL handle");
  if (a->cache_bs == 0) return fail(PA_EINVAL, "pa_prefix_cache_insert: cache not enabled");
  if (num_tokens < 0 || (num_tokens > 0 && !tokens))
    return fail(PA_EINVAL, "pa_prefix_cache_insert: bad token list");
  const int32_t full = num_tokens / a->cache_bs;
  if (num_blocks < full || (full > 0 && !block_ids))
    return fail(PA_EINVAL, "pa_prefix_cache_insert: %d full blocks but %d block ids",
                full, num_blocks);
  // validate the whole request before any change
  std::unordered_map<int32_t, int32_t> seen;
  int32_t node = -1;
  bool on_path = true;  // the trie already holds the prefix up to block j
  for (int32_t j = 0; j < full; ++j) {
    const int32_t id = block_ids[j];
    if (id < 0 || id >= a->n)
      return fail(PA_EINVAL, "pa_prefix_cache_insert: block %d out of range", id);
    if (a->refcount[id] == 0)
      return fail(PA_EINVAL, "pa_prefix_cache_insert: block %d is free", id);
    if (!seen.emplace(id, j).second)
      return fail(PA_EINVAL, "pa_prefix_cache_insert: block %d listed twice", id);
    int32_t child = -1;
    if (on_path) {
      child = a->find_child(node, tokens + int64_t(j) * a->cache_bs);
      on_path = child >= 0;
      node = child;
    }
    if (a->block_node[id] >= 0 && a->block_node[id] != child)
      return fail(PA_EINVAL,
                  "pa_prefix_cache_insert: block %d already caches another prefix", id);
  }
  node = -1;
  for (int32_t j = 0; j < full; ++j) {
    const int32_t id = block_ids[j];
    node = a->child_or_new(node, tokens + int64_t(j) * a->cache_bs);
    Node& nd = a->nodes[node];
    if (nd.block < 0) {  // first block to hold this prefix
      nd.block = id;
      a->block_node[id] = node;
      ++a->cached;
    }
    // else: this prefix is cached already (by id itself, or by another block,
    // which stays the cached copy; id then stays uncached)
  }
  return PA_OK;
}

extern "C" int pa_prefix_cache_export(const pa_allocator* a, int32_t* cached_out,
                                      int64_t* stats_out) {
  if (!a) return fail(PA_EINVAL, "pa_prefix_cache_export: NULL handle");
  if (cached_out)
    for (int32_t i = 0; i < a->n; ++i) cached_out[i] = a->block_node[i] >= 0 ? 1 : 0;
  if (stats_out) {
    stats_out[0] = a->cached;
    stats_out[1] = a->hits;
    stats_out[2] = a->evictions;
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

// ---------------------------------------------------------------------------
// decode work plan and the host half of a decode step
// ---------------------------------------------------------------------------
namespace {

// Partitions of max_seq_len tokens (1 when there is no split).
int64_t plan_parts(int32_t max_seq_len, int32_t partition_size) {
  if (partition_size <= 0 || max_seq_len <= 0) return 1;
  return (int64_t(max_seq_len) + partition_size - 1) / partition_size;
}

// Division by a positive divisor fixed for a call: shifts when it is a
// power of two (block sizes and partition sizes usually are), else the
// plain operators.
struct Divisor {
  int32_t d;
  int shift = -1;
  explicit Divisor(int32_t v) : d(v) {
    if (v > 0 && (v & (v - 1)) == 0) shift = __builtin_ctz(uint32_t(v));
  }
  int32_t div(int32_t x) const { return shift >= 0 ? x >> shift : x / d; }
  int32_t mod(int32_t x) const { return shift >= 0 ? x & (d - 1) : x % d; }
};

// Entries of one sequence of length L (an empty sequence still gets one,
// its zero output row).
inline int64_t plan_items(int32_t L, int64_t P, const Divisor& part) {
  if (P <= 1 || L == 0) return 1;
  return part.div(L + part.d - 1);
}

// Writes the plan of lengths L[0..B) (validated by the caller) into plan:
// entries (part << 16) | b ordered by tokens descending, then part, then b.
// Without a split every sequence is one item of L tokens.  With one, the
// full partitions (partition_size tokens, more than any other item) come
// first in (part, b) order, listed part by part over the sequences that
// still have one; then each sequence's last, shorter partition (or its
// single empty item).  Those are ordered by one sort of 64-bit keys
// (tokens inverted, part, b), which is the entry itself in the low bits.
void write_plan(const int32_t* L, int32_t B, int64_t P, const Divisor& part, int32_t* plan) {
  static thread_local std::vector<uint64_t> tail;
  static thread_local std::vector<std::pair<int32_t, int32_t>> active;   // (b, full partitions)
  tail.clear();
  auto key = [](int32_t tokens, int32_t part, int32_t b) {
    return (uint64_t(uint32_t(0x7FFFFFFF - tokens)) << 32) | (uint64_t(uint32_t(part)) << 16) |
           uint64_t(uint32_t(b));
  };
  int64_t k = 0;
  if (P <= 1) {
    for (int32_t b = 0; b < B; ++b) tail.push_back(key(L[b], 0, b));
  } else {
    active.clear();
    for (int32_t b = 0; b < B; ++b) {
      const int32_t full = part.div(L[b]), rem = part.mod(L[b]);
      if (full > 0) active.emplace_back(b, full);
      if (rem > 0 || L[b] == 0) tail.push_back(key(rem, full, b));
    }
    for (int32_t p = 0; !active.empty(); ++p) {
      size_t keep = 0;
      for (const auto& bf : active) {
        plan[k++] = int32_t(uint32_t(p) << 16 | uint32_t(bf.first));
        if (bf.second > p + 1) active[keep++] = bf;
      }
      active.resize(keep);
    }
  }
  std::sort(tail.begin(), tail.end());
  for (uint64_t e : tail) plan[k++] = int32_t(uint32_t(e));
}

}  // namespace

extern "C" int pa_decode_plan(const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
                              int32_t partition_size, int32_t* plan, int32_t capacity,
                              int32_t* num_entries) {
  if (B < 0 || max_seq_len < 0 || partition_size < 0 || partition_size % 16 || capacity < 0)
    return fail(PA_EINVAL, "pa_decode_plan: bad sizes");
  if (B > 65535) return fail(PA_ENOTSUP, "pa_decode_plan: B %d > 65535", B);
  if (B > 0 && !seq_lens) return fail(PA_EINVAL, "pa_decode_plan: NULL seq_lens");
  const int64_t P = plan_parts(max_seq_len, partition_size);
  if (P > 65535) return fail(PA_ENOTSUP, "pa_decode_plan: too many partitions");
  const Divisor part(partition_size > 0 ? partition_size : 1);
  int64_t n = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t L = seq_lens[b];
    if (L < 0 || L > max_seq_len)
      return fail(PA_EINVAL, "pa_decode_plan: seq_lens[%d] = %d outside [0, %d]", b, L, max_seq_len);
    n += plan_items(L, P, part);
  }
  if (num_entries) *num_entries = int32_t(n);
  if (n > capacity)
    return fail(PA_EINVAL, "pa_decode_plan: %lld entries, capacity %d", (long long)n, capacity);
  if (n > 0 && !plan) return fail(PA_EINVAL, "pa_decode_plan: NULL plan");
  write_plan(seq_lens, B, P, part, plan);
  return PA_OK;
}

extern "C" int pa_decode_step_prepare(pa_allocator* a, int32_t* block_tables,
                                      int32_t max_blocks_per_seq, int32_t* seq_lens, int32_t B,
                                      int32_t block_size, int32_t max_seq_len,
                                      int32_t partition_size, int64_t* slots, int32_t* plan,
                                      int32_t plan_capacity, int32_t* num_entries) {
  const char* fn = "pa_decode_step_prepare";
  if (num_entries) *num_entries = 0;
  if (!a) return fail(PA_EINVAL, "%s: NULL allocator", fn);
  if (B < 0 || block_size <= 0 || max_blocks_per_seq < 0 || max_seq_len < 0 ||
      partition_size < 0 || partition_size % 16 || plan_capacity < 0)
    return fail(PA_EINVAL, "%s: bad sizes", fn);
  if (B > 65535) return fail(PA_ENOTSUP, "%s: B %d > 65535", fn, B);
  if (B > 0 && (!block_tables || !seq_lens || !slots)) return fail(PA_EINVAL, "%s: NULL array", fn);
  const int64_t P = plan_parts(max_seq_len, partition_size);
  if (plan && P > 65535) return fail(PA_ENOTSUP, "%s: too many partitions", fn);
  const Divisor blk(block_size), part(partition_size > 0 ? partition_size : 1);
  // validate everything before changing anything
  int64_t need = 0, n = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t p = seq_lens[b];   // position of the new token
    if (p < 0 || p >= max_seq_len)
      return fail(PA_EINVAL, "%s: sequence %d: new token at %d, max_seq_len %d", fn, b, p,
                  max_seq_len);
    const int32_t j = blk.div(p);
    if (j >= max_blocks_per_seq)
      return fail(PA_EINVAL, "%s: sequence %d: position %d beyond its table", fn, b, p);
    const int32_t id = block_tables[int64_t(b) * max_blocks_per_seq + j];
    if (blk.mod(p) == 0) {
      if (id >= 0)
        return fail(PA_EINVAL, "%s: sequence %d: table entry %d already holds block %d", fn, b,
                    j, id);
      ++need;
    } else if (id < 0 || id >= a->n) {
      return fail(PA_EINVAL, "%s: sequence %d: position %d has no block", fn, b, p);
    }
    if (plan) n += plan_items(p + 1, P, part);
  }
  if (plan) {
    if (num_entries) *num_entries = int32_t(n);
    if (n > plan_capacity)
      return fail(PA_EINVAL, "%s: %lld plan entries, capacity %d", fn, (long long)n,
                  plan_capacity);
  }
  if (need > a->count)
    return fail(PA_ENOBLOCKS, "%s: need %lld blocks, %d free", fn, (long long)need, a->count);
  // blocks for the sequences whose new token opens one, in sequence order
  // (as one pa_allocator_allocate of that many blocks)
  for (int32_t b = 0; b < B; ++b) {
    const int32_t p = seq_lens[b];
    int32_t* row = block_tables + int64_t(b) * max_blocks_per_seq;
    const int32_t j = blk.div(p), off = blk.mod(p);
    if (off == 0) {
      const int32_t id = a->pop_head();
      if (a->block_node[id] >= 0) a->evict(id);
      a->refcount[id] = 1;
      row[j] = id;
    }
    slots[b] = int64_t(row[j]) * block_size + off;
    seq_lens[b] = p + 1;
  }
  if (plan) write_plan(seq_lens, B, P, part, plan);
  return PA_OK;
}
