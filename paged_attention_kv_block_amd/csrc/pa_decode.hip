// pa_decode host side: argument checks, work plans, workspaces, launches.
// The kernels and the design notes are in pa_decode_dev.h.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "pa.h"
#include "pa_common.h"
#include "pa_internal.h"
#include "pa_decode_dev.h"

namespace pa {

constexpr int kMaxMultiRows = 64;  // query rows per sequence of pa_decode_multi

// Zero-fills a decode workspace (its arrival counters must start at zero).
__global__ void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Scratch of pa_decode_append_noalloc: the split-K arrival counters and
// partial records of its launches live in this file-scope device array
// instead of a caller workspace.  Each device the library runs on holds its
// own copy until the process ends.  Host code never takes its address
// directly (in host code the name is only a stand-in): noalloc_scratch()
// asks the runtime for the device address, once per device.
constexpr size_t kNoallocScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Workgroups of one decode kernel variant that fit on the device at once
// (cached per device and variant): the persistent grid never exceeds this.
template <int D, int G, bool BF16, int NW, bool APPEND, bool KV8, bool MULTI, bool SHARED>
static int resident_workgroups() {
  constexpr int kMaxDev = 64;
  static int cached[kMaxDev] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) dev = 0;
  if (cached[dev] > 0) return cached[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu,
                                                   decode_kernel<D, G, BF16, NW, APPEND, KV8, MULTI,
                                                                 SHARED>,
                                                   NW * kWave, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  cached[dev] = cus * per_cu;
  if (std::getenv("PA_DEBUG"))
    std::fprintf(stderr, "pa: device %d: %d CUs x %d resident workgroups\n", dev, cus, per_cu);
  return cached[dev];
}

template <int D, int G, bool BF16, int NW, bool APPEND, bool KV8, bool MULTI, bool SHARED>
static void launch_decode_variant(const DecodeParams& a, hipStream_t s) {
  auto k = decode_kernel<D, G, BF16, NW, APPEND, KV8, MULTI, SHARED>;
  // With a plan every item is real: one workgroup each, so the hardware
  // dispatcher balances them and overlaps one item's merge with another's
  // loads.  Without one, a persistent grid skips the empty virtual items.
  const int grid = a.plan ? a.num_items
                          : std::max(1, std::min(a.num_items,
                                                 4 * resident_workgroups<D, G, BF16, NW, APPEND, KV8,
                                                                         MULTI, SHARED>()));
  hipLaunchKernelGGL(k, dim3(grid), dim3(NW * kWave), 0, s, a);
}

// Multi-row launches with several column groups and many items (the
// 2-wave regime, ALLOW_SHARED) use ordinary loads: the groups of one item
// run on one XCD together, and with that many workgroups in flight
// non-temporal lines leave the XCD's L2 before the sibling group reads
// them (long context, 4 rows at G = 8: 1.77 -> 1.32 ms).  With fewer
// items (TinyLlama-shaped, 4 rows: 24.3 against 26.3 us) or one group,
// non-temporal loads are faster.
template <int D, int G, bool BF16, int NW, bool KV8, bool MULTI, bool ALLOW_SHARED = false>
static void launch_decode_nw(const DecodeParams& a, hipStream_t s) {
  if constexpr (MULTI) {
    if constexpr (ALLOW_SHARED) {
      if (a.col_groups > 1) {
        launch_decode_variant<D, G, BF16, NW, false, KV8, true, true>(a, s);
        return;
      }
    }
    launch_decode_variant<D, G, BF16, NW, false, KV8, true, false>(a, s);
  } else if (a.new_k) {
    launch_decode_variant<D, G, BF16, NW, true, KV8, false, false>(a, s);
  } else {
    launch_decode_variant<D, G, BF16, NW, false, KV8, false, false>(a, s);
  }
}

// Compute units of the current device (cached per device).
static int device_cus() {
  constexpr int kMaxDev = 64;
  static int cached[kMaxDev] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) dev = 0;
  if (cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  cached[dev] = cus;
  return cus;
}

// Waves per workgroup from the items per compute unit: at most one item
// per compute unit gets 8 waves (a long item's blocks spread over more SIMD
// slots; an 8-wave workgroup holds its compute unit alone, so with more
// items than compute units the surplus would wait for a second round:
// TinyLlama-shaped batch at 1024-token partitions, 376 items, 24.3 us with
// 8 waves against 20.6 us with 4); many items
// get small workgroups, so that several items share a compute unit and one
// item's start and merge latency hides behind the others' loads.
// With many items, long items (whole sequences, or partitions of >= 1024
// tokens) still run best on 4-wave workgroups, which keep more of one
// item's blocks in flight; short partitions on 2-wave ones (measured on the
// Llama-3-shaped batch: one pass 248 us with 4 waves against 282 us with 2;
// 512-token partitions 258 against 265 us; long context, 1024-token
// partitions: 990 against 1011 us; the same with 2 query rows per
// sequence: 1027 against 1050 us).  FP8 launches (551 against 546 us) and
// multi-row launches with several column groups (whose shared loads need
// the 2-wave regime) keep 2 waves there.
template <int D, int G, bool BF16, bool KV8, bool MULTI = false>
static void launch_decode(const DecodeParams& a, hipStream_t s) {
  const int64_t cus = device_cus();
  const bool long_items = !KV8 && (!MULTI || a.col_groups == 1) &&
                          (a.part_blocks == 0 || a.part_blocks >= 64);
  if (a.num_items <= cus)
    launch_decode_nw<D, G, BF16, 8, KV8, MULTI>(a, s);
  else if (a.num_items < 8 * cus || long_items)
    launch_decode_nw<D, G, BF16, 4, KV8, MULTI>(a, s);
  else
    launch_decode_nw<D, G, BF16, 2, KV8, MULTI, true>(a, s);
}

// Columns of one multi-row work item: 16 (one matrix tile), or 32 (two tiles
// sharing each K and V operand) at head size 64 when the rows need more
// than one tile; an item holds as many of the sequence's query rows as fit
// those columns with their G heads each.
inline int multi_columns(int rows, int G, int head_size) {
  return head_size == 64 && G <= 16 && rows > 16 / G ? 32 : 16;
}
inline int multi_rows_per_group(int G, int cols = 16) { return G >= cols ? 1 : cols / G; }

// The split-K merge launch after a decode launch with defer_merge: one
// workgroup per (sequence, KV head), or four (each a quarter of the output
// columns) when there are fewer than two slots per compute unit, so that
// a few long sequences' merges still spread over the chip.
template <int D, bool BF16>
static bool launch_merge(int G, const DecodeParams& a, hipStream_t s) {
  const int64_t slots = int64_t(a.B) * a.num_kv_heads;
  const bool split = slots < 2 * device_cus();
  const dim3 block(kMergeWaves * kWave);
#define PA_MERGE_CASE(GG)                                                                    \
  case GG:                                                                                   \
    if (split)                                                                               \
      hipLaunchKernelGGL((merge_kernel<D, GG, BF16, 4>), dim3(slots * 4), block, 0, s, a);    \
    else                                                                                     \
      hipLaunchKernelGGL((merge_kernel<D, GG, BF16, 1>), dim3(slots), block, 0, s, a);        \
    return true;
  switch (G) {
    PA_MERGE_CASE(1)
    PA_MERGE_CASE(2)
    PA_MERGE_CASE(4)
    PA_MERGE_CASE(8)
    case 16:
      if constexpr (D == 64) {
        if (split)
          hipLaunchKernelGGL((merge_kernel<D, 16, BF16, 4>), dim3(slots * 4), block, 0, s, a);
        else
          hipLaunchKernelGGL((merge_kernel<D, 16, BF16, 1>), dim3(slots), block, 0, s, a);
        return true;
      }
      return false;
    default: return false;
  }
#undef PA_MERGE_CASE
}

template <int D, bool BF16, bool KV8 = false>
static bool dispatch_g(int G, const DecodeParams& a, hipStream_t s) {
  switch (G) {
    case 1: launch_decode<D, 1, BF16, KV8>(a, s); return true;
    case 2: launch_decode<D, 2, BF16, KV8>(a, s); return true;
    case 4: launch_decode<D, 4, BF16, KV8>(a, s); return true;
    case 8: launch_decode<D, 8, BF16, KV8>(a, s); return true;
    case 16:
      if constexpr (D == 64) { launch_decode<D, 16, BF16, KV8>(a, s); return true; }
      return false;
    default: return false;
  }
}

}  // namespace pa

using namespace pa;

extern "C" size_t pa_decode_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_size, int32_t max_seq_len,
                                            int32_t partition_size) {
  if (B <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0) return 0;
  const int64_t P = parts_for(max_seq_len, partition_size);
  if (P <= 1) return 0;
  return size_t(ws_layout(B, num_q_heads, num_kv_heads, head_size, P).total);
}

extern "C" size_t pa_decode_multi_workspace_bytes(int32_t B, int32_t rows, int32_t num_q_heads,
                                                  int32_t num_kv_heads, int32_t head_size,
                                                  int32_t max_seq_len, int32_t partition_size) {
  if (B <= 0 || rows <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
      num_q_heads % num_kv_heads || num_q_heads / num_kv_heads > 16)
    return 0;
  if (rows == 1)
    return pa_decode_workspace_bytes(B, num_q_heads, num_kv_heads, head_size, max_seq_len,
                                     partition_size);
  const int64_t P = parts_for(max_seq_len, partition_size);
  if (P <= 1) return 0;
  const int G = num_q_heads / num_kv_heads;
  const int cols = multi_columns(rows, G, head_size);
  const int rpg = multi_rows_per_group(G, cols);
  const int64_t groups = (rows + rpg - 1) / rpg;
  return size_t(ws_layout(int64_t(B) * groups, int64_t(cols) * num_kv_heads, num_kv_heads,
                          head_size, P).total);
}

extern "C" int pa_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes == 0) return PA_OK;
  if (!workspace) return fail(PA_EINVAL, "pa_decode_workspace_init: NULL workspace");
  if ((uintptr_t(workspace) & 255) || (workspace_bytes & 3))
    return fail(PA_EINVAL, "pa_decode_workspace_init: workspace must be 256-byte aligned, "
                           "size a multiple of 4");
  const int64_t n = int64_t(workspace_bytes / 4);
  const int64_t grid = (n + 255) / 256;
  if (grid > 0x7FFFFFFF) return fail(PA_EINVAL, "pa_decode_workspace_init: too large");
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<uint32_t*>(workspace), n);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PA_EHIP, "pa_decode_workspace_init: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

static int decode_call(const char* fn, void* out, float* lse_out, const void* query,
                       const void* new_key, const void* new_value, const void* kv_cache,
                       int32_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                       int32_t block_size, float scale, float k_scale, float v_scale,
                       int32_t partition_size, const int32_t* plan, int32_t plan_entries,
                       void* workspace, size_t workspace_bytes, int32_t dtype, void* stream,
                       int32_t rows = 1) {
  if (B < 0 || num_blocks < 0 || max_seq_len < 0 || max_blocks_per_seq < 0 || plan_entries < 0)
    return fail(PA_EINVAL, "%s: negative size", fn);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return fail(PA_EINVAL, "%s: H_q %d not a multiple of H_kv %d", fn, num_q_heads, num_kv_heads);
  if (dtype != PA_F32 && dtype != PA_BF16 && dtype != PA_FP8)
    return fail(PA_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (!(k_scale > 0.f && k_scale < INFINITY && v_scale > 0.f && v_scale < INFINITY))
    return fail(PA_EINVAL, "%s: cache scales must be positive and finite", fn);
  if (block_size != kBlockSize) return fail(PA_ENOTSUP, "%s: block_size %d (only 16)", fn, block_size);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ENOTSUP, "%s: head_size %d (64 or 128)", fn, head_size);
  if (partition_size < 0 || partition_size % kBlockSize)
    return fail(PA_EINVAL, "%s: partition_size %d must be a multiple of 16", fn, partition_size);
  if (int64_t(max_blocks_per_seq) * kBlockSize < max_seq_len)
    return fail(PA_EINVAL, "%s: max_seq_len %d exceeds the table (%d blocks)", fn, max_seq_len,
                max_blocks_per_seq);
  if (!(scale == scale)) return fail(PA_EINVAL, "%s: scale is NaN", fn);
  if (B == 0) return PA_OK;
  if (!out || !query || !block_tables || !seq_lens || (!kv_cache && num_blocks > 0))
    return fail(PA_EINVAL, "%s: NULL pointer", fn);
  if ((uintptr_t(out) | uintptr_t(query) | uintptr_t(kv_cache)) & 15)
    return fail(PA_EINVAL, "%s: out/query/cache must be 16-byte aligned", fn);
  if ((uintptr_t(block_tables) | uintptr_t(seq_lens) | uintptr_t(lse_out) | uintptr_t(plan)) & 3)
    return fail(PA_EINVAL, "%s: int/float arrays must be 4-byte aligned", fn);
  if ((new_key == nullptr) != (new_value == nullptr))
    return fail(PA_EINVAL, "%s: new_key and new_value go together", fn);
  if ((uintptr_t(new_key) | uintptr_t(new_value)) & 15)
    return fail(PA_EINVAL, "%s: new_key/new_value must be 16-byte aligned", fn);
  if (num_blocks == 0 && max_seq_len > 0)
    return fail(PA_EINVAL, "%s: empty pool but max_seq_len %d", fn, max_seq_len);
  if (plan && (B > 65535 || plan_entries == 0))
    return fail(PA_EINVAL, "%s: a plan needs B <= 65535 and at least one entry", fn);
  const int G = num_q_heads / num_kv_heads;
  const bool multi = rows > 1;
  if (rows < 1 || rows > kMaxMultiRows)
    return fail(PA_EINVAL, "%s: rows %d outside [1, %d]", fn, rows, kMaxMultiRows);
  if (multi && dtype != PA_BF16 && dtype != PA_FP8)
    return fail(PA_ENOTSUP, "%s: several rows per sequence need a bf16 or FP8 cache", fn);
  if (multi && G > 16) return fail(PA_ENOTSUP, "%s: group size %d > 16", fn, G);
  const int cols = multi ? multi_columns(rows, G, head_size) : G;
  const int rpg = multi ? multi_rows_per_group(G, cols) : 1;
  const int groups = (rows + rpg - 1) / rpg;
  const int64_t P = parts_for(max_seq_len, partition_size);
  if (P > 65535) return fail(PA_EINVAL, "%s: too many partitions (%lld)", fn, (long long)P);
  const int64_t per_group = plan ? int64_t(plan_entries) : int64_t(B) * P;
  // multi-row items come in runs of 8 per column group (see decode_kernel)
  const int64_t items = multi ? (per_group * num_kv_heads + 7) / 8 * 8 * groups
                              : per_group * num_kv_heads;
  if (items > 0x7FFFFFFF) return fail(PA_ENOTSUP, "%s: too many work items", fn);
  const size_t need =
      pa_decode_multi_workspace_bytes(B, rows, num_q_heads, num_kv_heads, head_size, max_seq_len,
                                      partition_size);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
  if (need > 0 && (uintptr_t(workspace) & 255))
    return fail(PA_EINVAL, "%s: workspace must be 256-byte aligned", fn);
  if (P > 1 && int64_t(B) * num_kv_heads * groups > kCounterCap)
    return fail(PA_ENOTSUP, "%s: split-K supports B * H_kv * column groups <= %lld", fn,
                (long long)kCounterCap);

  DecodeParams a{};
  a.out = out;
  a.lse_out = lse_out;
  a.query = query;
  a.cache = static_cast<const uint8_t*>(kv_cache);
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.plan = plan;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.num_kv_heads = num_kv_heads;
  a.B = B;
  a.scale_log2 = scale * k_scale * kLog2e;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.new_k = new_key;
  a.new_v = new_value;
  a.part_blocks = P > 1 ? partition_size / kBlockSize : 0;
  a.max_parts = int(P);
  a.num_items = int(items);
  a.rows = rows;
  a.group = G;
  a.rows_per_group = rpg;
  a.col_groups = groups;
  a.items_per_group = int(per_group);
  // One-row split-K over long partitions (>= 1024 tokens): the items only
  // write their records and a second launch merges them.  A workgroup that
  // merges in place first waits for its records' stores and an arrival
  // count, idle while the other items stream; with long items that idle
  // time costs more than the second launch (long-context batch, 1024-token
  // partitions: 986 -> 958 us).  Short partitions keep the in-place merge
  // (Llama-3-shaped batch, 512-token partitions: 257 us in place, 260 us
  // with the second launch).
  a.defer_merge = P > 1 && !multi && B > 0 && partition_size >= 64 * kBlockSize;
  if (P > 1) {
    const WsLayout w = multi ? ws_layout(int64_t(B) * groups, int64_t(cols) * num_kv_heads,
                                         num_kv_heads, head_size, P)
                             : ws_layout(B, num_q_heads, num_kv_heads, head_size, P);
    uint8_t* base = static_cast<uint8_t*>(workspace);
    a.ws_count = reinterpret_cast<int*>(base + w.count_off);
    a.ws_rec = base + w.rec_off;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  bool ok;
  if (multi && dtype == PA_FP8 && cols == 32)
    ok = (launch_decode<64, 32, true, true, true>(a, st), true);
  else if (multi && dtype == PA_FP8)
    ok = head_size == 64 ? (launch_decode<64, 16, true, true, true>(a, st), true)
                         : (launch_decode<128, 16, true, true, true>(a, st), true);
  else if (multi && cols == 32)
    ok = (launch_decode<64, 32, true, false, true>(a, st), true);
  else if (multi)
    ok = head_size == 64 ? (launch_decode<64, 16, true, false, true>(a, st), true)
                         : (launch_decode<128, 16, true, false, true>(a, st), true);
  else if (dtype == PA_FP8)
    ok = head_size == 64 ? dispatch_g<64, true, true>(G, a, st)
                         : dispatch_g<128, true, true>(G, a, st);
  else if (dtype == PA_BF16)
    ok = head_size == 64 ? dispatch_g<64, true>(G, a, st) : dispatch_g<128, true>(G, a, st);
  else
    ok = head_size == 64 ? dispatch_g<64, false>(G, a, st) : dispatch_g<128, false>(G, a, st);
  if (!ok) return fail(PA_ENOTSUP, "%s: group size %d with head_size %d", fn, G, head_size);
  if (a.defer_merge) {
    const bool bf16_recs = dtype != PA_F32;   // FP8 caches run the bf16 path
    const bool merged = head_size == 64
                            ? (bf16_recs ? launch_merge<64, true>(G, a, st)
                                         : launch_merge<64, false>(G, a, st))
                            : (bf16_recs ? launch_merge<128, true>(G, a, st)
                                         : launch_merge<128, false>(G, a, st));
    if (!merged) return fail(PA_ENOTSUP, "%s: group size %d with head_size %d", fn, G, head_size);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return PA_OK;
}

extern "C" int pa_decode(void* out, float* lse_out, const void* query, const void* kv_cache,
                         int32_t num_blocks, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B,
                         int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_size, int32_t block_size, float scale,
                         int32_t partition_size, const int32_t* plan, int32_t plan_entries,
                         void* workspace, size_t workspace_bytes, int32_t dtype, void* stream) {
  if (dtype == PA_FP8)
    return fail(PA_EINVAL, "pa_decode: an FP8 cache needs pa_decode_fp8 (its scales)");
  return decode_call("pa_decode", out, lse_out, query, nullptr, nullptr, kv_cache, num_blocks,
                     block_tables, max_blocks_per_seq, seq_lens, B, max_seq_len, num_q_heads,
                     num_kv_heads, head_size, block_size, scale, 1.f, 1.f, partition_size, plan,
                     plan_entries, workspace, workspace_bytes, dtype, stream);
}

extern "C" int pa_decode_fp8(void* out, float* lse_out, const void* query, const void* kv_cache,
                             int32_t num_blocks, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B,
                             int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_size, int32_t block_size, float scale, float k_scale,
                             float v_scale, int32_t partition_size, const int32_t* plan,
                             int32_t plan_entries, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return decode_call("pa_decode_fp8", out, lse_out, query, nullptr, nullptr, kv_cache, num_blocks,
                     block_tables, max_blocks_per_seq, seq_lens, B, max_seq_len, num_q_heads,
                     num_kv_heads, head_size, block_size, scale, k_scale, v_scale,
                     partition_size, plan, plan_entries, workspace, workspace_bytes, PA_FP8,
                     stream);
}

extern "C" int pa_decode_append_fp8(void* out, float* lse_out, const void* query,
                                    const void* new_key, const void* new_value, void* kv_cache,
                                    int32_t num_blocks, const int32_t* block_tables,
                                    int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                    int32_t B, int32_t max_seq_len, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                    float scale, float k_scale, float v_scale,
                                    int32_t partition_size, const int32_t* plan,
                                    int32_t plan_entries, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (B > 0 && (!new_key || !new_value))
    return fail(PA_EINVAL, "pa_decode_append_fp8: NULL new_key/new_value");
  return decode_call("pa_decode_append_fp8", out, lse_out, query, new_key, new_value, kv_cache,
                     num_blocks, block_tables, max_blocks_per_seq, seq_lens, B, max_seq_len,
                     num_q_heads, num_kv_heads, head_size, block_size, scale, k_scale, v_scale,
                     partition_size, plan, plan_entries, workspace, workspace_bytes, PA_FP8,
                     stream);
}

extern "C" int pa_decode_append(void* out, float* lse_out, const void* query,
                                const void* new_key, const void* new_value, void* kv_cache,
                                int32_t num_blocks, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B,
                                int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_size, int32_t block_size, float scale,
                                int32_t partition_size, const int32_t* plan,
                                int32_t plan_entries, void* workspace, size_t workspace_bytes,
                                int32_t dtype, void* stream) {
  if (dtype == PA_FP8)
    return fail(PA_EINVAL, "pa_decode_append: an FP8 cache needs pa_decode_append_fp8");
  if (B > 0 && (!new_key || !new_value))
    return fail(PA_EINVAL, "pa_decode_append: NULL new_key/new_value");
  return decode_call("pa_decode_append", out, lse_out, query, new_key, new_value, kv_cache,
                     num_blocks, block_tables, max_blocks_per_seq, seq_lens, B, max_seq_len,
                     num_q_heads, num_kv_heads, head_size, block_size, scale, 1.f, 1.f,
                     partition_size, plan, plan_entries, workspace, workspace_bytes, dtype,
                     stream);
}


extern "C" int pa_decode_multi(void* out, float* lse_out, const void* query, const void* kv_cache,
                               int32_t num_blocks, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B,
                               int32_t max_seq_len, int32_t rows, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                               float scale, int32_t partition_size, const int32_t* plan,
                               int32_t plan_entries, void* workspace, size_t workspace_bytes,
                               int32_t dtype, void* stream) {
  if (dtype == PA_FP8)
    return fail(PA_EINVAL, "pa_decode_multi: an FP8 cache needs pa_decode_multi_fp8 (its scales)");
  return decode_call("pa_decode_multi", out, lse_out, query, nullptr, nullptr, kv_cache,
                     num_blocks, block_tables, max_blocks_per_seq, seq_lens, B, max_seq_len,
                     num_q_heads, num_kv_heads, head_size, block_size, scale, 1.f, 1.f,
                     partition_size, plan, plan_entries, workspace, workspace_bytes, dtype,
                     stream, rows);
}

extern "C" int pa_decode_multi_fp8(void* out, float* lse_out, const void* query,
                                   const void* kv_cache, int32_t num_blocks,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
                                   int32_t rows, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size, float scale,
                                   float k_scale, float v_scale, int32_t partition_size,
                                   const int32_t* plan, int32_t plan_entries, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return decode_call("pa_decode_multi_fp8", out, lse_out, query, nullptr, nullptr, kv_cache,
                     num_blocks, block_tables, max_blocks_per_seq, seq_lens, B, max_seq_len,
                     num_q_heads, num_kv_heads, head_size, block_size, scale, k_scale, v_scale,
                     partition_size, plan, plan_entries, workspace, workspace_bytes, PA_FP8,
                     stream, rows);
}

// Device address of this device's scratch array, looked up once per device
// (with that device current), and its arrival counters cleared on the
// caller's stream by a fill kernel at that first call: every completed
// call leaves them at zero again.  nullptr on a runtime error.
static uint8_t* noalloc_scratch(hipStream_t stream) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static uint8_t* ptrs[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    fail(PA_EHIP, "pa_decode_append_noalloc: no current device (or more than %d)", kMaxDev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev]) return ptrs[dev];
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    fail(PA_EHIP, "pa_decode_append_noalloc: hipGetSymbolAddress(scratch) failed: %s",
         hipGetErrorString(e));
    return nullptr;
  }
  const int64_t n = ws_layout(1, 1, 1, 64, 1).rec_off / 4;   // the counter region
  hipLaunchKernelGGL(fill_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                     static_cast<uint32_t*>(p), n);
  const hipError_t le = hipGetLastError();
  if (le != hipSuccess) {
    fail(PA_EHIP, "pa_decode_append_noalloc: clearing the scratch failed: %s",
         hipGetErrorString(le));
    return nullptr;
  }
  ptrs[dev] = static_cast<uint8_t*>(p);
  return ptrs[dev];
}

extern "C" int pa_decode_append_noalloc(void* out, float* lse_out, const void* query,
                                        const void* new_key, const void* new_value,
                                        void* kv_cache, int32_t num_blocks,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_size, int32_t block_size, float scale,
                                        int32_t partition_size, const int32_t* plan,
                                        int32_t plan_entries, int32_t dtype, void* stream) {
  const char* fn = "pa_decode_append_noalloc";
  if (dtype == PA_FP8)
    return fail(PA_EINVAL, "%s: an FP8 cache needs pa_decode_append_fp8 (its scales)", fn);
  if (B > 0 && (!new_key || !new_value)) return fail(PA_EINVAL, "%s: NULL new_key/new_value", fn);
  if (B < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 || partition_size < 0)
    return fail(PA_EINVAL, "%s: bad sizes", fn);
  const size_t need = pa_decode_workspace_bytes(B, num_q_heads, num_kv_heads, head_size,
                                                max_seq_len, partition_size);
  if (need > kNoallocScratchBytes)
    return fail(PA_EINVAL, "%s: split-K needs %zu bytes of scratch, the static scratch holds %zu "
                "(fewer sequences or partitions, or pa_decode_append with a workspace)",
                fn, need, kNoallocScratchBytes);
  uint8_t* ws = nullptr;
  if (need > 0 && B > 0) {
    ws = noalloc_scratch(reinterpret_cast<hipStream_t>(stream));
    if (!ws) return PA_EHIP;
  }
  return decode_call(fn, out, lse_out, query, new_key, new_value, kv_cache, num_blocks,
                     block_tables, max_blocks_per_seq, seq_lens, B, max_seq_len, num_q_heads,
                     num_kv_heads, head_size, block_size, scale, 1.f, 1.f, partition_size, plan,
                     plan_entries, ws, ws ? kNoallocScratchBytes : 0, dtype, stream);
}
