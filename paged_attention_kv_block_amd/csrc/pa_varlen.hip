// One launch over a flattened batch that mixes decode rows and prefill
// chunks.
//
// The engine forms a step by flattening every scheduled sequence's new
// tokens into one sequence of query rows: decode requests contribute one
// row, prefill requests a chunk of their prompt ("Inside vLLM", "Generate
// function" and the continuous-batching discussion under "LLM Engine &
// Engine Core"; "Im Inneren von vLLM", "Fortgeschrittene Funktionen" for
// chunked prefill).  Both kinds of rows compute the same causal attention
// over the sequence's cached tokens; what differs is the shape of the work:
// a chunk of C_b >= 2 rows is a dense contraction (wide_tile, the prefill
// tile: MFMA over 128 (token, head) rows per workgroup), a single row is a stream over the
// sequence's blocks (decode_item: the matrix-core decode, optionally split
// into partitions merged by the last workgroup to finish).
//
// A host plan (pa_varlen_plan) lists the work items: first the prefill
// query tiles, grouped by sequence, then the decode (sequence, partition)
// items, longest first.  The grid has one workgroup per (item, KV head),
// item-major, so the dispatcher starts the heavy tiles first and the decode
// items fill the compute units as tiles finish.  With the KV heads a
// multiple of the 8 XCDs, all tiles of one (sequence, KV head) run on one
// XCD, one after another, and share the blocks they stream (a common prefix
// included) through that XCD's L2.
//
// Both kinds of work are bound by the same per-CU path from memory (the
// decode rows stream from HBM, the query tiles re-read their blocks from
// L2 into LDS), so running them side by side does not make either faster:
// the launch takes about as long as pa_prefill_chunk and pa_decode one
// after the other, and saves the second launch and its host call.
#include <algorithm>
#include <vector>

#include "pa.h"
#include "pa_common.h"
#include "pa_internal.h"
#include "pa_decode_dev.h"
#include "pa_prefill_wide_dev.h"

namespace pa {

constexpr int kVarlenWaves = kWideWaves;  // decode items run with the prefill workgroup

template <int D, int G>
union VarlenSmem {
  // the prefill tile's LDS ring and vote words
  __attribute__((aligned(1024))) uint8_t pf[kWideBufs * WideCfg<D, G>::BUF + 64];
  DecodeSmem<D, G, true, kVarlenWaves, false> dc;
  DecodeSmem<D, 16, true, kVarlenWaves, false> mc;
};

// A chunk this short runs on the multi-row decode path: 16 / G rows per
// item, at most kShortGroups items per (sequence, KV head).
constexpr int kShortGroups = 4;
inline int varlen_rows_per_group(int G) { return 16 / G; }

// plan entries: (1 << 31) | (tile << 16) | b for a prefill query tile,
// (part << 16) | b for a decode partition (part < 2^14), and
// (1 << 30) | (cg << 16) | b for column group cg of a short chunk (one pass
// over the sequence's blocks, no split-K)
template <int D, int G>
__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void varlen_kernel(const DecodeParams a, const int* __restrict__ qsl) {
  __shared__ VarlenSmem<D, G> sm;
  const int item = blockIdx.x / a.num_kv_heads;
  const int g = blockIdx.x % a.num_kv_heads;
  const int e = a.plan[item];
  const int b = e & 0xFFFF;
  const int x = (e >> 16) & 0x7FFF;
  if (b >= a.B) return;  // not an entry of this batch
  if (e < 0) {
    wide_tile<D, G>(sm.pf, static_cast<uint16_t*>(a.out), a.lse_out,
                    static_cast<const uint16_t*>(a.query), qsl,
                    reinterpret_cast<const uint16_t*>(a.cache), a.num_blocks, a.block_tables,
                    a.max_blocks_per_seq, a.seq_lens, a.max_seq_len, a.num_kv_heads,
                    a.scale_log2, b, g, x);
    return;
  }
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int nblk = (L + 15) >> 4;
  if (e & (1 << 30)) {  // column group of a short chunk
    const int cg = x & 0x3FFF;
    const int rows = qsl[b + 1] - qsl[b];
    if (cg * a.rows_per_group >= rows) return;
    decode_item<D, 16, true, kVarlenWaves, false, false, true>(
        a, sm.mc, b, qsl[b] + cg * a.rows_per_group, g, 0, L, nblk, nblk > 0 ? nblk : 1, 1, cg,
        rows);
    return;
  }
  const int pb = a.part_blocks > 0 ? a.part_blocks : (nblk > 0 ? nblk : 1);
  const int nparts = (nblk + pb - 1) / pb;
  if (x > 0 && x >= nparts) return;
  decode_item<D, G, true, kVarlenWaves, false, false>(a, sm.dc, b, qsl[b], g, x, L, nblk, pb,
                                                      nparts);
}

template <int D>
static bool launch_varlen(int G, const DecodeParams& a, const int* qsl, hipStream_t s) {
  const dim3 grid(a.num_items), block(kWideThreads);
  switch (G) {
    case 1: hipLaunchKernelGGL((varlen_kernel<D, 1>), grid, block, 0, s, a, qsl); return true;
    case 2: hipLaunchKernelGGL((varlen_kernel<D, 2>), grid, block, 0, s, a, qsl); return true;
    case 4: hipLaunchKernelGGL((varlen_kernel<D, 4>), grid, block, 0, s, a, qsl); return true;
    case 8: hipLaunchKernelGGL((varlen_kernel<D, 8>), grid, block, 0, s, a, qsl); return true;
    default: return false;
  }
}

}  // namespace pa

using namespace pa;

extern "C" int pa_varlen_plan(const int32_t* query_start_loc, const int32_t* seq_lens, int32_t B,
                              int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t partition_size, int32_t* plan, int32_t capacity,
                              int32_t* num_entries, int32_t* num_prefill_entries) {
  if (B < 0 || max_seq_len < 0 || partition_size < 0 || partition_size % kBlockSize ||
      capacity < 0)
    return fail(PA_EINVAL, "pa_varlen_plan: bad sizes");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return fail(PA_EINVAL, "pa_varlen_plan: H_q %d not a multiple of H_kv %d", num_q_heads,
                num_kv_heads);
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PA_ENOTSUP, "pa_varlen_plan: group size %d", G);
  if (B > 65535) return fail(PA_ENOTSUP, "pa_varlen_plan: B %d > 65535", B);
  if (B > 0 && (!seq_lens || !query_start_loc))
    return fail(PA_EINVAL, "pa_varlen_plan: NULL metadata");
  if (B > 0 && query_start_loc[0] != 0)
    return fail(PA_EINVAL, "pa_varlen_plan: query_start_loc[0] = %d", query_start_loc[0]);
  const int64_t P = parts_for(max_seq_len, partition_size);
  if (P > 16383) return fail(PA_ENOTSUP, "pa_varlen_plan: too many partitions");
  const int TQ = kWideRows / G;  // query tokens per prefill tile
  const int RPG = varlen_rows_per_group(G);
  // (work, b, x) of every item; work orders them; x carries the multi-row flag
  struct Item { int64_t work; int32_t b, x; };
  std::vector<Item> pre, dec;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t L = seq_lens[b];
    const int64_t Cb = int64_t(query_start_loc[b + 1]) - query_start_loc[b];
    if (L < 0 || L > max_seq_len)
      return fail(PA_EINVAL, "pa_varlen_plan: seq_lens[%d] = %d outside [0, %d]", b, L,
                  max_seq_len);
    if (Cb < 0 || Cb > L)
      return fail(PA_EINVAL, "pa_varlen_plan: sequence %d has %lld query rows for %d tokens", b,
                  (long long)Cb, L);
    if (Cb == 1) {
      const int32_t ptok = P > 1 ? partition_size : L;
      const int32_t np = (L + ptok - 1) / ptok;
      for (int32_t p = 0; p < np; ++p) dec.push_back({std::min(ptok, L - p * ptok), b, p});
    } else if (Cb > 1 && (Cb + RPG - 1) / RPG <= kShortGroups) {
      // a short chunk (e.g. the tokens of a speculative step): column groups
      // of RPG rows on the decode path, each one pass over the L tokens
      for (int32_t cg = 0; cg < int32_t((Cb + RPG - 1) / RPG); ++cg)
        dec.push_back({L, b, (1 << 14) | cg});
    } else if (Cb > 1) {
      const int64_t tiles = (Cb + TQ - 1) / TQ;
      if (tiles > 32767) return fail(PA_ENOTSUP, "pa_varlen_plan: chunk of %lld rows", (long long)Cb);
      const int64_t ctx = L - Cb;
      for (int32_t t = 0; t < int32_t(tiles); ++t) {
        const int64_t rows = std::min<int64_t>(TQ, Cb - int64_t(t) * TQ);
        pre.push_back({rows * (ctx + int64_t(t) * TQ + rows), b, t});  // rows x keys seen
      }
    }
  }
  auto longest_first = [](const Item& p, const Item& q) {
    if (p.work != q.work) return p.work > q.work;
    if (p.x != q.x) return p.x < q.x;
    return p.b < q.b;
  };
  // Query tiles stay grouped by sequence (consecutive workgroups, and on
  // one XCD per KV head when H_kv is a multiple of 8), so the tiles that
  // re-read a sequence's blocks run together and find them in L2; the
  // sequences go by their total work, longest first, and a sequence's
  // tiles longest first.
  std::vector<int64_t> seq_work(size_t(B), 0);
  for (const Item& it : pre) seq_work[size_t(it.b)] += it.work;
  std::stable_sort(pre.begin(), pre.end(), [&](const Item& p, const Item& q) {
    const int64_t wp = seq_work[size_t(p.b)], wq = seq_work[size_t(q.b)];
    if (wp != wq) return wp > wq;
    if (p.b != q.b) return p.b < q.b;
    return p.x > q.x;
  });
  std::stable_sort(dec.begin(), dec.end(), longest_first);
  const int64_t n = int64_t(pre.size()) + int64_t(dec.size());
  if (num_entries) *num_entries = int32_t(std::min<int64_t>(n, 0x7FFFFFFF));
  if (num_prefill_entries) *num_prefill_entries = int32_t(pre.size());
  if (n > capacity)
    return fail(PA_EINVAL, "pa_varlen_plan: %lld entries, capacity %d", (long long)n, capacity);
  if (n > 0 && !plan) return fail(PA_EINVAL, "pa_varlen_plan: NULL plan");
  size_t i = 0;
  for (const Item& it : pre) plan[i++] = int32_t(0x80000000u | uint32_t(it.x << 16) | uint32_t(it.b));
  for (const Item& it : dec) plan[i++] = int32_t((uint32_t(it.x) << 16) | uint32_t(it.b));
  return PA_OK;
}

extern "C" int pa_attention_varlen(void* out, float* lse_out, const void* query,
                                   const int32_t* query_start_loc, int32_t total_query_tokens,
                                   const void* kv_cache, int32_t num_blocks,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                                   int32_t block_size, float scale, int32_t partition_size,
                                   const int32_t* plan, int32_t plan_entries, void* workspace,
                                   size_t workspace_bytes, int32_t dtype, void* stream) {
  const char* fn = "pa_attention_varlen";
  if (B < 0 || num_blocks < 0 || max_seq_len < 0 || max_blocks_per_seq < 0 ||
      total_query_tokens < 0 || plan_entries < 0)
    return fail(PA_EINVAL, "%s: negative size", fn);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return fail(PA_EINVAL, "%s: H_q %d not a multiple of H_kv %d", fn, num_q_heads, num_kv_heads);
  if (dtype != PA_BF16)
    return fail(dtype == PA_F32 ? PA_ENOTSUP : PA_EINVAL, "%s: dtype %d (bf16 only)", fn, dtype);
  if (block_size != kBlockSize) return fail(PA_ENOTSUP, "%s: block_size %d (only 16)", fn, block_size);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ENOTSUP, "%s: head_size %d (64 or 128)", fn, head_size);
  if (partition_size < 0 || partition_size % kBlockSize)
    return fail(PA_EINVAL, "%s: partition_size %d must be a multiple of 16", fn, partition_size);
  if (int64_t(max_blocks_per_seq) * kBlockSize < max_seq_len)
    return fail(PA_EINVAL, "%s: max_seq_len %d exceeds the table", fn, max_seq_len);
  if (is_nan_bits(scale)) return fail(PA_EINVAL, "%s: scale is NaN", fn);
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(PA_ENOTSUP, "%s: group size %d", fn, G);
  if (B > 65535) return fail(PA_ENOTSUP, "%s: B %d > 65535", fn, B);
  if (B == 0 || plan_entries == 0 || total_query_tokens == 0) return PA_OK;
  if (!out || !query || !query_start_loc || !block_tables || !seq_lens || !plan ||
      (!kv_cache && num_blocks > 0))
    return fail(PA_EINVAL, "%s: NULL pointer", fn);
  if ((uintptr_t(out) | uintptr_t(query) | uintptr_t(kv_cache)) & 15)
    return fail(PA_EINVAL, "%s: out/query/cache must be 16-byte aligned", fn);
  if ((uintptr_t(block_tables) | uintptr_t(seq_lens) | uintptr_t(query_start_loc) |
       uintptr_t(lse_out) | uintptr_t(plan)) & 3)
    return fail(PA_EINVAL, "%s: int/float arrays must be 4-byte aligned", fn);
  if (num_blocks == 0) return fail(PA_EINVAL, "%s: empty pool", fn);
  if (max_blocks_per_seq > (1 << 28))
    return fail(PA_ENOTSUP, "%s: max_blocks_per_seq %d too large", fn, max_blocks_per_seq);
  const int64_t P = parts_for(max_seq_len, partition_size);
  if (P > 16383) return fail(PA_EINVAL, "%s: too many partitions (%lld)", fn, (long long)P);
  const int64_t items = int64_t(plan_entries) * num_kv_heads;
  if (items > 0x7FFFFFFF) return fail(PA_ENOTSUP, "%s: too many work items", fn);
  const size_t need =
      pa_decode_workspace_bytes(B, num_q_heads, num_kv_heads, head_size, max_seq_len, partition_size);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
  if (need > 0 && (uintptr_t(workspace) & 255))
    return fail(PA_EINVAL, "%s: workspace must be 256-byte aligned", fn);
  if (P > 1 && int64_t(B) * num_kv_heads > kCounterCap)
    return fail(PA_ENOTSUP, "%s: split-K supports B * H_kv <= %lld", fn, (long long)kCounterCap);

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
  a.scale_log2 = scale * kLog2e;
  a.k_scale = 1.f;
  a.v_scale = 1.f;
  a.part_blocks = P > 1 ? partition_size / kBlockSize : 0;
  a.max_parts = int(P);
  a.num_items = int(items);
  a.group = G;                                  // short chunks' column groups
  a.rows_per_group = varlen_rows_per_group(G);
  if (P > 1) {
    const WsLayout w = ws_layout(B, num_q_heads, num_kv_heads, head_size, P);
    uint8_t* base = static_cast<uint8_t*>(workspace);
    a.ws_count = reinterpret_cast<int*>(base + w.count_off);
    a.ws_rec = base + w.rec_off;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool ok = head_size == 64 ? launch_varlen<64>(G, a, query_start_loc, st)
                                  : launch_varlen<128>(G, a, query_start_loc, st);
  if (!ok) return fail(PA_ENOTSUP, "%s: group size %d", fn, G);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return PA_OK;
}
