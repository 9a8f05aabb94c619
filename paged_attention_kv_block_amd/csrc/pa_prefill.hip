// pa_prefill_chunk host side: argument checks and launches.  The kernel and
// the design notes are in pa_prefill_wide_dev.h.
#include "pa.h"
#include "pa_common.h"
#include "pa_internal.h"
#include "pa_prefill_wide_dev.h"

namespace pa {

template <int D>
static bool launch_prefill(int G, int max_query_len, int B, hipStream_t s, uint16_t* out,
                           float* lse, const uint16_t* q, const int* qsl, const uint16_t* cache,
                           int nb, const int* bt, int mbps, const int* sl, int msl, int hkv,
                           float sc) {
#define PA_PREFILL_CASE(GG)                                                                     \
  case GG: {                                                                                    \
    const int tiles = (max_query_len + WideCfg<D, GG>::TQ - 1) / WideCfg<D, GG>::TQ;            \
    const int groups = B * hkv;                                                                 \
    hipLaunchKernelGGL((prefill_wide_kernel<D, GG>), dim3(tiles * groups), dim3(kWideThreads),  \
                       0, s, out, lse, q, qsl, cache, nb, bt, mbps, sl, msl, hkv, sc, tiles,    \
                       groups);                                                                 \
    return true;                                                                                \
  }
  switch (G) {
    PA_PREFILL_CASE(1)
    PA_PREFILL_CASE(2)
    PA_PREFILL_CASE(4)
    PA_PREFILL_CASE(8)
    default: return false;
  }
#undef PA_PREFILL_CASE
}

}  // namespace pa

using namespace pa;

extern "C" int pa_prefill_chunk(void* out, float* lse_out, const void* query,
                                const int32_t* query_start_loc, int32_t max_query_len,
                                int32_t total_query_tokens, const void* kv_cache,
                                int32_t num_blocks, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B,
                                int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_size, int32_t block_size, float scale, int32_t dtype,
                                void* stream) {
  if (B < 0 || num_blocks < 0 || max_seq_len < 0 || max_blocks_per_seq < 0 ||
      max_query_len < 0 || total_query_tokens < 0)
    return fail(PA_EINVAL, "pa_prefill_chunk: negative size");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return fail(PA_EINVAL, "pa_prefill_chunk: H_q %d not a multiple of H_kv %d", num_q_heads,
                num_kv_heads);
  if (dtype != PA_BF16)
    return fail(dtype == PA_F32 ? PA_ENOTSUP : PA_EINVAL,
                "pa_prefill_chunk: dtype %d (bf16 only)", dtype);
  if (block_size != kBlockSize)
    return fail(PA_ENOTSUP, "pa_prefill_chunk: block_size %d (only 16)", block_size);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ENOTSUP, "pa_prefill_chunk: head_size %d (64 or 128)", head_size);
  if (int64_t(max_blocks_per_seq) * kBlockSize < max_seq_len)
    return fail(PA_EINVAL, "pa_prefill_chunk: max_seq_len %d exceeds the table", max_seq_len);
  if (max_query_len > max_seq_len)
    return fail(PA_EINVAL, "pa_prefill_chunk: max_query_len %d > max_seq_len %d", max_query_len,
                max_seq_len);
  if (is_nan_bits(scale)) return fail(PA_EINVAL, "pa_prefill_chunk: scale is NaN");
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PA_ENOTSUP, "pa_prefill_chunk: group size %d", G);
  if (B == 0 || max_query_len == 0 || total_query_tokens == 0) return PA_OK;
  if (!out || !query || !query_start_loc || !block_tables || !seq_lens ||
      (!kv_cache && num_blocks > 0))
    return fail(PA_EINVAL, "pa_prefill_chunk: NULL pointer");
  if ((uintptr_t(out) | uintptr_t(query) | uintptr_t(kv_cache)) & 15)
    return fail(PA_EINVAL, "pa_prefill_chunk: out/query/cache must be 16-byte aligned");
  if ((uintptr_t(block_tables) | uintptr_t(seq_lens) | uintptr_t(query_start_loc) |
       uintptr_t(lse_out)) & 3)
    return fail(PA_EINVAL, "pa_prefill_chunk: int/float arrays must be 4-byte aligned");
  if (num_blocks == 0) return fail(PA_EINVAL, "pa_prefill_chunk: empty pool");
  if (num_kv_heads > 65535 || B > 65535) return fail(PA_ENOTSUP, "pa_prefill_chunk: grid too large");
  if (max_blocks_per_seq > (1 << 28))
    return fail(PA_ENOTSUP, "pa_prefill_chunk: max_blocks_per_seq %d too large", max_blocks_per_seq);
  if (int64_t(max_query_len) * num_kv_heads * B > 0x7FFFFFFF)
    return fail(PA_ENOTSUP, "pa_prefill_chunk: grid too large");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto o = static_cast<uint16_t*>(out);
  auto q = static_cast<const uint16_t*>(query);
  auto c = static_cast<const uint16_t*>(kv_cache);
  const float sl2 = scale * kLog2eP;
  bool ok = head_size == 64
                ? launch_prefill<64>(G, max_query_len, B, s, o, lse_out, q, query_start_loc, c, num_blocks,
                                     block_tables, max_blocks_per_seq, seq_lens, max_seq_len,
                                     num_kv_heads, sl2)
                : launch_prefill<128>(G, max_query_len, B, s, o, lse_out, q, query_start_loc, c, num_blocks,
                                      block_tables, max_blocks_per_seq, seq_lens, max_seq_len,
                                      num_kv_heads, sl2);
  if (!ok) return fail(PA_ENOTSUP, "pa_prefill_chunk: group size %d", G);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PA_EHIP, "pa_prefill_chunk: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}
