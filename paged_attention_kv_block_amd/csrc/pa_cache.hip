// pa_reshape_and_cache: scatter new keys/values into the paged pool.
//
// "Inside vLLM: Anatomy of a High-Throughput LLM Inference System", section
// "LLM Engine constructor": the KV cache is one allocation reshaped and bound
// to the attention layers; section "LLM Engine & Engine Core": blocks map a
// sequence's tokens to their KV-cache blocks.  Token t goes to slot
// slot_mapping[t] = block * 16 + offset of the pool
// [num_blocks][2][H_kv][16][D]; values are copied bit for bit.
//
// HBM-bound copy: each thread moves one 16-byte vector of K and one of V, so
// a wave reads whole 256-byte (or 128-byte) head rows and writes them to one
// contiguous row of a block; reads and writes are coalesced.
#include "pa.h"
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

template <int VPR>  // 16-byte vectors per head row (D * elem_bytes / 16)
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value,
    const int64_t* __restrict__ slot_mapping, int num_tokens, uint4* __restrict__ cache,
    int64_t num_slots, int num_kv_heads) {
  const int64_t per_token = int64_t(num_kv_heads) * VPR;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= per_token * num_tokens) return;
  const int64_t t = idx / per_token;
  const int rem = int(idx - t * per_token);
  const int h = rem / VPR, v = rem % VPR;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // skipped token (or out of range: no write)
  const int64_t blk = slot / kBlockSize;
  const int off = int(slot % kBlockSize);
  // vectors per block = 2 * H_kv * 16 * VPR; K half first, then V half
  const int64_t kbase = ((blk * 2) * num_kv_heads + h) * (kBlockSize * VPR) + off * VPR + v;
  const int64_t vbase = kbase + int64_t(num_kv_heads) * kBlockSize * VPR;
  const uint4 kx = key[idx];
  const uint4 vx = value[idx];
  cache[kbase] = kx;
  cache[vbase] = vx;
}

// FP8 cache write: each thread quantises one 16-byte vector of 8 bf16 inputs
// into 8 bytes of the pool [num_blocks][2][H_kv][16][D] (one byte per
// element) with quantize4_e4m3 (the E4M3 reading is stated there).
__device__ __forceinline__ uint2 quantize8(const uint4& x, float scale) {
  return make_uint2(quantize4_e4m3(x.x, x.y, scale), quantize4_e4m3(x.z, x.w, scale));
}

template <int VPR>  // 16-byte input vectors per head row (D / 8)
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value,
    const int64_t* __restrict__ slot_mapping, int num_tokens, uint2* __restrict__ cache,
    int64_t num_slots, int num_kv_heads, float k_scale, float v_scale) {
  const int64_t per_token = int64_t(num_kv_heads) * VPR;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= per_token * num_tokens) return;
  const int64_t t = idx / per_token;
  const int rem = int(idx - t * per_token);
  const int h = rem / VPR, v = rem % VPR;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / kBlockSize;
  const int off = int(slot % kBlockSize);
  // 8-byte units: a cache row of D bytes is VPR units, as the input row is
  // VPR 16-byte vectors
  const int64_t kbase = ((blk * 2) * num_kv_heads + h) * (kBlockSize * VPR) + off * VPR + v;
  const int64_t vbase = kbase + int64_t(num_kv_heads) * kBlockSize * VPR;
  cache[kbase] = quantize8(key[idx], k_scale);
  cache[vbase] = quantize8(value[idx], v_scale);
}

}  // namespace pa

using namespace pa;

extern "C" int pa_reshape_and_cache_fp8(const void* key, const void* value,
                                        const int64_t* slot_mapping, int32_t num_tokens,
                                        void* kv_cache, int32_t num_blocks, int32_t block_size,
                                        int32_t num_kv_heads, int32_t head_size, float k_scale,
                                        float v_scale, void* stream) {
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0)
    return fail(PA_EINVAL,
                "pa_reshape_and_cache_fp8: bad sizes (tokens %d, blocks %d, kv heads %d)",
                num_tokens, num_blocks, num_kv_heads);
  if (block_size != kBlockSize)
    return fail(PA_ENOTSUP, "pa_reshape_and_cache_fp8: block_size %d (only 16)", block_size);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ENOTSUP, "pa_reshape_and_cache_fp8: head_size %d (64 or 128)", head_size);
  if (!(k_scale > 0.f && k_scale < INFINITY && v_scale > 0.f && v_scale < INFINITY))
    return fail(PA_EINVAL, "pa_reshape_and_cache_fp8: scales must be positive and finite");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !slot_mapping || !kv_cache)
    return fail(PA_EINVAL, "pa_reshape_and_cache_fp8: NULL pointer");
  if ((uintptr_t(key) | uintptr_t(value) | uintptr_t(kv_cache)) & 15)
    return fail(PA_EINVAL, "pa_reshape_and_cache_fp8: key/value/cache must be 16-byte aligned");
  if (uintptr_t(slot_mapping) & 7)
    return fail(PA_EINVAL, "pa_reshape_and_cache_fp8: slot_mapping must be 8-byte aligned");
  const int vpr = head_size / 8;
  const int64_t total = int64_t(num_tokens) * num_kv_heads * vpr;
  const int64_t grid = (total + 255) / 256;
  if (grid > 0x7FFFFFFF) return fail(PA_EINVAL, "pa_reshape_and_cache_fp8: too many tokens");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t num_slots = int64_t(num_blocks) * kBlockSize;
  auto k = static_cast<const uint4*>(key);
  auto v = static_cast<const uint4*>(value);
  auto c = static_cast<uint2*>(kv_cache);
  if (vpr == 8)
    hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<8>, dim3(grid), dim3(256), 0, s, k, v,
                       slot_mapping, num_tokens, c, num_slots, num_kv_heads, k_scale, v_scale);
  else
    hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<16>, dim3(grid), dim3(256), 0, s, k, v,
                       slot_mapping, num_tokens, c, num_slots, num_kv_heads, k_scale, v_scale);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PA_EHIP, "pa_reshape_and_cache_fp8: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

extern "C" int pa_reshape_and_cache(const void* key, const void* value,
                                    const int64_t* slot_mapping, int32_t num_tokens,
                                    void* kv_cache, int32_t num_blocks, int32_t block_size,
                                    int32_t num_kv_heads, int32_t head_size, int32_t dtype,
                                    void* stream) {
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0)
    return fail(PA_EINVAL, "pa_reshape_and_cache: bad sizes (tokens %d, blocks %d, kv heads %d)",
                num_tokens, num_blocks, num_kv_heads);
  if (dtype != PA_F32 && dtype != PA_BF16)
    return fail(PA_EINVAL, "pa_reshape_and_cache: unknown dtype %d", dtype);
  if (block_size != kBlockSize)
    return fail(PA_ENOTSUP, "pa_reshape_and_cache: block_size %d (only 16)", block_size);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ENOTSUP, "pa_reshape_and_cache: head_size %d (64 or 128)", head_size);
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !slot_mapping || !kv_cache)
    return fail(PA_EINVAL, "pa_reshape_and_cache: NULL pointer");
  if ((uintptr_t(key) | uintptr_t(value) | uintptr_t(kv_cache)) & 15)
    return fail(PA_EINVAL, "pa_reshape_and_cache: key/value/cache must be 16-byte aligned");
  if (uintptr_t(slot_mapping) & 7)
    return fail(PA_EINVAL, "pa_reshape_and_cache: slot_mapping must be 8-byte aligned");
  const int es = dtype == PA_F32 ? 4 : 2;
  const int vpr = head_size * es / 16;
  const int64_t total = int64_t(num_tokens) * num_kv_heads * vpr;
  const int64_t grid = (total + 255) / 256;
  if (grid > 0x7FFFFFFF) return fail(PA_EINVAL, "pa_reshape_and_cache: too many tokens");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t num_slots = int64_t(num_blocks) * kBlockSize;
  auto k = static_cast<const uint4*>(key);
  auto v = static_cast<const uint4*>(value);
  auto c = static_cast<uint4*>(kv_cache);
  switch (vpr) {
    case 8:
      hipLaunchKernelGGL(reshape_and_cache_kernel<8>, dim3(grid), dim3(256), 0, s, k, v,
                         slot_mapping, num_tokens, c, num_slots, num_kv_heads);
      break;
    case 16:
      hipLaunchKernelGGL(reshape_and_cache_kernel<16>, dim3(grid), dim3(256), 0, s, k, v,
                         slot_mapping, num_tokens, c, num_slots, num_kv_heads);
      break;
    case 32:
      hipLaunchKernelGGL(reshape_and_cache_kernel<32>, dim3(grid), dim3(256), 0, s, k, v,
                         slot_mapping, num_tokens, c, num_slots, num_kv_heads);
      break;
    default:
      return fail(PA_ENOTSUP, "pa_reshape_and_cache: row of %d vectors", vpr);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PA_EHIP, "pa_reshape_and_cache: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}
