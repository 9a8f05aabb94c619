// Decode-step graphs for a set of warm-up batch sizes.
//
// "Inside vLLM: Anatomy of a High-Throughput LLM Inference System", section
// "LLM Engine constructor": when the engine starts it captures a graph of
// the forward pass for each of a list of warm-up batch sizes, and a decode
// step later replays the graph of a batch size that fits instead of issuing
// its launches one by one.  Here the captured step is the attention half of
// a decode step for num_layers layers: per layer, pa_decode_append (the new
// tokens' K/V written into that layer's cache and attended to with the
// rest), over static buffers the caller owns and sizes for the largest
// batch.  A replay of B sequences takes the smallest captured size Bc >= B;
// rows B..Bc-1 are padding with seq_len 0, for which the decode writes
// nothing into the cache, a zero output row and lse -inf.
//
// A graph fixes its launch shapes, so the captured calls have no plan
// (whose length follows the step's lengths): the persistent grid walks
// every (sequence, partition up to max_seq_len) pair and skips the empty
// ones on the device, which makes one graph valid for any lengths up to
// max_seq_len.  The padding lengths are written by a fill kernel before the
// graph launch (a memset node in a graph is avoided on purpose).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace pa {

__global__ void zero_lens_kernel(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace pa

using namespace pa;

struct pa_decode_graphs {
  int device = -1;
  int32_t* seq_lens = nullptr;           // the caller's device array
  std::vector<int32_t> sizes;            // ascending
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> execs;

  ~pa_decode_graphs() {
    for (hipGraphExec_t e : execs) (void)hipGraphExecDestroy(e);
    for (hipGraph_t g : graphs) (void)hipGraphDestroy(g);
  }
};

extern "C" int pa_decode_graphs_create(
    void* out, float* lse_out, const void* query, const void* new_key, const void* new_value,
    void* const* kv_caches, int32_t num_layers, int32_t num_blocks, const int32_t* block_tables,
    int32_t max_blocks_per_seq, int32_t* seq_lens, int32_t max_seq_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size, float scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t dtype,
    const int32_t* batch_sizes, int32_t num_sizes, void* stream, pa_decode_graphs** handle) {
  const char* fn = "pa_decode_graphs_create";
  if (!handle) return fail(PA_EINVAL, "%s: NULL handle", fn);
  *handle = nullptr;
  if (num_layers <= 0 || !kv_caches) return fail(PA_EINVAL, "%s: no layers", fn);
  if (dtype != PA_BF16 && dtype != PA_F32)
    return fail(PA_EINVAL, "%s: dtype %d (bf16 or fp32 caches)", fn, dtype);
  if (!out || !query || !new_key || !new_value) return fail(PA_EINVAL, "%s: NULL pointer", fn);
  if (num_sizes <= 0 || !batch_sizes) return fail(PA_EINVAL, "%s: no batch sizes", fn);
  std::vector<int32_t> sizes(batch_sizes, batch_sizes + num_sizes);
  std::sort(sizes.begin(), sizes.end());
  sizes.erase(std::unique(sizes.begin(), sizes.end()), sizes.end());
  if (sizes.front() <= 0 || sizes.back() > 65535)
    return fail(PA_EINVAL, "%s: batch sizes must lie in [1, 65535]", fn);
  if (!stream)
    return fail(PA_EINVAL, "%s: capture needs a stream other than the null stream", fn);
  if (!seq_lens) return fail(PA_EINVAL, "%s: NULL seq_lens", fn);
  // the captured calls' workspace must hold the largest batch's split-K layout
  const size_t need = pa_decode_workspace_bytes(sizes.back(), num_q_heads, num_kv_heads,
                                                head_size, max_seq_len, partition_size);
  if (need > workspace_bytes)
    return fail(PA_EINVAL, "%s: workspace of %zu bytes needed for batch %d, %zu given", fn, need,
                sizes.back(), workspace_bytes);
  auto* g = new pa_decode_graphs();
  if (hipGetDevice(&g->device) != hipSuccess) {
    delete g;
    return fail(PA_EHIP, "%s: no current device", fn);
  }
  g->seq_lens = seq_lens;
  g->sizes = sizes;
  // layer l's rows start l * Bmax rows into out, lse, query and the new K/V
  const int64_t Bmax = sizes.back(), esz = dtype == PA_BF16 ? 2 : 4;
  const int64_t q_layer = Bmax * num_q_heads * head_size * esz;
  const int64_t kv_layer = Bmax * num_kv_heads * head_size * esz;
  const int64_t lse_layer = Bmax * num_q_heads;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int32_t Bc : sizes) {
    hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed);
    if (e != hipSuccess) {
      delete g;
      return fail(PA_EHIP, "%s: begin capture: %s", fn, hipGetErrorString(e));
    }
    // per layer, in order on the stream, the first Bc rows of every
    // per-sequence buffer (the layers share the workspace: each call leaves
    // its counters at zero before the next one starts)
    int rc = PA_OK;
    for (int32_t l = 0; l < num_layers && rc == PA_OK; ++l)
      rc = pa_decode_append(
          static_cast<uint8_t*>(out) + l * q_layer, lse_out ? lse_out + l * lse_layer : nullptr,
          static_cast<const uint8_t*>(query) + l * q_layer,
          new_key ? static_cast<const uint8_t*>(new_key) + l * kv_layer : nullptr,
          new_value ? static_cast<const uint8_t*>(new_value) + l * kv_layer : nullptr,
          kv_caches[l], num_blocks, block_tables, max_blocks_per_seq, seq_lens, Bc, max_seq_len,
          num_q_heads, num_kv_heads, head_size, block_size, scale, partition_size, nullptr, 0,
          workspace, workspace_bytes, dtype, stream);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(s, &graph);
    if (rc != PA_OK) {  // the message of the failed call stands
      if (graph) (void)hipGraphDestroy(graph);
      delete g;
      return rc;
    }
    if (e != hipSuccess || !graph) {
      if (graph) (void)hipGraphDestroy(graph);
      delete g;
      return fail(PA_EHIP, "%s: end capture (batch %d): %s", fn, Bc, hipGetErrorString(e));
    }
    g->graphs.push_back(graph);
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      delete g;
      return fail(PA_EHIP, "%s: instantiate (batch %d): %s", fn, Bc, hipGetErrorString(e));
    }
    g->execs.push_back(exec);
  }
  *handle = g;
  return PA_OK;
}

extern "C" int pa_decode_graphs_replay(pa_decode_graphs* g, int32_t B, void* stream,
                                       int32_t* graph_batch) {
  const char* fn = "pa_decode_graphs_replay";
  if (!g) return fail(PA_EINVAL, "%s: NULL handle", fn);
  if (graph_batch) *graph_batch = 0;
  if (B < 0 || B > g->sizes.back())
    return fail(PA_EINVAL, "%s: batch %d outside [0, %d] (the largest captured size)", fn, B,
                g->sizes.back());
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != g->device)
    return fail(PA_EINVAL, "%s: current device %d, graphs captured on %d", fn, dev, g->device);
  if (B == 0) return PA_OK;
  const size_t i = size_t(std::lower_bound(g->sizes.begin(), g->sizes.end(), B) - g->sizes.begin());
  const int32_t Bc = g->sizes[i];
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (B < Bc) {
    const int n = Bc - B;
    hipLaunchKernelGGL(zero_lens_kernel, dim3((n + 255) / 256), dim3(256), 0, s, g->seq_lens + B, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_EHIP, "%s: padding fill: %s", fn, hipGetErrorString(e));
  }
  const hipError_t e = hipGraphLaunch(g->execs[i], s);
  if (e != hipSuccess) return fail(PA_EHIP, "%s: graph launch: %s", fn, hipGetErrorString(e));
  if (graph_batch) *graph_batch = Bc;
  return PA_OK;
}

extern "C" int32_t pa_decode_graphs_count(const pa_decode_graphs* g, int32_t* batch_sizes,
                                          int32_t capacity) {
  if (!g) return -1;
  const int32_t n = int32_t(g->sizes.size());
  if (batch_sizes)
    for (int32_t k = 0; k < n && k < capacity; ++k) batch_sizes[k] = g->sizes[k];
  return n;
}

extern "C" void pa_decode_graphs_destroy(pa_decode_graphs* g) { delete g; }
