// pa_prefill_chunk: causal chunked prefill over a paged KV cache on gfx950
// matrix cores.
//
// What is computed: "Im Inneren von vLLM: Anatomie eines Hochdurchsatz-LLM-
// Inferenzsystems", section "Fortgeschrittene Funktionen" (chunked prefill:
// long prompts are cut into chunks; prefix caching: KV of shared prompt
// prefixes is reused) and "Inside vLLM: Anatomy of a High-Throughput LLM
// Inference System", section "Generate function" (the batch is flattened into
// one sequence of tokens).  Sequence b owns packed query rows
// [qsl[b], qsl[b+1]); these C_b queries are its last C_b tokens, and query i
// at position p = seq_len[b] - C_b + i attends to tokens 0..p through the
// block table (scaled-dot-product softmax attention, the standard
// transformer's, cited in "Inside vLLM", "LLM Engine & Engine Core").
//
// Design (MFMA-bound: ~1400 flop per unique KV byte):
//   * one workgroup (4 waves) per (query tile, KV head, sequence); the rows
//     of a tile are (token, head) pairs of the G query heads that share the
//     KV head, token-major, 128 rows per workgroup and 32 per wave;
//   * keys advance 32 at a time (two blocks).  K and V of the step are
//     loaded by the whole workgroup (coalesced 16-byte vectors, gathered
//     through the block table), double-buffered in padded LDS;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = Q^T
//     held in registers for the whole loop).  The S^T output layout puts one
//     query row per lane and 4 keys per lane group, which is exactly the
//     B-operand layout of O^T = V^T P^T over those keys, so P never leaves
//     registers; only V^T is gathered from LDS (8 keys of one column per lane);
//   * online softmax in the log2 domain per row (row = lane % 16); the
//     causal mask is applied only on steps that reach the diagonal; the
//     denominator sums the same bf16-rounded P that multiplies V.
#include "pa.h"
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPrefillWaves = 4;
constexpr float kLog2eP = 1.4426950408889634f;
constexpr float kLn2P = 0.6931471805599453f;

template <int D, int G>
struct PrefillCfg {
  static constexpr int ROWS = 128;            // (token, head) rows per workgroup
  static constexpr int TQ = ROWS / G;         // query tokens per workgroup
  static constexpr int RW = ROWS / kPrefillWaves;  // rows per wave
  static constexpr int NT = RW / 16;          // 16-row MFMA tiles per wave
  static constexpr int KSTEP = 32;            // keys per step (two blocks)
  static constexpr int DS = D / 32;           // K-dim steps of S^T = K Q^T
  static constexpr int DT = D / 16;           // 16-column tiles of O^T
  static constexpr int LROW = D + 8;          // padded LDS row in bf16 elements
  static constexpr int CH = D / 8;            // 16-byte chunks per K/V row
  static constexpr int LOADS = KSTEP * CH / (kPrefillWaves * kWave);  // per thread, per K or V
  static_assert(LOADS >= 1 && KSTEP * CH % (kPrefillWaves * kWave) == 0, "load split");
  static_assert(RW % 16 == 0, "rows per wave");
};

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int D, int G>
__global__ __launch_bounds__(kPrefillWaves * kWave) void prefill_chunk_kernel(
    uint16_t* __restrict__ out, float* __restrict__ lse_out, const uint16_t* __restrict__ query,
    const int* __restrict__ qsl, const uint16_t* __restrict__ cache, int num_blocks,
    const int* __restrict__ block_tables, int max_blocks_per_seq, const int* __restrict__ seq_lens,
    int max_seq_len, int num_kv_heads, float scale_log2) {
  using C = PrefillCfg<D, G>;
  const int qtile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int H_q = num_kv_heads * G;
  const int q0 = qsl[b];
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
  int Cb = qsl[b + 1] - q0;
  Cb = Cb < 0 ? 0 : (Cb > L ? L : Cb);
  const int t0 = qtile * C::TQ;
  if (t0 >= Cb) return;
  const int ctx = L - Cb;                       // position of the chunk's first query
  const int ntok = min(C::TQ, Cb - t0);
  const int kend = ctx + t0 + ntok;             // keys [0, kend) are visible to some row
  const int nsteps = (kend + C::KSTEP - 1) / C::KSTEP;
  const int nblk = (kend + 15) >> 4;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane >> 4;                     // lane group 0..3
  const int lr = lane & 15;                     // row / column within a 16-tile

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][C::KSTEP * C::LROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][C::KSTEP * C::LROW];

  const int64_t tile_elems = int64_t(16) * D;
  const int64_t block_elems = int64_t(2) * num_kv_heads * tile_elems;
  const int* bt_row = block_tables + int64_t(b) * max_blocks_per_seq;

  // ---- rows of this wave: r = wave*RW + nt*16 + lr  ->  (token r/G, head r%G)
  int row_pos[C::NT];   // absolute position of the row's query, or -1 if inactive
  u32x4 qt[C::NT][C::DS];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    const int r = wave * C::RW + nt * 16 + lr;
    const int i = r / G, hh = r % G;
    const bool active = t0 + i < Cb;
    row_pos[nt] = active ? ctx + t0 + i : -1;
    const uint16_t* qrow = query + (int64_t(q0 + t0 + i) * H_q + g * G + hh) * D;
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (active) v = *reinterpret_cast<const u32x4*>(qrow + ds * 32 + lq * 8);
      qt[nt][ds] = v;
    }
  }

  // ---- staging of one step's K and V (registers -> LDS)
  u32x4 kreg[C::LOADS], vreg[C::LOADS];
  auto load_step = [&](int s, u32x4 (&kr)[C::LOADS], u32x4 (&vr)[C::LOADS]) {
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const int c = u * kPrefillWaves * kWave + tid;   // chunk index in the step
      const int key = c / C::CH, ch = c % C::CH;
      const int kabs = s * C::KSTEP + key;
      const int j = kabs >> 4;
      u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
      if (kabs < kend) {        // past kend: never needed (and may be unwritten)
        int phys = j < nblk ? bt_row[j] : 0;
        phys = (phys < 0 || phys >= num_blocks) ? 0 : phys;
        const uint16_t* kt = cache + int64_t(phys) * block_elems + int64_t(g) * tile_elems;
        const uint16_t* vt = kt + int64_t(num_kv_heads) * tile_elems;
        const int off = (kabs & 15) * D + ch * 8;
        kx = *reinterpret_cast<const u32x4*>(kt + off);
        vx = *reinterpret_cast<const u32x4*>(vt + off);
      }
      kr[u] = kx;
      vr[u] = vx;
    }
  };
  auto store_step = [&](int buf, const u32x4 (&kr)[C::LOADS], const u32x4 (&vr)[C::LOADS]) {
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const int c = u * kPrefillWaves * kWave + tid;
      const int key = c / C::CH, ch = c % C::CH;
      *reinterpret_cast<u32x4*>(&Ks[buf][key * C::LROW + ch * 8]) = kr[u];
      *reinterpret_cast<u32x4*>(&Vs[buf][key * C::LROW + ch * 8]) = vr[u];
    }
  };

  f32x4 acc[C::DT][C::NT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) acc[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[C::NT], l_part[C::NT];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) { m_run[nt] = -INFINITY; l_part[nt] = 0.f; }

  // smallest query position of this wave's active rows (rows are token-major)
  const int wave_min_pos = ctx + t0 + (wave * C::RW) / G;

  load_step(0, kreg, vreg);
  store_step(0, kreg, vreg);
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < nsteps;
    if (more) load_step(s + 1, kreg, vreg);

    // ---- S^T = K Q^T for the step's two 16-key tiles
    f32x4 sacc[2][C::NT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) sacc[kt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int ds = 0; ds < C::DS; ++ds) {
        const u32x4 a =
            *reinterpret_cast<const u32x4*>(&Ks[buf][(kt * 16 + lr) * C::LROW + ds * 32 + lq * 8]);
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) sacc[kt][nt] = mfma16x16x32(a, qt[nt][ds], sacc[kt][nt]);
      }
    }

    // ---- online softmax; lane holds row lr of tile nt, keys kt*16 + 4*lq + i
    const int key0 = s * C::KSTEP;
    const bool need_mask = key0 + C::KSTEP - 1 > wave_min_pos;
    u32x4 pb[C::NT];   // P^T as the B operand: 8 bf16 keys of this lane's row
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      float x[8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sacc[kt][nt][i] * scale_log2;
          if (need_mask) {
            const int key = key0 + kt * 16 + lq * 4 + i;
            v = key <= row_pos[nt] ? v : -INFINITY;
          }
          x[kt * 4 + i] = v;
        }
      float mloc = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mloc = fmaxf(mloc, x[e]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
      const float m_new = fmaxf(m_run[nt], mloc);
      const float mref = m_new == -INFINITY ? 0.f : m_new;   // rows with nothing visible yet
      const float alpha = exp2f(m_run[nt] - mref);
      m_run[nt] = m_new;
      uint32_t pw[4];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t lo = f32_to_bf16_rne(exp2f(x[e] - mref));
        const uint32_t hi = f32_to_bf16_rne(exp2f(x[e + 1] - mref));
        psum += __uint_as_float(lo << 16) + __uint_as_float(hi << 16);
        pw[e / 2] = lo | (hi << 16);
      }
      l_part[nt] = l_part[nt] * alpha + psum;
      pb[nt] = u32x4{pw[0], pw[1], pw[2], pw[3]};
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) acc[dt][nt] *= alpha;
    }

    // ---- O^T += V^T P^T; lane (lq, lr) supplies V[key][dt*16 + lr] for the
    // keys 4*lq + i and 16 + 4*lq + i (i = 0..3), matching P^T's key slots
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const uint16_t* vcol = &Vs[buf][dt * 16 + lr];
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int k0 = (e < 4 ? 0 : 16) + lq * 4 + (e & 3);
        w[e / 2] = uint32_t(vcol[k0 * C::LROW]) | (uint32_t(vcol[(k0 + 1) * C::LROW]) << 16);
      }
      const u32x4 a = u32x4{w[0], w[1], w[2], w[3]};
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) acc[dt][nt] = mfma16x16x32(a, pb[nt], acc[dt][nt]);
    }

    if (more) store_step(buf ^ 1, kreg, vreg);
    __syncthreads();
  }

  // ---- normalise and write: lane holds O^T[dt*16 + 4*lq + i][row lr of tile nt]
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    float l = l_part[nt];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (row_pos[nt] < 0) continue;
    const int r = wave * C::RW + nt * 16 + lr;
    const int i = r / G, hh = r % G;
    const int64_t orow = int64_t(q0 + t0 + i) * H_q + g * G + hh;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const uint32_t w0 = f32_to_bf16_rne(acc[dt][nt][0] * inv) | (f32_to_bf16_rne(acc[dt][nt][1] * inv) << 16);
      const uint32_t w1 = f32_to_bf16_rne(acc[dt][nt][2] * inv) | (f32_to_bf16_rne(acc[dt][nt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(out + orow * D + dt * 16 + lq * 4) = make_uint2(w0, w1);
    }
    if (lse_out && lq == 0) lse_out[orow] = l > 0.f ? m_run[nt] * kLn2P + logf(l) : -INFINITY;
  }
}

template <int D>
static bool launch_prefill(int G, dim3 grid, hipStream_t s, uint16_t* out, float* lse,
                           const uint16_t* q, const int* qsl, const uint16_t* cache, int nb,
                           const int* bt, int mbps, const int* sl, int msl, int hkv, float sc) {
#define PA_PREFILL_CASE(GG)                                                                     \
  case GG:                                                                                      \
    grid.x = (grid.x + PrefillCfg<D, GG>::TQ - 1) / PrefillCfg<D, GG>::TQ;                      \
    hipLaunchKernelGGL((prefill_chunk_kernel<D, GG>), grid, dim3(kPrefillWaves * kWave), 0, s,  \
                       out, lse, q, qsl, cache, nb, bt, mbps, sl, msl, hkv, sc);                \
    return true;
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
  if (!(scale == scale)) return fail(PA_EINVAL, "pa_prefill_chunk: scale is NaN");
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
  dim3 grid(max_query_len, num_kv_heads, B);  // x is divided by the tile size at launch
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto o = static_cast<uint16_t*>(out);
  auto q = static_cast<const uint16_t*>(query);
  auto c = static_cast<const uint16_t*>(kv_cache);
  const float sl2 = scale * kLog2eP;
  bool ok = head_size == 64
                ? launch_prefill<64>(G, grid, s, o, lse_out, q, query_start_loc, c, num_blocks,
                                     block_tables, max_blocks_per_seq, seq_lens, max_seq_len,
                                     num_kv_heads, sl2)
                : launch_prefill<128>(G, grid, s, o, lse_out, q, query_start_loc, c, num_blocks,
                                      block_tables, max_blocks_per_seq, seq_lens, max_seq_len,
                                      num_kv_heads, sl2);
  if (!ok) return fail(PA_ENOTSUP, "pa_prefill_chunk: group size %d", G);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PA_EHIP, "pa_prefill_chunk: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}
