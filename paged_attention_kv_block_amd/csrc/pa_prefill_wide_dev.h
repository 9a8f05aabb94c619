// Causal chunked prefill over a paged KV cache on the gfx950 32x32x16 bf16
// matrix instructions: the device code of pa_prefill_chunk, and of the
// chunk rows of pa_attention_varlen.
//
// What is computed: "Im Inneren von vLLM: Anatomie eines Hochdurchsatz-LLM-
// Inferenzsystems", section "Fortgeschrittene Funktionen" (chunked prefill:
// long prompts are cut into chunks; prefix caching: KV of shared prompt
// prefixes is reused) and "Inside vLLM: Anatomy of a High-Throughput LLM
// Inference System", section "Generate function" (the batch is flattened
// into one sequence of tokens).  Sequence b owns packed query rows
// [qsl[b], qsl[b+1]); these C_b queries are its last C_b tokens, and query i
// at position p = seq_len[b] - C_b + i attends to tokens 0..p through the
// block table (scaled-dot-product softmax attention, the standard
// transformer's, cited in "Inside vLLM", "LLM Engine & Engine Core").
//
// Design (MFMA-bound: ~1400 flop per distinct KV byte):
//   * one workgroup of 4 waves (one per SIMD, about 250 registers each, two
//     workgroups per compute unit) per (query tile, KV head, sequence); a
//     tile is 128 (token, head) rows of the G query heads sharing the KV
//     head, token-major, 32 rows per wave;
//   * keys advance 32 per step (two cache blocks).  Every step's K and V
//     tiles travel from memory straight into a 4-step LDS ring (buffer
//     loads with the LDS destination, no registers), issued three steps
//     ahead; one barrier per step.  Rows are stored as 16-byte chunks
//     permuted by an XOR of the row index, so that both operand reads below
//     hit distinct LDS banks;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims of K
//     from LDS, B = Q^T held in registers for the whole loop.  A lane of the
//     result holds 16 keys of one query row, the other 16 sit in lane ^ 32;
//     those 16 values, rounded to bf16, are exactly the lane's B operand of
//     O^T = V^T P^T over the same keys, so P never leaves registers;
//   * the V^T operand comes from the row-major V tile through the
//     transposing LDS read (ds_read_b64_tr_b16), 4 keys of one head
//     dimension per lane per read;
//   * online softmax in the log2 domain, in two passes of which the second
//     rarely runs: the fast pass fixes each row's reference at the exact
//     max of the first step and never rescales; if a later score is so far
//     above it that P, the denominator or the accumulators overflow, the
//     workgroup redoes the tile with a pass that moves the reference
//     whenever a score exceeds it by 2^8 and rescales the row.  The causal
//     mask is applied only on steps that reach the diagonal of the wave's
//     rows; steps past the wave's last row are skipped; the denominator
//     sums the same bf16-rounded P that multiplies V.
#pragma once

#include <type_traits>

#include "pa.h"
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
#define PA_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kWideWaves = 4;
constexpr int kWideThreads = kWideWaves * kWave;
constexpr int kWideBufs = 4;  // LDS ring of K/V steps
constexpr int kWideRows = kWideWaves * 32;  // (token, head) rows per workgroup
constexpr float kLog2eP = 1.4426950408889634f;
constexpr float kLn2P = 0.6931471805599453f;
constexpr float kPrefillSlack = 8.f;  // log2 units a row max may exceed the reference

template <int D, int G>
struct WideCfg {
  static constexpr int RW = 32;                   // query rows per wave
  static constexpr int ROWS = kWideRows;          // rows per workgroup
  static constexpr int TQ = ROWS / G;             // query tokens per tile
  static constexpr int NC = RW / 32;              // 32-row column tiles per wave
  static constexpr int KSTEP = 32;                // keys per step
  static constexpr int KS = D / 16;               // contraction steps of S^T = K Q^T
  static constexpr int DT = D / 32;               // 32-row head-dimension tiles of O^T
  static constexpr int RB = D * 2;                // bytes per K / V row
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int TILE = KSTEP * RB;         // bytes of a step's K (or V) tile
  static constexpr int BUF = 2 * TILE;            // one ring slot: K, then V
  static constexpr int WL = KSTEP * CPR / kWave;  // 1 KiB wave-loads per tile
  static constexpr int LOADS = (WL + kWideWaves - 1) / kWideWaves;  // per loading wave per tile
  static constexpr int LOAD_WAVES = WL / LOADS;   // waves that load (the others only compute)
  static constexpr int ROWS_PER_WL = kWave / CPR;
  static_assert(WL % LOADS == 0 && LOAD_WAVES <= kWideWaves, "load split");
  static_assert(16 % ROWS_PER_WL == 0, "a wave-load stays inside one cache block");
  static_assert(ROWS == kWideWaves * RW, "rows per workgroup");
};

// Physical 16-byte chunk of logical chunk c in row r (an involution).  K:
// the 16 rows read by one 16-lane group at one chunk land on 16 distinct
// bank groups.  V: the 4 rows x 32 bytes of one 16-lane transposing read
// (and the 8 rows of a half-wave) land on distinct banks.
template <int D>
__device__ __forceinline__ int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int v_swz(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// max / sum of x over lanes l and l ^ 32 (gfx950 lane-swap move)
__device__ __forceinline__ float xor32_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] at their
// maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) alone: this wave's LDS stores have completed.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Workgroup barrier for the LDS ring without a memory fence.  A fence here
// would also wait for every buffer load still streaming into the ring
// (they count as LDS writes), i.e. drain the prefetch at every step; the
// ring's ordering is kept by hand instead: before the barrier each wave
// waits for its own loads of the step about to be read (wait_vmcnt) and
// for its own LDS stores (wait_lgkmcnt0), and every LDS read is consumed
// before the barrier that precedes the slot's reuse.  The empty asm keeps
// the compiler from moving memory operations across it.
__device__ __forceinline__ void ring_barrier() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// One query tile `qtile` of sequence b, KV head g; called by the whole
// workgroup (kWideThreads threads) with smem holding kWideBufs * BUF + 64
// bytes.
template <int D, int G>
__device__ __forceinline__ void wide_tile(
    uint8_t* __restrict__ smem, uint16_t* __restrict__ out, float* __restrict__ lse_out,
    const uint16_t* __restrict__ query, const int* __restrict__ qsl,
    const uint16_t* __restrict__ cache, int num_blocks, const int* __restrict__ block_tables,
    int max_blocks_per_seq, const int* __restrict__ seq_lens, int max_seq_len, int num_kv_heads,
    float scale_log2, int b, int g, int qtile) {
  using C = WideCfg<D, G>;
  const int H_q = num_kv_heads * G;
  const int q0 = qsl[b];
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
  int Cb = qsl[b + 1] - q0;
  Cb = Cb < 0 ? 0 : (Cb > L ? L : Cb);
  const int t0 = qtile * C::TQ;
  if (t0 >= Cb) return;                         // uniform over the workgroup
  const int ctx = L - Cb;                       // position of the chunk's first query
  const int ntok = min(C::TQ, Cb - t0);
  const int kend = ctx + t0 + ntok;             // keys [0, kend) are visible to some row
  const int nsteps = (kend + C::KSTEP - 1) / C::KSTEP;
  const int nblk = (kend + 15) >> 4;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;                     // half of the wave
  const int ln = lane & 31;                     // query row within a 32-row column tile

  // ---- this wave's rows: r = RW wave + 32 nc + ln -> (token r / G, head r % G)
  int row_pos[C::NC];   // absolute position of the row's query, -1 if the row is padding
  u32x4 qt[C::NC][C::KS];
#pragma unroll
  for (int nc = 0; nc < C::NC; ++nc) {
    const int r = wave * C::RW + nc * 32 + ln;
    const int i = r / G, hh = r % G;
    const bool active = t0 + i < Cb;
    row_pos[nc] = active ? ctx + t0 + i : -1;
    const uint16_t* qrow = query + (int64_t(q0 + t0 + i) * H_q + g * G + hh) * D;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (active) v = *reinterpret_cast<const u32x4*>(qrow + ks * 16 + hl * 8);
      qt[nc][ks] = v;
    }
  }
  // first and last query position among the wave's rows (token-major rows)
  const int wtok0 = (wave * C::RW) / G;
  const int wtok1 = min((wave * C::RW + C::RW - 1) / G, ntok - 1);
  const int wave_steps = wtok0 < ntok ? (ctx + t0 + wtok1) / C::KSTEP + 1 : 0;
  const int s_diag = min((ctx + t0 + wtok0 + 1) / C::KSTEP, nsteps);

  // ---- loads: block ids through scalar loads, issued a step before their
  // use right after a barrier (no LDS operation is outstanding there, so
  // their shared wait counter costs nothing; a vector load's result would
  // make the compiler wait for the ring's buffer loads too), and the K/V
  // tiles straight into the LDS ring
  const int* bt_row = block_tables + int64_t(b) * max_blocks_per_seq;
  auto step_ids = [&](int s) -> int2 {
    const int j = __builtin_amdgcn_readfirstlane(min(2 * s, nblk - 1));
    const int k = __builtin_amdgcn_readfirstlane(min(2 * s + 1, nblk - 1));
    return make_int2(__builtin_nontemporal_load(bt_row + j), __builtin_nontemporal_load(bt_row + k));
  };
  const int64_t tile_elems = int64_t(16) * D;          // one (block, head) K or V tile
  const int block_bytes = int(2 * num_kv_heads * tile_elems * 2);
  uint32_t koff[C::LOADS], voff[C::LOADS];             // bytes from the block's start
#pragma unroll
  for (int u = 0; u < C::LOADS; ++u) {
    const int ci = (wave * C::LOADS + u) * kWave + lane;   // chunk slot within the tile
    const int r = ci / C::CPR, pc = ci % C::CPR;
    koff[u] = uint32_t((g * tile_elems + (r & 15) * D + (pc ^ k_swz<D>(r)) * 8) * 2);
    voff[u] = uint32_t(((num_kv_heads + g) * tile_elems + (r & 15) * D + (pc ^ v_swz<D>(r)) * 8) * 2);
  }
  const uint8_t* cache_bytes = reinterpret_cast<const uint8_t*>(cache);
  auto load_step = [&](int s, int2 ids) __attribute__((always_inline)) {
    uint8_t* slot = smem + (s & (kWideBufs - 1)) * C::BUF;
    int id0 = __builtin_amdgcn_readfirstlane(ids.x);
    int id1 = __builtin_amdgcn_readfirstlane(ids.y);
    id0 = (id0 < 0 || id0 >= num_blocks) ? 0 : id0;    // out-of-range ids read block 0
    id1 = (id1 < 0 || id1 >= num_blocks) ? 0 : id1;
    const __amdgpu_buffer_rsrc_t r0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(cache_bytes + int64_t(id0) * block_bytes), 0, block_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(cache_bytes + int64_t(id1) * block_bytes), 0, block_bytes, 0x00020000);
    if (wave >= C::LOAD_WAVES) return;
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const int wl = wave * C::LOADS + u;
      const bool second = wl * C::ROWS_PER_WL >= 16;    // rows 16..31: the step's second block
      uint8_t* kdst = slot + wl * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? r1 : r0, PA_LDS_PTR(void, kdst), 16,
                                               koff[u], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? r1 : r0,
                                               PA_LDS_PTR(void, kdst + C::TILE), 16, voff[u], 0,
                                               0, 0);
    }
  };
  constexpr int kVmemPerStep = 2 * C::LOADS;       // K/V loads of one step

  // ---- per-lane operand offsets within a ring slot
  // K (A of S^T): row ln (key), chunk 2 ks + hl (head dims 16 ks + 8 hl ..)
  uint32_t kofs[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    kofs[ks] = uint32_t(ln * C::RB + (((2 * ks + hl) ^ k_swz<D>(ln)) * 16));
  // V^T (A of O^T), transposing read: 16-lane group gi covers head dims
  // 32 dt + 16 (gi & 1) + 0..15 for keys of lane half gi >> 1; its lane
  // li = 4 jj + q points at row 4 (gi >> 1) + jj (+ 16 kh + 8 p), dims
  // 32 dt + 16 (gi & 1) + 4 q .. + 3, and receives 4 keys of one dim.
  const int gi = lane >> 4, li = lane & 15, jj = li >> 2, qq = li & 3;
  const int vrow0 = 4 * (gi >> 1) + jj;
  uint32_t vofs[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    const int ub = 8 * dt + 4 * (gi & 1) + qq;       // 8-byte unit within the row
    vofs[dt] = uint32_t(C::TILE + vrow0 * C::RB + (((ub >> 1) ^ v_swz<D>(vrow0)) * 16) + (ub & 1) * 8);
  }

  f32x16 acc[C::DT][C::NC];
  float m_run[C::NC], m_thr[C::NC], l_part[C::NC];

  // S^T of a step for both column tiles: its K operands from the ring slot
  // (read_k), then the matrix products (mfma_s)
  // (the *_at forms take the ring slot as a compile-time constant, so its
  // offset folds into the LDS instructions' immediate field)
  auto read_k_at = [&](auto slot_tag, u32x4 (&ka)[C::KS]) __attribute__((always_inline)) {
    const uint8_t* slot = smem + decltype(slot_tag)::value * C::BUF;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) ka[ks] = *reinterpret_cast<const u32x4*>(slot + kofs[ks]);
  };
  auto read_k = [&](int s, u32x4 (&ka)[C::KS]) __attribute__((always_inline)) {
    const uint8_t* slot = smem + (s & (kWideBufs - 1)) * C::BUF;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) ka[ks] = *reinterpret_cast<const u32x4*>(slot + kofs[ks]);
  };
  auto mfma_s = [&](const u32x4 (&ka)[C::KS], f32x16 (&sacc)[C::NC]) __attribute__((always_inline)) {
#pragma unroll
    for (int nc = 0; nc < C::NC; ++nc) {
      sacc[nc] = mfma32x32x16(ka[0], qt[nc][0], f32x16{});
#pragma unroll
      for (int ks = 1; ks < C::KS; ++ks) sacc[nc] = mfma32x32x16(ka[ks], qt[nc][ks], sacc[nc]);
    }
  };
  auto scores = [&](int s, f32x16 (&sacc)[C::NC]) __attribute__((always_inline)) {
    u32x4 ka[C::KS];
    read_k(s, ka);
    mfma_s(ka, sacc);
  };

  // Softmax of step s, in place on its scores: lane value 4 j + i of
  // column tile nc is key 8 j + 4 hl + i of row ln.  check() applies the
  // causal mask (diagonal steps) and reports whether any of the lane's
  // scores exceeds its row's threshold (lmax keeps the lane's maxima).
  float lmax[C::NC];
  auto check = [&](int s, f32x16 (&x)[C::NC], auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int key0 = s * C::KSTEP + 4 * hl;
    bool grow = false;
#pragma unroll
    for (int nc = 0; nc < C::NC; ++nc) {
      if constexpr (MASK) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          x[nc][e] = key0 + 8 * (e >> 2) + (e & 3) <= row_pos[nc] ? x[nc][e] : -INFINITY;
      }
      float m = x[nc][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) m = fmaxf(m, x[nc][e]);
      lmax[nc] = m * scale_log2;                 // scale > 0 keeps the order
      grow |= lmax[nc] > m_thr[nc];
    }
    return grow;
  };
  // mask(): the causal mask alone (the fast pass checks no maxima)
  auto mask = [&](int s, f32x16 (&x)[C::NC], auto mask_tag) __attribute__((always_inline)) {
    if constexpr (decltype(mask_tag)::value) {
      const int key0 = s * C::KSTEP + 4 * hl;
#pragma unroll
      for (int nc = 0; nc < C::NC; ++nc)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          x[nc][e] = key0 + 8 * (e >> 2) + (e & 3) <= row_pos[nc] ? x[nc][e] : -INFINITY;
    }
  };
  // rescale(): rows whose max grew past the threshold move their reference
  // and scale their accumulators (rescaling pass only)
  auto rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nc = 0; nc < C::NC; ++nc) {
      const float rm = xor32_max(lmax[nc]);      // the row's max over both lane halves
      if (rm > m_thr[nc]) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[nc] - rm);
        m_run[nc] = rm;
        m_thr[nc] = rm + kPrefillSlack;
        l_part[nc] *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) acc[dt][nc] *= alpha;
      }
    }
  };
  // probs(): bf16 P^T B operands (keys 16 kh + 4 hl + 0..3 and + 8) under
  // the current reference, adding the same rounded values to each row's
  // denominator; mfma_pv(): O^T += V^T P^T.
  auto probs = [&](const f32x16 (&x)[C::NC], u32x4 (&pb)[C::NC][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int nc = 0; nc < C::NC; ++nc) {
      uint32_t pw[8];
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[nc][e], scale_log2, -m_run[nc]));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[nc][e + 1], scale_log2, -m_run[nc]));
        pw[e / 2] = pack_bf16x2(p0, p1);
        l_part[nc] = dot2_bf16(pw[e / 2], 0x3F803F80u, l_part[nc]);
      }
      pb[nc][0] = u32x4{pw[0], pw[1], pw[2], pw[3]};
      pb[nc][1] = u32x4{pw[4], pw[5], pw[6], pw[7]};
    }
  };
  // V^T operands of a step from its ring slot (read_v_slot), then
  // O^T += V^T P^T (mfma_pv_ops)
  auto read_v_slot = [&](const uint8_t* slot, u32x4 (&va)[C::DT][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const uint8_t* p = slot + vofs[dt] + (16 * kh) * C::RB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(PA_LDS_PTR(i16x4, p));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(PA_LDS_PTR(i16x4, p + 8 * C::RB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        va[dt][kh] = u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
  };
  auto mfma_pv_ops = [&](const u32x4 (&va)[C::DT][2], const u32x4 (&pb)[C::NC][2])
      __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int nc = 0; nc < C::NC; ++nc)
          acc[dt][nc] = mfma32x32x16(va[dt][kh], pb[nc][kh], acc[dt][nc]);
  };
  auto mfma_pv_slot = [&](const uint8_t* slot, const u32x4 (&pb)[C::NC][2])
      __attribute__((always_inline)) {
    u32x4 va[C::DT][2];
    read_v_slot(slot, va);
    mfma_pv_ops(va, pb);
  };
  auto mfma_pv = [&](int s, const u32x4 (&pb)[C::NC][2]) __attribute__((always_inline)) {
    mfma_pv_slot(smem + (s & (kWideBufs - 1)) * C::BUF, pb);
  };
  auto mfma_pv_at = [&](auto slot_tag, const u32x4 (&pb)[C::NC][2]) __attribute__((always_inline)) {
    mfma_pv_slot(smem + decltype(slot_tag)::value * C::BUF, pb);
  };

  // V rows at and past kend in the last step's slot may hold unwritten
  // cache slots (NaN): they are zeroed once that step's loads have landed
  // (its P there is 0 and must not meet a NaN).
  const int zlast = nsteps - 1;
  auto zero_tail_v = [&]() __attribute__((always_inline)) {
    const int r0 = kend - zlast * C::KSTEP;   // first row to clear (1..32)
    if (r0 >= C::KSTEP) return;
    uint8_t* vt = smem + (zlast & (kWideBufs - 1)) * C::BUF + C::TILE;
    for (int c = r0 * C::CPR + tid; c < C::KSTEP * C::CPR; c += kWideThreads)
      *reinterpret_cast<u32x4*>(vt + c * 16) = u32x4{0u, 0u, 0u, 0u};
    wait_lgkmcnt0();
  };

  // Iteration s: loads of step s + 3 (ids of step s + 4), S^T of step s + 1,
  // softmax and P V of step s, then every load issued before this
  // iteration has landed (step s + 2) and one barrier (tail).  Loads past
  // the last step repeat the last block into a slot nobody reads, so the
  // wait count is constant.  Every wave runs all nsteps iterations.
  int2 ids_next;
  auto head = [&](int s) __attribute__((always_inline)) {
    const int2 ids = ids_next;
    ids_next = step_ids(s + 4);
    load_step(s + 3, ids);
  };
  auto tail = [&](int s) __attribute__((always_inline)) {
    if (s == zlast - 1 && zlast >= 2) zero_tail_v();
    wait_vmcnt<kVmemPerStep>();
    ring_barrier();
  };

  // One pass over the tile's keys.  The fast pass never rescales and
  // checks no maxima: every row's reference is the exact max of step 0
  // (which holds key 0, visible to every query; padding rows take 0), and a
  // later score above it is harmless as long as P, the denominators and the
  // accumulators stay finite (bf16 and fp32 keep their relative precision
  // up to 2^127).  If any of them overflowed, the wave raises a flag at the
  // end, and a flag anywhere in the workgroup makes every wave redo the
  // tile with the rescaling pass (reference moved whenever a score exceeds
  // it by 2^8).  So the fast pass's steps are
  // straight-line code: K operands of step s + 1 first, the softmax of step
  // s while they arrive, then both matrix products.
  auto pass = [&](auto slow_tag) __attribute__((always_inline)) -> bool {
    constexpr bool SLOW = decltype(slow_tag)::value;
    const float slack = kPrefillSlack;   // used by the rescaling pass only
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int nc = 0; nc < C::NC; ++nc) acc[dt][nc] = f32x16{};
#pragma unroll
    for (int nc = 0; nc < C::NC; ++nc) { m_run[nc] = 0.f; m_thr[nc] = 0.f; l_part[nc] = 0.f; }

    // prologue: ids of steps 0..3, K/V of steps 0..2; steps 0 and 1 landed
    const int2 ids0 = step_ids(0), ids1 = step_ids(1), ids2 = step_ids(2);
    ids_next = step_ids(3);
    load_step(0, ids0);
    load_step(1, ids1);
    load_step(2, ids2);
    wait_vmcnt<2 * C::LOADS>();
    ring_barrier();
    if (zlast <= 1) zero_tail_v();
    ring_barrier();
    f32x16 sa[C::NC], sb[C::NC];
    if (wave_steps > 0) {
      scores(0, sa);
      if (s_diag > 0) check(0, sa, std::false_type{});
      else check(0, sa, std::true_type{});
#pragma unroll
      for (int nc = 0; nc < C::NC; ++nc) {
        const float rm = xor32_max(lmax[nc]);
        m_run[nc] = rm == -INFINITY ? 0.f : rm;
        m_thr[nc] = m_run[nc] + slack;
      }
    }
    bool flag = false;
    int s = 0;
    // a full step (S^T of step s + 1 and P V of step s); SL: the ring slot
    // of step s when known at compile time (-1: computed from s)
    auto full_step = [&](f32x16 (&cur)[C::NC], f32x16 (&nxt)[C::NC], auto mask_tag,
                         auto slot_tag) __attribute__((always_inline)) {
      constexpr int SL = decltype(slot_tag)::value;
      head(s);
      // every LDS operand read of the step first (K of step s + 1, V of
      // step s), held there by a scheduling barrier: the softmax below
      // then covers their latency instead of each product waiting on its
      // own read
      u32x4 ka[C::KS];
      u32x4 va[C::DT][2];
      if constexpr (SL >= 0) {
        read_k_at(std::integral_constant<int, (SL + 1) & (kWideBufs - 1)>{}, ka);
        read_v_slot(smem + SL * C::BUF, va);
      } else {
        read_k(s + 1, ka);
        read_v_slot(smem + (s & (kWideBufs - 1)) * C::BUF, va);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (SLOW) {
        if (__builtin_amdgcn_ballot_w64(check(s, cur, mask_tag)) != 0) rescale();
      } else {
        mask(s, cur, mask_tag);
      }
      u32x4 pb[C::NC][2];
      probs(cur, pb);
      mfma_s(ka, nxt);
      mfma_pv_ops(va, pb);
      tail(s);
      ++s;
    };
    using Dyn = std::integral_constant<int, -1>;
    // full steps: singles up to a multiple of the ring size, then groups of
    // four with static slots (the score buffers also swap roles without
    // copies), then singles
    auto full_steps = [&](int end, auto mask_tag) __attribute__((always_inline)) {
      while (s < end && (s & (kWideBufs - 1)) != 0) {
        full_step(sa, sb, mask_tag, Dyn{});
#pragma unroll
        for (int nc = 0; nc < C::NC; ++nc) sa[nc] = sb[nc];
      }
      for (; s + kWideBufs - 1 < end;) {
        full_step(sa, sb, mask_tag, std::integral_constant<int, 0>{});
        full_step(sb, sa, mask_tag, std::integral_constant<int, 1>{});
        full_step(sa, sb, mask_tag, std::integral_constant<int, 2>{});
        full_step(sb, sa, mask_tag, std::integral_constant<int, 3>{});
      }
      while (s < end) {
        full_step(sa, sb, mask_tag, Dyn{});
#pragma unroll
        for (int nc = 0; nc < C::NC; ++nc) sa[nc] = sb[nc];
      }
    };
    auto other_step = [&](auto mask_tag) __attribute__((always_inline)) {
      head(s);
      if (s + 1 < wave_steps) scores(s + 1, sb);
      if (s < wave_steps) {
        if constexpr (SLOW) {
          if (__builtin_amdgcn_ballot_w64(check(s, sa, mask_tag)) != 0) rescale();
        } else {
          mask(s, sa, mask_tag);
        }
        u32x4 pb[C::NC][2];
        probs(sa, pb);
        mfma_pv(s, pb);
      }
      tail(s);
#pragma unroll
      for (int nc = 0; nc < C::NC; ++nc) sa[nc] = sb[nc];
      ++s;
    };
    const int full_end = max(wave_steps - 1, 0);
    const int e1 = min(s_diag, full_end);
    full_steps(e1, std::false_type{});
    while (s < s_diag) other_step(std::false_type{});
    const int e2 = max(min(nsteps, full_end), s);
    full_steps(e2, std::true_type{});
    while (s < nsteps) other_step(std::true_type{});
    wait_vmcnt<0>();   // every load has landed before the ring is reused or released
    if constexpr (!SLOW) {
      // A score far above its row's reference overflows P, the denominator
      // or the accumulators to inf (or NaN): one sum per row shows it.
#pragma unroll
      for (int nc = 0; nc < C::NC; ++nc) {
        float t = l_part[nc];
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) t += acc[dt][nc][e];
        // the bits pass through an empty asm: this file is built without
        // NaN semantics, under which the compiler would reduce the exponent
        // test to |t| == inf and miss a NaN
        uint32_t tb = __float_as_uint(t);
        __asm__ __volatile__("" : "+v"(tb));
        flag |= (tb & 0x7F800000u) == 0x7F800000u;
      }
    }
    return flag;
  };

  // the workgroup agrees on a redo through one LDS word per wave (outside
  // the ring)
  int* wave_flags = reinterpret_cast<int*>(smem + kWideBufs * C::BUF);
  const bool flag = pass(std::false_type{});
  const bool wave_flag = __builtin_amdgcn_ballot_w64(flag) != 0;   // all lanes take part
  if (lane == 0) wave_flags[wave] = wave_flag;
  wait_lgkmcnt0();
  ring_barrier();
  bool redo = false;
#pragma unroll
  for (int w = 0; w < kWideWaves; ++w) redo |= wave_flags[w] != 0;
  ring_barrier();
  if (redo) pass(std::true_type{});

  // ---- normalise and write: lane holds O^T[32 dt + 8 j + 4 hl + i][row ln]
#pragma unroll
  for (int nc = 0; nc < C::NC; ++nc) {
    const float l = xor32_sum(l_part[nc]);
    if (row_pos[nc] < 0) continue;
    const int r = wave * C::RW + nc * 32 + ln;
    const int i = r / G, hh = r % G;
    const int64_t orow = int64_t(q0 + t0 + i) * H_q + g * G + hh;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& a = acc[dt][nc];
        const uint32_t w0 = pack_bf16x2(a[4 * j] * inv, a[4 * j + 1] * inv);
        const uint32_t w1 = pack_bf16x2(a[4 * j + 2] * inv, a[4 * j + 3] * inv);
        *reinterpret_cast<uint2*>(out + orow * D + dt * 32 + j * 8 + hl * 4) = make_uint2(w0, w1);
      }
    if (lse_out && hl == 0) lse_out[orow] = l > 0.f ? m_run[nc] * kLn2P + logf(l) : -INFINITY;
  }
}

template <int D, int G>
__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
prefill_wide_kernel(uint16_t* __restrict__ out, float* __restrict__ lse_out,
                    const uint16_t* __restrict__ query, const int* __restrict__ qsl,
                    const uint16_t* __restrict__ cache, int num_blocks,
                    const int* __restrict__ block_tables, int max_blocks_per_seq,
                    const int* __restrict__ seq_lens, int max_seq_len, int num_kv_heads,
                    float scale_log2, int tiles, int num_groups) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kWideBufs * WideCfg<D, G>::BUF + 64];
  // Workgroup -> (query tile, KV head g, sequence b), with all query tiles of
  // a (sequence, KV head) on one XCD when the groups split evenly over the 8
  // (the dispatcher deals workgroups to the XCDs in turn): they share the
  // blocks they stream through that XCD's L2.
  const int wg = blockIdx.x;
  int grp, qtile;
  if ((num_groups & 7) == 0) {
    const int r = wg >> 3;
    grp = (r / tiles) * 8 + (wg & 7);
    qtile = r % tiles;
  } else {
    grp = wg / tiles;
    qtile = wg % tiles;
  }
  const int g = grp % num_kv_heads, b = grp / num_kv_heads;
  wide_tile<D, G>(smem, out, lse_out, query, qsl, cache, num_blocks, block_tables,
                  max_blocks_per_seq, seq_lens, max_seq_len, num_kv_heads, scale_log2, b, g,
                  qtile);
}

}  // namespace pa
