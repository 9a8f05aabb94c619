// pa_prefill_chunk device code: causal chunked prefill over a paged KV
// cache on gfx950 matrix cores.
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
//     loaded by the whole workgroup (16-byte vectors gathered through the
//     block table) and double-buffered in LDS: K row-major, V transposed
//     (one row per head dimension) with its keys permuted into the order in
//     which P^T holds them, so every MFMA operand is one 16-byte LDS read;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = Q^T
//     held in registers for the whole loop).  The S^T output layout puts one
//     query row per lane and 4 keys per lane group, which is the B-operand
//     layout of O^T = V^T P^T over those keys, so P never leaves registers;
//   * online softmax in the log2 domain per row (row = lane % 16), row
//     maxima reduced across the four lane groups with lane-swap moves; the
//     reference moves only when a row's max exceeds it by 2^8, so the
//     accumulators are rarely rescaled; the causal mask is applied only on
//     steps that reach the diagonal; the denominator sums the same
//     bf16-rounded P that multiplies V.
#pragma once

#include <type_traits>

#include "pa.h"
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPrefillWaves = 4;
constexpr int kPrefillThreads = kPrefillWaves * kWave;
constexpr int kPrefillBufs = 3;  // LDS ring of K/V steps
constexpr int kPrefillRows = 128;  // (token, head) rows per workgroup: 128 / G query tokens
constexpr float kLog2eP = 1.4426950408889634f;
constexpr float kLn2P = 0.6931471805599453f;
constexpr float kPrefillSlack = 8.f;  // log2 units a row max may exceed the reference

template <int D, int G>
struct PrefillCfg {
  static constexpr int ROWS = kPrefillRows;   // (token, head) rows per workgroup
  static constexpr int TQ = ROWS / G;         // query tokens per workgroup
  static constexpr int RW = ROWS / kPrefillWaves;  // rows per wave
  static constexpr int NT = RW / 16;          // 16-row MFMA tiles per wave
  static constexpr int KSTEP = 32;            // keys per step (two blocks)
  static constexpr int DS = D / 32;           // K-dim steps of S^T = K Q^T
  static constexpr int DT = D / 16;           // 16-column tiles of O^T
  static constexpr int LROW = D + 8;          // padded K row in LDS (bf16 elements)
  static constexpr int VROW = KSTEP + 8;      // padded V^T row in LDS (bf16 elements)
  static constexpr int CH = D / 8;            // 16-byte chunks per K/V row
  static constexpr int KLOADS = KSTEP * CH / kPrefillThreads;   // K chunks per thread
  static constexpr int VPAIRS = KSTEP / 2 * CH;                 // V (key pair, chunk) items
  static_assert(KLOADS >= 1 && KSTEP * CH % kPrefillThreads == 0, "K load split");
  static_assert(VPAIRS <= kPrefillThreads, "V pair split");
  static_assert(RW % 16 == 0, "rows per wave");
};

// Position of key k (0..31 of a step) in a V^T row: P^T gives lane group lq
// the keys 4*lq + i and 16 + 4*lq + i (i = 0..3) as its 8 B-operand slots.
__device__ __forceinline__ constexpr int vt_pos(int k) {
  return 8 * ((k & 15) >> 2) + 4 * (k >> 4) + (k & 3);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Max / sum of x over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane
// groups), with the lane-swap moves of gfx950.
__device__ __forceinline__ float group4_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS of one prefill workgroup: the ring of K steps (row-major) and V^T steps.
template <int D, int G>
struct PrefillSmem {
  using C = PrefillCfg<D, G>;
  __attribute__((aligned(16))) uint16_t Ks[kPrefillBufs][C::KSTEP * C::LROW];
  __attribute__((aligned(16))) uint16_t Vt[kPrefillBufs][D * C::VROW];
};

// One query tile `qtile` of sequence b, KV head g; called by the whole
// workgroup (kPrefillThreads threads).
template <int D, int G>
__device__ __forceinline__ void prefill_tile(
    PrefillSmem<D, G>& sm, uint16_t* __restrict__ out, float* __restrict__ lse_out,
    const uint16_t* __restrict__ query, const int* __restrict__ qsl,
    const uint16_t* __restrict__ cache, int num_blocks, const int* __restrict__ block_tables,
    int max_blocks_per_seq, const int* __restrict__ seq_lens, int max_seq_len, int num_kv_heads,
    float scale_log2, int b, int g, int qtile) {
  using C = PrefillCfg<D, G>;
  auto& Ks = sm.Ks;
  auto& Vt = sm.Vt;
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

  // ---- staging of one step's K and V (registers -> LDS).  K: thread tid
  // takes chunks tid, tid + 256, ... (row-major).  V: thread t takes chunk
  // vch of the key pair (2 vkp, 2 vkp + 1), so that it can write the pair's
  // values of each head dimension as one 32-bit word of V^T (with fewer
  // pairs than threads the others load a duplicate and store nothing).
  // Every load is issued unconditionally (block indices clamped to the last
  // block, V zeroed past the last visible key), so the loop's wait counts
  // stay exact.
  const int vsrc = tid % C::VPAIRS;
  const int vkp = vsrc % (C::KSTEP / 2), vch = vsrc / (C::KSTEP / 2);
  const bool vthread = tid < C::VPAIRS;
  // The step's two block ids (same in all lanes), read as vector buffer
  // loads: a scalar load would share its wait counter with the LDS reads.
  const __amdgpu_buffer_rsrc_t bt_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int*>(bt_row), 0, max_blocks_per_seq * 4, 0x00020000);
  auto step_ids = [&](int s) -> int2 {
    return make_int2(__builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, min(2 * s, nblk - 1) * 4, 0, 0),
                     __builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, min(2 * s + 1, nblk - 1) * 4, 0, 0));
  };
  auto block_ptr = [&](int id) -> const uint16_t* {
    id = __builtin_amdgcn_readfirstlane(id);
    id = (id < 0 || id >= num_blocks) ? 0 : id;  // out-of-range ids read block 0
    return cache + int64_t(id) * block_elems + int64_t(g) * tile_elems;
  };
  auto load_step = [&](int s, int2 ids, u32x4 (&kreg)[C::KLOADS], u32x4 (&vreg)[2])
      __attribute__((always_inline)) {
    const uint16_t* k0 = block_ptr(ids.x);
    const uint16_t* k1 = block_ptr(ids.y);
#pragma unroll
    for (int u = 0; u < C::KLOADS; ++u) {
      const int c = u * kPrefillThreads + tid;
      const int key = c / C::CH;
      const uint16_t* kt = key < 16 ? k0 : k1;
      kreg[u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kt + (key & 15) * D + (c % C::CH) * 8));
    }
    const int64_t vofs = int64_t(num_kv_heads) * tile_elems;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int key = 2 * vkp + e;
      const uint16_t* vt = (key < 16 ? k0 : k1) + vofs;
      const u32x4 vx = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(vt + (key & 15) * D + vch * 8));
      const bool in = s * C::KSTEP + key < kend;  // past kend: may be unwritten
      vreg[e] = u32x4{in ? vx.x : 0u, in ? vx.y : 0u, in ? vx.z : 0u, in ? vx.w : 0u};
    }
  };
  auto store_step = [&](int buf, const u32x4 (&kreg)[C::KLOADS], const u32x4 (&vreg)[2])
      __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < C::KLOADS; ++u) {
      const int c = u * kPrefillThreads + tid;
      *reinterpret_cast<u32x4*>(&Ks[buf][(c / C::CH) * C::LROW + (c % C::CH) * 8]) = kreg[u];
    }
    if (vthread) {
      uint32_t* vt = reinterpret_cast<uint32_t*>(&Vt[buf][vch * 8 * C::VROW + vt_pos(2 * vkp)]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // head dims 8 vch + 2w (low halves) and 8 vch + 2w + 1 (high halves)
        vt[(2 * w) * (C::VROW / 2)] = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x05040100u);
        vt[(2 * w + 1) * (C::VROW / 2)] = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x07060302u);
      }
    }
  };

  f32x4 acc[C::DT][C::NT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) acc[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[C::NT], m_thr[C::NT], l_part[C::NT];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) { m_run[nt] = -INFINITY; m_thr[nt] = -INFINITY; l_part[nt] = 0.f; }

  // smallest query position of this wave's active rows (rows are token-major);
  // steps from s_diag on reach it and need the causal mask
  const int wave_min_pos = ctx + t0 + (wave * C::RW) / G;
  const int s_diag = (wave_min_pos + 1) / C::KSTEP;

  // S^T = K Q^T for a step's two 16-key tiles, K from LDS buffer buf
  auto scores = [&](int buf, f32x4 (&sacc)[2][C::NT]) __attribute__((always_inline)) {
    u32x4 ka[2][C::DS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ds = 0; ds < C::DS; ++ds)
        ka[kt][ds] =
            *reinterpret_cast<const u32x4*>(&Ks[buf][(kt * 16 + lr) * C::LROW + ds * 32 + lq * 8]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) sacc[kt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) sacc[kt][nt] = mfma16x16x32(ka[kt][ds], qt[nt][ds], sacc[kt][nt]);
  };

  // online softmax of step s and O^T += V^T P^T with V from LDS buffer buf
  auto softmax_pv = [&](int s, const f32x4 (&sacc)[2][C::NT], int buf, auto mask_tag)
      __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // lane holds row lr of tile nt, keys kt*16 + 4*lq + i
    const int key0 = s * C::KSTEP;
    float x[C::NT][8];
    float mloc[C::NT];
    bool grow = false;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sacc[kt][nt][i];
          if constexpr (MASK) v = key0 + kt * 16 + lq * 4 + i <= row_pos[nt] ? v : -INFINITY;
          x[nt][kt * 4 + i] = v;
        }
      const float m = fmaxf(fmaxf(fmaxf(x[nt][0], x[nt][1]), fmaxf(x[nt][2], x[nt][3])),
                            fmaxf(fmaxf(x[nt][4], x[nt][5]), fmaxf(x[nt][6], x[nt][7])));
      mloc[nt] = group4_max(m) * scale_log2;   // scale > 0 keeps the order
      grow |= mloc[nt] > m_thr[nt];
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // wave-uniform, rare after the first step
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {
        if (mloc[nt] > m_thr[nt]) {
          const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - mloc[nt]);  // 0 on the first step
          m_run[nt] = mloc[nt];
          m_thr[nt] = mloc[nt] + kPrefillSlack;
          l_part[nt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) acc[dt][nt] *= alpha;
        }
      }
    }
    u32x4 pb[C::NT];   // P^T as the B operand: 8 bf16 keys of this lane's row
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      const float mref = m_run[nt] == -INFINITY ? 0.f : m_run[nt];  // rows with nothing visible
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[nt][e], scale_log2, -mref));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[nt][e + 1], scale_log2, -mref));
        pw[e / 2] = pack_bf16x2(p0, p1);
        l_part[nt] = dot2_bf16(pw[e / 2], 0x3F803F80u, l_part[nt]);
      }
      pb[nt] = u32x4{pw[0], pw[1], pw[2], pw[3]};
    }
    // lane (lq, lr) reads head dim dt*16 + lr at the eight V^T positions of
    // its P^T key slots
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const u32x4 va = *reinterpret_cast<const u32x4*>(&Vt[buf][(dt * 16 + lr) * C::VROW + lq * 8]);
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) acc[dt][nt] = mfma16x16x32(va, pb[nt], acc[dt][nt]);
    }
  };

  // Pipeline over a ring of three LDS buffers: while the VALU runs step s's
  // softmax, the MFMA pipe already computes step s + 1's scores; step s + 2's
  // K/V are loaded meanwhile and stored to the third buffer after it.  The
  // block ids of a step are loaded one step before its K/V, so no K/V load
  // waits on a table read.  Steps before s_diag run without the causal
  // mask, the rest with it (two loops: a branch between the variants inside
  // one loop costs registers); each iteration has one barrier, so every
  // wave meets the same barriers.
  u32x4 kreg[C::KLOADS], vreg[2];
  load_step(0, step_ids(0), kreg, vreg);
  store_step(0, kreg, vreg);
  load_step(1, step_ids(1), kreg, vreg);
  store_step(1, kreg, vreg);
  int2 ids_next = step_ids(2);
  __syncthreads();
  f32x4 s_cur[2][C::NT], s_next[2][C::NT];
  scores(0, s_cur);
  int b_cur = 0;  // LDS buffer of step s
  auto iteration = [&](int s, auto mask_tag) __attribute__((always_inline)) {
    const int b_next = b_cur == kPrefillBufs - 1 ? 0 : b_cur + 1;
    const int b_load = b_next == kPrefillBufs - 1 ? 0 : b_next + 1;
    const int2 ids = ids_next;
    ids_next = step_ids(s + 3);
    load_step(s + 2, ids, kreg, vreg);   // past the last step: clamped, never stored
    scores(b_next, s_next);              // past the last step: stale buffer, never used
    softmax_pv(s, s_cur, b_cur, mask_tag);
    if (s + 2 < nsteps) store_step(b_load, kreg, vreg);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) s_cur[kt][nt] = s_next[kt][nt];
    b_cur = b_next;
    __syncthreads();
  };
  int s = 0;
  for (const int sd = min(s_diag, nsteps); s < sd; ++s) iteration(s, std::false_type{});
  for (; s < nsteps; ++s) iteration(s, std::true_type{});

  // ---- normalise and write: lane holds O^T[dt*16 + 4*lq + i][row lr of tile nt]
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    const float l = group4_sum(l_part[nt]);
    if (row_pos[nt] < 0) continue;
    const int r = wave * C::RW + nt * 16 + lr;
    const int i = r / G, hh = r % G;
    const int64_t orow = int64_t(q0 + t0 + i) * H_q + g * G + hh;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const uint32_t w0 = pack_bf16x2(acc[dt][nt][0] * inv, acc[dt][nt][1] * inv);
      const uint32_t w1 = pack_bf16x2(acc[dt][nt][2] * inv, acc[dt][nt][3] * inv);
      *reinterpret_cast<uint2*>(out + orow * D + dt * 16 + lq * 4) = make_uint2(w0, w1);
    }
    if (lse_out && lq == 0) lse_out[orow] = l > 0.f ? m_run[nt] * kLn2P + logf(l) : -INFINITY;
  }
}

template <int D, int G>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_chunk_kernel(
    uint16_t* __restrict__ out, float* __restrict__ lse_out, const uint16_t* __restrict__ query,
    const int* __restrict__ qsl, const uint16_t* __restrict__ cache, int num_blocks,
    const int* __restrict__ block_tables, int max_blocks_per_seq, const int* __restrict__ seq_lens,
    int max_seq_len, int num_kv_heads, float scale_log2, int tiles, int num_groups) {
  __shared__ PrefillSmem<D, G> sm;
  // Workgroup -> (query tile, KV head g, sequence b).  The dispatcher hands
  // consecutive workgroups to the 8 XCDs in turn; when the (sequence, KV
  // head) groups split evenly over them, all query tiles of a group go to
  // one XCD, so they share the KV blocks they stream through that XCD's L2.
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
  prefill_tile<D, G>(sm, out, lse_out, query, qsl, cache, num_blocks, block_tables,
                     max_blocks_per_seq, seq_lens, max_seq_len, num_kv_heads, scale_log2, b, g,
                     qtile);
}

}  // namespace pa
