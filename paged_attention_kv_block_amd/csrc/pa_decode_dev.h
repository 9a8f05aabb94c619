// pa_decode device code: one query token per sequence attending to its
// paged KV cache, grouped-query heads, optional split-K over context
// partitions with a log-sum-exp reduce pass.
//
// What is computed ("Inside vLLM: Anatomy of a High-Throughput LLM Inference
// System", section "LLM Engine & Engine Core": paged attention over blocks
// that map tokens to their KV-cache blocks; the attention is the standard
// transformer's): for sequence b and query head h with KV head g = h / G,
//   s_t = scale * <q[b,h], K_b[t,g]>,  o = sum_t softmax(s)_t V_b[t,g],
//   lse = ln sum_t exp(s_t),  t = 0 .. seq_len[b]-1,
// with K_b[t] / V_b[t] read from physical block block_tables[b][t/16],
// offset t%16.  Paging only moves where keys/values live ("vLLM: Ein tiefer
// Einblick ...", section "Tiefenanalyse"), so results do not depend on the
// physical block ids: the arithmetic order below depends only on logical
// token positions.
//
// Design (gfx950, HBM-bound: 4-8 flop per byte of KV):
//   * one workgroup of NW waves (8, 4 or 2, fewer when there are many work
//     items) per work item = (partition, KV head, sequence), taken from a
//     host-built plan; the G query heads of a KV head share every K/V byte
//     loaded, so each byte of the cache is read from HBM once per call;
//   * wave w of the workgroup takes logical blocks w, w+NW, ... of its
//     partition and keeps its own online-softmax state; the states are
//     merged through LDS at the end; with split-K the last workgroup of a
//     (sequence, KV head) to finish merges the partitions' partials by
//     log-sum-exp weights in the same launch;
//   * each wave keeps two blocks in flight in registers (non-temporal
//     loads: the cache is streamed once); every load instruction covers
//     whole cache rows, because a compute unit streams at a rate set by the
//     cache lines it requests;
//   * scores are in the log2 domain and the softmax reference moves lazily
//     (only when a block's max exceeds it by 2^8), so most blocks need no
//     max reduction and no rescale of the accumulated output;
//   * bf16 (mfma_blocks): S^T = K Q^T and O += P V on the matrix cores;
//     K goes through a small LDS tile into operand order, the S^T result is
//     already the P operand, V is loaded in operand order; P is rounded to
//     bf16 for the product and the denominator sums the same rounded values;
//   * fp32 (valu_blocks): q.k with v_fma through the LDS K tile and a
//     cross-lane sum over d-parts, P through LDS, P.V with v_fma.
#pragma once

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "pa.h"
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// How far (in log2 units) a block's max may exceed the softmax reference
// before the reference moves; P then stays <= 2^8.
constexpr float kRescaleSlack = 8.f;

// Split-K partial of one (sequence, KV head, partition): the G heads'
// normalised outputs [G][D] in the cache's precision (bf16 or fp32), then
// their maxima [G] and denominators [G] in fp32 in a 128-byte line of their
// own.  One work item writes one contiguous record; writes into a
// read-saturated HBM cost far more than their bytes, so bf16 outputs are
// not widened.  Records are sized for fp32 outputs.
constexpr int64_t ws_record_bytes(int64_t G, int64_t D) { return G * D * 4 + 128; }

// Host side of split-K: partitions per sequence and the workspace layout.
inline int64_t parts_for(int max_seq_len, int partition_size) {
  if (partition_size <= 0 || max_seq_len <= 0) return 1;
  return (int64_t(max_seq_len) + partition_size - 1) / partition_size;
}

// Workspace layout:
//   [arrival counters: kCounterCap int32][records: B * H_kv * partitions]
// with one split-K record per (sequence, KV head, partition) (see
// ws_record_bytes).  Counter (b, g) sits at index
// b * H_kv + g of a region of fixed size, so calls of any shape can share
// one workspace without their partials overlapping another shape's
// counters.  Only the counters need a defined initial value (zero); every
// completed call leaves them at zero.
constexpr int64_t kCounterCap = 65536;
struct WsLayout {
  int64_t count_off, rec_off, total;
};
inline int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }
inline WsLayout ws_layout(int64_t B, int64_t H_q, int64_t H_kv, int64_t D, int64_t P) {
  WsLayout w{};
  w.count_off = 0;
  w.rec_off = round256(kCounterCap * 4);
  w.total = w.rec_off + B * H_kv * P * ws_record_bytes(H_q / H_kv, D);
  return w;
}


// Shapes of the fp32 block loop on the vector ALUs.  The K tile goes
// through LDS and is read back as (token, head group, d-part) per lane, so
// q.k needs a cross-lane sum over the d-parts only; for P.V each lane owns
// D / 64 output columns of every head.
template <int D, int G>
struct F32Cfg {
  static constexpr int RB = D * 4;                 // bytes per K/V row
  static constexpr int CPR = RB / 16;              // 16-byte chunks per row
  static constexpr int TILE_VEC = 16 * CPR;        // 16-byte vectors per tile
  static constexpr int LOADS = TILE_VEC / kWave;   // vector loads per lane per tile
  static constexpr int HG = G >= 4 ? 4 : G;        // head groups across lanes
  static constexpr int HPL = G / HG;               // heads per lane
  static constexpr int QCH_NEED = HPL * CPR;       // q chunks a lane would need with DP = 1
  static constexpr int DP_Q = QCH_NEED <= 8 ? 1 : QCH_NEED / 8;  // keep q <= 8 chunks (32 VGPRs)
  static constexpr int DP_MIN = 4 / HG;
  static constexpr int DP = DP_Q > DP_MIN ? DP_Q : DP_MIN;  // lanes sharing one token row
  static constexpr int TPP = kWave / (HG * DP);    // tokens per pass
  static constexpr int NPASS = 16 / TPP;
  static constexpr int CPL = CPR / DP;             // chunks per lane per row
  static constexpr int LDS_ROW = RB + 16;          // padded row (bank spread)
  static constexpr int LDS_TILE = 16 * LDS_ROW;
  static constexpr int DPL = D / kWave;            // output columns (= V dwords) per lane
  static constexpr int P_BYTES = G * 16 * 4;
  // K chunks (16 bytes each) read from LDS together
  static constexpr int KGRP_MAX = D == 64 ? 8 : (G >= 8 ? 2 : 4);
  static constexpr int KGRP = NPASS * CPL < KGRP_MAX ? NPASS * CPL : KGRP_MAX;
  static constexpr int PD = 2;                     // blocks in flight per wave (register ring)
  static_assert(DP >= HPL, "every head of a lane group needs a lane to follow it");
  static_assert((NPASS * CPL) % KGRP == 0, "read groups must tile");
  static_assert(CPR % DP == 0 && TPP >= 1 && 16 % TPP == 0, "bad decode lane split");
  static_assert(HG * DP * TPP == kWave, "lane split must cover the wave");
  static_assert(TILE_VEC % kWave == 0, "tile must be a whole number of wave loads");
};

// Agent-scope relaxed stores: coherent across the L2 caches of all XCDs,
// used for split-K partials.
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes of a decode workspace (raw buffer,
// 32-bit elements; reads past the end return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const float* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, 0x00020000);
}
constexpr int kSc1 = 16;  // cache policy bit sc1
__device__ __forceinline__ float ws_load(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kSc1));
}
__device__ __forceinline__ f32x4 ws_load4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kSc1));
}
// Four bf16 values (8 bytes) widened to fp32.
__device__ __forceinline__ f32x4 ws_load_bf16x4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t w = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, kSc1));
  return f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
}

template <bool BF16>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (BF16)
    reinterpret_cast<uint16_t*>(out)[idx] = uint16_t(f32_to_bf16_rne(v));
  else
    reinterpret_cast<float*>(out)[idx] = v;
}

// q.k partial over one 16-byte chunk (four fp32 values)
__device__ __forceinline__ float chunk_dot(const u32x4& q, const u32x4& k, float acc) {
  acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

// Registers of one block: the K tile as coalesced 16-byte vectors (lane i
// holds vectors i, i+64, ...) and this lane's V columns of all 16 rows.
// Each KV byte is read once per call, so the loads are non-temporal (they
// stream past the caches instead of displacing other lines).
template <class C>
struct BlockRegs {
  u32x4 k[C::LOADS];
  uint32_t v[16][C::DPL];
};

template <class C>
__device__ __forceinline__ BlockRegs<C> load_block_regs(const uint8_t* __restrict__ cache, int phys,
                                                        int64_t block_bytes, int g,
                                                        int num_kv_heads, int64_t tile_bytes,
                                                        int lane) {
  const uint8_t* kbase = cache + int64_t(phys) * block_bytes + int64_t(g) * tile_bytes;
  const uint8_t* vbase = kbase + int64_t(num_kv_heads) * tile_bytes;
  BlockRegs<C> r;
  const u32x4* kt = reinterpret_cast<const u32x4*>(kbase);
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) r.k[i] = __builtin_nontemporal_load(kt + i * kWave + lane);
  const uint32_t* vt = reinterpret_cast<const uint32_t*>(vbase);
#pragma unroll
  for (int row = 0; row < 16; ++row)
#pragma unroll
    for (int w = 0; w < C::DPL; ++w)
      r.v[row][w] = __builtin_nontemporal_load(vt + row * (C::RB / 4) + lane * C::DPL + w);
  return r;
}

// Online-softmax state of one wave.  Each lane follows one query head of
// its head group for the softmax (lanes dp and dp + HPL are replicas): the
// running reference m_run and the threshold m_run + slack (log2 domain),
// and its share of the denominator.  The unnormalised output columns cover
// all G heads.
template <class C, int G>
struct DecodeState {
  float m_run, m_thr, l;
  float o[G][C::DPL];
  __device__ __forceinline__ void init() {
    m_run = -INFINITY;
    m_thr = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < C::DPL; ++j) o[h][j] = 0.f;
  }
};

// Lane roles inside a wave.
struct LaneRoles {
  int dp;    // d-part of the QK split
  int tq;    // token within a QK pass
  int hg;    // head group
  int head;  // softmax head of this lane within the KV head's G query heads
};

// The stages of one 16-token block, in order:
//   block_scores   K tile through LDS, q.k of this lane's head and token(s);
//   block_softmax  lazily moved softmax reference, P to LDS;
//   pv_rescale     o *= alpha when the block moved the reference;
//   pv_accumulate  P of each head from LDS, P.V into the lane's columns.
// TAIL: only the first `valid` tokens of the block are inside the sequence
// (1 <= valid <= 16).

// Scores (log2 domain) of this lane's head for its token of each pass.
template <int D, int G, bool TAIL>
__device__ __forceinline__ void block_scores(const BlockRegs<F32Cfg<D, G>>& cur, int valid,
                                             const u32x4 (&q)[F32Cfg<D, G>::HPL]
                                                             [F32Cfg<D, G>::CPL],
                                             uint8_t* kt_lds, float scale_log2, const LaneRoles& r,
                                             float (&x)[F32Cfg<D, G>::NPASS]) {
  using C = F32Cfg<D, G>;
  const int lane = threadIdx.x & (kWave - 1);

  // K tile -> LDS (padded rows)
  wave_lds_sync();  // previous block's reads of the tile are done
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int v = i * kWave + lane;
    const int row = v / C::CPR, ch = v % C::CPR;
    *reinterpret_cast<u32x4*>(kt_lds + row * C::LDS_ROW + ch * 16) = cur.k[i];
  }
  wave_lds_sync();

  // K chunks are read from LDS in groups of KGRP (registers permitting) so
  // that the reads of a group overlap one another
  float sacc[C::NPASS][C::HPL];
#pragma unroll
  for (int ps = 0; ps < C::NPASS; ++ps)
#pragma unroll
    for (int hh = 0; hh < C::HPL; ++hh) sacc[ps][hh] = 0.f;
  constexpr int NCH = C::NPASS * C::CPL;
#pragma unroll
  for (int base = 0; base < NCH; base += C::KGRP) {
    u32x4 kv[C::KGRP];
#pragma unroll
    for (int i = 0; i < C::KGRP; ++i) {
      const int ps = (base + i) / C::CPL, c = (base + i) % C::CPL;
      kv[i] = reinterpret_cast<const u32x4*>(kt_lds + (ps * C::TPP + r.tq) * C::LDS_ROW)[r.dp * C::CPL + c];
    }
#pragma unroll
    for (int i = 0; i < C::KGRP; ++i) {
      const int ps = (base + i) / C::CPL, c = (base + i) % C::CPL;
#pragma unroll
      for (int hh = 0; hh < C::HPL; ++hh) sacc[ps][hh] = chunk_dot(q[hh][c], kv[i], sacc[ps][hh]);
    }
  }
#pragma unroll
  for (int ps = 0; ps < C::NPASS; ++ps) {
    const int row = ps * C::TPP + r.tq;
    const float (&s)[C::HPL] = sacc[ps];
    float v = allreduce_sum<0, ilog2(C::DP)>(s[0]);
#pragma unroll
    for (int hh = 1; hh < C::HPL; ++hh) {
      const float w = allreduce_sum<0, ilog2(C::DP)>(s[hh]);
      v = (r.dp % C::HPL) == hh ? w : v;
    }
    v *= scale_log2;
    if constexpr (TAIL) v = row < valid ? v : -INFINITY;
    x[ps] = v;
  }
}

// Online softmax with a lazily moved reference: m_run moves only when the
// block's max exceeds it by more than kRescaleSlack (log2 units), so
// P = 2^(s - m_run) <= 2^kRescaleSlack and most blocks neither reduce their
// max across lanes nor rescale the accumulated output.  Writes P to LDS
// ([head][token]; replica lanes store the same value to the same word) and,
// when the reference moved, each
// head's alpha; returns whether it moved (wave-uniform).  The caller orders
// the P stores after any earlier reads of P (wave_lds_sync).
template <int D, int G>
__device__ __forceinline__ bool block_softmax(const float (&x)[F32Cfg<D, G>::NPASS],
                                              DecodeState<F32Cfg<D, G>, G>& st,
                                              uint32_t* p_lds, float* alpha_lds, const LaneRoles& r) {
  using C = F32Cfg<D, G>;
  float t = x[0];
#pragma unroll
  for (int ps = 1; ps < C::NPASS; ++ps) t = fmaxf(t, x[ps]);
  const bool rescale = __builtin_amdgcn_ballot_w64(t > st.m_thr) != 0;  // wave-uniform
  if (rescale) {
    // lanes of other d-parts follow other heads: exact xor partners
    const float mb = allreduce_max_xor<ilog2(C::DP), ilog2(C::DP * C::TPP)>(t);
    // mb is finite: token 0 of the block is inside the sequence
    const bool grow = mb > st.m_thr;
    const float alpha = grow ? __builtin_amdgcn_exp2f(st.m_run - mb) : 1.f;
    st.m_run = grow ? mb : st.m_run;
    st.m_thr = st.m_run + kRescaleSlack;
    st.l *= alpha;
    if (r.tq == 0 && r.dp < C::HPL) alpha_lds[r.head] = alpha;
  }
  float* pf = reinterpret_cast<float*>(p_lds);
#pragma unroll
  for (int ps = 0; ps < C::NPASS; ++ps) {
    const float p = __builtin_amdgcn_exp2f(x[ps] - st.m_run);
    st.l += p;
    pf[r.head * 16 + ps * C::TPP + r.tq] = p;
  }
  return rescale;
}

template <int D, int G>
__device__ __forceinline__ void pv_rescale(bool rescale, DecodeState<F32Cfg<D, G>, G>& st,
                                           const float* alpha_lds) {
  using C = F32Cfg<D, G>;
  if (rescale) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float a = alpha_lds[h];
#pragma unroll
      for (int jj = 0; jj < C::DPL; ++jj) st.o[h][jj] *= a;
    }
  }
}

// Rows past the sequence may hold anything: zero them in a tail block.
template <int D, int G>
__device__ __forceinline__ void mask_tail_rows(BlockRegs<F32Cfg<D, G>>& cur, int valid) {
  using C = F32Cfg<D, G>;
#pragma unroll
  for (int row = 0; row < 16; ++row)
#pragma unroll
    for (int w = 0; w < C::DPL; ++w) cur.v[row][w] = row < valid ? cur.v[row][w] : 0u;
}

// P.V: each head's 16 P values are read from LDS (four 16-byte reads, the
// same words for every lane) and multiply the lane's V columns.
template <int D, int G>
__device__ __forceinline__ void pv_accumulate(const BlockRegs<F32Cfg<D, G>>& cur,
                                              const uint32_t* p_lds,
                                              DecodeState<F32Cfg<D, G>, G>& st) {
  using C = F32Cfg<D, G>;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float p[16];
#pragma unroll
    for (int k4 = 0; k4 < 16; k4 += 4) {
      const u32x4 t4 = *reinterpret_cast<const u32x4*>(p_lds + h * 16 + k4);
      p[k4] = __uint_as_float(t4.x);
      p[k4 + 1] = __uint_as_float(t4.y);
      p[k4 + 2] = __uint_as_float(t4.z);
      p[k4 + 3] = __uint_as_float(t4.w);
    }
#pragma unroll
    for (int row = 0; row < 16; ++row)
#pragma unroll
      for (int w = 0; w < C::DPL; ++w) st.o[h][w] = fmaf(p[row], __uint_as_float(cur.v[row][w]), st.o[h][w]);
  }
}

// One block, stage after stage.
template <int D, int G, bool TAIL>
__device__ __forceinline__ void process_block(BlockRegs<F32Cfg<D, G>>& cur, int valid,
                                            const u32x4 (&q)[F32Cfg<D, G>::HPL]
                                                            [F32Cfg<D, G>::CPL],
                                            DecodeState<F32Cfg<D, G>, G>& st,
                                            uint8_t* kt_lds, uint32_t* p_lds, float* alpha_lds,
                                            float scale_log2, const LaneRoles& r) {
  using C = F32Cfg<D, G>;
  float x[C::NPASS];
  block_scores<D, G, TAIL>(cur, valid, q, kt_lds, scale_log2, r, x);
  const bool rescale = block_softmax<D, G>(x, st, p_lds, alpha_lds, r);
  wave_lds_sync();
  if constexpr (TAIL) mask_tail_rows<D, G>(cur, valid);
  pv_rescale<D, G>(rescale, st, alpha_lds);
  pv_accumulate<D, G>(cur, p_lds, st);
}

// Arguments of one decode launch (passed by value as the kernel argument).
struct DecodeParams {
  void* out;
  float* lse_out;
  const void* query;
  const uint8_t* cache;
  const int* block_tables;
  const int* seq_lens;
  const int* plan;        // (part << 16 | b) entries, or nullptr: virtual grid
  int* ws_count;
  uint8_t* ws_rec;        // split-K records, [b * H_kv + g][max_parts]
  const void* new_k;      // append mode: the new token's K/V per sequence, [B][H_kv][D];
  const void* new_v;      // nullptr: the cache already holds token L - 1
  int num_blocks, max_blocks_per_seq, max_seq_len, num_kv_heads, B;
  int part_blocks, max_parts, num_items;
  float scale_log2;       // scale * log2(e), times the key scale for an FP8 cache
  float k_scale, v_scale;  // FP8 cache: key / value scales
  // Several query rows per sequence (the multi-row kernel variant only):
  // sequence b's `rows` query rows are its last `rows` tokens, packed at
  // rows b * rows ...; a work item covers `rows_per_group` of them for the
  // `group` query heads of one KV head (columns = (row, head) pairs); there
  // are col_groups items per (sequence, KV head, partition), and
  // items_per_group items (plan entries or virtual (b, part)) per column group.
  int rows, group, rows_per_group, col_groups, items_per_group;
  // 1: split items only write their records, and a second launch
  // (merge_kernel) merges them; 0: the last item of a slot to finish merges
  int defer_merge;
};

// Append mode: the new token (position L - 1 of sequence b, KV head g)
// replaces its row of the block held in registers and is stored to the
// cache at the same place, so the call equals pa_reshape_and_cache of the
// token followed by pa_decode.  A block id out of range is read as block 0
// and not written.
template <class C>
__device__ __forceinline__ void append_new_token(BlockRegs<C>& rg, const DecodeParams& a, int b,
                                                 int g, int row, int phys, int64_t block_bytes,
                                                 int64_t tile_bytes, int lane) {
  const int64_t src = (int64_t(b) * a.num_kv_heads + g) * C::RB;
  const bool store = phys >= 0 && phys < a.num_blocks;
  uint8_t* kbase = const_cast<uint8_t*>(a.cache) + int64_t(store ? phys : 0) * block_bytes +
                   int64_t(g) * tile_bytes;
  uint8_t* vbase = kbase + int64_t(a.num_kv_heads) * tile_bytes;
  const u32x4* nk = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.new_k) + src);
  const uint32_t* nv = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(a.new_v) + src);
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int v = i * kWave + lane;
    if (v / C::CPR == row) {
      const u32x4 x = nk[v % C::CPR];
      rg.k[i] = x;
      if (store) reinterpret_cast<u32x4*>(kbase)[v] = x;
    }
  }
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    if (rr == row) {
#pragma unroll
      for (int w = 0; w < C::DPL; ++w) {
        const uint32_t x = nv[lane * C::DPL + w];
        rg.v[rr][w] = x;
        if (store) reinterpret_cast<uint32_t*>(vbase)[row * (C::RB / 4) + lane * C::DPL + w] = x;
      }
    }
  }
}

// Shapes of the bf16 (matrix-core) block loop; see mfma_blocks.
// KV8: the cache holds FP8 E4M3 codes (converted to bf16 operands, exactly).
template <int D, bool KV8 = false>
struct MfmaCfg {
  static_assert(D == 64 || D == 128, "head size");
  static constexpr int EB = KV8 ? 1 : 2;  // bytes of a cache element
  static constexpr int KS = D / 32;   // S^T products per block
  static constexpr int NPV = D / 16;  // P V products per block (16 columns each)
  static constexpr int RB = EB * D;   // bytes of a cache row
  static constexpr int CPR = RB / 16;  // 16-byte chunks per row
  static constexpr int KLD = RB / 64;  // 16-byte vectors of the K tile per lane
  static constexpr int VWD = RB / 64;  // dwords of a V row per lane (16 lanes per row)
  static constexpr int LROW = RB + 16;  // padded LDS row: conflict-free operand reads
  static constexpr int TILE = 16 * LROW;
  static constexpr int PD = 2;        // blocks in flight per wave
};

// LDS of one workgroup: K tiles during the block loop, then the per-wave
// outputs, the merge weights and the split-K subset sums; fp32 P (the bf16
// loop keeps P in registers); and the merge state.
template <int D, int G, bool BF16, int NW, bool KV8 = false>
struct DecodeSmem {
  using C = F32Cfg<D, G>;
  static constexpr int kTiles = NW * (BF16 ? MfmaCfg<D, KV8>::TILE : C::LDS_TILE);
  static constexpr int kOStage = NW * G * D * 4;
  static constexpr int kSubsets = NW * kWave * 16;
  static constexpr int kBytes = std::max(kTiles, std::max(kOStage, kSubsets));
  __attribute__((aligned(16))) uint8_t k[kBytes];
  __attribute__((aligned(16))) uint32_t p[BF16 ? 1 : NW][BF16 ? 1 : C::P_BYTES / 4];
  float alpha[NW][G];
  float m[NW][G];
  float l[NW][G];
  float M[G], W[G];
  int last;
};

// ---------------------------------------------------------------------------
// bf16 blocks on the matrix cores.  Per 16-token block of one KV head, a
// wave forms S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (rows: the block's
// tokens; columns: the G query heads, padded to 16 with zero queries;
// contraction over D, 32 at a time) and accumulates O += P V with
// v_mfma_f32_16x16x16_bf16 (rows: heads; columns: 16 output columns;
// contraction over the block's 16 tokens).  With lane = 16 * grp + n:
//   * K operand: token n, 16-byte d-chunk 4 * s + grp of product s.  The K
//     tile is loaded coalesced (each load instruction covers whole rows: a
//     compute unit streams at a rate set by the cache lines it requests, and
//     the operand layout would split every line between two requests),
//     written to a padded per-wave LDS tile and read back in operand layout;
//     the Q^T operand holds the same chunk of query head n;
//   * the S^T result gives the lane tokens 4 * grp + i (i < 4) of head n,
//     which is exactly where P V wants P (row n, contraction slots i), so
//     the softmax runs in place and P never leaves the registers;
//   * V operand: the same four tokens at output column 2 * (VWD * n + w) + hb,
//     built with v_perm from the lane's dwords of those rows (16 lanes read a
//     whole row as one coalesced segment);
//   * the O result holds heads 4 * grp + i at columns (D / 16) * n + p.
// P and V never touch LDS; the softmax reference moves lazily as in the
// fp32 path, now one head per lane column n.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));


// K: lane holds 16-byte vectors lane + 64 j of the tile (D / 32 of them);
// V: operand layout (rows 4 grp + i, dwords VWD n ..).
template <int D, bool KV8 = false>
struct MfmaBlock {
  u32x4 k[MfmaCfg<D, KV8>::KLD];
  uint32_t v[4][MfmaCfg<D, KV8>::VWD];
};

template <int D>
struct MfmaState {
  float m_run, m_thr, l;  // head n's reference, threshold; this lane's share of l
  f32x4 o[MfmaCfg<D>::NPV];
};

__device__ __forceinline__ f32x4 mfma_k32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_k16(const u32x2& a, const u32x2& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Two FP8 E4M3 codes (bytes 0-1, or 2-3 when `hi`) as a bf16 pair, element
// 0 in the low half.  E4M3 values are exact in bf16 (3 mantissa bits,
// exponents 2^-9 .. 2^8), and the scale here is 1.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Loads of one block's K and V operands: non-temporal when the cache is
// streamed once per call (NT); ordinary loads when other workgroups on the
// same XCD read the same blocks at about the same time (the column groups
// of a multi-row item), so the lines stay in that XCD's L2 for them.
// (A compile-time choice: a select between the two loads of one address
// is folded into a single load without the non-temporal hint.)
template <bool NT, class T>
__device__ __forceinline__ T kv_load(const T* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}
template <int D, bool KV8 = false, bool NT = true>
__device__ __forceinline__ MfmaBlock<D, KV8> load_mfma_block(const uint8_t* __restrict__ cache,
                                                             int phys, int64_t block_bytes, int g,
                                                             int num_kv_heads, int64_t tile_bytes,
                                                             int lane) {
  using M = MfmaCfg<D, KV8>;
  const uint8_t* kbase = cache + int64_t(phys) * block_bytes + int64_t(g) * tile_bytes;
  const uint8_t* vbase = kbase + int64_t(num_kv_heads) * tile_bytes;
  const int n = lane & 15, grp = lane >> 4;
  MfmaBlock<D, KV8> r;
  const u32x4* kt = reinterpret_cast<const u32x4*>(kbase);
#pragma unroll
  for (int j = 0; j < M::KLD; ++j) r.k[j] = kv_load<NT>(kt + j * kWave + lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t* vp = vbase + (4 * grp + i) * M::RB + n * (M::VWD * 4);
    if constexpr (M::VWD == 1) {
      r.v[i][0] = kv_load<NT>(reinterpret_cast<const uint32_t*>(vp));
    } else if constexpr (M::VWD == 2) {
      const u32x2 x = kv_load<NT>(reinterpret_cast<const u32x2*>(vp));
      r.v[i][0] = x.x;
      r.v[i][1] = x.y;
    } else {
      const u32x4 x = kv_load<NT>(reinterpret_cast<const u32x4*>(vp));
      r.v[i][0] = x.x;
      r.v[i][1] = x.y;
      r.v[i][2] = x.z;
      r.v[i][3] = x.w;
    }
  }
  return r;
}

// Token `row` of the registers of the sequence's last block becomes the new
// key/value (new_k / new_v row (b, g)), which is also stored to the cache
// (skipped when the block id is out of range).
template <int D>
__device__ __forceinline__ void append_new_token_mfma(MfmaBlock<D>& rg, const DecodeParams& a,
                                                      int b, int g, int row, int phys,
                                                      int64_t block_bytes, int64_t tile_bytes,
                                                      int lane) {
  using M = MfmaCfg<D>;
  const int64_t src = (int64_t(b) * a.num_kv_heads + g) * M::RB;
  const bool store = phys >= 0 && phys < a.num_blocks;
  uint8_t* kbase = const_cast<uint8_t*>(a.cache) + int64_t(store ? phys : 0) * block_bytes +
                   int64_t(g) * tile_bytes;
  uint8_t* vbase = kbase + int64_t(a.num_kv_heads) * tile_bytes;
  const uint8_t* nk = static_cast<const uint8_t*>(a.new_k) + src;
  const uint8_t* nv = static_cast<const uint8_t*>(a.new_v) + src;
  const int n = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int j = 0; j < M::KS; ++j) {
    const int v = j * kWave + lane;
    if (v / M::CPR == row) {
      const u32x4 x = reinterpret_cast<const u32x4*>(nk)[v % M::CPR];
      rg.k[j] = x;
      if (store) reinterpret_cast<u32x4*>(kbase)[v] = x;
    }
  }
  const int off = n * (M::VWD * 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (4 * grp + i == row) {
#pragma unroll
      for (int w = 0; w < M::VWD; ++w) {
        const uint32_t x = reinterpret_cast<const uint32_t*>(nv + off)[w];
        rg.v[i][w] = x;
        if (store) reinterpret_cast<uint32_t*>(vbase + row * M::RB + off)[w] = x;
      }
    }
  }
}

// The same for an FP8 cache: the new bf16 key/value row is quantised with
// the key/value scale (quantize4_e4m3, as pa_reshape_and_cache_fp8 does)
// into the registers and the cache.
template <int D>
__device__ __forceinline__ void append_new_token_fp8(MfmaBlock<D, true>& rg,
                                                     const DecodeParams& a, int b, int g, int row,
                                                     int phys, int64_t block_bytes,
                                                     int64_t tile_bytes, int lane) {
  using M = MfmaCfg<D, true>;
  const int64_t src = (int64_t(b) * a.num_kv_heads + g) * (2 * D);  // bf16 input rows
  const bool store = phys >= 0 && phys < a.num_blocks;
  uint8_t* kbase = const_cast<uint8_t*>(a.cache) + int64_t(store ? phys : 0) * block_bytes +
                   int64_t(g) * tile_bytes;
  uint8_t* vbase = kbase + int64_t(a.num_kv_heads) * tile_bytes;
  const uint8_t* nk = static_cast<const uint8_t*>(a.new_k) + src;
  const uint8_t* nv = static_cast<const uint8_t*>(a.new_v) + src;
  const int n = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int j = 0; j < M::KLD; ++j) {
    const int v = j * kWave + lane;  // 16 codes: elements 16 c .. 16 c + 15 of row v / CPR
    if (v / M::CPR == row) {
      const u32x4* in = reinterpret_cast<const u32x4*>(nk) + 2 * (v % M::CPR);
      const u32x4 x0 = in[0], x1 = in[1];
      const u32x4 c = {quantize4_e4m3(x0.x, x0.y, a.k_scale), quantize4_e4m3(x0.z, x0.w, a.k_scale),
                       quantize4_e4m3(x1.x, x1.y, a.k_scale), quantize4_e4m3(x1.z, x1.w, a.k_scale)};
      rg.k[j] = c;
      if (store) reinterpret_cast<u32x4*>(kbase)[v] = c;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (4 * grp + i == row) {
#pragma unroll
      for (int w = 0; w < M::VWD; ++w) {
        const int dw = M::VWD * n + w;  // dword of the row: elements 4 dw .. 4 dw + 3
        const u32x2 x = reinterpret_cast<const u32x2*>(nv)[dw];
        const uint32_t c = quantize4_e4m3(x.x, x.y, a.v_scale);
        rg.v[i][w] = c;
        if (store) reinterpret_cast<uint32_t*>(vbase + row * M::RB)[dw] = c;
      }
    }
  }
}

// One block.  TAIL: only the first `valid` tokens (1 <= valid <= 16) are in
// the sequence; the others get score -inf and their V rows are zeroed (they
// may hold anything).
// MULTI: lane column n of tile c sees the block's tokens below lim[c] (its
// own causal limit, relative to the block's first token; may be <= 0 or
// >= 16).  CT tiles of 16 columns share the K operand and the V operand.
template <int D, bool TAIL, bool KV8 = false, bool MULTI = false, int CT = 1>
__device__ __forceinline__ void mfma_block(MfmaBlock<D, KV8>& cur, int valid,
                                           const u32x4 (&qbt)[CT][MfmaCfg<D>::KS],
                                           MfmaState<D> (&stt)[CT], uint8_t* kt_lds,
                                           float scale_log2, int lane, const int (&lim)[CT]) {
  using M = MfmaCfg<D, KV8>;
  const int n = lane & 15, grp = lane >> 4;
  // K tile -> LDS -> operand layout
  wave_lds_sync();  // the previous block's operand reads are done
#pragma unroll
  for (int j = 0; j < M::KLD; ++j) {
    const int v = j * kWave + lane;
    *reinterpret_cast<u32x4*>(kt_lds + (v / M::CPR) * M::LROW + (v % M::CPR) * 16) = cur.k[j];
  }
  wave_lds_sync();
  u32x4 ka[M::KS];
#pragma unroll
  for (int s = 0; s < M::KS; ++s) {
    // 8 elements of token n, d-chunk 4 s + grp
    const uint8_t* src = kt_lds + n * M::LROW + (4 * s + grp) * 8 * M::EB;
    if constexpr (KV8) {
      const u32x2 c = *reinterpret_cast<const u32x2*>(src);
      ka[s] = u32x4{fp8x2_to_bf16x2<false>(c.x), fp8x2_to_bf16x2<true>(c.x),
                    fp8x2_to_bf16x2<false>(c.y), fp8x2_to_bf16x2<true>(c.y)};
    } else {
      ka[s] = *reinterpret_cast<const u32x4*>(src);
    }
  }
  u32x2 pat[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
  const u32x4 (&qb)[MfmaCfg<D>::KS] = qbt[c];
  MfmaState<D>& st = stt[c];
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < M::KS; ++s) sc = mfma_k32(ka[s], qb[s], sc);
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = sc[i] * scale_log2;
    if constexpr (TAIL) v = 4 * grp + i < valid ? v : -INFINITY;
    if constexpr (MULTI) v = 4 * grp + i < lim[c] ? v : -INFINITY;
    x[i] = v;
  }
  const float t = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  if (__builtin_amdgcn_ballot_w64(t > st.m_thr) != 0) {  // wave-uniform
    // max over the head's 16 tokens (lanes n, n + 16, n + 32, n + 48); it
    // is finite: token 0 of the block is in the sequence (MULTI: a column
    // may see none of the block; its reference then starts at a finite
    // -1e30, so the block's weights are exp2(-inf) = 0, never NaN)
    const float mb = allreduce_max_xor<4, 6>(t);
    const bool grow = mb > st.m_thr;
    const float alpha = grow ? __builtin_amdgcn_exp2f(st.m_run - mb) : 1.f;
    st.m_run = grow ? mb : st.m_run;
    st.m_thr = st.m_run + kRescaleSlack;
    st.l *= alpha;
    // output rows are heads 4 * grp + i; lane 4 * grp + i holds their alpha
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(alpha, 4 * grp + i, kWave);
#pragma unroll
      for (int p = 0; p < M::NPV; ++p) st.o[p][i] *= ai;
    }
  }
  u32x2 pa;
  pa.x = pack_bf16x2(__builtin_amdgcn_exp2f(x[0] - st.m_run), __builtin_amdgcn_exp2f(x[1] - st.m_run));
  pa.y = pack_bf16x2(__builtin_amdgcn_exp2f(x[2] - st.m_run), __builtin_amdgcn_exp2f(x[3] - st.m_run));
  st.l = dot2_bf16(pa.x, 0x3F803F80u, st.l);  // the rounded values that multiply V
  st.l = dot2_bf16(pa.y, 0x3F803F80u, st.l);
  pat[c] = pa;
  }  // column tiles
  if constexpr (TAIL) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int w = 0; w < M::VWD; ++w) cur.v[i][w] = 4 * grp + i < valid ? cur.v[i][w] : 0u;
  }
  if constexpr (KV8) {
    // dword w of a row holds output columns 4 (VWD n + w) + c, c < 4: bytes
    // c of the four rows pair up with v_perm and widen to bf16 pairs
#pragma unroll
    for (int w = 0; w < M::VWD; ++w) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {  // columns (2 c2, 2 c2 + 1)
        const uint32_t sel = c2 ? 0x07030602u : 0x05010400u;
        const uint32_t t01 = __builtin_amdgcn_perm(cur.v[1][w], cur.v[0][w], sel);
        const uint32_t t23 = __builtin_amdgcn_perm(cur.v[3][w], cur.v[2][w], sel);
        const int p = 4 * w + 2 * c2;
        const u32x2 vlo = {fp8x2_to_bf16x2<false>(t01), fp8x2_to_bf16x2<false>(t23)};
        const u32x2 vhi = {fp8x2_to_bf16x2<true>(t01), fp8x2_to_bf16x2<true>(t23)};
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          stt[c].o[p] = mfma_k16(pat[c], vlo, stt[c].o[p]);
          stt[c].o[p + 1] = mfma_k16(pat[c], vhi, stt[c].o[p + 1]);
        }
      }
    }
  } else {
#pragma unroll
    for (int w = 0; w < M::VWD; ++w) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const uint32_t sel = hb ? 0x07060302u : 0x05040100u;  // high or low bf16 of each dword
        u32x2 vb;
        vb.x = __builtin_amdgcn_perm(cur.v[1][w], cur.v[0][w], sel);  // tokens 4 grp + 0, + 1
        vb.y = __builtin_amdgcn_perm(cur.v[3][w], cur.v[2][w], sel);  // tokens 4 grp + 2, + 3
#pragma unroll
        for (int c = 0; c < CT; ++c)
          stt[c].o[2 * w + hb] = mfma_k16(pat[c], vb, stt[c].o[2 * w + hb]);
      }
    }
  }
}

// The bf16 block loop of one wave, then its (m, l) into sm.m / sm.l and its
// unnormalised output rows into the LDS output stage; synchronises the
// workgroup.
// MULTI: column n is query row qrow + n / a.group, head g * a.group + n %
// a.group, for n < ncols; that row sits at position L - rows + row_in_seq
// (rows: the sequence's query rows) and sees the tokens up to it.
// SHARED: ordinary (L2-allocating) loads, see load_mfma_block.
template <int D, int G, int NW, bool APPEND, bool KV8 = false, bool MULTI = false,
          bool SHARED = false>
__device__ __forceinline__ void mfma_blocks(const DecodeParams& a,
                                            DecodeSmem<D, G, true, NW, KV8>& sm, int b, int qrow,
                                            int g, int L, int nblk, int blk_lo, int blk_hi,
                                            int row0 = 0, int ncols = G, int rows = 1) {
  using M = MfmaCfg<D, KV8>;
  // columns in tiles of 16: G = 32 (multi-row items at head size 64) uses two
  constexpr int CT = G > 16 ? 2 : 1;
  static_assert(G <= 16 * CT && CT <= 2, "query heads per KV head");
  const uint8_t* __restrict__ cache = a.cache;
  const int num_blocks = a.num_blocks, num_kv_heads = a.num_kv_heads;
  const float scale_log2 = a.scale_log2;
  const int H_q = num_kv_heads * G;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, grp = lane >> 4;

  // Q^T operand: head n of this KV head (zero past G), d-chunks 4 s + grp
  u32x4 qb[CT][M::KS];
  int lim[CT];  // MULTI: this lane column's causal limit (exclusive), per tile
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int nc = n + 16 * c;  // the column this lane follows in tile c
    lim[c] = L;
    int64_t qoff;
    bool qvalid;
    if constexpr (MULTI) {
      const int gr = a.group;
      const int nn = nc < ncols ? nc : 0;
      qoff = (int64_t(qrow + nn / gr) * (num_kv_heads * gr) + g * gr + nn % gr) * (D / 8);
      qvalid = nc < ncols;
      if (qvalid) lim[c] = L - rows + row0 + nc / gr + 1;
    } else {
      qoff = (int64_t(qrow) * H_q + g * G + (nc < G ? nc : 0)) * (D / 8);
      qvalid = nc < G;
    }
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.query) + qoff;
#pragma unroll
    for (int s = 0; s < M::KS; ++s) {
      const u32x4 v = qp[4 * s + grp];
      qb[c][s] = qvalid ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const int64_t tile_bytes = int64_t(16) * M::RB;
  const int64_t block_bytes = int64_t(2) * num_kv_heads * tile_bytes;
  const int* bt_row = a.block_tables + int64_t(b) * a.max_blocks_per_seq;

  uint8_t* kt_lds = sm.k + wave * M::TILE;
  MfmaState<D> st[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    st[c].m_run = MULTI ? -1e30f : -INFINITY;
    st[c].m_thr = MULTI ? -1e30f : -INFINITY;
    st[c].l = 0.f;
#pragma unroll
    for (int p = 0; p < M::NPV; ++p) st[c].o[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Register ring of PD blocks in flight, block ids one group ahead; the
  // same scheme as the fp32 loop (see there).
  constexpr int PD = M::PD;
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int s = 0; s < M::KS; ++s) asm volatile("" ::"v"(qb[c][s]));
  const int first = blk_lo + wave;
  const int nmine = blk_hi > first ? (blk_hi - first + NW - 1) / NW : 0;
  if (nmine > 0) {
    auto id_group = [&](int base) -> int {
      const int k = min(base + (lane & (PD - 1)), nmine - 1);
      int id = bt_row[first + k * NW];
      return (id < 0 || id >= num_blocks) ? 0 : id;  // out-of-range ids read block 0
    };
    const int ids_cur = id_group(0);
    int ids_next = id_group(PD);
    MfmaBlock<D, KV8> buf[PD];
#pragma unroll
    for (int s = 0; s < PD; ++s)
      buf[s] = load_mfma_block<D, KV8, !SHARED>(cache, __builtin_amdgcn_readlane(ids_cur, s), block_bytes,
                                       g, num_kv_heads, tile_bytes, lane);
    const int j_last = first + (nmine - 1) * NW;
    const int tail_valid = L - j_last * 16;
    const bool seq_last = APPEND && j_last == nblk - 1;
    const int nfull = (tail_valid < 16 || seq_last) ? nmine - 1 : nmine;
    for (int k0 = 0; k0 < nfull; k0 += PD) {
      const int ids_after = id_group(k0 + 2 * PD);
#pragma unroll
      for (int s = 0; s < PD; ++s) {
        if (k0 + s < nfull)
        {
          int lr[CT];
#pragma unroll
          for (int c = 0; c < CT; ++c) lr[c] = lim[c] - 16 * (first + (k0 + s) * NW);
          mfma_block<D, false, KV8, MULTI, CT>(buf[s], 16, qb, st, kt_lds, scale_log2, lane, lr);
        }
        buf[s] = load_mfma_block<D, KV8, !SHARED>(cache, __builtin_amdgcn_readlane(ids_next, s),
                                         block_bytes, g, num_kv_heads, tile_bytes, lane);
      }
      ids_next = ids_after;
    }
    if (nfull < nmine) {  // buf[0] holds the last block (later loads were clamped to it)
      if constexpr (APPEND) {
        if (seq_last) {
          if constexpr (KV8)
            append_new_token_fp8<D>(buf[0], a, b, g, (L - 1) & 15, bt_row[nblk - 1],
                                    block_bytes, tile_bytes, lane);
          else
            append_new_token_mfma<D>(buf[0], a, b, g, (L - 1) & 15, bt_row[nblk - 1],
                                     block_bytes, tile_bytes, lane);
        }
      }
      int lr[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) lr[c] = lim[c] - 16 * j_last;
      mfma_block<D, true, KV8, MULTI, CT>(buf[0], min(tail_valid, 16), qb, st, kt_lds,
                                          scale_log2, lane, lr);
    }
  }

  if constexpr (KV8) {  // values are codes times v_scale
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int p = 0; p < M::NPV; ++p) st[c].o[p] *= a.v_scale;
  }
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const float lsum = allreduce_sum<4, 6>(st[c].l);  // over the head's four lanes
    if (lane < 16 && lane + 16 * c < G) {
      sm.m[wave][lane + 16 * c] = st[c].m_run;
      sm.l[wave][lane + 16 * c] = lsum;
    }
  }
  __syncthreads();  // every wave is done with its K tile: reuse the LDS for o
  float* o_lds = reinterpret_cast<float*>(sm.k);  // [wave][G][D]
#pragma unroll
  for (int c = 0; c < CT; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = 4 * grp + i + 16 * c;
      if (head < G) {
        float* dst = o_lds + (wave * G + head) * D + M::NPV * n;
#pragma unroll
        for (int p = 0; p < M::NPV; p += 4)
          *reinterpret_cast<f32x4*>(dst + p) =
              f32x4{st[c].o[p][i], st[c].o[p + 1][i], st[c].o[p + 2][i], st[c].o[p + 3][i]};
      }
    }
  }
  __syncthreads();
}

// fp32 blocks on the vector ALUs: q.k through the LDS K tile, P through
// LDS.  Leaves this wave's (m, l) in sm.m / sm.l and its unnormalised output
// rows in the LDS output stage, then synchronises the workgroup.
template <int D, int G, int NW, bool APPEND>
__device__ __forceinline__ void valu_blocks(const DecodeParams& a, DecodeSmem<D, G, false, NW>& sm,
                                            int b, int qrow, int g, int L, int nblk, int blk_lo,
                                            int blk_hi) {
  using C = F32Cfg<D, G>;
  const uint8_t* __restrict__ cache = a.cache;
  const int num_blocks = a.num_blocks, num_kv_heads = a.num_kv_heads;
  const float scale_log2 = a.scale_log2;
  const int H_q = num_kv_heads * G;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  LaneRoles r;
  r.dp = lane % C::DP;
  r.tq = (lane / C::DP) % C::TPP;
  r.hg = lane / (C::DP * C::TPP);
  r.head = r.hg * C::HPL + r.dp % C::HPL;
  const int dp = r.dp, hg = r.hg;

  // ---- query chunks for this lane: heads hg*HPL + hh, chunks dp*CPL + c
  u32x4 q[C::HPL][C::CPL];
  {
    const u32x4* qb = reinterpret_cast<const u32x4*>(a.query) + int64_t(qrow) * H_q * C::CPR;
#pragma unroll
    for (int hh = 0; hh < C::HPL; ++hh) {
      const int h = g * G + hg * C::HPL + hh;
#pragma unroll
      for (int c = 0; c < C::CPL; ++c) q[hh][c] = qb[h * C::CPR + dp * C::CPL + c];
    }
  }

  const int64_t tile_bytes = int64_t(16) * C::RB;
  const int64_t block_bytes = int64_t(2) * num_kv_heads * tile_bytes;
  const int* bt_row = a.block_tables + int64_t(b) * a.max_blocks_per_seq;

  DecodeState<C, G> st;
  st.init();

  uint8_t* kt_lds = sm.k + wave * C::LDS_TILE;
  uint32_t* p_lds = sm.p[wave];

  // Each wave keeps PD blocks in flight in a register ring: while block k is
  // computed, blocks k+1 .. k+PD are loading.  Block ids come one group of
  // PD ahead of the data (lane s of an id vector holds the id of the group's
  // block s), loaded before the group's data so reading them never waits on
  // data.  Loads past the wave's last block are clamped to that block (cache
  // hits, never computed): every iteration issues the same loads, so the
  // compiler's wait counts stay exact.
  constexpr int PD = C::PD;
  // The query must have arrived before the block loop: waiting for it inside
  // the loop would also wait for the prefetched blocks issued after it.
#pragma unroll
  for (int hh = 0; hh < C::HPL; ++hh)
#pragma unroll
    for (int c = 0; c < C::CPL; ++c) asm volatile("" ::"v"(q[hh][c]));
  const int first = blk_lo + wave;
  const int nmine = blk_hi > first ? (blk_hi - first + NW - 1) / NW : 0;
  if (nmine > 0) {
    auto id_group = [&](int base) -> int {
      const int k = min(base + (lane & (PD - 1)), nmine - 1);
      int id = bt_row[first + k * NW];
      return (id < 0 || id >= num_blocks) ? 0 : id;  // out-of-range ids read block 0
    };
    const int ids_cur = id_group(0);
    int ids_next = id_group(PD);  // issued before the data, as in the loop
    BlockRegs<C> buf[PD];
#pragma unroll
    for (int s = 0; s < PD; ++s)
      buf[s] = load_block_regs<C>(cache, __builtin_amdgcn_readlane(ids_cur, s), block_bytes, g,
                                  num_kv_heads, tile_bytes, lane);
    // Only the sequence's last block can be partial; it is the last block of
    // the wave that owns it and is processed after the loop, so the loop
    // body needs no masking.  In append mode that block (partial or not)
    // also takes the new token there.
    const int j_last = first + (nmine - 1) * NW;
    const int tail_valid = L - j_last * 16;
    const bool seq_last = APPEND && j_last == nblk - 1;
    const int nfull = (tail_valid < 16 || seq_last) ? nmine - 1 : nmine;
    for (int k0 = 0; k0 < nfull; k0 += PD) {
      const int ids_after = id_group(k0 + 2 * PD);
#pragma unroll
      for (int s = 0; s < PD; ++s) {
        if (k0 + s < nfull)
          process_block<D, G, false>(buf[s], 16, q, st, kt_lds, p_lds, sm.alpha[wave],
                                           scale_log2, r);
        buf[s] = load_block_regs<C>(cache, __builtin_amdgcn_readlane(ids_next, s), block_bytes, g,
                                    num_kv_heads, tile_bytes, lane);
      }
      ids_next = ids_after;
    }
    // Loads past the last block were clamped to it, so buf[0] now holds it.
    if (nfull < nmine) {
      if constexpr (APPEND) {
        if (seq_last)
          append_new_token<C>(buf[0], a, b, g, (L - 1) & 15, bt_row[nblk - 1], block_bytes,
                              tile_bytes, lane);
      }
      process_block<D, G, true>(buf[0], min(tail_valid, 16), q, st, kt_lds, p_lds,
                                      sm.alpha[wave], scale_log2, r);
    }
  }

  // ---- merge: this wave's denominator, then the waves of the workgroup
  {
    // sum over the token lanes of this lane's head
    float lsum = st.l;
#pragma unroll
    for (int bit = ilog2(C::DP); bit < ilog2(C::DP * C::TPP); ++bit)
      lsum += __shfl_xor(lsum, 1 << bit, kWave);
    if (r.tq == 0 && dp < C::HPL) {
      sm.m[wave][r.head] = st.m_run;
      sm.l[wave][r.head] = lsum;
    }
  }
  __syncthreads();  // all waves done with their tiles: reuse smem_k for o
  float* o_lds = reinterpret_cast<float*>(sm.k);  // [wave][G][D]
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int jj = 0; jj < C::DPL; ++jj) o_lds[(wave * G + h) * D + lane * C::DPL + jj] = st.o[h][jj];
  __syncthreads();
}

// Merges the split-K records of one (sequence, KV head[, column group]) into
// its output rows: M = max_p m_p, W = sum_p 2^(m_p - M) l_p and
// O = sum_p 2^(m_p - M) l_p o_p / W per head.  Called by the whole
// workgroup (NW waves); sm supplies M[G], W[G] and the scratch k[] (at
// least NW * 64 * 16 bytes).  recs: the nparts records of the slot.  With
// QSPLIT > 1 the slot's G * D / 4 output quads are shared by QSPLIT
// workgroups and this one writes those of part qs.
template <int D, int G, bool BF16, int NW, bool MULTI, int QSPLIT = 1, int MB = 8, class SM,
          class OutRow>
__device__ __forceinline__ void merge_records(const DecodeParams& a, SM& sm,
                                              const uint8_t* __restrict__ recs, int nparts,
                                              int ncols, OutRow out_row, int qs = 0) {
  void* __restrict__ out = a.out;
  float* __restrict__ lse_out = a.lse_out;
  const int max_parts = a.max_parts;
  constexpr int REC = int(ws_record_bytes(G, D));
  constexpr int ML = G * D * (BF16 ? 2 : 4);  // offset of the maxima within a record
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x;
  // The partials of this KV head's G query-head rows, read through buffer
  // resources with the sc1 cache policy: like agent-scope atomic loads they
  // fetch past this XCD's L2 (which may hold stale lines from an earlier
  // call), but as plain loads many of them can be in flight at once.
  const __amdgpu_buffer_rsrc_t rr = ws_rsrc(reinterpret_cast<const float*>(recs), max_parts * REC);
  auto m_off = [&](int h, int p) { return p * REC + ML + h * 4; };
  auto l_off = [&](int h, int p) { return p * REC + ML + (G + h) * 4; };

  // O = sum_p w_p o_p / W with w_p = 2^(m_p - M) l_p, M = max_p m_p and
  // W = sum_p w_p.  Each thread owns 16-byte quads of the output rows; when
  // there are more threads than quads, S threads share a quad and take
  // every S-th partition, and their sums meet in LDS.  Partials are loaded
  // MB at a time.
  constexpr int NT = NW * kWave;
  constexpr int Q = G * D / 4 / QSPLIT;   // quads of this workgroup
  static_assert(Q >= 1 && (G * D / 4) % QSPLIT == 0, "quad split");
  constexpr int S = NT > Q ? NT / Q : 1;
  constexpr int QPT = Q > NT ? Q / NT : 1;
  static_assert(NT * 16 <= int(sizeof(sm.k)), "LDS too small for the subset sums");
  float* lds = reinterpret_cast<float*>(sm.k);
  const int sub = S > 1 ? tid / Q : 0;
  f32x4 acc[QPT];
#pragma unroll
  for (int qi = 0; qi < QPT; ++qi) acc[qi] = f32x4{0.f, 0.f, 0.f, 0.f};
  // partitions [p0, p0 + pc) with weight(h, p - p0)
  auto accumulate = [&](int p0, int pc, auto weight) __attribute__((always_inline)) {
#pragma unroll
    for (int qi = 0; qi < QPT; ++qi) {
      const int quad = qs * Q + (S > 1 ? tid % Q : tid) + qi * NT;
      const int h = quad / (D / 4), d4 = quad % (D / 4);
      for (int pp = sub; pp < pc; pp += S * MB) {
        f32x4 v[MB];
        float w[MB];
#pragma unroll
        for (int j = 0; j < MB; ++j) {
          const int p = pp + j * S;
          const int pl = p < pc ? p : pc - 1;  // in range; weight 0 past the chunk
          if constexpr (BF16)
            v[j] = ws_load_bf16x4(rr, (p0 + pl) * REC + (h * D + d4 * 4) * 2);
          else
            v[j] = ws_load4(rr, (p0 + pl) * REC + (h * D + d4 * 4) * 4);
          w[j] = p < pc ? weight(h, pl) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < MB; ++j) acc[qi] += w[j] * v[j];
      }
    }
  };
  // maxima and sums of every partition fit LDS at once: one pass of loads
  // stages them, the weights replace the maxima in place, and no record
  // field is read twice
  constexpr int FCAP = int(sizeof(sm.k) / sizeof(float)) / (2 * G);
  if (nparts <= FCAP) {
    const int n = nparts * 2 * G;          // [p][m_0..m_{G-1}, l_0..l_{G-1}]
    for (int i0 = tid; i0 < n; i0 += 4 * NT) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * NT;
        v[u] = i < n ? ws_load(rr, (i / (2 * G)) * REC + ML + (i % (2 * G)) * 4) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + u * NT < n) lds[i0 + u * NT] = v[u];
    }
    __syncthreads();
    for (int h = wave; h < G; h += NW) {   // one wave per head
      float M = -INFINITY;
      for (int p = lane; p < nparts; p += kWave) M = fmaxf(M, lds[p * 2 * G + h]);
      M = allreduce_max<0, 6>(M);
      float W = 0.f;
      for (int p = lane; p < nparts; p += kWave) {
        const float w = exp2f(lds[p * 2 * G + h] - M) * lds[p * 2 * G + G + h];
        lds[p * 2 * G + h] = w;
        W += w;
      }
      W = allreduce_sum<0, 6>(W);
      if (lane == 0) { sm.M[h] = M; sm.W[h] = W; }
    }
    __syncthreads();
    accumulate(0, nparts, [&](int h, int p) { return lds[p * 2 * G + h]; });
    __syncthreads();
  } else {
    // per head: M and W over all partitions (one wave per head), then the
    // weights staged through LDS in chunks of WCAP partitions per head
    for (int h = wave; h < G; h += NW) {
      float M = -INFINITY;
      for (int p = lane; p < nparts; p += kWave) M = fmaxf(M, ws_load(rr, m_off(h, p)));
      M = allreduce_max<0, 6>(M);
      float W = 0.f;
      for (int p = lane; p < nparts; p += kWave)
        W += exp2f(ws_load(rr, m_off(h, p)) - M) * ws_load(rr, l_off(h, p));
      W = allreduce_sum<0, 6>(W);
      if (lane == 0) { sm.M[h] = M; sm.W[h] = W; }
    }
    __syncthreads();
    constexpr int WCAP = int(sizeof(sm.k) / sizeof(float)) / G;
    for (int p0 = 0; p0 < nparts; p0 += WCAP) {
      const int pc = min(WCAP, nparts - p0);
      for (int idx = tid; idx < G * pc; idx += NT) {
        const int h = idx / pc, pp = idx % pc;
        lds[h * WCAP + pp] =
            exp2f(ws_load(rr, m_off(h, p0 + pp)) - sm.M[h]) * ws_load(rr, l_off(h, p0 + pp));
      }
      __syncthreads();
      accumulate(p0, pc, [&](int h, int p) { return lds[h * WCAP + p]; });
      __syncthreads();
    }
  }
  if constexpr (S > 1) {
    f32x4* red = reinterpret_cast<f32x4*>(sm.k);  // [S][Q]
    red[tid] = acc[0];
    __syncthreads();
    if (sub == 0) {
#pragma unroll
      for (int t = 1; t < S; ++t) acc[0] += red[t * Q + tid];
    }
  }
  if (sub == 0) {
#pragma unroll
    for (int qi = 0; qi < QPT; ++qi) {
      const int quad = qs * Q + tid + qi * NT;
      const int h = quad / (D / 4), d4 = quad % (D / 4);
      if (MULTI && h >= ncols) continue;
      const int64_t row = out_row(h);
      // a MULTI row before position 0 (seq_len < rows) sees nothing: W = 0
      const float inv = (!MULTI || sm.W[h] > 0.f) ? 1.f / sm.W[h] : 0.f;
      store_out<BF16>(out, row * D + d4 * 4 + 0, acc[qi].x * inv);
      store_out<BF16>(out, row * D + d4 * 4 + 1, acc[qi].y * inv);
      store_out<BF16>(out, row * D + d4 * 4 + 2, acc[qi].z * inv);
      store_out<BF16>(out, row * D + d4 * 4 + 3, acc[qi].w * inv);
      if (lse_out && d4 == 0)
        lse_out[row] = (!MULTI || sm.W[h] > 0.f) ? sm.M[h] * kLn2 + logf(sm.W[h]) : -INFINITY;
    }
  }
}

// One work item: KV head g of sequence b, partition `part` (blocks
// [part * pb, min((part + 1) * pb, nblk))).  The query and output rows are
// those of packed row `qrow` (b itself in a decode batch; the sequence's
// first query row in a flattened batch).  Called by the whole workgroup.
// MULTI (bf16 only): the item's columns are (query row, head) pairs of
// column group cg of the sequence's `rows` query rows (see DecodeParams);
// qrow is the group's first query row.
template <int D, int G, bool BF16, int NW, bool APPEND, bool KV8 = false, bool MULTI = false,
          bool SHARED = false>
__device__ __forceinline__ void decode_item(const DecodeParams& a,
                                            DecodeSmem<D, G, BF16, NW, KV8>& sm,
                                            int b, int qrow, int g, int part, int L, int nblk,
                                            int pb, int nparts, int cg = 0, int rows = 1) {
  void* __restrict__ out = a.out;
  float* __restrict__ lse_out = a.lse_out;
  const int num_kv_heads = a.num_kv_heads, max_parts = a.max_parts;
  int* __restrict__ ws_count = a.ws_count;
  constexpr int REC = int(ws_record_bytes(G, D));
  constexpr int ML = G * D * (BF16 ? 2 : 4);  // offset of the maxima within a record
  const int H_q = num_kv_heads * G;
  const int blk_lo = part * pb;
  const int blk_hi = min(blk_lo + pb, nblk);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  static_assert(!MULTI || (BF16 && !APPEND), "multi-row items: bf16, no append");
  int row0 = 0, ncols = G;  // MULTI: first row of the group within the sequence, live columns
  if constexpr (MULTI) {
    row0 = cg * a.rows_per_group;
    ncols = min(a.rows_per_group, rows - row0) * a.group;
  }
  // output row of column h
  auto out_row = [&](int h) -> int64_t {
    if constexpr (MULTI)
      return int64_t(qrow + h / a.group) * (num_kv_heads * a.group) + g * a.group + h % a.group;
    else
      return int64_t(qrow) * H_q + g * G + h;
  };
  const int slot = MULTI ? (b * num_kv_heads + g) * a.col_groups + cg : b * num_kv_heads + g;
  if constexpr (BF16)
    mfma_blocks<D, G, NW, APPEND, KV8, MULTI, SHARED>(a, sm, b, qrow, g, L, nblk, blk_lo, blk_hi,
                                                      row0, ncols, rows);
  else
    valu_blocks<D, G, NW, APPEND>(a, sm, b, qrow, g, L, nblk, blk_lo, blk_hi);
  float* o_lds = reinterpret_cast<float*>(sm.k);  // [wave][G][D]

  const bool single = nparts <= 1;
  const int tid = threadIdx.x;
  // head h's (M, sum l, sum o[d]) over the waves, each wave weighted by
  // 2^(m_w - M) (0 for a wave with no tokens)
  auto wave_merge = [&](int h, int d, float& M, float& lsum, float& acc) {
    M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][h]);
    lsum = 0.f;
    acc = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float wt = __builtin_amdgcn_exp2f(sm.m[w][h] - M);
        lsum += wt * sm.l[w][h];
        acc += wt * o_lds[(w * G + h) * D + d];
      }
    }
  };
  if (single) {
    for (int e = tid; e < ncols * D; e += NW * kWave) {
      const int h = e / D, d = e % D;
      float M, lsum, acc;
      wave_merge(h, d, M, lsum, acc);
      const int64_t row = out_row(h);
      store_out<BF16>(out, row * D + d, lsum > 0.f ? acc / lsum : 0.f);
      if (lse_out && d == 0) lse_out[row] = lsum > 0.f ? M * kLn2 + logf(lsum) : -INFINITY;
    }
    return;
  }
  // this partition's record: the outputs, then the maxima and sums
  uint8_t* __restrict__ recs = a.ws_rec + int64_t(slot) * max_parts * REC;
  uint8_t* rec = recs + int64_t(part) * REC;
  constexpr int PER = BF16 ? 2 : 1;  // outputs per 4-byte store
  for (int e = tid; e < G * D / PER; e += NW * kWave) {
    const int h = e / (D / PER), d = PER * (e % (D / PER));
    float M, lsum, a0;
    wave_merge(h, d, M, lsum, a0);
    if constexpr (BF16) {
      float a1;
      wave_merge(h, d + 1, M, lsum, a1);
      const float o0 = lsum > 0.f ? a0 / lsum : 0.f, o1 = lsum > 0.f ? a1 / lsum : 0.f;
      coherent_store_u32(reinterpret_cast<uint32_t*>(rec + (h * D + d) * 2),
                         (f32_to_bf16_rne(o0) & 0xFFFFu) | (f32_to_bf16_rne(o1) << 16));
    } else {
      coherent_store(reinterpret_cast<float*>(rec) + h * D + d, lsum > 0.f ? a0 / lsum : 0.f);
    }
    if (d == 0) {
      sm.M[h] = M;
      sm.W[h] = lsum;
    }
  }
  __syncthreads();
  if (tid < 2 * G)  // the maxima and sums in one store
    coherent_store(reinterpret_cast<float*>(rec + ML) + tid, tid < G ? sm.M[tid] : sm.W[tid - G]);
  if (a.defer_merge) return;  // merge_kernel combines the records after this launch

  // ---- split-K: the last workgroup of this (sequence, KV head) to finish
  // merges all partitions.  Partials are written and read with accesses that
  // are coherent across the XCDs' L2 caches (agent scope), and this
  // workgroup's writes have completed before its arrival is counted, so the
  // workgroup that counts last sees every partial.  No L2 flush is needed.
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(&ws_count[slot], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    sm.last = old == nparts - 1;
  }
  __syncthreads();
  if (!sm.last) return;
  if (tid == 0)  // ready for the next call
    __hip_atomic_store(&ws_count[slot], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  merge_records<D, G, BF16, NW, MULTI>(a, sm, recs, nparts, ncols, out_row);
}


// Decode kernel: each workgroup walks work items t = blockIdx.x,
// blockIdx.x + gridDim.x, ...  With a plan the items are its (b, part)
// entries times the KV heads (one workgroup per item); without one they are
// the virtual grid (part, b, g) walked by a grid of a few times the resident
// workgroups, and items past a sequence's last partition are skipped in the
// loop instead of being dispatched as empty workgroups.
// 4-wave bf16 variants of head size 64 are held to 168 VGPRs (three waves
// per SIMD, so three workgroups share a compute unit when there are many
// items); head size 128 and fp32 need more registers than that.  An 8-wave
// workgroup holds a compute unit alone at two or three waves per SIMD, so
// its registers are left free for loads in flight.
// 2-wave variants with 16 or more columns (the multi-row kernel) are held to
// two waves per SIMD, like the other 2-wave variants; the 4-wave head-size-64
// variants with up to 16 columns to three (the 32-column one needs more).
template <int D, int G, bool BF16, int NW>
constexpr int decode_min_waves() {
  return NW == 4 && BF16 && D == 64 && G <= 16 ? 3
                                               : (NW == 2 && BF16 && G >= 16 ? 2 : 1);
}
template <int D, int G, bool BF16, int NW>
constexpr int decode_max_waves() { return NW == 8 ? 2 : 8; }

// MULTI: the column groups of one (entry, KV head) item s are 8 item
// indices apart, inside runs of 8 * col_groups indices: the dispatcher deals
// workgroups to the 8 XCDs in turn, so they run on one XCD at about the same
// time and the later ones can read the blocks from that XCD's L2.
template <int D, int G, bool BF16, int NW, bool APPEND, bool KV8 = false, bool MULTI = false,
          bool SHARED = false>
__global__ __launch_bounds__(NW * kWave)
__attribute__((amdgpu_waves_per_eu(decode_min_waves<D, G, BF16, NW>(), decode_max_waves<D, G, BF16, NW>())))
void decode_kernel(const DecodeParams a) {
  __shared__ DecodeSmem<D, G, BF16, NW, KV8> sm;
  for (int t = blockIdx.x; t < a.num_items; t += gridDim.x) {
    int s = t, cg = 0;
    if constexpr (MULTI) {
      const int run = 8 * a.col_groups;
      const int blk = t / run, rem = t - blk * run;
      cg = rem >> 3;
      s = blk * 8 + (rem & 7);
      if (s >= a.items_per_group * a.num_kv_heads) continue;  // padding of the last run
    }
    const int g = s % a.num_kv_heads;
    const int r = s / a.num_kv_heads;
    int b, part;
    if (a.plan) {
      const int e = a.plan[r];
      b = e & 0xFFFF;
      part = (e >> 16) & 0xFFFF;
      if (b >= a.B) continue;  // not an entry of this batch
    } else {
      b = r % a.B;
      part = r / a.B;
    }
    int L = a.seq_lens[b];
    L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
    const int nblk = (L + 15) >> 4;
    const int pb = a.part_blocks > 0 ? a.part_blocks : (nblk > 0 ? nblk : 1);
    const int nparts = (nblk + pb - 1) / pb;
    if (part > 0 && part >= nparts) continue;
    const int qrow = MULTI ? b * a.rows + cg * a.rows_per_group : b;
    decode_item<D, G, BF16, NW, APPEND, KV8, MULTI, SHARED>(a, sm, b, qrow, g, part, L, nblk, pb,
                                                            nparts, cg, a.rows);
    __syncthreads();  // LDS is reused by the next item
  }
}

// Split-K merge as its own launch (decode launches with defer_merge): one
// workgroup per (slot, quad part), slot = b * H_kv + g; slots whose
// sequence fits one partition were written by their single item.  The
// records were written by the previous launch on the stream, so they are
// complete when this one starts.
constexpr int kMergeWaves = 4;

template <int G>
struct MergeSmem {
  __attribute__((aligned(16))) uint8_t k[16384];
  float M[G], W[G];
};

template <int D, int G, bool BF16, int QSPLIT>
__global__ __launch_bounds__(kMergeWaves * kWave) void merge_kernel(const DecodeParams a) {
  __shared__ MergeSmem<G> sm;
  const int slot = blockIdx.x / QSPLIT, qs = blockIdx.x % QSPLIT;
  const int b = slot / a.num_kv_heads, g = slot % a.num_kv_heads;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int nblk = (L + 15) >> 4;
  const int pb = a.part_blocks > 0 ? a.part_blocks : (nblk > 0 ? nblk : 1);
  const int nparts = (nblk + pb - 1) / pb;
  if (nparts <= 1) return;
  const int H_q = a.num_kv_heads * G;
  auto out_row = [&](int h) -> int64_t { return int64_t(b) * H_q + g * G + h; };
  const uint8_t* recs = a.ws_rec + int64_t(slot) * a.max_parts * ws_record_bytes(G, D);
  merge_records<D, G, BF16, kMergeWaves, false, QSPLIT, 16>(a, sm, recs, nparts, G, out_row, qs);
}

}  // namespace pa
