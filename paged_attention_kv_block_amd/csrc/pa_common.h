// Device-side helpers shared by the libpa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;
constexpr int kBlockSize = 16;  // tokens per KV-cache block supported by the kernels

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Native 4 x 32-bit vector (a first-class LLVM vector, unlike HIP's uint4
// struct, so arrays of it stay in registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (inputs here are never NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// (lo, hi) -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// a.lo*b.lo + a.hi*b.hi + c on packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                          __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Lane-crossing moves through DPP.  Control codes (GFX9 DPP encoding):
//   quad_perm = 2-bit selectors; row_shl:n = 0x100+n; row_ror:n = 0x120+n;
//   row_mirror = 0x140; row_half_mirror = 0x141.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // i <-> 7-i within 8 lanes
constexpr int kRowMirror = 0x140;     // i <-> 15-i within 16 lanes

// Butterfly step over lane bit `BIT` for a value that is already uniform
// over the lower bits of its 2^(BIT+1)-lane group (true after the steps for
// the lower bits, or when those bits index replicas).  Bits 0-3 use DPP;
// bits 4-5 cross DPP rows and use a shuffle.
template <int BIT>
__device__ __forceinline__ float partner(float x) {
  if constexpr (BIT == 0) return dpp_f<kQuadXor1>(x);
  else if constexpr (BIT == 1) return dpp_f<kQuadXor2>(x);
  else if constexpr (BIT == 2) return dpp_f<kRowHalfMirror>(x);
  else if constexpr (BIT == 3) return dpp_f<kRowMirror>(x);
  else return __shfl_xor(x, 1 << BIT, kWave);
}

// Value of lane (this lane xor 2^BIT), for any x.  Bits 2 and 3 compose two
// DPP moves: half_mirror is xor 7 and mirror is xor 15 within their rows.
constexpr int kQuadRev = 0x1B;        // quad_perm [3,2,1,0] = xor 3
template <int BIT>
__device__ __forceinline__ float xor_partner(float x) {
  if constexpr (BIT == 0) return dpp_f<kQuadXor1>(x);
  else if constexpr (BIT == 1) return dpp_f<kQuadXor2>(x);
  else if constexpr (BIT == 2) return dpp_f<kQuadRev>(dpp_f<kRowHalfMirror>(x));
  else if constexpr (BIT == 3) return dpp_f<kRowHalfMirror>(dpp_f<kRowMirror>(x));
  else return __shfl_xor(x, 1 << BIT, kWave);
}

// Max over lane bits [LO, HI) for values that may differ across the bits
// below LO.
template <int LO, int HI>
__device__ __forceinline__ float allreduce_max_xor(float x) {
  if constexpr (LO < HI) {
    x = fmaxf(x, xor_partner<LO>(x));
    return allreduce_max_xor<LO + 1, HI>(x);
  } else {
    return x;
  }
}

template <int LO, int HI>
__device__ __forceinline__ float allreduce_max(float x) {
  if constexpr (LO < HI) {
    x = fmaxf(x, partner<LO>(x));
    return allreduce_max<LO + 1, HI>(x);
  } else {
    return x;
  }
}

template <int LO, int HI>
__device__ __forceinline__ float allreduce_sum(float x) {
  if constexpr (LO < HI) {
    x += partner<LO>(x);
    return allreduce_sum<LO + 1, HI>(x);
  } else {
    return x;
  }
}

// Orders this wave's LDS traffic: writes before the call are visible to
// reads after it (LDS executes one wave's requests in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// FP8 (OCP E4M3) codes of four bf16 cache inputs (elements w0.lo, w0.hi,
// w1.lo, w1.hi -> bytes 0..3) under a per-tensor scale: each input divided by
// the scale in fp32 (IEEE division), saturated at +-448 and rounded to
// nearest even by the hardware conversion, sign kept.  "vLLM: Ein tiefer
// Einblick ...", section "Tiefenanalyse", lists FP8 among the engine's
// quantisation formats without a format or scale: E4M3 with per-tensor
// scales is the reading.
// A NaN input (either sign) is stored as the code 0x7F: the clamp would
// otherwise turn it into -448 or 448, a large finite key nothing can detect.
// +-inf saturate to +-448 like any other out-of-range value.
__device__ __forceinline__ float e4m3_input(uint32_t f32_bits, float scale) {
  const float q = __uint_as_float(f32_bits) / scale;
  return fminf(fmaxf(q, -448.f), 448.f);
}
__device__ __forceinline__ uint32_t e4m3_nan_byte(uint32_t f32_bits, uint32_t byte_mask) {
  return (f32_bits & 0x7FFFFFFFu) > 0x7F800000u ? byte_mask : 0u;
}
__device__ __forceinline__ uint32_t quantize4_e4m3(uint32_t w0, uint32_t w1, float scale) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_input(w0 << 16, scale),
                                         e4m3_input(w0 & 0xFFFF0000u, scale), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_input(w1 << 16, scale),
                                     e4m3_input(w1 & 0xFFFF0000u, scale), r, true);
  const uint32_t nan = e4m3_nan_byte(w0 << 16, 0xFFu) | e4m3_nan_byte(w0 & 0xFFFF0000u, 0xFF00u) |
                       e4m3_nan_byte(w1 << 16, 0xFF0000u) |
                       e4m3_nan_byte(w1 & 0xFFFF0000u, 0xFF000000u);
  return (uint32_t(r) & ~nan) | (0x7F7F7F7Fu & nan);
}

}  // namespace pa
