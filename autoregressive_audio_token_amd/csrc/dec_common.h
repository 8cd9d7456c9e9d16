// Shared device helpers for the decode-step kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dec {

constexpr int kWave = 64;

// ---- cross-lane moves (DPP within 16-lane rows, ds_swizzle/bpermute beyond) -------

// DPP control codes (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowRor8 = 0x128;     // row_ror:8  == lane ^ 8 inside a 16-lane row
constexpr int kDppRowMirror = 0x140;   // lane 15 - i inside a 16-lane row
constexpr int kDppHalfMirror = 0x141;  // lane 7 - i inside an 8-lane half row

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G = 8, 16 or 32); every lane of a group gets the sum.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 8 || G == 16 || G == 32, "group of 8, 16 or 32 lanes");
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  if constexpr (G >= 16) v += dpp_f32<kDppRowMirror>(v);
  if constexpr (G == 32) v += __shfl_xor(v, 16);
  return v;
}

// Butterfly across lanes that differ in bit positions [log2(FROM), 6): combines the
// values held by lanes lane ^ FROM, lane ^ 2*FROM, ... (all lanes end with the result).
// (The gfx950 permlane16/32 swaps do the 16- and 32-lane steps in one VALU op each,
// bit for bit the same; in the attention kernel they measured slower than these
// shuffles, the compiler then holding more scalar state in lanes of VGPRs.)
template <int FROM>
__device__ __forceinline__ float xor_max_from(float v) {
  if constexpr (FROM <= 8) v = fmaxf(v, dpp_f32<kDppRowRor8>(v));
  if constexpr (FROM <= 16) v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}

template <int FROM>
__device__ __forceinline__ float xor_sum_from(float v) {
  if constexpr (FROM <= 8) v += dpp_f32<kDppRowRor8>(v);
  if constexpr (FROM <= 16) v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Maximum over the wave, returned to every lane: DPP within each 16-lane row,
// then the four row results through readlane.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Inclusive prefix sums over the 64 lanes in lane order, with DPP row shifts and
// row broadcasts (the lanes a step does not update take a zero addend).  The
// addition order is fixed, so results are reproducible.
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr3 = 0x113;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ int dpp_i32_masked(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, BANK_MASK, true);
}

__device__ __forceinline__ int wave_inclusive_sum_int(int v, int /*lane*/) {
  const int x = v;
  v += dpp_i32_masked<kDppRowShr1, 0xF, 0xF>(x);
  v += dpp_i32_masked<kDppRowShr2, 0xF, 0xF>(x);
  v += dpp_i32_masked<kDppRowShr3, 0xF, 0xF>(x);
  v += dpp_i32_masked<kDppRowShr4, 0xF, 0xE>(v);
  v += dpp_i32_masked<kDppRowShr8, 0xF, 0xC>(v);
  v += dpp_i32_masked<kDppRowBcast15, 0xA, 0xF>(v);
  v += dpp_i32_masked<kDppRowBcast31, 0xC, 0xF>(v);
  return v;
}

__device__ __forceinline__ float wave_inclusive_sum(float v, int /*lane*/) {
  const int x = __builtin_bit_cast(int, v);
  auto add = [](float a, int b) { return a + __builtin_bit_cast(float, b); };
  v = add(v, dpp_i32_masked<kDppRowShr1, 0xF, 0xF>(x));
  v = add(v, dpp_i32_masked<kDppRowShr2, 0xF, 0xF>(x));
  v = add(v, dpp_i32_masked<kDppRowShr3, 0xF, 0xF>(x));
  v = add(v, dpp_i32_masked<kDppRowShr4, 0xF, 0xE>(__builtin_bit_cast(int, v)));
  v = add(v, dpp_i32_masked<kDppRowShr8, 0xF, 0xC>(__builtin_bit_cast(int, v)));
  v = add(v, dpp_i32_masked<kDppRowBcast15, 0xA, 0xF>(__builtin_bit_cast(int, v)));
  v = add(v, dpp_i32_masked<kDppRowBcast31, 0xC, 0xF>(__builtin_bit_cast(int, v)));
  return v;
}

// The same scan over doubles: each DPP move carries both halves of a value.
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ double dpp_f64_masked(double v) {
  const uint64_t bits = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)dpp_i32_masked<CTRL, ROW_MASK, BANK_MASK>((int)(uint32_t)bits);
  const uint32_t hi =
      (uint32_t)dpp_i32_masked<CTRL, ROW_MASK, BANK_MASK>((int)(uint32_t)(bits >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double wave_inclusive_sum_f64(double v) {
  const double x = v;
  v += dpp_f64_masked<kDppRowShr1, 0xF, 0xF>(x);
  v += dpp_f64_masked<kDppRowShr2, 0xF, 0xF>(x);
  v += dpp_f64_masked<kDppRowShr3, 0xF, 0xF>(x);
  v += dpp_f64_masked<kDppRowShr4, 0xF, 0xE>(v);
  v += dpp_f64_masked<kDppRowShr8, 0xF, 0xC>(v);
  v += dpp_f64_masked<kDppRowBcast15, 0xA, 0xF>(v);
  v += dpp_f64_masked<kDppRowBcast31, 0xC, 0xF>(v);
  return v;
}

// Lane `src`'s double, in every lane.
__device__ __forceinline__ double readlane_f64(double v, int src) {
  const uint64_t bits = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bits, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bits >> 32), src);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int wave_exclusive_sum_int(int v, int lane) {
  return wave_inclusive_sum_int(v, lane) - v;
}

// ---- element decoding ------------------------------------------------------------

// bfloat16 pair packed in a 32-bit word (little endian: element 2i in the low half).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// ---- order-preserving key for float32 (host and device) ---------------------------
// Monotone: a < b implies key(a) < key(b); -0 is folded onto +0 so equal values tie.
__host__ __device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace dec
