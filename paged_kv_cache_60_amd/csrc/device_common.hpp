// Device-side helpers shared by the gfx950 kernels of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N = 1, 2, 4, 8, 16); every lane of the
// group receives the group's total. Uses DPP butterflies: xor 1, xor 2, then
// the half-row and row mirrors, which pair each quad (half row) with the other.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group size");
  if constexpr (N >= 2) v += dpp_f32<kDppQuadXor1>(v);
  if constexpr (N >= 4) v += dpp_f32<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp_f32<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f32<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ float shfl_xor_f32(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Host-side argument check: the kernels read and write K/V rows, queries,
// outputs, host-pool blocks and workspaces with 16-byte vector accesses, and
// index arrays element by element, so each pointer must be aligned to
// kVecAlign or to its element size. A null pointer passes (null checks are
// separate).
constexpr uintptr_t kVecAlign = 16;
inline bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline bool vec_aligned(const void* p) { return aligned_to(p, kVecAlign); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// dot of two packed fp16 pairs, accumulated in fp32
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

__device__ __forceinline__ float h_lo(uint32_t a) { return (float)__builtin_bit_cast(f16x2, a).x; }
__device__ __forceinline__ float h_hi(uint32_t a) { return (float)__builtin_bit_cast(f16x2, a).y; }

// e4m3fn bytes to fp16 pairs with gfx950's v_cvt_scalef32_pk_f16_fp8 at scale
// 1.0: exact, since every e4m3 value is an fp16 value (checked on the device
// for all 256 codes in every byte position). lo: bytes 0, 1; hi: bytes 2, 3.
__device__ __forceinline__ uint32_t fp8x2_lo_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ uint32_t fp8x2_hi_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// Cache element formats: fp16, OCP fp8 e4m3fn, OCP fp8 e5m2 (the values of
// pkv_kv_dtype).
enum KvFmt { kF16 = 0, kE4M3 = 1, kE5M2 = 2 };

// e5m2 bytes to fp16 pairs: e5m2 is the top byte of an fp16 with the same
// exponent layout, so each byte moves to the high byte of its half (exact).
// v_perm_b32 with the word in both sources: selector 0x0C writes 0x00.
__device__ __forceinline__ uint32_t e5m2x2_lo_to_f16x2(uint32_t w) {
  return __builtin_amdgcn_perm(w, w, 0x010C000Cu);  // bytes [0, b0, 0, b1]
}
__device__ __forceinline__ uint32_t e5m2x2_hi_to_f16x2(uint32_t w) {
  return __builtin_amdgcn_perm(w, w, 0x030C020Cu);  // bytes [0, b2, 0, b3]
}

// Bytes 0, 1 (lo) or 2, 3 (hi) of a word of fp8 codes as an fp16 pair.
template <int FMT>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w, bool hi) {
  static_assert(FMT == kE4M3 || FMT == kE5M2, "fp8 format");
  if constexpr (FMT == kE4M3)
    return hi ? fp8x2_hi_to_f16x2(w) : fp8x2_lo_to_f16x2(w);
  else
    return hi ? e5m2x2_hi_to_f16x2(w) : e5m2x2_lo_to_f16x2(w);
}

}  // namespace pkv
