// Device-side building blocks shared by the HiLS kernels (gfx950, wave64).
//
// MFMA fragment conventions (16x16 family, verified on gfx950):
//   A operand: lane l holds row (l % 16) and KPL consecutive k-slots of group g = l / 16;
//   B operand: lane l holds column (l % 16) and the same KPL k-slots of group g;
//   C/D:       lane l holds column (l % 16) and rows 4*g + r, r = 0..3.
// bf16: v_mfma_f32_16x16x32_bf16 (KPL = 8, K = 32 per instruction).
// fp32: v_mfma_f32_16x16x4_f32   (KPL = 1, K = 4 per instruction).
// Any assignment of real k indices to (g, slot) works as long as A and B use the same one.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kChunk = 64;  // chunk size C (the only one this library builds)

// ------------------------------------------------------------------------------------------
// Scalar conversions
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

// fp32 -> bf16, round to nearest, ties to even (gfx950: v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16 bf16_rne(float x) { return static_cast<bf16>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return bf16_rne(x); }

// Order-preserving map of a float to uint32 (larger float -> larger key), for finite values.
__device__ __forceinline__ uint32_t f32_key(float x) {
  uint32_t u = __float_as_uint(x);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k ^ 0x80000000u) : ~k;
  return __uint_as_float(u);
}

// ------------------------------------------------------------------------------------------
// MFMA 16x16 wrappers
// ------------------------------------------------------------------------------------------
template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
  static constexpr int KPL = 8;   // k-slots per lane
  static constexpr int K = 32;    // k per instruction
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  static constexpr int K = 4;
  typedef float frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Load one fragment (KPL consecutive elements) from memory (global or LDS).
template <typename T> __device__ __forceinline__ typename Mfma<T>::frag load_frag(const T* p);
template <> __device__ __forceinline__ bf16x8 load_frag<bf16>(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <> __device__ __forceinline__ float load_frag<float>(const float* p) { return *p; }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ------------------------------------------------------------------------------------------
// Cross-lane helpers
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ uint32_t shfl_xor_u(uint32_t v, int m) {
  return (uint32_t)__shfl_xor((int)v, m, kWave);
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = shfl_xor_u((uint32_t)v, m), hi = shfl_xor_u((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// Partner values across 16- and 32-lane halves without the LDS crossbar (gfx950
// v_permlane16_swap / v_permlane32_swap with both operands holding v): the two results hold, at
// every lane l, the values of lanes l and l^16 (resp. l^32) in some order.
__device__ __forceinline__ void swap16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Reductions over the four lanes {l, l^16, l^32, l^48} that share column l % 16.
__device__ __forceinline__ float col_max(float v) {
  float a, b;
  swap16(v, a, b);
  swap32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float col_sum(float v) {
  float a, b;
  swap16(v, a, b);
  swap32(a + b, a, b);
  return a + b;
}
__device__ __forceinline__ int col_sum_i(int v) {
  v += shfl_xor_i(v, 16);
  return v + shfl_xor_i(v, 32);
}
__device__ __forceinline__ uint32_t col_min_u(uint32_t v) {
  v = min(v, shfl_xor_u(v, 16));
  return min(v, shfl_xor_u(v, 32));
}
__device__ __forceinline__ uint32_t col_max_u(uint32_t v) {
  v = max(v, shfl_xor_u(v, 16));
  return max(v, shfl_xor_u(v, 32));
}
// Exclusive prefix of v over the column's four lanes in group order g = 0..3.
__device__ __forceinline__ int col_exclusive_prefix(int v, int g) {
  int a = shfl_xor_i(v, 16);                 // partner in the other group of the pair
  int pair = v + a;                          // sum of groups {g & ~1, g | 1}
  int lower_in_pair = (g & 1) ? a : 0;
  int other_pair = shfl_xor_i(pair, 32);     // sum of the other pair
  int lower_pairs = (g & 2) ? other_pair : 0;
  return lower_pairs + lower_in_pair;
}

// Wave-wide reductions (all 64 lanes).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
  return v;
}

// Remap a workgroup id so that consecutive logical tiles run on the same XCD.  Workgroups are
// dispatched round-robin over the 8 XCDs; this is a bijection on [0, total).
// Key/value (and landmark) pair of query pair bh = b * H + h when G consecutive query heads
// share one key/value head (grouped-query attention; G = 1 is one head each).
__device__ __forceinline__ int kv_pair(int bh, int H, int G) {
  return G == 1 ? bh : (bh / H) * (H / G) + (bh % H) / G;
}

__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t total) {
  const uint32_t nx = 8;
  uint32_t x = bid % nx, slot = bid / nx;
  uint32_t per = total / nx, rem = total % nx;
  return x * per + min(x, rem) + slot;
}

}  // namespace hils
