// Device-side helpers shared by the paged-attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;

// 16-byte vector moved as one global load / store.
struct alignas(16) Vec16 {
  uint32_t w[4];
};

__device__ __forceinline__ Vec16 load16(const void* p) {
  return *reinterpret_cast<const Vec16*>(p);
}

// Streaming load: the non-temporal hint keeps data that is read once (a
// sequence's K/V rows in a decode step) from displacing reusable lines.
__device__ __forceinline__ Vec16 load16_nt(const void* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return Vec16{{v.x, v.y, v.z, v.w}};
}

__device__ __forceinline__ void store16(void* p, const Vec16& v) {
  *reinterpret_cast<Vec16*>(p) = v;
}

// bf16 stored as its 16-bit pattern. Widening is exact: the pattern becomes
// the upper half of an fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Element storage traits: how many elements one 16-byte vector holds and how
// to widen element e of it to fp32.
template <typename T> struct Elem;

struct BF16Tag {};

template <> struct Elem<float> {
  static constexpr int kPerVec = 4;
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float get(const Vec16& v, int e) { return __uint_as_float(v.w[e]); }
  __device__ __forceinline__ static void to_f32(const Vec16& v, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v.w[e]);
  }
  __device__ __forceinline__ static uint32_t from_f32_word(const float* f, int w) {
    return __float_as_uint(f[w]);
  }
};

template <> struct Elem<BF16Tag> {
  static constexpr int kPerVec = 8;
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static void to_f32(const Vec16& v, float* f) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f[2 * w] = bf16_lo(v.w[w]);
      f[2 * w + 1] = bf16_hi(v.w[w]);
    }
  }
  __device__ __forceinline__ static uint32_t from_f32_word(const float* f, int w) {
    return pack_bf16x2(f[2 * w], f[2 * w + 1]);
  }
};

}  // namespace pa
