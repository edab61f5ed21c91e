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

// 4-byte vector: four fp8 cache elements.
struct alignas(4) Vec4 {
  uint32_t w[1];
};

// 8-byte vector: eight fp8 cache elements.
struct alignas(8) Vec8 {
  uint32_t w[2];
};

__device__ __forceinline__ Vec8 load8(const void* p) {
  return *reinterpret_cast<const Vec8*>(p);
}

__device__ __forceinline__ Vec8 load8_nt(const void* p) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return Vec8{{v.x, v.y}};
}

__device__ __forceinline__ void store8(void* p, const Vec8& v) {
  *reinterpret_cast<Vec8*>(p) = v;
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

// ---- fp8 cache elements: OCP E4M3 (sign, 4 exponent bits with bias 7,
// 3 mantissa bits; no infinities; 0x7F / 0xFF are NaN; largest value 448) ----

// fp32 -> E4M3 code: round to nearest, ties to even mantissa; magnitudes of
// 448 and above (infinities included) saturate to +-448; NaN stays NaN with
// its sign. Integer arithmetic on the fp32 fields, so the result does not
// depend on the hardware conversion's rounding or clamping modes.
__host__ __device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;   // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |x| >= 448 = 1.75 * 2^8
  if (a < 0x3c800000u) {
    // below 2^-6: subnormal codes are multiples of 2^-9; scaling by 2^9 is
    // exact and v_rndne rounds half to even (8 lands on the smallest normal)
    return sign | static_cast<uint32_t>(__builtin_rintf(__builtin_bit_cast(float, a) * 512.f));
  }
  // normal: rebias the exponent (127 -> 7), then drop 20 mantissa bits with
  // round to nearest even; a carry moves into the exponent as it should
  const uint32_t v = a - (120u << 23);
  return sign | ((v + 0x7ffffu + ((v >> 20) & 1u)) >> 20);
}

// Codes in bytes (2 * HI, 2 * HI + 1) of w -> packed bf16 pair (exact: every
// E4M3 value is a bf16 value; v_cvt_scalef32_pk_bf16_fp8 with scale 1).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// Whether a non-negative fp32 value (bits u) is exactly a rounding midpoint
// between two neighbouring E4M3 values: in the normal range (2^-6 .. 448)
// the 20 mantissa bits below the kept 3 read 1000..0; below 2^-6 the value
// is an odd multiple of 2^-10 (so u * 512 has fraction one half; the
// product and the fraction are exact).
__host__ __device__ __forceinline__ bool e4m3_midpoint(uint32_t u) {
  if (u >= 0x3c800000u) return u < 0x43e00000u && (u & 0xfffffu) == 0x80000u;
  const float t = __builtin_bit_cast(float, u) * 512.f;
  return t - __builtin_floorf(t) == 0.5f;
}

// Cache code of x under a per-tensor scale: the E4M3 code nearest the exact
// quotient |x| / scale, carrying x's sign bit (so -0 and NaN keep their
// sign whatever sign the hardware gives a NaN quotient).
// The correctly rounded fp32 quotient q lies in the same E4M3 rounding
// interval as the exact quotient unless q is itself a midpoint; there the
// exact quotient may be on either side. Its side is the sign of the remainder
// |x| - q * scale, which fp64 gives exactly (q * scale has at most 48
// significant bits, and the two terms are within a factor of two of each
// other), and q is moved one fp32 ulp that way before it is rounded, so a
// true tie (remainder 0) still goes to the even code.
__host__ __device__ __forceinline__ uint32_t e4m3_quantize(float x, float scale) {
  const uint32_t sign = (__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u;
  const float a = fabsf(x);
  const float q = a / scale;
  uint32_t qb = __builtin_bit_cast(uint32_t, q);
  if (e4m3_midpoint(qb)) {
    const double r = static_cast<double>(a) - static_cast<double>(q) * static_cast<double>(scale);
    qb += (r > 0.0) ? 1u : 0u;
    qb -= (r < 0.0) ? 1u : 0u;
  }
  return sign | (f32_to_e4m3(__builtin_bit_cast(float, qb)) & 0x7fu);
}

// E4M3 codes of eight consecutive elements of a bf16 row under a scale.
__device__ __forceinline__ Vec8 quantize8(const Vec16& x, float scale) {
  Vec8 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t word = x.w[2 * w + e / 2];
      const float f = (e & 1) ? bf16_hi(word) : bf16_lo(word);
      c |= e4m3_quantize(f, scale) << (8 * e);
    }
    r.w[w] = c;
  }
  return r;
}

// Cache element traits for the decode kernels: the vector one lane moves per
// load (eight elements for 16-bit and fp8 caches, four for fp32), bytes per
// cache element and per query / output element, and widening to fp32.
template <typename T> struct Elem;

struct BF16Tag {};
struct Fp8Tag {};  // E4M3 cache elements; queries and outputs are bf16

template <> struct Elem<float> {
  using Vec = Vec16;
  static constexpr int kPerVec = 4;
  static constexpr int kBytes = 4;
  static constexpr int kQBytes = 4;
  __device__ __forceinline__ static Vec load_nt(const void* p) { return load16_nt(p); }
  __device__ __forceinline__ static void to_f32(const Vec& v, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v.w[e]);
  }
};

template <> struct Elem<BF16Tag> {
  using Vec = Vec16;
  static constexpr int kPerVec = 8;
  static constexpr int kBytes = 2;
  static constexpr int kQBytes = 2;
  __device__ __forceinline__ static Vec load_nt(const void* p) { return load16_nt(p); }
  __device__ __forceinline__ static void to_f32(const Vec& v, float* f) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f[2 * w] = bf16_lo(v.w[w]);
      f[2 * w + 1] = bf16_hi(v.w[w]);
    }
  }
};

template <> struct Elem<Fp8Tag> {
  using Vec = Vec8;
  static constexpr int kPerVec = 8;
  static constexpr int kBytes = 1;
  static constexpr int kQBytes = 2;
  __device__ __forceinline__ static Vec load_nt(const void* p) { return load8_nt(p); }
  // v_cvt_pk_f32_fp8: two codes (one 16-bit half of the word) per instruction, exact
  __device__ __forceinline__ static void to_f32(const Vec& v, float* f) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v.w[w]), false);
      const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v.w[w]), true);
      f[4 * w] = lo.x;
      f[4 * w + 1] = lo.y;
      f[4 * w + 2] = hi.x;
      f[4 * w + 3] = hi.y;
    }
  }
};

}  // namespace pa
