// Device helpers shared by the gfx950 kernels of libmoefp8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moefp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // 16 bytes in registers
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// OCP E4M3FN encoding of two fp32 values: round to nearest, ties to even mantissa,
// sign kept, saturating at 448 (0x7E), NaN -> 0x7F | sign.  The gfx950 conversion
// instruction (v_cvt_pk_fp8_f32) rounds to nearest even into the OCP format; the
// values are clamped to +-448 first (the format has no infinity, so saturation is
// the clamp) and NaN inputs are patched after.  Returns code(a) | code(b) << 8.
__device__ __forceinline__ uint32_t e4m3_encode2(float a, float b) {
  const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  const float cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
  const uint32_t na = ((__float_as_uint(a) >> 24) & 0x80u) | 0x7Fu;
  const uint32_t nb = ((__float_as_uint(b) >> 16) & 0x8000u) | 0x7F00u;
  r = a != a ? (r & 0xFF00u) | na : r;
  r = b != b ? (r & 0x00FFu) | nb : r;
  return r;
}

__device__ __forceinline__ uint32_t e4m3_encode(float f) { return e4m3_encode2(f, 0.0f) & 0xFFu; }

// Codes of four values packed into a word, v0 in the low byte.
__device__ __forceinline__ uint32_t e4m3_encode4(float v0, float v1, float v2, float v3) {
  return e4m3_encode2(v0, v1) | (e4m3_encode2(v2, v3) << 16);
}

// Scale of one quantisation tile (amax >= 0): fp32(amax / 448), correctly rounded, and at least
// the smallest normal fp32 2^-126 (so that v / s stays within +-448 and 1 / s is finite even for
// tiles of subnormal values); or, with pow2 (power-of-two "UE8M0" scales), the smallest 2^k,
// k in [-127, 127], with amax <= 448 * 2^k.  For amax = m * 2^E (m in [1, 2)),
// 448 * 2^k = 1.75 * 2^(k + 8) covers amax exactly when k >= E - 8, or k >= E - 7 when m > 1.75;
// subnormal amax takes the clamp.  1 for amax == 0.
__device__ __forceinline__ float tile_scale(float amax, bool pow2) {
  if (amax == 0.0f) return 1.0f;
  if (!pow2) {
    const float s = amax / 448.0f;
    return s < 0x1p-126f ? 0x1p-126f : s;       // (a NaN amax stays NaN)
  }
  const uint32_t b = __float_as_uint(amax);
  const int ef = (int)(b >> 23);
  int k = ef == 0 ? -127 : ef - 135 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  k = k < -127 ? -127 : (k > 127 ? 127 : k);
  return k >= -126 ? __uint_as_float((uint32_t)(k + 127) << 23) : __uint_as_float(0x400000u);   // 2^-127: subnormal
}

// Error-free sum (Knuth's TwoSum): s + e == a + b exactly, s = fl(a + b).
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// 8 e4m3 bytes (two dwords) -> 8 bf16.  Every e4m3 value, subnormals included,
// is exactly representable in bf16 (3 <= 7 fraction bits, 2^-9 .. 448 in range),
// so the conversion (gfx950 v_cvt_scalef32_pk_bf16_fp8 with scale 1) is exact.
__device__ __forceinline__ v8bf e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return v8bf{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// The same with the values multiplied by a power of two `scale` during the conversion (gfx950
// v_cvt_scalef32_pk_bf16_fp8): exact while the scaled values stay in bf16's normal range.
__device__ __forceinline__ v8bf e4m3x8_to_bf16_scaled(uint32_t w0, uint32_t w1, float scale) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true);
  return v8bf{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// E8M0 byte of a power-of-two fp32 scale 2^k, k in [-127, 127]: the biased exponent k + 127
// (2^-127 is the fp32 subnormal 0x00400000, whose exponent field 0 is that byte too).
__device__ __forceinline__ int e8m0_of(float pow2) { return (int)(__float_as_uint(pow2) >> 23); }

template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, W));
  return v;
}

__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

// 1x128 quantisation of tile `tile` (row-major over rows x cols / 128 tiles) by a 16-lane group,
// lane `sub` holding 8 consecutive elements (one 16-byte load for bf16, two for fp32; one 8-byte
// store of codes): amax = max |v|, s = fp32(amax / 448) (correctly rounded division),
// q = e4m3(fp32(v / s)); an all-zero tile has s = 1.  Every lane of the group must call it (the
// amax is reduced across the group); a tile index past the end stores nothing.
template <bool kBf16>
__device__ __forceinline__ void quant_1x128_tile(const void* __restrict__ x, int rows, int cols, int ld_x,
                                                 uint8_t* __restrict__ q, int ld_q, float* __restrict__ s, int pow2,
                                                 long tile, int sub) {
  const int tpr = cols >> 7;
  const long ntiles = (long)rows * tpr;
  const bool valid = tile < ntiles;
  const long r = valid ? tile / tpr : 0;
  const int tc = valid ? (int)(tile - r * tpr) : 0;
  const int c0 = tc * 128 + sub * 8;
  float v[8];
  if (valid) {
    if (kBf16) {
      const uint4 p = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + r * ld_x + c0);
      const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + r * ld_x + c0);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = group_max<16>(amax);
  const float sc = tile_scale(amax, pow2 != 0);
  const uint32_t lo = e4m3_encode4(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc);
  const uint32_t hi = e4m3_encode4(v[4] / sc, v[5] / sc, v[6] / sc, v[7] / sc);
  if (valid) {
    *reinterpret_cast<uint2*>(q + r * ld_q + c0) = make_uint2(lo, hi);
    if (sub == 0) s[r * tpr + tc] = sc;
  }
}

// silu(z) * u in fp32: z / (1 + e^-z) * u, the quotient taken with the hardware reciprocal (1 ulp, like
// the exponential).  The result is requantised to e4m3, whose rounding absorbs errors of this size
// except within a few fp32 ulps of a rounding midpoint.
__device__ __forceinline__ float swiglu(float z, float u) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)) * u;
}

}  // namespace moefp8
