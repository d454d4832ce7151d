// Fine-granularity FP8 quantisation kernels (onlylabs "DeepSeek v3 and R1 Model
// Architecture", headings "Fine granularity quantization" and "Online
// Quantization"; aguasto "DeepSeek-R1", "Quantization": blockwise FP8).
//
// Per tile: amax = max |v|, s = fp32(amax / 448) (correctly rounded division),
// q = e4m3(fp32(v / s)); an all-zero tile has s = 1.
#include "common.h"
#include "launch.h"

namespace moefp8 {

// One 16-lane group per 128-wide tile (quant_1x128_tile), 16 tiles per workgroup.
template <bool kBf16>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const void* __restrict__ x, int rows, int cols, int ld_x,
                                                          uint8_t* __restrict__ q, int ld_q, float* __restrict__ s,
                                                          int pow2) {
  quant_1x128_tile<kBf16>(x, rows, cols, ld_x, q, ld_q, s, pow2, (long)blockIdx.x * 16 + (threadIdx.x >> 4),
                          threadIdx.x & 15);
}

// One workgroup per 128x128 block; thread t holds row t/2, columns (t%2)*64 .. +64;
// the block's amax is reduced per wave, then across the 4 waves through LDS.
__global__ __launch_bounds__(256) void quant_128x128_kernel(const float* __restrict__ w, int rows, int cols,
                                                            uint8_t* __restrict__ q, float* __restrict__ s, int pow2) {
  __shared__ float red[4];
  const int bc = blockIdx.x, br = blockIdx.y;
  const int tid = threadIdx.x;
  const int rr = tid >> 1;
  const int cc = (tid & 1) * 64;
  const float* src = w + (long)(br * 128 + rr) * cols + bc * 128 + cc;
  float v[64];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 a = reinterpret_cast<const float4*>(src)[i];
    v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = tile_scale(amax, pow2 != 0);
  uint8_t* dst = q + (long)(br * 128 + rr) * cols + bc * 128 + cc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t wd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* vv = v + 16 * i + 4 * j;
      wd[j] = e4m3_encode4(vv[0] / sc, vv[1] / sc, vv[2] / sc, vv[3] / sc);
    }
    reinterpret_cast<uint4*>(dst)[i] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }
  if (tid == 0) s[br * (cols >> 7) + bc] = sc;
}

// Row-major e4m3 [G][N][K] -> MFMA-fragment order.  Block (g, n16, kb) holds
// rows 16 n16 .. +15, columns 128 kb .. +127 in 2 KB: byte
// (h * 1024 + (16 q + r) * 16 + b) = B[16 n16 + r][128 kb + 64 h + 16 q + b], so
// lane l = r + 16 q of a 16x16x128 MFMA fragment finds its two 16-byte pieces at
// h * 1024 + 16 l: one wave-wide load covers 1 KB of consecutive bytes in lane
// order (bank-conflict free from LDS).
__global__ __launch_bounds__(256) void pack_kernel(const uint4* __restrict__ src, long nchunks, int N, int K,
                                                   uint4* __restrict__ dst) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;   // destination 16-byte chunk
  if (i >= nchunks) return;
  const int nkb = K >> 7;
  const long blk = i >> 7;                                // 2 KB block index (g, n16, kb)
  const int w = (int)(i & 127);
  const int h = w >> 6, r = w & 15, q = (w >> 4) & 3;
  const int kb = (int)(blk % nkb);
  const long gn16 = blk / nkb;                            // g * (N/16) + n16
  const long row = gn16 * 16 + r;                         // g * N + n
  dst[i] = src[(row * K + kb * 128 + 64 * h + 16 * q) >> 4];
}

hipError_t launch_pack(const uint8_t* src, int G, int N, int K, uint8_t* dst, hipStream_t st) {
  const long nchunks = (long)G * N * K / 16;
  if (nchunks == 0) return hipSuccess;
  pack_kernel<<<(unsigned)((nchunks + 255) / 256), 256, 0, st>>>(reinterpret_cast<const uint4*>(src), nchunks, N, K,
                                                                  reinterpret_cast<uint4*>(dst));
  return hipGetLastError();
}

hipError_t launch_quant_1x128(const void* x, bool bf16, int rows, int cols, int ld_x, uint8_t* q, int ld_q, float* s,
                              bool pow2, hipStream_t st) {
  const long ntiles = (long)rows * (cols / 128);
  if (ntiles == 0) return hipSuccess;
  const unsigned grid = (unsigned)((ntiles + 15) / 16);
  if (bf16)
    quant_1x128_kernel<true><<<grid, 256, 0, st>>>(x, rows, cols, ld_x, q, ld_q, s, pow2);
  else
    quant_1x128_kernel<false><<<grid, 256, 0, st>>>(x, rows, cols, ld_x, q, ld_q, s, pow2);
  return hipGetLastError();
}

hipError_t launch_quant_128x128(const float* w, int rows, int cols, uint8_t* q, float* s, bool pow2, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  dim3 grid(cols / 128, rows / 128);
  quant_128x128_kernel<<<grid, 256, 0, st>>>(w, rows, cols, q, s, pow2);
  return hipGetLastError();
}

// Exactly rounded fp64 sum of the squares of a bf16 row (cols = 128 * tpr), for the
// workgroup of rmsnorm_quant_kernel: double-double (TwoSum) accumulation per lane, the
// same through the wave and across the 4 waves (red_hi / red_lo: 4 doubles each in LDS).
// Every thread returns the sum.  It runs only when the plain fp64 sum cannot decide the
// fp32 result, and reads the row again from memory (L2) rather than from the caller's
// registers, which keeps the common path's register count (and occupancy) as it is.
__device__ __forceinline__ double exact_row_sum(const uint16_t* xr, int tpr, double* red_hi, double* red_lo) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = tid >> 4, sub = tid & 15;
  double hi = 0.0, lo = 0.0;
  for (int tc = grp; tc < tpr; tc += 16) {
    const uint4 p = *reinterpret_cast<const uint4*>(xr + tc * 128 + sub * 8);
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const double v = (double)__uint_as_float(h ? (w[i] & 0xFFFF0000u) : (w[i] << 16));
        double t, e;
        two_sum(hi, v * v, t, e);
        hi = t;
        lo += e;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double oh = __shfl_xor(hi, o), ol = __shfl_xor(lo, o);
    double t, e;
    two_sum(hi, oh, t, e);
    hi = t;
    lo = lo + ol + e;
  }
  if (lane == 0) {
    red_hi[wave] = hi;
    red_lo[wave] = lo;
  }
  __syncthreads();
  hi = red_hi[0];
  lo = red_lo[0];
#pragma unroll
  for (int w2 = 1; w2 < 4; ++w2) {
    double t, e;
    two_sum(hi, red_hi[w2], t, e);
    hi = t;
    lo = lo + red_lo[w2] + e;
  }
  return hi + lo;
}

// RMSNorm fused with the 1x128 quantisation (llm-architectures-explained,
// "DeepSeek-R1", facts rows "Norm placement" / "Norm type": RMSNorm right before
// the MLP).  One workgroup (16 groups of 16 lanes) per row; group g handles the
// 128-column tiles g, g + 16, ...; each lane 8 consecutive values of a tile.
//   the sum of squares: squares of bf16 values are exact in fp64.  The sum is
//     first taken with plain fp64 adds; its relative error is below cols * 2^-53
//     whatever the order, so fp32(inv) below is the one the exact sum gives
//     unless the fp64 inv lies that close to a rounding midpoint of the fp32
//     grid.  Then (rarely; a uniform branch for the workgroup) the sum is taken
//     again in double-double (TwoSum per lane, pairwise reduction), which gives
//     the exactly rounded fp64 sum for any realistic row, so the result never
//     depends on the summation order;
//   inv = fp32(1 / sqrt(sum / cols + eps)) in fp64;
//   y = bf16(fp32(fp32(x * inv) * gamma)), written out if asked, and quantised
//     per 128 columns like quant_1x128.
// NT > 0: the row stays in registers between the two steps (NT tiles per group,
// cols <= 16 * NT * 128), one read of x; NT == 0: any width, the second step
// reads the row again (from L2).
template <int NT>
__global__ __launch_bounds__(256) void rmsnorm_quant_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ gamma, float eps, int cols,
                                                            int ld_x, uint16_t* __restrict__ y, int ld_y,
                                                            uint8_t* __restrict__ q, int ld_q, float* __restrict__ s,
                                                            int pow2) {
  constexpr int R = NT > 0 ? NT : 1;
  __shared__ double red_hi[4], red_lo[4];
  const long row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = tid >> 4, sub = tid & 15;
  const int tpr = cols >> 7;
  const uint16_t* xr = x + row * ld_x;
  uint4 keep[R], gkeep[R];                      // the row's x and gamma pieces (NT > 0)
  if constexpr (NT > 0) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int tc = grp + 16 * i;
      keep[i] = tc < tpr ? *reinterpret_cast<const uint4*>(xr + tc * 128 + sub * 8) : make_uint4(0, 0, 0, 0);
      // gamma is read before the reduction, so its latency hides under the row's
      gkeep[i] = tc < tpr ? *reinterpret_cast<const uint4*>(gamma + tc * 128 + sub * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  // the row's sum of squares with plain fp64 adds
  double hi = 0.0;
  auto accumulate = [&](const uint4 p) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double a = (double)__uint_as_float(w[i] << 16), b = (double)__uint_as_float(w[i] & 0xFFFF0000u);
      hi += a * a;
      hi += b * b;
    }
  };
  if constexpr (NT > 0) {
#pragma unroll
    for (int i = 0; i < NT; ++i) accumulate(keep[i]);       // zeros add nothing
  } else {
    for (int tc = grp; tc < tpr; tc += 16) accumulate(*reinterpret_cast<const uint4*>(xr + tc * 128 + sub * 8));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) hi += __shfl_xor(hi, o);
  if (lane == 0) red_hi[wave] = hi;
  __syncthreads();
  const double ss_fast = ((red_hi[0] + red_hi[1]) + red_hi[2]) + red_hi[3];
  const double inv64 = 1.0 / sqrt(ss_fast / (double)cols + (double)eps);
  float inv = (float)inv64;
  {
    // distance of inv64 from the fp32 rounding midpoints on either side of inv, against a
    // bound on the fast sum's effect (relative error < (cols / 2 + 3) * 2^-53 in inv64)
    const uint32_t ib = __float_as_uint(inv);
    const double below = 0.5 * ((double)inv + (double)__uint_as_float(ib - 1u));
    const double above = 0.5 * ((double)inv + (double)__uint_as_float(ib + 1u));
    const double margin = fmin(inv64 - below, above - inv64);
    if (margin <= inv64 * ((double)cols * 0x1p-53 + 0x1p-50)) {   // same value in every thread
      __syncthreads();                         // every thread has read the fast sum's partials
      inv = (float)(1.0 / sqrt(exact_row_sum(xr, tpr, red_hi, red_lo) / (double)cols + (double)eps));
    }
  }

  auto emit = [&](int tc, const uint4 px, const uint4 pg) {
    const int c0 = tc * 128 + sub * 8;
    const uint32_t wx[4] = {px.x, px.y, px.z, px.w}, wg[4] = {pg.x, pg.y, pg.z, pg.w};
    float v[8];
    uint32_t yb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t pair = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float xv = __uint_as_float(h ? (wx[i] & 0xFFFF0000u) : (wx[i] << 16));
        const float gv = __uint_as_float(h ? (wg[i] & 0xFFFF0000u) : (wg[i] << 16));
        const float t = xv * inv;
        const uint16_t b = f32_to_bf16_rne(t * gv);
        v[2 * i + h] = bf16_to_f32(b);
        pair |= (uint32_t)b << (16 * h);
      }
      yb[i] = pair;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = group_max<16>(amax);
    const float sc = tile_scale(amax, pow2 != 0);
    const uint32_t lo4 = e4m3_encode4(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc);
    const uint32_t hi4 = e4m3_encode4(v[4] / sc, v[5] / sc, v[6] / sc, v[7] / sc);
    if (y) *reinterpret_cast<uint4*>(y + row * ld_y + c0) = make_uint4(yb[0], yb[1], yb[2], yb[3]);
    *reinterpret_cast<uint2*>(q + row * ld_q + c0) = make_uint2(lo4, hi4);
    if (sub == 0) s[row * tpr + tc] = sc;
  };
  if constexpr (NT > 0) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
      if (grp + 16 * i < tpr) emit(grp + 16 * i, keep[i], gkeep[i]);   // uniform within each 16-lane group
  } else {
    for (int tc = grp; tc < tpr; tc += 16)
      emit(tc, *reinterpret_cast<const uint4*>(xr + tc * 128 + sub * 8),
           *reinterpret_cast<const uint4*>(gamma + tc * 128 + sub * 8));
  }
}

hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps, int rows, int cols, int ld_x,
                                uint16_t* y, int ld_y, uint8_t* q, int ld_q, float* s, bool pow2, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (cols <= 16 * 4 * 128)
    rmsnorm_quant_kernel<4><<<rows, 256, 0, st>>>(x, gamma, eps, cols, ld_x, y, ld_y, q, ld_q, s, pow2);
  else
    rmsnorm_quant_kernel<0><<<rows, 256, 0, st>>>(x, gamma, eps, cols, ld_x, y, ld_y, q, ld_q, s, pow2);
  return hipGetLastError();
}

}  // namespace moefp8
