// Gating kernels: router GEMM + sigmoid, and group-limited top-k selection
// (onlylabs "DeepSeek v3 and R1 Model Architecture", "Local Balanced Routing to
// Experts": token-to-expert affinity plus a routing-only bias term).
#include <climits>

#include "common.h"
#include "launch.h"

namespace moefp8 {

// scores[t][e] = sigmoid(sum_d x[t][d] * w[e][d]); bf16 operands on the gfx950
// 16x16x32 bf16 MFMA, fp32 accumulation.  A workgroup is 4 waves over 64
// tokens (16 per wave) and shares one slice of 16*NT experts; operands are read
// straight from global memory (the slice of router weights stays in L2).
template <int NT>
__global__ __launch_bounds__(256) void router_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                     int T, int E, int D, float* __restrict__ scores) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * 64 + wave * 16;
  const int e0 = blockIdx.y * 16 * NT;
  const int ta = min(t0 + r16, T - 1);
  const uint16_t* xa = x + (long)ta * D + 8 * q;
  const uint16_t* wb[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) wb[j] = w + (long)(e0 + 16 * j + r16) * D + 8 * q;
  v4f acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < D; k += 32) {
    const v8bf a = *reinterpret_cast<const v8bf*>(xa + k);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const v8bf b = *reinterpret_cast<const v8bf*>(wb[j] + k);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
  }
  // lane holds rows (tokens) 4q..4q+3 of the wave's 16, column (expert) r16
#pragma unroll
  for (int j = 0; j < NT; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * q + i;
      if (t < T) scores[(long)t * E + e0 + 16 * j + r16] = 1.0f / (1.0f + expf(-acc[j][i]));
    }
  }
}

// One wave per token.  Biased scores live in LDS; lane g < n_group scores
// group g; groups are ranked with ties to the lower index; then top_k rounds
// of a wave-wide argmax (ties to the lower expert id) over the kept groups.
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ scores, const float* __restrict__ bias,
                                                    int T, int E, int k, int G, int gk, int rule, float routed_scale,
                                                    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  extern __shared__ float sh[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  const bool valid = t < T;
  float* b = sh + wave * E;
  const float* s = scores + (long)(valid ? t : 0) * E;
  for (int e = lane; e < E; e += 64) b[e] = s[e] + (bias ? bias[e] : 0.0f);
  __syncthreads();
  const int gsz = E / G;
  float gscore = -INFINITY;
  if (lane < G) {
    float t1 = -INFINITY, t2 = -INFINITY;
    for (int i = 0; i < gsz; ++i) {
      const float v = b[lane * gsz + i];
      if (v > t1) {
        t2 = t1;
        t1 = v;
      } else if (v > t2) {
        t2 = v;
      }
    }
    gscore = (rule == 1 || gsz == 1) ? t1 : t1 + t2;
  }
  int rank = 0;
  for (int g = 0; g < G; ++g) {
    const float o = __shfl(gscore, g);
    rank += (o > gscore || (o == gscore && g < lane)) ? 1 : 0;
  }
  const unsigned long long kept = __ballot(lane < G && rank < gk);
  unsigned taken = 0;   // bit i: expert lane + 64 i already chosen
  int mine = 0;
  for (int j = 0; j < k; ++j) {
    float best = -INFINITY;
    int bi = INT_MAX;
    for (int i = 0, e = lane; e < E; ++i, e += 64) {
      if (((kept >> (e / gsz)) & 1ull) && !((taken >> i) & 1u)) {
        const float v = b[e];
        if (v > best || (v == best && e < bi)) {
          best = v;
          bi = e;
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(best, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > best || (ov == best && oi < bi)) {
        best = ov;
        bi = oi;
      }
    }
    if (bi == INT_MAX) bi = 0;   // no candidate left: only with NaN scores, outside the contract
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) mine = bi;
  }
  // weights from the unbiased scores, normalised by their fp32 sum in slot order
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += s[__shfl(mine, j)];
  if (valid && lane < k) {
    topk_idx[(long)t * k + lane] = mine;
    topk_w[(long)t * k + lane] = (s[mine] / sum) * routed_scale;
  }
}

hipError_t launch_router(const uint16_t* x, const uint16_t* w, int T, int E, int D, float* scores, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const unsigned gx = (unsigned)((T + 63) / 64);
  if (E % 64 == 0 && T > 256) {
    router_kernel<4><<<dim3(gx, E / 64), 256, 0, st>>>(x, w, T, E, D, scores);
  } else {
    router_kernel<1><<<dim3(gx, E / 16), 256, 0, st>>>(x, w, T, E, D, scores);
  }
  return hipGetLastError();
}

hipError_t launch_route(const float* scores, const float* bias, int T, int E, int k, int G, int gk, int rule,
                        float routed_scale, int32_t* topk_idx, float* topk_w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  route_kernel<<<(T + 3) / 4, 256, 4 * E * sizeof(float), st>>>(scores, bias, T, E, k, G, gk, rule, routed_scale,
                                                                topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moefp8
