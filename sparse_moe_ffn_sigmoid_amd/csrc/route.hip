// Gating kernels: router GEMM + sigmoid, and group-limited top-k selection
// (onlylabs "DeepSeek v3 and R1 Model Architecture", "Local Balanced Routing to
// Experts": token-to-expert affinity plus a routing-only bias term).
#include <climits>

#include "common.h"
#include "launch.h"

namespace moefp8 {

// scores[t][e] = sigmoid(sum_d x[t][d] * w[e][d]); bf16 operands on the gfx950
// 16x16x32 bf16 MFMA, fp32 accumulation.  A workgroup covers 16*MTK tokens x
// 16*NT experts; its NW waves split the hidden dimension (in 32-wide steps) and
// add their partial logits through LDS in a fixed order (deterministic).  Each
// wave issues the loads of U steps before their MFMAs, straight from global
// memory (the router weights stay in L2).  Small batches use many waves per
// workgroup (the 3.7 MB of router weights spread over many CUs); large ones a
// 64 x 64 tile, so each token row is read once per 64 experts and each router
// weight row once per 64 tokens, with 8 waves (two per SIMD: 11 us faster than
// 4 at 4096 tokens, the loads being latency-bound).
template <int NW, int NT, int MTK, int U>
__global__ __launch_bounds__(64 * NW) void router_splitk_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ w, int T, int E, int D,
                                                                float* __restrict__ scores) {
  __shared__ v4f part[NW][MTK * NT][64];
  // wave-uniform wave index: the K-step bounds derive from it and guard MFMAs, which write every
  // lane whatever EXEC holds, so those branches must be scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * 16 * MTK, e0 = blockIdx.y * 16 * NT;
  const int steps = D >> 5;                     // 32-wide K steps, split as evenly as possible
  const int s0 = (steps * wave) / NW, s1 = (steps * (wave + 1)) / NW;
  const uint16_t* xa[MTK];
#pragma unroll
  for (int i = 0; i < MTK; ++i) xa[i] = x + (long)min(t0 + 16 * i + r16, T - 1) * D + 8 * q;
  const uint16_t* wb[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) wb[j] = w + (long)(e0 + 16 * j + r16) * D + 8 * q;
  v4f acc[MTK][NT];
#pragma unroll
  for (int i = 0; i < MTK; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  int k = s0;
  for (; k + U <= s1; k += U) {
    v8bf a[MTK][U], b[NT][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int i = 0; i < MTK; ++i) a[i][u] = *reinterpret_cast<const v8bf*>(xa[i] + 32 * (k + u));
#pragma unroll
      for (int j = 0; j < NT; ++j) b[j][u] = *reinterpret_cast<const v8bf*>(wb[j] + 32 * (k + u));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MTK; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][u], b[j][u], acc[i][j], 0, 0, 0);
  }
  if (k < s1) {                                 // the last, partial batch: all its loads first
    v8bf a[MTK][U] = {}, b[NT][U] = {};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k + u < s1) {
#pragma unroll
        for (int i = 0; i < MTK; ++i) a[i][u] = *reinterpret_cast<const v8bf*>(xa[i] + 32 * (k + u));
#pragma unroll
        for (int j = 0; j < NT; ++j) b[j][u] = *reinterpret_cast<const v8bf*>(wb[j] + 32 * (k + u));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k + u < s1) {
#pragma unroll
        for (int i = 0; i < MTK; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][u], b[j][u], acc[i][j], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < MTK; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) part[wave][i * NT + j][lane] = acc[i][j];
  __syncthreads();
  // tile (i, j) is finished by wave (i * NT + j) % NW: fixed-order sum over the waves, then the sigmoid
  for (int tile = wave; tile < MTK * NT; tile += NW) {
    v4f t = part[0][tile][lane];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) t += part[w2][tile][lane];
    const int i = tile / NT, j = tile % NT;
    // lane holds rows (tokens) 4q..4q+3 of token tile i, column (expert) r16 of expert tile j
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tt = t0 + 16 * i + 4 * q + r;
      if (tt < T) scores[(long)tt * E + e0 + 16 * j + r16] = 1.0f / (1.0f + expf(-t[r]));
    }
  }
}

// Register-resident routing for the common layouts: lane l holds experts
// l*EPL .. l*EPL+EPL-1 (EPL = E/64, or 1 when E <= 64), a group is LPG
// consecutive lanes.  Group top-2 merges pairs across the group's lanes with
// xor shuffles; the top_k rounds are wave-wide argmaxes (ties to the lower id).
template <int EPL>
__global__ __launch_bounds__(256) void route_reg_kernel(const float* __restrict__ scores,
                                                        const float* __restrict__ bias, int T, int E, int k, int G,
                                                        int gk, int rule, float routed_scale,
                                                        int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;                               // whole wave: no block-level barrier below
  const float* s = scores + (long)t * E;
  const int e0 = lane * EPL;
  const bool live = e0 < E;
  float sv[EPL], b[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    sv[i] = live ? s[e0 + i] : 0.0f;
    b[i] = live ? sv[i] + (bias ? bias[e0 + i] : 0.0f) : -INFINITY;
  }
  const int gsz = E / G;
  const int lpg = gsz / EPL;                        // lanes per group (a power of two here)
  float t1 = b[0], t2 = -INFINITY;
#pragma unroll
  for (int i = 1; i < EPL; ++i) {
    if (b[i] > t1) {
      t2 = t1;
      t1 = b[i];
    } else if (b[i] > t2) {
      t2 = b[i];
    }
  }
  for (int o = 1; o < lpg; o <<= 1) {               // merge the two largest of two multisets
    const float u1 = __shfl_xor(t1, o), u2 = __shfl_xor(t2, o);
    const float hi = fmaxf(t1, u1), lo = fminf(t1, u1);
    t2 = fmaxf(lo, fmaxf(t2, u2));
    t1 = hi;
  }
  const float gscore = (rule == 1 || gsz == 1) ? t1 : t1 + t2;
  const int mygroup = lane / lpg;
  int rank = 0;
  for (int g = 0; g < G; ++g) {
    const float o = __shfl(gscore, g * lpg);
    rank += (o > gscore || (o == gscore && g < mygroup)) ? 1 : 0;
  }
  const bool kept = live && rank < gk;
  // each round's winner carries its unbiased score along, so the weights need no second
  // read of the scores
  unsigned taken = 0;
  int mine = 0;
  float mine_s = 0.0f;
  for (int j = 0; j < k; ++j) {
    float best = -INFINITY, best_s = 0.0f;
    int bi = INT_MAX;
    if (kept) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        if (!((taken >> i) & 1u) && (b[i] > best || bi == INT_MAX)) {
          best = b[i];
          best_s = sv[i];
          bi = e0 + i;
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(best, o), os = __shfl_xor(best_s, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > best || (ov == best && oi < bi)) {
        best = ov;
        best_s = os;
        bi = oi;
      }
    }
    if (bi == INT_MAX) bi = 0;                      // only with NaN scores, outside the contract
    if (bi >= e0 && bi < e0 + EPL) taken |= 1u << (bi - e0);
    if (lane == j) {
      mine = bi;
      mine_s = best_s;
    }
  }
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __shfl(mine_s, j);
  if (lane < k) {
    topk_idx[(long)t * k + lane] = mine;
    topk_w[(long)t * k + lane] = (mine_s / sum) * routed_scale;
  }
}

// General layouts (any E <= 1024 and group size): one wave per token.  Biased scores live in LDS; lane g < n_group scores
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
  if (T <= 512)
    router_splitk_kernel<16, 1, 1, 8><<<dim3((T + 15) / 16, E / 16), 1024, 0, st>>>(x, w, T, E, D, scores);
  else if (E % 64 == 0)
    router_splitk_kernel<8, 4, 4, 2><<<dim3((T + 63) / 64, E / 64), 512, 0, st>>>(x, w, T, E, D, scores);
  else
    router_splitk_kernel<4, 1, 4, 4><<<dim3((T + 63) / 64, E / 16), 256, 0, st>>>(x, w, T, E, D, scores);
  return hipGetLastError();
}

hipError_t launch_route(const float* scores, const float* bias, int T, int E, int k, int G, int gk, int rule,
                        float routed_scale, int32_t* topk_idx, float* topk_w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const unsigned grid = (unsigned)((T + 3) / 4);
  const int epl = E <= 64 ? 1 : E / 64;
  const bool reg_layout = (E <= 64 || E % 64 == 0) && (E / G) % epl == 0;
  const int lpg = reg_layout ? (E / G) / epl : 0;
  if (reg_layout && (lpg & (lpg - 1)) == 0 && (epl == 1 || epl == 2 || epl == 4 || epl == 8 || epl == 16)) {
    switch (epl) {
      case 1: route_reg_kernel<1><<<grid, 256, 0, st>>>(scores, bias, T, E, k, G, gk, rule, routed_scale, topk_idx, topk_w); break;
      case 2: route_reg_kernel<2><<<grid, 256, 0, st>>>(scores, bias, T, E, k, G, gk, rule, routed_scale, topk_idx, topk_w); break;
      case 4: route_reg_kernel<4><<<grid, 256, 0, st>>>(scores, bias, T, E, k, G, gk, rule, routed_scale, topk_idx, topk_w); break;
      case 8: route_reg_kernel<8><<<grid, 256, 0, st>>>(scores, bias, T, E, k, G, gk, rule, routed_scale, topk_idx, topk_w); break;
      default: route_reg_kernel<16><<<grid, 256, 0, st>>>(scores, bias, T, E, k, G, gk, rule, routed_scale, topk_idx, topk_w); break;
    }
  } else {
    route_kernel<<<grid, 256, 4 * E * sizeof(float), st>>>(scores, bias, T, E, k, G, gk, rule, routed_scale,
                                                           topk_idx, topk_w);
  }
  return hipGetLastError();
}

}  // namespace moefp8
