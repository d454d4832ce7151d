// Gating kernels: router GEMM + sigmoid, and group-limited top-k selection
// (onlylabs "DeepSeek v3 and R1 Model Architecture", "Local Balanced Routing to
// Experts": token-to-expert affinity plus a routing-only bias term).
#include <algorithm>
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
// PARTIAL: the hidden dimension is also split over gridDim.z workgroups (block z
// takes the z-th of gridDim.z near-equal ranges of K steps), each writing its raw
// partial logits to out[z][T][E]; router_finish_kernel adds them in order of z and
// applies the sigmoid.  Small batches use it, so that the router's loads are spread
// over every CU.
template <int NW, int NT, int MTK, int U, bool PARTIAL>
__global__ __launch_bounds__(64 * NW) void router_splitk_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ w, int T, int E, int D,
                                                                float* __restrict__ scores) {
  __shared__ v4f part[NW][MTK * NT][64];
  // wave-uniform wave index: the K-step bounds derive from it and guard MFMAs, which write every
  // lane whatever EXEC holds, so those branches must be scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * 16 * MTK, e0 = blockIdx.y * 16 * NT;
  // 32-wide K steps: this workgroup's range (all of them unless PARTIAL), split as evenly as
  // possible over its waves
  const int z = PARTIAL ? (int)blockIdx.z : 0, nz = PARTIAL ? (int)gridDim.z : 1;
  const int all = D >> 5, kz0 = (all * z) / nz, steps = (all * (z + 1)) / nz - kz0;
  const int s0 = kz0 + (steps * wave) / NW, s1 = kz0 + (steps * (wave + 1)) / NW;
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
      if (tt < T) {
        if constexpr (PARTIAL) scores[((long)z * T + tt) * E + e0 + 16 * j + r16] = t[r];
        else scores[(long)tt * E + e0 + 16 * j + r16] = 1.0f / (1.0f + expf(-t[r]));
      }
    }
  }
}

// Workgroup barrier after this wave's LDS accesses have completed (lgkmcnt(0)), leaving its global
// loads in flight (__syncthreads() would also wait for every one of them).
__device__ __forceinline__ void router_lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);           // vmcnt 63 and expcnt 7: no wait; lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Large batches: a workgroup of 8 waves covers 128 tokens x 256 experts, so each token row is read
// once and each router weight row once per 128 tokens; the hidden dimension goes through LDS in
// chunks of 64 (A 16 KB + B 32 KB per stage, two stages), each chunk's loads issued two chunks
// ahead into registers and written to LDS one chunk ahead.  Rows are stored as 128-byte lines with
// the 16-byte piece index XORed by row % 8, so a fragment read (16 rows, one piece) spreads over
// the banks.  Wave (wm, wn) computes tokens 64 wm .. +63 x experts 64 wn .. +63.  gridDim.z > 1
// splits the chunks into near-equal ranges over workgroups (raw partial logits to
// out[z][T][E], added in order of z by router_finish_kernel); with one range the kernel applies
// the sigmoid itself.  Every output is one MFMA chain in chunk order: deterministic.
__global__ __launch_bounds__(512) void router_lds_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w, int T, int E, int D,
                                                         float* __restrict__ out) {
  constexpr int A_BYTES = 128 * 128, STAGE = A_BYTES + 256 * 128;
  __shared__ __attribute__((aligned(16))) uint8_t lds0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[STAGE];
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, q = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), wm = wave & 1, wn = wave >> 1;
  const int t0 = blockIdx.x * 128, e0 = blockIdx.y * 256;
  const int z = blockIdx.z, nz = gridDim.z, nch = D >> 6;
  const int c0 = (nch * z) / nz, nk = (nch * (z + 1)) / nz - c0;   // >= 1: the host keeps nz <= nch
  // this thread's 16-byte pieces of a chunk: A (x) pieces tid and tid + 512 of 1024 (8 per row),
  // B (router weight) pieces tid + 512 i of 2048; sources clamp rows past the batch to its last
  const uint16_t* a_src[2];
  int a_dst[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + 512 * i, r = p >> 3, c = p & 7;
    a_src[i] = x + (long)min(t0 + r, T - 1) * D + (long)c0 * 64 + 8 * c;
    a_dst[i] = r * 128 + 16 * (c ^ (r & 7));
  }
  const uint16_t* b_src[4];
  int b_dst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 512 * i, r = p >> 3, c = p & 7;
    b_src[i] = w + (long)(e0 + r) * D + (long)c0 * 64 + 8 * c;
    b_dst[i] = A_BYTES + r * 128 + 16 * (c ^ (r & 7));
  }
  // chunk j of this range into registers (past the range: its last chunk again, never stored)
  auto gload = [&](int j, u32x4 (&ra)[2], u32x4 (&rb)[4]) __attribute__((always_inline)) {
    const long off = (long)min(j, nk - 1) * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = *reinterpret_cast<const u32x4*>(b_src[i] + off);
  };
  auto swrite = [&](uint8_t* st, const u32x4 (&ra)[2], const u32x4 (&rb)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(st + a_dst[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(st + b_dst[i]) = rb[i];
  };
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // the lane's fragment rows: token 64 wm + 16 i + r16, expert 64 wn + 16 j + r16 (row % 8 = r16 % 8)
  const int swz = r16 & 7;
  auto compute = [&](const uint8_t* st) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {               // two 32-wide K steps per chunk
      const int piece = 16 * ((4 * s + q) ^ swz);
      v8bf a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const v8bf*>(st + (64 * wm + 16 * i + r16) * 128 + piece);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const v8bf*>(st + A_BYTES + (64 * wn + 16 * j + r16) * 128 + piece);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };
  u32x4 ra0[2], rb0[4], ra1[2], rb1[4];
  gload(0, ra0, rb0);
  gload(1, ra1, rb1);
  swrite(lds0, ra0, rb0);
  gload(2, ra0, rb0);
  router_lds_barrier();
  // at the top of each round: stage 0 holds chunk c, registers set 1 chunk c + 1 and set 0 chunk
  // c + 2 (both in flight)
  int c = 0;
  for (; c + 2 <= nk; c += 2) {
    compute(lds0);
    swrite(lds1, ra1, rb1);
    gload(c + 3, ra1, rb1);
    router_lds_barrier();
    compute(lds1);
    swrite(lds0, ra0, rb0);
    gload(c + 4, ra0, rb0);
    router_lds_barrier();
  }
  if (c < nk) compute(lds0);                    // an odd count: the last chunk
  // lane holds tokens 4q .. 4q + 3 of token tile i, expert r16 of expert tile j
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tt = t0 + 64 * wm + 16 * i + 4 * q + r;
      if (tt < T) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = e0 + 64 * wn + 16 * j + r16;
          const float v = acc[i][j][r];
          if (nz > 1) out[((long)z * T + tt) * E + e] = v;
          else out[(long)tt * E + e] = 1.0f / (1.0f + expf(-v));
        }
      }
    }
}

// Wave-wide maximum of a 64-bit key, every lane receiving it: DPP exchanges within each row of 16
// lanes (pairs, quads, half rows mirrored, rows mirrored), then the four rows' maxima read as
// scalars.  DPP moves are VALU operations; the LDS-routed lane shuffles they replace wait on the
// LDS pipe at every step of the argmax rounds below.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, true);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o = dpp_u64<0xB1>(v);                  // quad_perm [1, 0, 3, 2]
  v = o > v ? o : v;
  o = dpp_u64<0x4E>(v);                           // quad_perm [2, 3, 0, 1]
  v = o > v ? o : v;
  o = dpp_u64<0x141>(v);                          // row_half_mirror
  v = o > v ? o : v;
  o = dpp_u64<0x140>(v);                          // row_mirror
  v = o > v ? o : v;
  uint64_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * i) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * i);
  const uint64_t a = r[0] > r[1] ? r[0] : r[1], b = r[2] > r[3] ? r[2] : r[3];
  return a > b ? a : b;
}

// Order-preserving key of a biased score and its expert: a larger score wins, equal scores (-0 and
// +0 equal) go to the lower expert id; 0 is below every key.
__device__ __forceinline__ uint64_t route_key(float b, int e) {
  const uint32_t f = __float_as_uint(b + 0.0f);   // -0 -> +0
  const uint32_t u = (f & 0x80000000u) ? ~f : (f | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0x7FFFFFFF - e);
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
  for (int g = 0; g < G; ++g) {                     // g * lpg is the same in every lane: a scalar read
    const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gscore), g * lpg));
    rank += (o > gscore || (o == gscore && g < mygroup)) ? 1 : 0;
  }
  const bool kept = live && rank < gk;
  // each round's winner carries its unbiased score along (read from the lane that holds it), so
  // the weights need no second read of the scores
  unsigned taken = 0;
  int mine = 0;
  float mine_s = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t key = 0;
    float key_s = 0.0f;
    if (kept) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const uint64_t c = route_key(b[i], e0 + i);
        if (!((taken >> i) & 1u) && c > key) {
          key = c;
          key_s = sv[i];
        }
      }
    }
    const uint64_t best = wave_max_u64(key);
    // no candidate left: only with NaN scores, outside the contract
    const int bi = best ? 0x7FFFFFFF - (int)(uint32_t)best : 0;
    const float best_s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(key_s), bi / EPL));
    if (bi >= e0 && bi < e0 + EPL) taken |= 1u << (bi - e0);
    if (lane == j) {
      mine = bi;
      mine_s = best_s;
    }
  }
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine_s), j));
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

// scores = sigmoid(part[0] + part[1] + ... + part[nz-1]), added in that order; n = T * E (a
// multiple of 4), float4 i of them.
__device__ __forceinline__ void finish_logits(const float* __restrict__ part, int nz, long n,
                                              float* __restrict__ scores, long i) {
  if (4 * i >= n) return;
  v4f a = reinterpret_cast<const v4f*>(part)[i];
  for (int z = 1; z < nz; ++z) a += reinterpret_cast<const v4f*>(part + z * n)[i];
  v4f o;
#pragma unroll
  for (int r = 0; r < 4; ++r) o[r] = 1.0f / (1.0f + expf(-a[r]));
  reinterpret_cast<v4f*>(scores)[i] = o;
}

__global__ __launch_bounds__(256) void router_finish_kernel(const float* __restrict__ part, int nz, long n,
                                                            float* __restrict__ scores) {
  finish_logits(part, nz, n, scores, blockIdx.x * 256L + threadIdx.x);
}

// The same, with the layer input's 1x128 quantisation in the workgroups past the first nfin
// (16 tiles each, as quant_1x128_kernel): both are short and latency-bound at small batches,
// and neither reads what the other writes, so one launch does both.
__global__ __launch_bounds__(256) void router_finish_quant_kernel(const float* __restrict__ part, int nz, long n,
                                                                  float* __restrict__ scores, unsigned nfin,
                                                                  const uint16_t* __restrict__ x, int rows, int cols,
                                                                  uint8_t* __restrict__ q, float* __restrict__ s,
                                                                  int pow2) {
  if (blockIdx.x < nfin) {
    finish_logits(part, nz, n, scores, blockIdx.x * 256L + threadIdx.x);
    return;
  }
  quant_1x128_tile<true>(x, rows, cols, cols, q, cols, s, pow2, (long)(blockIdx.x - nfin) * 16 + (threadIdx.x >> 4),
                         threadIdx.x & 15);
}

// Up to 512 tokens: 16 x 16 tiles of 16 waves; with a partial-logit buffer of kRouterSplit * T * E
// floats (the forward lends one) and a hidden dimension of at least 4096 the hidden dimension is
// also split 4 ways (at T = 64: 256 workgroups instead of 64).  Larger batches with a
// partial-logit buffer (the forward's) and a multiple of 256 experts: router_lds_kernel, its K
// range split over up to 16 workgroups so that the grid fills the chip (T = 4096: 32 token tiles
// x 8); V3 router,
// route + permutation stage: T = 1280 0.079 -> 0.050 ms, 4096 0.083 -> 0.067, 16384 0.271 ->
// 0.134.  Otherwise (moe_route's router, other expert counts) the 16 x 16 tiles up to 1024 tokens
// (at T = 640 the route + permutation stage took 68 against 80 us with the 64 x 64 tiles, equal
// at 1024, 80 against 109 us at 1536), then 64 x 64 token x expert tiles.
constexpr int kRouterSplit = 4, kRouterLdsSplitMax = 16;

bool router_small_split(int T, int E, int D, const float* part, size_t part_floats) {
  return T > 0 && T <= 512 && part && D >= 4096 && part_floats >= (size_t)kRouterSplit * (size_t)T * (size_t)E;
}

hipError_t launch_router(const uint16_t* x, const uint16_t* w, int T, int E, int D, float* scores, float* part,
                         size_t part_floats, const RouterQuant* xq, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const long n = (long)T * E;
  if (router_small_split(T, E, D, part, part_floats)) {
    router_splitk_kernel<16, 1, 1, 8, true><<<dim3((T + 15) / 16, E / 16, kRouterSplit), 1024, 0, st>>>(x, w, T, E, D,
                                                                                                         part);
    const unsigned nfin = (unsigned)((n / 4 + 255) / 256);
    if (xq) {
      const long ntiles = (long)T * (D / 128);
      router_finish_quant_kernel<<<nfin + (unsigned)((ntiles + 15) / 16), 256, 0, st>>>(
          part, kRouterSplit, n, scores, nfin, x, T, D, xq->q, xq->s, xq->pow2 ? 1 : 0);
    } else {
      router_finish_kernel<<<nfin, 256, 0, st>>>(part, kRouterSplit, n, scores);
    }
  } else if (T > 512 && part && E % 256 == 0 && D % 64 == 0) {
    const int tiles = ((T + 127) / 128) * (E / 256);
    int nz = std::min(kRouterLdsSplitMax, std::max(1, 256 / tiles));
    nz = (int)std::min<size_t>((size_t)std::min(nz, D / 64), part_floats / (size_t)n);
    const dim3 grid((T + 127) / 128, E / 256, nz > 1 ? nz : 1);
    if (nz > 1) {
      router_lds_kernel<<<grid, 512, 0, st>>>(x, w, T, E, D, part);
      router_finish_kernel<<<(unsigned)((n / 4 + 255) / 256), 256, 0, st>>>(part, nz, n, scores);
    } else {
      router_lds_kernel<<<grid, 512, 0, st>>>(x, w, T, E, D, scores);
    }
  } else if (T <= 1024) {
    router_splitk_kernel<16, 1, 1, 8, false><<<dim3((T + 15) / 16, E / 16), 1024, 0, st>>>(x, w, T, E, D, scores);
  } else if (E % 64 == 0) {
    router_splitk_kernel<8, 4, 4, 2, false><<<dim3((T + 63) / 64, E / 64), 512, 0, st>>>(x, w, T, E, D, scores);
  } else {
    router_splitk_kernel<4, 1, 4, 4, false><<<dim3((T + 63) / 64, E / 16), 256, 0, st>>>(x, w, T, E, D, scores);
  }
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
