// Sorting token-expert assignments by expert (stable: by expert, then by
// assignment index a = t*k + j) and the inverse / weighted combine.
//
// Deterministic three-pass counting sort over chunks of 1024 assignments:
//   count   - per-chunk expert histogram (LDS atomics: counts do not depend on order);
//   scan    - per expert, exclusive prefix over chunks; offsets = exclusive scan over experts;
//   scatter - each wave ranks its 64 lanes among equal expert ids with ballots
//             (lower lane first) and places them after everything earlier.
#include "common.h"
#include "launch.h"

namespace moefp8 {

constexpr int kChunk = 1024;          // assignments per workgroup (4 waves x 4 steps x 64 lanes)

__global__ __launch_bounds__(256) void perm_count_kernel(const int32_t* __restrict__ idx, int n, int E,
                                                         int32_t* __restrict__ chunk_counts) {
  extern __shared__ int cnt[];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int a0 = c * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += 256) {
    const int a = a0 + i;
    if (a < n) atomicAdd(&cnt[idx[a]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(long)c * E + e] = cnt[e];
}

// One workgroup of 1024 threads.  chunk_counts becomes the exclusive prefix over
// chunks (per expert); offsets[e] = exclusive prefix over experts, offsets[E] = n.
// A thread reads its expert's counts 16 chunks at a time before writing their
// prefixes, so a batch costs one memory round trip (V3 prefill, 32 chunks: a
// load-store chain per chunk took 10 us).
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ chunk_counts, int nchunks, int E,
                                                         int32_t* __restrict__ offsets) {
  constexpr int kBatch = 16;
  __shared__ int tot[1024];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = c0 + j < nchunks ? chunk_counts[(long)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (c0 + j < nchunks) chunk_counts[(long)(c0 + j) * E + e] = run;
        run += v[j];
      }
    }
  }
  tot[e] = run;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {   // inclusive Hillis-Steele scan
    const int v = e >= o ? tot[e - o] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  if (e < E) offsets[e] = tot[e] - run;
  if (e == E - 1) offsets[E] = tot[e];
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ idx, int n, int k, int E,
                                                           const int32_t* __restrict__ chunk_base,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_assign,
                                                           int32_t* __restrict__ assign_pos,
                                                           int32_t* __restrict__ sorted_token,
                                                           const float* __restrict__ topk_w,
                                                           float* __restrict__ sorted_w) {
  extern __shared__ int wcnt[];      // [4][E]: per wave, then start position per (wave, expert)
  const int c = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int* mycnt = wcnt + wave * E;
  for (int e = lane; e < E; e += 64) mycnt[e] = 0;
  __syncthreads();
  const int a_wave = c * kChunk + wave * 256;
  for (int s = 0; s < 4; ++s) {
    const int a = a_wave + s * 64 + lane;
    if (a < n) atomicAdd(&mycnt[idx[a]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    int run = offsets[e] + chunk_base[(long)c * E + e];
    for (int w = 0; w < 4; ++w) {
      const int v = wcnt[w * E + e];
      wcnt[w * E + e] = run;
      run += v;
    }
  }
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
  int nbits = 1;
  while ((1 << nbits) <= E) ++nbits;   // enough bits for ids 0..E (E marks an idle lane)
  for (int s = 0; s < 4; ++s) {
    const int a = a_wave + s * 64 + lane;
    const bool valid = a < n;
    const int e = valid ? idx[a] : E;
    unsigned long long peers = ~0ull;
    for (int bit = 0; bit < nbits; ++bit) {
      const unsigned long long m = __ballot((e >> bit) & 1);
      peers &= ((e >> bit) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    const int gsize = __popcll(peers);
    int pos = 0;
    if (valid) pos = mycnt[e] + rank;
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == gsize - 1) mycnt[e] += gsize;
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      sorted_assign[pos] = a;
      assign_pos[a] = pos;
      if (sorted_token) sorted_token[pos] = a / k;
      if (sorted_w) sorted_w[pos] = topk_w[a];
    }
  }
}

// Small batches (n <= kSmallN, E <= kSmallE): the whole counting sort in one
// workgroup of 1024 threads (16 waves): LDS histogram, block scan into the
// offsets, then per 1024-assignment chunk: ballot ranks inside each wave, a
// prefix over the 16 waves per expert, positions = running base + prefix + rank.
// Beyond 2048 assignments the multi-workgroup path is faster (V3 layer, route +
// permutation: 4096 assignments 61.6 -> 59.0 us, 8192: 90.7 -> 77.8 us; 3072: 50.4
// against 51.1 us; measured on one box).
constexpr int kSmallN = 2048;
constexpr int kSmallE = 512;

__global__ __launch_bounds__(1024) void perm_small_kernel(const int32_t* __restrict__ idx, int n, int k, int E,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_assign,
                                                          int32_t* __restrict__ assign_pos,
                                                          int32_t* __restrict__ sorted_token,
                                                          const float* __restrict__ topk_w,
                                                          float* __restrict__ sorted_w) {
  __shared__ int base[kSmallE];
  __shared__ int wcnt[16][kSmallE];
  __shared__ int scan[1024];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e < E; e += 1024) base[e] = 0;
  __syncthreads();
  for (int a = tid; a < n; a += 1024) atomicAdd(&base[idx[a]], 1);
  __syncthreads();
  const int cnt = tid < E ? base[tid] : 0;
  scan[tid] = cnt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? scan[tid - o] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  if (tid < E) {
    base[tid] = scan[tid] - cnt;                    // exclusive prefix: first sorted row of expert tid
    offsets[tid] = scan[tid] - cnt;
  }
  if (tid == 0) offsets[E] = n;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int nbits = 1;
  while ((1 << nbits) <= E) ++nbits;
  for (int c0 = 0; c0 < n; c0 += 1024) {
    for (int i = tid; i < 16 * E; i += 1024) wcnt[i / E][i % E] = 0;
    __syncthreads();
    const int a = c0 + tid;
    const bool valid = a < n;
    const int e = valid ? idx[a] : E;
    unsigned long long peers = ~0ull;
    for (int bit = 0; bit < nbits; ++bit) {
      const unsigned long long m = __ballot((e >> bit) & 1);
      peers &= ((e >> bit) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    const int gsize = __popcll(peers);
    if (valid && rank == gsize - 1) wcnt[wave][e] = gsize;
    __syncthreads();
    for (int ee = tid; ee < E; ee += 1024) {
      int run = base[ee];
      for (int w = 0; w < 16; ++w) {
        const int v = wcnt[w][ee];
        wcnt[w][ee] = run;
        run += v;
      }
      base[ee] = run;
    }
    __syncthreads();
    if (valid) {
      const int pos = wcnt[wave][e] + rank;
      sorted_assign[pos] = a;
      assign_pos[a] = pos;
      if (sorted_token) sorted_token[pos] = a / k;
      if (sorted_w) sorted_w[pos] = topk_w[a];
    }
    __syncthreads();
  }
}

// rows_out[p] = rows_in[sorted_assign[p] / k], row_bytes % 16 == 0.
__global__ __launch_bounds__(256) void perm_gather_kernel(const uint4* __restrict__ rows_in, int row_vec, int n, int k,
                                                          const int32_t* __restrict__ sorted_assign,
                                                          uint4* __restrict__ rows_out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long total = (long)n * row_vec;
  if (i >= total) return;
  const long p = i / row_vec;
  const int c = (int)(i - p * row_vec);
  rows_out[i] = rows_in[(long)(sorted_assign[p] / k) * row_vec + c];
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));   // 8 bytes in registers

// 16 bytes read exactly once: a nontemporal load.
__device__ __forceinline__ float4 load_once(const float* p) {
  const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// out[t][c] = bf16(sum_j w[t][j] * y[assign_pos[t*k+j]][c] (+ shared[t][c])), fp32, slot order.
// KT > 0: k fixed at compile time, so a thread has all its index loads, then all its row loads, in
// flight together (two memory round trips); KT == 0: k at run time.  The sum is taken in the same
// order either way.  Every y and shared byte is read exactly once, so the rows are read with
// nontemporal loads (V3 prefill: 218 -> 197 us).
template <int KT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ ap,
                                                      const float* __restrict__ w, const float* __restrict__ shared,
                                                      int T, int k, int d, uint16_t* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;       // one float4 of output per thread
  const int dv = d >> 2;
  if (i >= (long)T * dv) return;
  const long t = i / dv;
  const int c = (int)(i - t * dv) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float wj, const float4& v) {
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  };
  if constexpr (KT > 0) {
    int pos[KT];
    float wv[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      pos[j] = ap[t * KT + j];
      wv[j] = w[t * KT + j];
    }
    float4 v[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j) v[j] = load_once(y + (long)pos[j] * d + c);
#pragma unroll
    for (int j = 0; j < KT; ++j) add(wv[j], v[j]);
  } else {
    for (int j = 0; j < k; ++j) add(w[t * k + j], load_once(y + (long)ap[t * k + j] * d + c));
  }
  if (shared) {
    const float4 v = load_once(shared + t * d + c);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  uint2 o;
  o.x = (uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
  o.y = (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
  // the layer output is written once and not read again here: a nontemporal store (V3 prefill
  // combine 196 -> 185 us)
  __builtin_nontemporal_store(u32x2{o.x, o.y}, reinterpret_cast<u32x2*>(out + t * d + c));
}

// out[t*k+j][:] = y[assign_pos[t*k+j]][:], rows of row_words 32-bit words.
__global__ __launch_bounds__(256) void unpermute_kernel(const uint32_t* __restrict__ y, const int32_t* __restrict__ ap,
                                                        long n, int row_words, uint32_t* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n * row_words) return;
  const long a = i / row_words;
  const int c = (int)(i - a * row_words);
  out[i] = y[(long)ap[a] * row_words + c];
}

// acc (fp32) -> bf16, round to nearest even.
__global__ __launch_bounds__(256) void cast_bf16_kernel(const float* __restrict__ in, long n4, uint16_t* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4 v = reinterpret_cast<const float4*>(in)[i];
  uint2 o;
  o.x = (uint32_t)f32_to_bf16_rne(v.x) | ((uint32_t)f32_to_bf16_rne(v.y) << 16);
  o.y = (uint32_t)f32_to_bf16_rne(v.z) | ((uint32_t)f32_to_bf16_rne(v.w) << 16);
  reinterpret_cast<uint2*>(out)[i] = o;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float4* __restrict__ p, long n4) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

size_t permute_scratch_bytes(int n, int E) {
  const long nchunks = (n + kChunk - 1) / kChunk;
  return (size_t)nchunks * E * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets, int32_t* sorted_assign,
                          int32_t* assign_pos, int32_t* sorted_token, const float* topk_w, float* sorted_w,
                          int32_t* scratch, hipStream_t st) {
  const int n = T * k;
  if (n <= kSmallN && E <= kSmallE) {
    perm_small_kernel<<<1, 1024, 0, st>>>(idx, n, k, E, offsets, sorted_assign, assign_pos, sorted_token, topk_w,
                                          sorted_w);
    return hipGetLastError();
  }
  const int nchunks = (n + kChunk - 1) / kChunk;
  if (nchunks > 0) perm_count_kernel<<<nchunks, 256, E * sizeof(int), st>>>(idx, n, E, scratch);
  perm_scan_kernel<<<1, 1024, 0, st>>>(scratch, nchunks, E, offsets);
  if (nchunks > 0)
    perm_scatter_kernel<<<nchunks, 256, 4 * E * sizeof(int), st>>>(idx, n, k, E, scratch, offsets, sorted_assign,
                                                                    assign_pos, sorted_token, topk_w, sorted_w);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* rows_in, int row_bytes, int n, int k, const int32_t* sorted_assign,
                              void* rows_out, hipStream_t st) {
  const int row_vec = row_bytes / 16;
  const long total = (long)n * row_vec;
  if (total == 0) return hipSuccess;
  perm_gather_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(
      reinterpret_cast<const uint4*>(rows_in), row_vec, n, k, sorted_assign, reinterpret_cast<uint4*>(rows_out));
  return hipGetLastError();
}

hipError_t launch_combine(const float* y, const int32_t* ap, const float* w, const float* shared, int T, int k, int d,
                          uint16_t* out, hipStream_t st) {
  const long total = (long)T * (d / 4);
  if (total == 0) return hipSuccess;
  const unsigned grid = (unsigned)((total + 255) / 256);
  switch (k) {
    case 8: combine_kernel<8><<<grid, 256, 0, st>>>(y, ap, w, shared, T, k, d, out); break;
    case 2: combine_kernel<2><<<grid, 256, 0, st>>>(y, ap, w, shared, T, k, d, out); break;
    default: combine_kernel<0><<<grid, 256, 0, st>>>(y, ap, w, shared, T, k, d, out); break;
  }
  return hipGetLastError();
}

hipError_t launch_unpermute(const void* y, const int32_t* ap, long n, int row_bytes, void* out, hipStream_t st) {
  const int row_words = row_bytes / 4;
  const long total = n * row_words;
  if (total == 0) return hipSuccess;
  unpermute_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(reinterpret_cast<const uint32_t*>(y), ap, n,
                                                                     row_words, reinterpret_cast<uint32_t*>(out));
  return hipGetLastError();
}

hipError_t launch_cast_bf16(const float* in, long n, uint16_t* out, hipStream_t st) {
  const long n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  cast_bf16_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>(in, n4, out);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, long n, hipStream_t st) {
  const long n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  fill_zero_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>(reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

}  // namespace moefp8

namespace moefp8 {

// Routing-bias balancing step (onlylabs "DeepSeek v3 and R1 Model Architecture",
// "Local Balanced Routing to Experts": an overloaded expert's bias goes down by
// gamma, an underloaded one's goes up).  One workgroup: the n = T*k expert ids
// are counted in LDS (integer atomics: exact), then, against the mean load
// n / E, bias[e] += gamma * sign(n - E * load_e) in fp32 (an expert exactly at
// the mean adds +0).  Ids outside [0, E) are not counted.
__global__ __launch_bounds__(1024) void bias_update_kernel(const int32_t* __restrict__ idx, long n, int E, float gamma,
                                                           float* __restrict__ bias, int32_t* __restrict__ counts) {
  __shared__ int cnt[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) cnt[e] = 0;
  __syncthreads();
  for (long i = tid; i < n; i += 1024) {
    const int e = idx[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    const long diff = n - (long)E * cnt[e];
    const float step = diff > 0 ? gamma : (diff < 0 ? -gamma : 0.0f);
    bias[e] = bias[e] + step;
    if (counts) counts[e] = cnt[e];
  }
}

hipError_t launch_bias_update(const int32_t* topk_idx, long n, int E, float gamma, float* bias, int32_t* counts,
                              hipStream_t st) {
  bias_update_kernel<<<1, 1024, 0, st>>>(topk_idx, n, E, gamma, bias, counts);
  return hipGetLastError();
}

}  // namespace moefp8
