// FP8 backward of the experts' grouped GEMMs (onlylabs "DeepSeek v3 and R1 Model
// Architecture", "First ever FP8 Precision OSS LLM pre-training": the model trains
// with FP8 matrix multiplications; headings "Fine granularity quantization",
// "Online Quantization", "Better Accumulation Precision").
//
// For a forward GEMM C_g = A_g . W_g^T over group g's rows:
//  * dgrad, dA = dC . W, is a forward-shaped grouped GEMM: dC quantised 1x128 along its
//    contraction dimension, W^T in 128x128 blocks (W's blocks transposed, same scales),
//    packed into MFMA-fragment order by pack_transposed_kernel;
//  * wgrad, dW_g = dC_g^T . A_g, contracts over the group's rows: both operands are
//    quantised in 128x1 tiles (quant_128x1_grouped_kernel: per column, per 128 rows of one
//    group) and stored transposed, [N][Mp] with every group padded to 128-row multiples,
//    so a 128x1 tile is a 1x128 tile of the transposed operand; wgrad_gemm_kernel
//    multiplies them, K = the group's padded rows, with the blocks' scales promoted into
//    the fp32 accumulator (or, for power-of-two scales, applied as the FP8 MFMA's E8M0
//    operands).
#include "common.h"
#include "launch.h"

namespace moefp8 {

// padded[g + 1] - padded[g] = round_up(offsets[g + 1] - offsets[g], 128); one workgroup, G <= 1024.
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t* __restrict__ offsets, int G,
                                                           int32_t* __restrict__ padded) {
  __shared__ int scan[1024];
  const int t = threadIdx.x;
  const int v = t < G ? (offsets[t + 1] - offsets[t] + 127) / 128 * 128 : 0;
  scan[t] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {          // inclusive Hillis-Steele scan
    const int y = t >= o ? scan[t - o] : 0;
    __syncthreads();
    scan[t] += y;
    __syncthreads();
  }
  if (t < G) padded[t + 1] = scan[t];
  if (t == 0) padded[0] = 0;
}

// One workgroup per (128-row tile of the padded rows, 64 columns).  The tile's rows come from
// one group (rows past the group's end are zeros).  Each wave loads 32 rows with 16-byte loads,
// all in flight together, and stages them transposed in LDS (fp32, rows padded by one word;
// 33 KB, so four workgroups share a CU); then thread t takes column t / 4, rows (t % 4) * 32 ..
// +31: the column's amax over the four quarters (lane shuffles), its scale, and 32 codes written
// as 32 contiguous bytes of the transposed output.
template <bool kBf16>
__global__ __launch_bounds__(256) void quant_128x1_grouped_kernel(const void* __restrict__ x, int ld_x,
                                                                  const int32_t* __restrict__ offsets, int G,
                                                                  const int32_t* __restrict__ padded, int N,
                                                                  uint8_t* __restrict__ qt, int ld_q,
                                                                  float* __restrict__ st, int pow2) {
  constexpr int kCols = 64;
  __shared__ float tile[kCols][129];
  const int tid = threadIdx.x;
  const int p0 = blockIdx.x * 128;               // first padded row of the tile
  if (p0 >= padded[G]) return;
  // the group holding padded row p0 (padded offsets never decrease): binary search
  int lo = 0, hi = G;                            // padded[lo] <= p0 < padded[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (padded[mid] <= p0) lo = mid;
    else hi = mid;
  }
  const int g = lo;
  const int r0 = offsets[g] + (p0 - padded[g]);  // first source row
  const int rows = min(128, offsets[g + 1] - r0);
  const int c0 = blockIdx.y * kCols;
  const int wave = tid >> 6, lane = tid & 63;
  // load: a 16-byte chunk per lane holds 8 bf16 or 4 fp32 columns; a row is 8 (bf16) or 16 (fp32)
  // chunks, so one wave load covers 8 or 4 rows and a wave's 32 rows take 4 or 8 loads
  constexpr int kPer = kBf16 ? 8 : 4;            // columns per chunk
  constexpr int kChunks = kCols / kPer;          // chunks per row
  constexpr int kRowsPer = 64 / kChunks;         // rows per wave load
  constexpr int kLoads = 32 / kRowsPer;
  const int ch = lane % kChunks, rl = lane / kChunks;
  uint4 v[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = wave * 32 + i * kRowsPer + rl;
    v[i] = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows) {
      const char* src = reinterpret_cast<const char*>(x) +
                        ((long)(r0 + r) * ld_x + c0 + ch * kPer) * (kBf16 ? 2 : 4);
      v[i] = *reinterpret_cast<const uint4*>(src);
    }
  }
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = wave * 32 + i * kRowsPer + rl;
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (kBf16) {
        tile[ch * 8 + 2 * j][r] = __uint_as_float(w[j] << 16);
        tile[ch * 8 + 2 * j + 1][r] = __uint_as_float(w[j] & 0xFFFF0000u);
      } else {
        tile[ch * 4 + j][r] = __uint_as_float(w[j]);
      }
    }
  }
  __syncthreads();
  const int col = tid >> 2, qtr = tid & 3;
  const float* vv = &tile[col][qtr * 32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(vv[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const float sc = tile_scale(amax, pow2 != 0);
  uint8_t* dst = qt + (long)(c0 + col) * ld_q + p0 + qtr * 32;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t wd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* e = vv + 16 * i + 4 * j;
      wd[j] = e4m3_encode4(e[0] / sc, e[1] / sc, e[2] / sc, e[3] / sc);
    }
    reinterpret_cast<uint4*>(dst)[i] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }
  if (qtr == 0) st[(long)(c0 + col) * (ld_q >> 7) + (p0 >> 7)] = sc;
}

// Row-major e4m3 W [G][N][K] -> W^T [G][K][N] in MFMA-fragment order (see pack_kernel): the
// destination's byte (h * 1024 + (16 q + r) * 16 + b) of block (g, n16, kb) is
// W^T[16 n16 + r][128 kb + 64 h + 16 q + b] = W[128 kb + 64 h + 16 q + b][16 n16 + r].
__global__ __launch_bounds__(256) void pack_transposed_kernel(const uint8_t* __restrict__ src, long nchunks, int N,
                                                              int K, uint4* __restrict__ dst) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;   // destination 16-byte chunk
  if (i >= nchunks) return;
  const int nkb = N >> 7;                                 // K blocks of W^T: W's rows
  const long blk = i >> 7;
  const int w = (int)(i & 127);
  const int h = w >> 6, r = w & 15, q = (w >> 4) & 3;
  const int kb = (int)(blk % nkb);
  const long gn16 = blk / nkb;                            // g * (K / 16) + n16
  const long g = gn16 / (K >> 4);
  const int col = (int)(gn16 - g * (K >> 4)) * 16 + r;    // W's column = W^T's row
  const uint8_t* s = src + (g * N + kb * 128 + 64 * h + 16 * q) * (long)K + col;
  uint32_t wd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wd[j] = (uint32_t)s[(4 * j) * (long)K] | ((uint32_t)s[(4 * j + 1) * (long)K] << 8) |
            ((uint32_t)s[(4 * j + 2) * (long)K] << 16) | ((uint32_t)s[(4 * j + 3) * (long)K] << 24);
  dst[i] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
}

// Block scales of W^T: s_t[g][kb][nb] = s[g][nb][kb].
__global__ __launch_bounds__(256) void transpose_scales_kernel(const float* __restrict__ s, long n, int NB, int KB,
                                                               float* __restrict__ s_t) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const long g = i / ((long)NB * KB);
  const int rem = (int)(i - g * NB * KB);
  const int kb = rem / NB, nb = rem - kb * NB;
  s_t[i] = s[(g * NB + nb) * KB + kb];
}

// ---------------------------------------------------------------------------
// wgrad: out[g][i][j] = sum over group g's padded rows k of A_t[i][k] * B_t[j][k], by 128-wide K
// blocks with their 128x1 tile scales.  Workgroup: 4 waves (2 x 2), output tile 128 (i) x 128
// (j), wave tile 64 x 64.  Both operands are row-major with K contiguous and go global -> LDS by
// LDS-DMA as whole 128-byte rows (8 rows per wave load), the 16-byte chunk index XORed by
// row % 8 (bank-conflict-free fragment reads); their per-row scales ride in the same stage.
// 2 stages of 33 KB, one barrier per K block: a group's K is a few blocks at most sizes, and the
// 66 KB let two workgroups share a CU, so one's loads overlap the other's fp32 stores (the
// output, not the K loop, is what costs: 64 KB of fp32 per tile against 32 KB of operands per
// K block).
namespace {
constexpr int kWgA = 128 * 128, kWgB = 128 * 128, kWgS = 256 * 4;   // bytes per stage
constexpr int kWgStage = kWgA + kWgB + kWgS;

__device__ __forceinline__ void wg_dma16(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void wg_dma4(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}
template <int N>
__device__ __forceinline__ void wg_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
}  // namespace

struct WgradArgs {
  const uint8_t* a_t;      // [Na][ld] e4m3
  const float* a_ts;       // [Na][ld / 128]
  const uint8_t* b_t;      // [Nb][ld]
  const float* b_ts;       // [Nb][ld / 128]
  const int32_t* padded;   // [G + 1] padded row offsets (multiples of 128)
  int G, Na, Nb, ld;
  float* out;              // [G][Na][Nb]
};

template <bool SCALED>
__global__ __launch_bounds__(256) void wgrad_gemm_kernel(const WgradArgs args) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[kWgStage];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[kWgStage];
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, q = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;       // 64-row, 64-column wave tile
  const int ti_n = args.Na >> 7, tj_n = (args.Nb + 127) >> 7;
  const int per_group = ti_n * tj_n;
  const int t = blockIdx.x;
  const int g = t / per_group, rem = t - g * per_group;
  const int ti = rem / tj_n, tj = rem - ti * tj_n;
  const int i0 = ti * 128, j0 = tj * 128;
  const int kb0 = args.padded[g] >> 7, nk = (args.padded[g + 1] >> 7) - kb0;
  const int ld = args.ld, lds_ = ld >> 7;

  // per-lane sources: wave load i covers A rows and B rows 8 li .. +7 (li = 4 wave + i)
  const uint8_t* a_src[4];
  const uint8_t* b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * (4 * wave + i) + (lane >> 3);
    a_src[i] = args.a_t + (long)(i0 + r) * ld + 16 * ((lane & 7) ^ (r & 7)) + (long)kb0 * 128;
    const int jr = min(j0 + r, args.Nb - 1);     // rows past Nb (a partial last tile) read the last row, discarded
    b_src[i] = args.b_t + (long)jr * ld + 16 * ((lane & 7) ^ (r & 7)) + (long)kb0 * 128;
  }
  // one 4-byte scale DMA per wave and K block: waves 0, 1 the A rows 64 w .. +63, waves 2, 3 the
  // B rows 64 (w - 2) .. +63
  const float* s_src;
  if (wave < 2) s_src = args.a_ts + (long)(i0 + 64 * wave + lane) * lds_ + kb0;
  else s_src = args.b_ts + (long)min(j0 + 64 * (wave - 2) + lane, args.Nb - 1) * lds_ + kb0;

#define WG_ISSUE(kb_, dst_)                                                                      \
  {                                                                                              \
    uint8_t* d_ = (dst_);                                                                        \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                              \
      wg_dma16(a_src[i] + (kb_) * 128, d_ + (4 * wave + i) * 1024);                              \
      wg_dma16(b_src[i] + (kb_) * 128, d_ + kWgA + (4 * wave + i) * 1024);                       \
    }                                                                                            \
    wg_dma4(s_src + (kb_), d_ + kWgA + kWgB + wave * 256);                                       \
  }

  v4f acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[mi][f] = v4f{0.f, 0.f, 0.f, 0.f};
  const int swz = r16 & 7;
  const int off_lo = r16 * 128 + 16 * (q ^ swz), off_hi = r16 * 128 + 16 * ((4 + q) ^ swz);
  auto frag = [&](const uint8_t* base, int blk16) {
    const v4i lo = *reinterpret_cast<const v4i*>(base + blk16 * 2048 + off_lo);
    const v4i hi = *reinterpret_cast<const v4i*>(base + blk16 * 2048 + off_hi);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto compute = [&](const uint8_t* st) __attribute__((always_inline)) {
    const float* sa = reinterpret_cast<const float*>(st + kWgA + kWgB);
    const float* sb = sa + 128;
    v8i bfr[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) bfr[f] = frag(st + kWgA, wn * 4 + f);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const v8i af = frag(st, wm * 4 + mi);
      const int rb = wm * 64 + mi * 16;
      if constexpr (SCALED) {
        const int ea = e8m0_of(sa[rb + r16]);
#pragma unroll
        for (int f = 0; f < 4; ++f)
          acc[mi][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bfr[f], acc[mi][f], 0, 0, 0, ea, 0,
                                                                        e8m0_of(sb[wn * 64 + 16 * f + r16]));
      } else {
        const float4 s4 = *reinterpret_cast<const float4*>(sa + rb + 4 * q);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bfr[f], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                            0, 0, 0, 0);
          const float sbf = sb[wn * 64 + 16 * f + r16];
          acc[mi][f][0] = fmaf(part[0], s4.x * sbf, acc[mi][f][0]);
          acc[mi][f][1] = fmaf(part[1], s4.y * sbf, acc[mi][f][1]);
          acc[mi][f][2] = fmaf(part[2], s4.z * sbf, acc[mi][f][2]);
          acc[mi][f][3] = fmaf(part[3], s4.w * sbf, acc[mi][f][3]);
        }
      }
    }
  };
  // K loop: block kb waits for its own loads (none other is in flight), barrier (every wave's
  // loads of kb have landed and every wave is done with kb - 1, whose stage kb + 1 now takes),
  // issue kb + 1, compute kb; run-time bounds (a group's K is a few blocks at most sizes)
  if (nk > 0) {
    WG_ISSUE(0, smem0);
    for (int kb = 0; kb < nk; kb += 2) {
#define WG_STEP(k_, cur_, nxt_)                                                                  \
  if ((k_) < nk) {                                                                               \
    wg_wait_vmcnt<0>();                                                                          \
    wg_barrier();                                                                                \
    if ((k_) + 1 < nk) WG_ISSUE((k_) + 1, nxt_);                                                 \
    compute(cur_);                                                                               \
  }
      WG_STEP(kb, smem0, smem1);
      WG_STEP(kb + 1, smem1, smem0);
#undef WG_STEP
    }
  }
#undef WG_ISSUE
  // epilogue: each wave's 64 x 64 fp32 tile through its own LDS slice (16 KB: the two stages
  // hold the four), read back by rows for 16-byte nontemporal stores; columns XOR-swizzled by row
  // bits 2-3 so the four quads' writes of a fragment row fall on distinct banks
  wg_barrier();                                   // every wave is past its last read of the stages
  uint8_t* const arr = wave < 2 ? smem0 : smem1;
  float* const wt = reinterpret_cast<float*>(arr + (wave % 2) * 16384);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mi * 16 + 4 * q + i, c = 16 * f + r16;
        wt[r * 64 + (c ^ (((r >> 2) & 3) << 4))] = acc[mi][f][i];
      }
  float* const out = args.out + (long)g * args.Na * args.Nb;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int tt = it * 64 + lane, r = tt >> 4, c = (tt & 15) * 4;
    const float4 v = *reinterpret_cast<const float4*>(wt + r * 64 + (c ^ (((r >> 2) & 3) << 4)));
    const int i = i0 + wm * 64 + r, j = j0 + wn * 64 + c;
    if (j < args.Nb)
      __builtin_nontemporal_store(v4f{v.x, v.y, v.z, v.w}, reinterpret_cast<v4f*>(out + (long)i * args.Nb + j));
  }
}

hipError_t launch_pad_offsets(const int32_t* offsets, int G, int32_t* padded, hipStream_t st) {
  pad_offsets_kernel<<<1, 1024, 0, st>>>(offsets, G, padded);
  return hipGetLastError();
}

hipError_t launch_quant_128x1_grouped(const void* x, bool bf16, int ld_x, const int32_t* offsets, int G,
                                      const int32_t* padded, int M_pad_max, int N, uint8_t* qt, int ld_q, float* st,
                                      bool pow2, hipStream_t s) {
  if (M_pad_max == 0 || N == 0) return hipSuccess;
  const dim3 grid((unsigned)(M_pad_max / 128), (unsigned)(N / 64));
  if (bf16)
    quant_128x1_grouped_kernel<true><<<grid, 256, 0, s>>>(x, ld_x, offsets, G, padded, N, qt, ld_q, st, pow2);
  else
    quant_128x1_grouped_kernel<false><<<grid, 256, 0, s>>>(x, ld_x, offsets, G, padded, N, qt, ld_q, st, pow2);
  return hipGetLastError();
}

hipError_t launch_pack_transposed(const uint8_t* src, const float* s, int G, int N, int K, uint8_t* dst, float* s_t,
                                  hipStream_t st) {
  const long nchunks = (long)G * N * K / 16;
  if (nchunks == 0) return hipSuccess;
  pack_transposed_kernel<<<(unsigned)((nchunks + 255) / 256), 256, 0, st>>>(src, nchunks, N, K,
                                                                           reinterpret_cast<uint4*>(dst));
  const long ns = (long)G * (N / 128) * (K / 128);
  transpose_scales_kernel<<<(unsigned)((ns + 255) / 256), 256, 0, st>>>(s, ns, N / 128, K / 128, s_t);
  return hipGetLastError();
}

hipError_t launch_wgrad(const uint8_t* a_t, const float* a_ts, const uint8_t* b_t, const float* b_ts,
                        const int32_t* padded, int G, int Na, int Nb, int ld, float* out, bool pow2, hipStream_t st) {
  const long tiles = (long)G * (Na / 128) * ((Nb + 127) / 128);
  if (tiles == 0) return hipSuccess;
  WgradArgs a{a_t, a_ts, b_t, b_ts, padded, G, Na, Nb, ld, out};
  if (pow2) wgrad_gemm_kernel<true><<<(unsigned)tiles, 256, 0, st>>>(a);
  else wgrad_gemm_kernel<false><<<(unsigned)tiles, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moefp8
