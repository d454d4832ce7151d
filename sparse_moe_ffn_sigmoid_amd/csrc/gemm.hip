// Block-scaled FP8 grouped GEMM for gfx950 (onlylabs "DeepSeek v3 and R1 Model
// Architecture", headings "Fine granularity quantization" and "Better
// Accumulation Precision"; aguasto "DeepSeek-R1", "Quantization").
//
//   C[m][n] = sum_kb a_s[row(m)][kb] * b_s[g][n/128][kb] * (sum_{k in kb} A[row(m)][k] * B[g][n][k])
//
// One 128-wide K block is exactly one V_MFMA_F32_16X16X128_F8F6F4 (e4m3 x
// e4m3 -> fp32) per 16x16 output tile.  Each block's partial is promoted into
// the fp32 accumulator with one FMA per element: acc = fma(part, sa * sb, acc).
//
// Accumulation precision: measured on MI355X, the FP8 MFMAs (this one and the
// 16x16x32 form alike) return a 128-term dot product with a relative error
// near 1e-5 of the sum of |products|, while the bf16 MFMA sums exactly decoded
// e4m3 values as an IEEE fp32 accumulation would.  Where the GEMM's output is
// requantised to e4m3 (the gate/up GEMM with the SwiGLU epilogue), 1e-5 shifts
// flip codes at rounding midpoints often enough to cost ~1e-3 of the layer's
// output, so that GEMM converts both tiles to bf16 in registers (exact) and runs
// four 16x16x32 bf16 MFMAs per K block instead ("exact" path).  The down GEMM,
// whose output is not requantised, keeps the native FP8 MFMA.
//
// B is stored in MFMA-fragment order (moe_pack_weights): for 16 B rows and one
// K block, 2 KB in which lane l of a wave finds its two 16-byte pieces at
// 16 l and 1024 + 16 l, so every fragment load is one 1 KB-contiguous wave
// access (coalesced from HBM, bank-conflict free in LDS).
//
// Two kernels:
//  * stream_gemm_kernel (groups of about 10 rows or fewer on average, decode): B
//    bypasses LDS and streams from HBM into registers; the weight bytes are the
//    whole cost.
//  * mfma_gemm_kernel (larger groups, prefill and dense layers): A and B tiles
//    go global -> LDS by LDS-DMA through a 3-stage pipeline, one barrier per
//    K block.
//
// Grouped rows: a static segment (the shared expert, or a plain GEMM) and a
// dynamic segment (routed experts, rows given by device-side offsets) share
// one launch; each wave finds its workgroup's tile with a cross-lane prefix sum
// over the groups' tile counts, and workgroups past the real tile count exit at
// once, so no device-to-host copy of the counts is needed.
#include "common.h"
#include "launch.h"

namespace moefp8 {

// Tiles of the dynamic segment: group g has ceil(rows_g / bm) tiles (its rows split evenly over
// them by the tile kernel, in whole 16-row blocks).  Each wave scans the per-group counts on its
// own, with cross-lane shuffles (no LDS, no barrier; every wave of a workgroup gets the same
// result): lane l owns groups l * per .. l * per + per - 1.
struct GroupTiles {
  int per;        // groups per lane (G <= 1024)
  int first;      // this lane's first tile: the tiles of all groups of the lanes below it
  int total;      // tiles of all groups (wave-uniform)
};

__device__ __forceinline__ int group_tiles(const GemmSeg& sd, int gi, int bm) {
  return (sd.offsets[gi + 1] - sd.offsets[gi] + bm - 1) / bm;
}

__device__ GroupTiles scan_group_tiles(const GemmSeg& sd, int bm) {
  const int lane = threadIdx.x & 63;
  const int per = (sd.G + 63) >> 6;
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int gi = lane * per + i;
    if (gi < sd.G) sum += group_tiles(sd, gi, bm);
  }
  int inc = sum;                                // inclusive scan over the lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  GroupTiles r;
  r.per = per;
  r.first = inc - sum;
  r.total = __builtin_amdgcn_readlane(inc, 63);
  return r;
}

// The group holding tile t (< total), its first tile and its tile count, all wave-uniform.
// The owning lane is the last one whose first tile is <= t (first tiles never decrease).
__device__ void locate_tile(const GemmSeg& sd, int bm, const GroupTiles& s, int t, int& g, int& start, int& count) {
  const unsigned long long m = __ballot(s.first <= t);
  const int L = __builtin_amdgcn_readfirstlane(63 - __builtin_clzll(m));
  int acc = __builtin_amdgcn_readlane(s.first, L);
  g = L * s.per;
  count = 0;
  for (int i = 0; i < s.per; ++i) {
    const int gi = L * s.per + i;
    const int c = group_tiles(sd, gi, bm);
    if (t < acc + c) {
      g = gi;
      count = c;
      break;
    }
    acc += c;
  }
  g = __builtin_amdgcn_readfirstlane(g);
  start = __builtin_amdgcn_readfirstlane(acc);
  count = __builtin_amdgcn_readfirstlane(count);
}

// Maps m tile v to (segment, group, first row, end row) for tiles of bm rows (one
// workgroup per m tile and n tile).  Static segment tiles come first.  Returns false (uniformly) for workgroups past the real
// tile count.  The tile coordinates are workgroup-uniform: readfirstlane lets
// the compiler keep them (and every address derived from them) in scalar
// registers.
__device__ bool find_tile(const GemmArgs& args, int bm, int v, int& si, int& g, int& m0, int& m_end) {
  if (v < args.seg[0].m_tiles) {
    si = 0;
    g = 0;
    m0 = v * bm;
    m_end = args.seg[0].m_rows;
    return true;
  }
  v -= args.seg[0].m_tiles;
  const GemmSeg& sd = args.seg[1];
  if (v >= sd.m_tiles) return false;
  const GroupTiles scan = scan_group_tiles(sd, bm);
  if (v >= scan.total) return false;
  int start, count;
  locate_tile(sd, bm, scan, v, g, start, count);
  si = 1;
  m0 = __builtin_amdgcn_readfirstlane(sd.offsets[g] + (v - start) * bm);
  m_end = __builtin_amdgcn_readfirstlane(sd.offsets[g + 1]);
  return true;
}

// Work order of the MFMA tile kernel.  A work item is one (m tile, n tile).
// Items are numbered segment 0 first, then segment 1 group by group; inside a
// group (or the static segment) the m tiles are taken in panels of up to
// kPanel, and a panel's items run n-major with its m tiles innermost: the
// items of one n tile, which read the same B tile, are adjacent, and a panel's
// A rows are reused by every n tile of the panel.  The items are then cut into
// 8 contiguous chunks of equal count, chunk x for XCD x: workgroups are
// dispatched to the 8 XCDs round-robin by workgroup id, so workgroup b runs
// item (b % 8) * chunk + b / 8, and each XCD's L2 sees a contiguous run of
// items (one expert's tiles land on one XCD and share its L2).
//
// Inside an XCD, workgroup j goes to shader engine j % 4 (measured on MI355X) and
// the dispatch is in order: a shader engine whose CUs are all busy holds back
// every later workgroup.  The m tiles of one n tile are therefore taken in an
// order rotated by the number of whole 4-item rounds before that n tile, so
// that each shader engine gets each m tile of a panel in turn.  The last m tile
// of a group is often nearly empty and costs less than half a full one; with
// two m tiles per group and no rotation, two shader engines would get every
// full tile and the other two every partial one, and sit idle half the time.
constexpr int kPanel = 4;

__device__ __forceinline__ void panel_map(int L, int c, int ny, int& mt, int& nt) {
  const int full = c / kPanel;                  // full panels of kPanel m tiles
  const int in_full = full * kPanel * ny;
  if (L < in_full) {
    const int p = L / (kPanel * ny), r = L - p * (kPanel * ny);
    nt = r / kPanel;
    mt = p * kPanel + (r - nt * kPanel + nt) % kPanel;
  } else {
    const int rem = c - full * kPanel, r = L - in_full;
    nt = r / rem;
    mt = full * kPanel + (r - nt * rem + rem * nt / 4) % rem;
  }
}

__device__ bool find_work(const GemmArgs& args, int bm, int ny0, int ny1, int& si, int& g, int& m0, int& m_end,
                          int& nt) {
  const GemmSeg& s0 = args.seg[0];
  const GemmSeg& sd = args.seg[1];
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;   // XCD, position in its sequence
  // static segment: panel p goes to XCD p % 8; this XCD's panels come first in its sequence
  const int panels = (s0.m_tiles + kPanel - 1) / kPanel, per_panel = kPanel * ny0;
  const int mine = panels > x ? (panels - 1 - x) / 8 + 1 : 0;
  const int last_m = s0.m_tiles - (panels - 1) * kPanel;   // m tiles of the last panel
  const int s_items = mine == 0 ? 0 : (mine - 1) * per_panel + ((x + 8 * (mine - 1)) == panels - 1 ? last_m * ny0 : per_panel);
  int mt;
  if (j < s_items) {
    const int kp = j / per_panel, L = j - kp * per_panel, p = x + 8 * kp;
    const int c = p == panels - 1 ? last_m : kPanel;
    nt = L / c;
    mt = p * kPanel + (L - nt * c);
    si = 0;
    g = 0;
    m0 = mt * bm;
    m_end = s0.m_rows;
  } else {
    // dynamic segment: 8 equal contiguous chunks, chunk x after this XCD's static panels
    GroupTiles scan{0, 0, 0};
    if (sd.m_tiles > 0) scan = scan_group_tiles(sd, bm);
    const int dyn = scan.total * ny1, chunk = (dyn + 7) >> 3;
    const int dj = j - s_items;
    if (dj >= chunk) return false;
    const int v = x * chunk + dj;
    if (v >= dyn) return false;
    int start, c;
    locate_tile(sd, bm, scan, v / ny1, g, start, c);
    panel_map(v - ny1 * start, c, ny1, mt, nt);
    si = 1;
    // a group's rows are split evenly over its c tiles, in whole 16-row blocks (150 rows: 80 + 70,
    // not 128 + 22): the tiles of one n tile stream the same B tile however the rows fall, and
    // two tiles of partial row blocks cost less than a full tile plus a nearly empty one
    const int off = sd.offsets[g], end = sd.offsets[g + 1];
    const int rb = c > 1 ? ((end - off + c - 1) / c + 15) & ~15 : bm;
    m0 = off + mt * rb;
    m_end = min(m0 + rb, end);
  }
  nt = __builtin_amdgcn_readfirstlane(nt);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  m_end = __builtin_amdgcn_readfirstlane(m_end);
  return true;
}

// ---------------------------------------------------------------------------
// Weight-streaming variant for decode-sized batches (16-row tiles; a group of more rows takes
// one tile per 16 rows, each streaming the group's weights).  Each B byte is used by exactly one wave, so B bypasses LDS: every
// lane loads its own MFMA fragments straight from HBM (fragment-ordered
// weights: two 1 KB contiguous wave loads per 16 rows and K block, and a wave's
// whole stream over K is one contiguous range), with P K blocks of loads in
// flight per wave; the waves never synchronise inside the K loop.  A (the <= 16 activation rows) comes from L2
// the same way.  Wave w covers NTW 16-column tiles of each of the NB B blocks;
// with NB = 2 (gate/up) a workgroup covers 128 h columns, the SwiGLU
// requantisation tile.
// NFAST: the grid is (n tiles, m tiles) with the n tile fastest-varying, so that a tile's n tiles
// are dispatched together and the static segment's first.  Workgroups go to the 8 XCDs
// round-robin by linear id, so with a multiple of 8 n tiles the m tiles of one n tile, which
// stream the same weights, run on one XCD at about the same time and share its L2: the shared
// expert's rows (T of them in T / 16 tiles) then read its weights from HBM about once.  Measured
// for the gate/up GEMM at decode (T = 64): 6.372 GB fetched per launch instead of 6.438 GB for
// 6.343 GB of algorithmic bytes, 0.924 instead of 0.935 ms.  The down GEMM ran 2.5% slower in
// that order, and keeps the grid (m tiles, n tiles).
// Launch bounds: the FP8 kernels with power-of-two scales (NB = 1, SCALED) ask for 3 waves per SIMD;
// left alone the compiler gave them 208 registers (2 waves), and the down GEMM at decode ran 0.498
// instead of 0.486 ms.
// MB: 16-row blocks per workgroup (1 or 2).  With 2, each streamed B fragment serves both row
// blocks (converted once per block for the exact path), so a group of up to 32 rows streams its
// weights once.
template <int NB, int NTW, int P, int EPI, bool SCALED, bool NFAST, int MB>
__device__ __forceinline__ void stream_gemm_body(const GemmArgs& args) {
  constexpr int NF = NB * NTW;                 // B fragments per lane per K block
  constexpr int CW = 16 * NTW;                 // columns per wave in each B block
  static_assert(EPI != kEpiSwiglu || NTW % 2 == 0, "the SwiGLU epilogue encodes h in pairs");
  static_assert(MB == 1 || MB == 2, "one or two row blocks");
  constexpr bool kExact = EPI == kEpiSwiglu;
  __shared__ float red[4][16 * MB];
  __shared__ __attribute__((aligned(16))) uint8_t stage[16 * MB * 128];

  // wave index made wave-uniform: the MFMAs below sit under branches on it, and an MFMA writes
  // every lane whatever EXEC holds, so those branches must be scalar
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, r16 = lane & 15,
            q = lane >> 4;
  // (m tile, n tile) of this workgroup.  NFAST: the grid's x is the n tile.  Otherwise the grid is
  // (m tiles, n tiles), and when the static segment (the shared expert) has 2..8 m tiles and the
  // n tiles come in multiples of 8, the first ms x ny workgroups in dispatch order take its tiles
  // so that the m tiles of one n tile are 8 workgroups apart: the same XCD (workgroups go to the
  // 8 XCDs round-robin), whose L2 then serves their shared weight stream; the other workgroups
  // take the dynamic segment's tiles in the grid's own order (m tile fastest).
  int tm = NFAST ? blockIdx.y : blockIdx.x, tn = NFAST ? blockIdx.x : blockIdx.y;
  if constexpr (!NFAST) {
    const int ms = args.seg[0].m_tiles, ny = gridDim.y, mt = gridDim.x;
    if (ms >= 2 && ms <= 8 && ny % 8 == 0 && mt > ms) {
      const int L = blockIdx.y * mt + blockIdx.x;   // dispatch order
      if (L < ms * ny) {
        const int b = L / (8 * ms), rem = L - b * 8 * ms;
        tm = rem >> 3;
        tn = 8 * b + (rem & 7);
      } else {
        const int L2 = L - ms * ny, md = mt - ms;
        tm = ms + L2 % md;
        tn = L2 / md;
      }
    }
  }
  int si, g, m0, m_end;
  if (!find_tile(args, 16 * MB, tm, si, g, m0, m_end)) return;
  const GemmSeg& s0 = args.seg[0];
  const GemmSeg& s1 = args.seg[1];
  const int K = si ? s1.K : s0.K, nkb = K >> 7;
  const int half = (si ? s1.N : s0.N) / NB;
  const int nbase = tn * 4 * CW;                 // first column of this workgroup in each block
  if (nbase >= half) return;
  const int ncol0 = nbase + wave * CW;         // first column of this wave in each block
  const bool wave_live = ncol0 < half;          // all waves live when half % (4 CW) == 0
  const uint8_t* const a_q = si ? s1.a_q : s0.a_q;
  const float* const a_s = si ? s1.a_s : s0.a_s;
  const int32_t* const gat = si ? s1.a_gather : s0.a_gather;
  const uint8_t* const bq = (si ? s1.b_q : s0.b_q) + (long long)g * (si ? s1.b_stride : s0.b_stride);
  const float* const bs = (si ? s1.b_s : s0.b_s) + (long long)g * (si ? s1.bs_stride : s0.bs_stride);

  // row block b: lane l loads row 16 b + l % 16 (rows past the group's end repeat row m0)
  const uint8_t* a_ptr[MB];
  const float* sa_ptr[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int my_m = m0 + 16 * b + r16 < m_end ? m0 + 16 * b + r16 : m0;
    const long src = gat ? (long)gat[my_m] : (long)my_m;
    a_ptr[b] = a_q + src * K + 16 * q;
    sa_ptr[b] = a_s + src * nkb;
  }
  const uint8_t* b_ptr[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int nb = f / NTW, j = f % NTW;
    const int n16 = wave_live ? (nb * half + ncol0) / 16 + j : 0;
    b_ptr[f] = bq + (long)n16 * nkb * 2048 + lane * 16;   // MFMA-fragment order: 1 KB per wave load
  }
  const float* sb_ptr[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) sb_ptr[nb] = bs + (long)((nb * half + (wave_live ? ncol0 : 0)) >> 7) * nkb;

  u32x4 al[P][MB], ah[P][MB], bl[P][NF], bh[P][NF];
  float sav[P][MB], sbv[P][NB];
#define STREAM_LOAD(p_, kb_)                                                                 \
  {                                                                                          \
    const int ko_ = (kb_) << 7;                                                              \
    _Pragma("unroll") for (int b = 0; b < MB; ++b) {                                        \
      al[p_][b] = *reinterpret_cast<const u32x4*>(a_ptr[b] + ko_);                           \
      ah[p_][b] = *reinterpret_cast<const u32x4*>(a_ptr[b] + ko_ + 64);                      \
    }                                                                                        \
    _Pragma("unroll") for (int f = 0; f < NF; ++f) {                                        \
      bl[p_][f] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b_ptr[f] + (long)(kb_) * 2048));        \
      bh[p_][f] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b_ptr[f] + (long)(kb_) * 2048 + 1024)); \
    }                                                                                        \
    _Pragma("unroll") for (int b = 0; b < MB; ++b) sav[p_][b] = sa_ptr[b][kb_];             \
    _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) sbv[p_][nb] = sb_ptr[nb][kb_];        \
  }

  v4f acc[MB][NF];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[b][f] = v4f{0.f, 0.f, 0.f, 0.f};
  if (wave_live) {
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (p < nkb) STREAM_LOAD(p, p);
    for (int kb0 = 0; kb0 < nkb; kb0 += P) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int kb = kb0 + p;
        if (kb < nkb) {
#pragma unroll
          for (int b = 0; b < MB; ++b) {
            const v8i af = v8i{(int)al[p][b].x, (int)al[p][b].y, (int)al[p][b].z, (int)al[p][b].w,
                               (int)ah[p][b].x, (int)ah[p][b].y, (int)ah[p][b].z, (int)ah[p][b].w};
            if constexpr (SCALED) {
              // power-of-two scales: applied exactly by the bf16 conversion (exact path) or as the
              // FP8 MFMA's E8M0 scale operands, so the MFMA accumulates straight into acc (this lane's
              // A row, r16 of block b, has scale sav[p][b]; its B column, of block f / NTW, sbv[p][f / NTW])
              if constexpr (kExact) {
                v8bf ab[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  ab[j] = e4m3x8_to_bf16_scaled((uint32_t)af[2 * j], (uint32_t)af[2 * j + 1], sav[p][b]);
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                  const v8i bfr = v8i{(int)bl[p][f].x, (int)bl[p][f].y, (int)bl[p][f].z, (int)bl[p][f].w,
                                      (int)bh[p][f].x, (int)bh[p][f].y, (int)bh[p][f].z, (int)bh[p][f].w};
                  const float sbf = sbv[p][f / NTW];
#pragma unroll
                  for (int j = 0; j < 4; ++j)
                    acc[b][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        ab[j], e4m3x8_to_bf16_scaled((uint32_t)bfr[2 * j], (uint32_t)bfr[2 * j + 1], sbf), acc[b][f],
                        0, 0, 0);
                }
              } else {
                const int ea = e8m0_of(sav[p][b]);
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                  const v8i bfr = v8i{(int)bl[p][f].x, (int)bl[p][f].y, (int)bl[p][f].z, (int)bl[p][f].w,
                                      (int)bh[p][f].x, (int)bh[p][f].y, (int)bh[p][f].z, (int)bh[p][f].w};
                  acc[b][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bfr, acc[b][f], 0, 0, 0, ea, 0,
                                                                               e8m0_of(sbv[p][f / NTW]));
                }
              }
            } else {
              v4f part[NF];
              if constexpr (kExact) {
                v8bf ab[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) ab[j] = e4m3x8_to_bf16((uint32_t)af[2 * j], (uint32_t)af[2 * j + 1]);
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                  const v8i bfr = v8i{(int)bl[p][f].x, (int)bl[p][f].y, (int)bl[p][f].z, (int)bl[p][f].w,
                                      (int)bh[p][f].x, (int)bh[p][f].y, (int)bh[p][f].z, (int)bh[p][f].w};
                  v4f t = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                  for (int j = 0; j < 4; ++j)
                    t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        ab[j], e4m3x8_to_bf16((uint32_t)bfr[2 * j], (uint32_t)bfr[2 * j + 1]), t, 0, 0, 0);
                  part[f] = t;
                }
              } else {
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                  const v8i bfr = v8i{(int)bl[p][f].x, (int)bl[p][f].y, (int)bl[p][f].z, (int)bl[p][f].w,
                                      (int)bh[p][f].x, (int)bh[p][f].y, (int)bh[p][f].z, (int)bh[p][f].w};
                  part[f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bfr, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                             0, 0, 0, 0);
                }
              }
              // row 4q+i's activation scale sits in lane 4q+i
              float srow[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) srow[i] = __shfl(sav[p][b], 4 * q + i);
#pragma unroll
              for (int f = 0; f < NF; ++f) {
                const float sbf = sbv[p][f / NTW];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[b][f][i] = fmaf(part[f][i], srow[i] * sbf, acc[b][f][i]);
              }
            }
          }
          if (kb + P < nkb) STREAM_LOAD(p, kb + P);
        }
      }
    }
  }
#undef STREAM_LOAD

  void* const out = si ? s1.out : s0.out;
  float* const out_s = si ? s1.out_s : s0.out_s;
  const int ld_out = si ? s1.ld_out : s0.ld_out;
  const int32_t* const dst_row = si ? s1.dst_row : s0.dst_row;
  const float* const row_w = si ? s1.row_w : s0.row_w;
  // lane holds rows m0 + 16 b + 4q + i, columns ncol0 + 16 j + r16 of each B block
  if constexpr (EPI == kEpiSwiglu) {
    float h[MB][NTW][4];
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) h[b][j][i] = swiglu(acc[b][j][i], acc[b][NTW + j][i]);
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = 0.0f;
#pragma unroll
        for (int j = 0; j < NTW; ++j) mx = fmaxf(mx, fabsf(h[b][j][i]));
        mx = group_max<16>(mx);
        if (r16 == 0) red[wave][16 * b + 4 * q + i] = mx;
      }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * b + 4 * q + i;
        const float amax = fmaxf(fmaxf(red[0][r], red[1][r]), fmaxf(red[2][r], red[3][r]));
        const float sc = tile_scale(amax, (si ? s1.pow2_scales : s0.pow2_scales) != 0);
        const float inv = 1.0f / sc;              // x * inv is within an ulp of x / sc (equal for power-of-two sc)
#pragma unroll
        for (int j = 0; j < NTW; j += 2) {
          const uint32_t c2 = e4m3_encode2(h[b][j][i] * inv, h[b][j + 1][i] * inv);
          stage[r * 128 + wave * CW + 16 * j + r16] = (uint8_t)c2;
          stage[r * 128 + wave * CW + 16 * (j + 1) + r16] = (uint8_t)(c2 >> 8);
        }
        if (wave == 0 && r16 == 0 && m0 + r < m_end) out_s[(long)(m0 + r) * (half >> 7) + (nbase >> 7)] = sc;
      }
    __syncthreads();
    if (tid < 128 * MB) {
      const int r = tid >> 3, c = tid & 7;
      if (m0 + r < m_end)
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(out) + (long)(m0 + r) * ld_out + nbase + c * 16) =
            *reinterpret_cast<const u32x4*>(stage + r * 128 + c * 16);
    }
  } else {
    if (!wave_live) return;
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 16 * b + 4 * q + i;
        if (m >= m_end) continue;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int n = ncol0 + 16 * f + r16;
          const float val = acc[b][f][i];
          if constexpr (EPI == kEpiF32) {
            reinterpret_cast<float*>(out)[(long)m * ld_out + n] = val;
          } else if constexpr (EPI == kEpiBf16) {
            reinterpret_cast<uint16_t*>(out)[(long)m * ld_out + n] = f32_to_bf16_rne(val);
          } else {
            const long dst = dst_row ? (long)dst_row[m] : (long)m;
            const float wgt = row_w ? row_w[m] : 1.0f;
            atomicAdd(reinterpret_cast<float*>(out) + dst * ld_out + n, wgt * val);
          }
        }
      }
  }
}

template <int NB, int NTW, int P, int EPI, bool SCALED, bool NFAST>
__global__ __launch_bounds__(256, (SCALED && NB == 1) ? 3 : 1) void stream_gemm_kernel(const GemmArgs args) {
  stream_gemm_body<NB, NTW, P, EPI, SCALED, NFAST, 1>(args);
}

// The same with 32-row tiles (two row blocks per workgroup), used for the gate/up GEMM.
template <int NB, int NTW, int P, int EPI, bool SCALED, bool NFAST>
__global__ __launch_bounds__(256) void stream_gemm2_kernel(const GemmArgs args) {
  stream_gemm_body<NB, NTW, P, EPI, SCALED, NFAST, 2>(args);
}

// The launch's scale format: power-of-two scales when its segments say so (the forward sets both
// segments alike; the C ABI's GEMM call has one segment).
static bool gemm_pow2(const GemmArgs& args) {
  return (args.seg[1].m_tiles > 0 ? args.seg[1] : args.seg[0]).pow2_scales != 0;
}

template <int MB, int PG, int PD>
static hipError_t launch_stream_mb(const GemmArgs& args, int epi, hipStream_t st);

// MB = 1 (groups of up to 16 rows per tile): the decode kernels; MB = 2: 32-row tiles, for the
// gate/up GEMM only (the FP8 down GEMM measured faster on the 64-row LDS tiles there).
static hipError_t launch_stream(const GemmArgs& args, int epi, hipStream_t st, int mb) {
  return mb == 2 ? launch_stream_mb<2, 3, 3>(args, epi, st) : launch_stream_mb<1, 6, 4>(args, epi, st);
}

// PG, PD: K blocks in flight per wave in the gate/up (SwiGLU) and the other kernels.
template <int MB, int PG, int PD>
static hipError_t launch_stream_mb(const GemmArgs& args, int epi, hipStream_t st) {
  const int mt = args.seg[0].m_tiles + args.seg[1].m_tiles;
  if (mt == 0) return hipSuccess;
  const bool swiglu = epi == kEpiSwiglu;
  const int cols = 4 * 16 * 2;                               // columns per workgroup in each block
  int ny = 0;
  for (int s = 0; s < 2; ++s) {
    const GemmSeg& S = args.seg[s];
    if (S.m_tiles > 0) {
      const int half = S.N / (swiglu ? 2 : 1);
      const int n = (half + cols - 1) / cols;
      ny = ny > n ? ny : n;
    }
  }
  if (ny == 0) return hipSuccess;
  const dim3 grid(ny, mt), grid_m(mt, ny);
  if constexpr (MB == 2) {                        // the gate/up (SwiGLU) GEMM only
    if (epi != kEpiSwiglu) return hipErrorInvalidValue;
    if (gemm_pow2(args)) stream_gemm2_kernel<2, 2, PG, kEpiSwiglu, true, true><<<grid, 256, 0, st>>>(args);
    else stream_gemm2_kernel<2, 2, PG, kEpiSwiglu, false, true><<<grid, 256, 0, st>>>(args);
    return hipGetLastError();
  } else {
#define STREAM_LAUNCH(NB_, P_, EPI_, SC_, NF_, G_) stream_gemm_kernel<NB_, 2, P_, EPI_, SC_, NF_><<<G_, 256, 0, st>>>(args)
    if (gemm_pow2(args)) {
      switch (epi) {
        case kEpiSwiglu: STREAM_LAUNCH(2, PG, kEpiSwiglu, true, true, grid); break;
        case kEpiF32: STREAM_LAUNCH(1, PD, kEpiF32, true, false, grid_m); break;
        case kEpiBf16: STREAM_LAUNCH(1, PD, kEpiBf16, true, false, grid_m); break;
        default: STREAM_LAUNCH(1, PD, kEpiScatter, true, false, grid_m); break;
      }
    } else {
      switch (epi) {
        case kEpiSwiglu: STREAM_LAUNCH(2, PG, kEpiSwiglu, false, true, grid); break;
        case kEpiF32: STREAM_LAUNCH(1, PD, kEpiF32, false, false, grid_m); break;
        case kEpiBf16: STREAM_LAUNCH(1, PD, kEpiBf16, false, false, grid_m); break;
        default: STREAM_LAUNCH(1, PD, kEpiScatter, false, false, grid_m); break;
      }
    }
#undef STREAM_LAUNCH
    return hipGetLastError();
  }
}

// ---------------------------------------------------------------------------
// MFMA tile kernel for groups of many rows (prefill, dense layers).
// Workgroup: WM x WN waves (2 x 2, or 2 x 4 for tiles of 64+ rows); tile
// 16*MT*WM rows x 256 B rows (plain: 256 output columns; SwiGLU: 128 gate +
// 128 up rows = one 128-column h tile).  Wave tile: 16*MT rows x 256/WN B rows.
// Staging: A and B tiles of a K block go global -> LDS directly
// (global_load_lds_dwordx4: each wave load writes 1 KB of LDS).  B arrives in
// fragment order, so each B operand read is one 1 KB-contiguous ds_read_b128;
// A arrives as whole 128-byte rows (8 rows per wave load) with the 16-byte
// chunk index XORed by (row & 7), which keeps the 16 lanes of a ds_read_b128
// phase on distinct banks.  3 LDS stages, one barrier per K block.  Per K block
// each wave issues the same number of loads (kLoads), so "my loads for block
// kb are done" is a constant vmcnt.  Tiles with fewer rows than BM (a group's
// last, or all of a small group's) compute only their row blocks, from copies
// of the K loop compiled per count of active row blocks (see the kernel).
constexpr int kStages = 3;

__device__ __forceinline__ void lds_dma16(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 4, 0, 0);
}
// Workgroup barrier without a memory fence: only the compiler is kept from
// moving memory operations across it.  LDS-DMA data is covered by the explicit
// vmcnt waits before it; __syncthreads() would also wait for every outstanding
// load (vmcnt(0)) and empty the prefetch pipeline.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier after this wave's LDS accesses have completed (lgkmcnt(0)), without the wait
// for every outstanding global load and store that __syncthreads() adds.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);           // vmcnt 63 and expcnt 7: no wait; lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) (gfx9 encoding: vmcnt low bits [3:0], high bits [15:14];
// expcnt and lgkmcnt left at their "no wait" maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int WM, int WN, int MT, int EPI, bool SCALED>
__global__ __launch_bounds__(64 * WM * WN) void mfma_gemm_kernel(const GemmArgs args) {
  constexpr int NW = WM * WN;                   // waves
  constexpr int NTW = 16 / WN;                  // 16-column tiles per wave (the workgroup covers 256 B rows)
  constexpr int BM = 16 * MT * WM;
  constexpr bool kExact = EPI == kEpiSwiglu;
  constexpr int A_BYTES = BM * 128, B_BYTES = 256 * 128, SA_BYTES = (BM / 32) * 256;
  constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;
  constexpr int A_LOADS = BM / 8 / NW;          // wave loads of A per wave per K block (2 per 16-row block)
  constexpr int B_LOADS = 32 / NW;              // 16 blocks x 2 halves
  constexpr int kLoads = A_LOADS + B_LOADS + 1; // + one scale load
  static_assert(A_LOADS * NW == BM / 8 && B_LOADS * NW == 32, "loads must split evenly over the waves");
  static_assert(BM / 32 <= NW && BM % 32 == 0, "one scale load per wave at most");
  static_assert(!kExact || (WN >= 2 && BM <= 64 * NW), "the SwiGLU epilogue's per-row scales: red[0..1], a thread per row");
  static_assert(!kExact || NTW % 4 == 0, "SwiGLU waves hold gate and up tiles in pairs and encode h in pairs");
  // one array per pipeline stage: the compiler can then tell the stages apart and does
  // not wait for every LDS-DMA load before each LDS read
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t smem2[STAGE];
  __shared__ float red[WN][BM];

  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, q = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar loads below
  const GemmSeg& s0 = args.seg[0];
  const GemmSeg& s1 = args.seg[1];
  const int ny0 = kExact ? s0.N / 256 : (s0.N + 255) / 256;   // n tiles per segment
  const int ny1 = kExact ? s1.N / 256 : (s1.N + 255) / 256;
  int si, g, m0, m_end, nt;
  if (!find_work(args, BM, ny0, ny1, si, g, m0, m_end, nt)) return;
  // Wave (wm, wn) computes row block wm and column block wn of the tile.  A partial tile (the last
  // tile of a group often is) takes wm = wave / WN: waves are placed on the CU's 4 SIMDs round-robin
  // by wave index, so every SIMD then holds waves of both row halves, and the work left when the
  // rows end in the first half is spread over all four SIMDs.  Full tiles keep wm = wave % WM,
  // measured a few percent faster for them.
  const bool partial = m_end - m0 < BM;
  const int wm = partial ? wave / WN : wave % WM, wn = partial ? wave % WN : wave / WM;
  const int K = si ? s1.K : s0.K, nkb = K >> 7;
  const int Nfull = si ? s1.N : s0.N;
  const int half = Nfull / (kExact ? 2 : 1);
  const uint8_t* const a_q = si ? s1.a_q : s0.a_q;
  const float* const a_s = si ? s1.a_s : s0.a_s;
  const int32_t* const gat = si ? s1.a_gather : s0.a_gather;
  const uint8_t* const bq = (si ? s1.b_q : s0.b_q) + (long long)g * (si ? s1.b_stride : s0.b_stride);
  const float* const bs = (si ? s1.b_s : s0.b_s) + (long long)g * (si ? s1.bs_stride : s0.bs_stride);

  // ---- per-lane global sources of this wave's loads (advanced by kb each K block) ----
  // A: wave load i covers tile rows 8 li .. 8 li + 7 (li = wave * A_LOADS + i) as whole
  //    128-byte rows (full cache lines): lane l takes row r = 8 li + l / 8 and fills slot l % 8 of
  //    that row in LDS with the row's 16-byte chunk (l % 8) ^ (r % 8).  The XOR spreads a fragment
  //    read (16 rows x one chunk) over the LDS banks (measured conflict-free on gfx950, where a
  //    plain row-major layout conflicts 4-way and an XOR with (r % 8) ^ (r / 8 % 2) 2-way).
  const uint8_t* a_src[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int li = wave * A_LOADS + i;
    const int r = 8 * li + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    int m = m0 + r;
    m = m < m_end ? m : m0;
    const long src = gat ? (long)gat[m] : (long)m;
    a_src[i] = a_q + src * K + 16 * c;
  }
  // where this lane's A fragment pieces sit inside a 16-row block (2 KB): row r16, chunks q and 4 + q
  const int a_swz = r16 & 7;
  const int a_off_lo = r16 * 128 + 16 * (q ^ a_swz);
  const int a_off_hi = r16 * 128 + 16 * ((4 + q) ^ a_swz);
  // B: wave load i covers local block bb = (wave * B_LOADS + i) / 2, half h = i % 2.
  const uint8_t* b_src[B_LOADS];
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int li = wave * B_LOADS + i;
    const int bb = li >> 1, h = li & 1;
    const int n16 = kExact ? ((bb >> 3) * half + nt * 128) / 16 + (bb & 7) : (nt * 256) / 16 + bb;
    const int n16c = n16 * 16 < Nfull ? n16 : 0;  // a partial last tile reads block 0 (discarded)
    b_src[i] = bq + (long)n16c * nkb * 2048 + h * 1024 + lane * 16;
  }
  // Scales, one 4-byte LDS-DMA per wave and K block into a 256 B slot: wave w loads the A-row
  // scales of the 32-row group min(w, BM/32 - 1) with lanes 0..31 (surplus waves rewrite the
  // last group with the same values, which keeps every wave's load count equal); lanes 32 and
  // 33 load the tile's two B-scale blocks (plain: columns nt*256 and nt*256 + 128; SwiGLU: the
  // gate and the up block), so the B scales arrive with the stage, under the same vmcnt wait;
  // lanes 34..63 repeat A rows.
  const int sgrp = wave < BM / 32 ? wave : BM / 32 - 1;
  const float* sa_src;
  if (lane == 32 || lane == 33) {
    int blk = kExact ? (lane == 32 ? nt : (half + nt * 128) / 128) : 2 * nt + (lane - 32);
    blk = blk * 128 < Nfull ? blk : 2 * nt;       // a partial last tile: the missing block is never stored
    sa_src = bs + (long)blk * nkb;
  } else {
    int m = m0 + sgrp * 32 + (lane & 31);
    m = m < m_end ? m : m0;
    sa_src = a_s + (gat ? (long)gat[m] : (long)m) * nkb;
  }
  // this wave's B-scale slot(s): plain: the 128-column block its columns fall in; SwiGLU: gate, up
  const int sb_slot = kExact ? 0 : (wn * NTW * 16) / 128;

#define MFMA_ISSUE(kb_, dst_)                                                                         \
  {                                                                                                   \
    uint8_t* st_ = (dst_);                                                                            \
    _Pragma("unroll") for (int i = 0; i < A_LOADS; ++i)                                              \
        lds_dma16(a_src[i] + (kb_) * 128, st_ + (wave * A_LOADS + i) * 1024);                         \
    _Pragma("unroll") for (int i = 0; i < B_LOADS; ++i)                                              \
        lds_dma16(b_src[i] + (long)(kb_) * 2048, st_ + A_BYTES + (wave * B_LOADS + i) * 1024);        \
    lds_dma4(sa_src + (kb_), st_ + A_BYTES + B_BYTES + sgrp * 256);                                   \
  }

  v4f acc[MT][NTW];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int f = 0; f < NTW; ++f) acc[mi][f] = v4f{0.f, 0.f, 0.f, 0.f};
  const int lane_off = lane * 16;
  // In a partial tile a wave computes only its 16-row blocks that hold rows of the group (nmi of
  // them, from its own copy of the K loop below), and a wave with none of them only loads and
  // synchronises.
  const int nmi = __builtin_amdgcn_readfirstlane(min(MT, max(0, (m_end - m0 - wm * 16 * MT + 15) / 16)));
  const bool wave_has_rows = nmi > 0;

  // MFMAs and scale promotion of one K block from the LDS stage at st (+ this lane's offset)
  auto compute = [&](const uint8_t* st, int nblk) __attribute__((always_inline)) {
    const uint8_t* const stb = st - lane_off;
    auto load_a = [&](int mi) {
      const int ab = wm * MT + mi;
      const v4i lo = *reinterpret_cast<const v4i*>(stb + ab * 2048 + a_off_lo);
      const v4i hi = *reinterpret_cast<const v4i*>(stb + ab * 2048 + a_off_hi);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // LDS reads in the order the MFMAs need them: the first A fragment, then the B fragments;
    // the next A fragment is read one row block ahead
    v8i af_next = load_a(0);
    const float* sbp = reinterpret_cast<const float*>(st - lane_off + A_BYTES + B_BYTES + 128);
    const float sb0 = sbp[sb_slot];
    const float sb1 = kExact ? sbp[1] : sb0;
    // B fragments of this wave: plain: local blocks NTW wn .. +NTW-1; SwiGLU: gate (NTW/2) wn .. and the
    // same up blocks (+8)
    v8i bf[NTW];
#pragma unroll
    for (int f = 0; f < NTW; ++f) {
      constexpr int H = NTW / 2;
      const int bb = kExact ? ((f / H) * 8 + wn * H + (f % H)) : (wn * NTW + f);
      const v4i lo = *reinterpret_cast<const v4i*>(st + A_BYTES + bb * 2048);
      const v4i hi = *reinterpret_cast<const v4i*>(st + A_BYTES + bb * 2048 + 1024);
      bf[f] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      if (mi >= nblk) break;                    // row blocks past the group's end (nblk: a constant per copy)
      const int ab = wm * MT + mi;
      const v8i af = af_next;
      if (mi + 1 < MT) af_next = load_a(mi + 1);
      const int r0 = ab * 16;                   // the lane's rows are r0 + 4q .. +3
      const float4 sa4 = *reinterpret_cast<const float4*>(st - lane_off + A_BYTES + B_BYTES + (r0 >> 5) * 256 +
                                                          (r0 & 31) * 4 + q * 16);
      if constexpr (SCALED) {
        // power-of-two scales: the lane's A row r0 + r16 has scale sa_in; applied exactly by the bf16
        // conversion (exact path) or as the FP8 MFMA's E8M0 scale operands, accumulating into acc
        const float sa_in = *reinterpret_cast<const float*>(st - lane_off + A_BYTES + B_BYTES + (r0 >> 5) * 256 +
                                                            ((r0 & 31) + r16) * 4);
        if constexpr (kExact) {
          v8bf ab8[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) ab8[j] = e4m3x8_to_bf16_scaled((uint32_t)af[2 * j], (uint32_t)af[2 * j + 1], sa_in);
#pragma unroll
          for (int f = 0; f < NTW; ++f) {
            const float sbf = f >= NTW / 2 ? sb1 : sb0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  e4m3x8_to_bf16_scaled((uint32_t)bf[f][2 * j], (uint32_t)bf[f][2 * j + 1], sbf), ab8[j], acc[mi][f], 0,
                  0, 0);
          }
        } else {
          const int ea = e8m0_of(sa_in), eb = e8m0_of(sb0);
#pragma unroll
          for (int f = 0; f < NTW; ++f)
            acc[mi][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[f], acc[mi][f], 0, 0, 0, ea, 0, eb);
        }
        continue;
      }
      if constexpr (kExact) {
        // the weights are the MFMA's first operand here, so the lane's 4 outputs of a tile are 4
        // columns of one row (r0 + r16) and share one scale product per K block: sa x sb_gate and
        // sa x sb_up for the row, two multiplies per row block instead of eight
        const float sa_row = *reinterpret_cast<const float*>(st - lane_off + A_BYTES + B_BYTES + (r0 >> 5) * 256 +
                                                             ((r0 & 31) + r16) * 4);
        const float cg = sa_row * sb0, cu = sa_row * sb1;
        v8bf ab8[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) ab8[j] = e4m3x8_to_bf16((uint32_t)af[2 * j], (uint32_t)af[2 * j + 1]);
#pragma unroll
        for (int f0 = 0; f0 < NTW; f0 += 4) {     // promote in groups of 4 tiles: fewer live partials
          v4f part[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int f = f0 + u;
            v4f t = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j)
              t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  e4m3x8_to_bf16((uint32_t)bf[f][2 * j], (uint32_t)bf[f][2 * j + 1]), ab8[j], t, 0, 0, 0);
            part[u] = t;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[mi][f0 + u][i] = fmaf(part[u][i], f0 + u >= NTW / 2 ? cu : cg, acc[mi][f0 + u][i]);
        }
        continue;
      }
      const float c0[4] = {sa4.x * sb0, sa4.y * sb0, sa4.z * sb0, sa4.w * sb0};
#pragma unroll
      for (int f0 = 0; f0 < NTW; f0 += 4) {       // promote in groups of 4 tiles: fewer live partials
        v4f part[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          part[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[f0 + u], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                     0, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mi][f0 + u][i] = fmaf(part[u][i], c0[i], acc[mi][f0 + u][i]);
      }
    }
  };

  // One K block: wait for this wave's loads of block kb (the loads of kb + 1 may stay in
  // flight), barrier (everyone's block kb has landed and everyone is done with block kb - 1,
  // whose stage the loads of kb + 2 now overwrite), issue kb + 2, compute kb.  The stage
  // arrays are named statically (K loop unrolled by the 3 stages) so the compiler can tell
  // them apart and keeps the other stages' loads in flight.  The main loop has no branches
  // inside: with control flow in the loop body the compiler's wait insertion loses track of
  // which stage a pending LDS-DMA load writes and waits for all of them before LDS reads.
  // The last one to four blocks run in a peeled tail.
#define MFMA_STEP(kb_, cur_, nxt_, nblk_)                                                             \
  {                                                                                                   \
    wait_vmcnt<kLoads>();                                                                             \
    block_barrier();                                                                                  \
    MFMA_ISSUE((kb_) + 2, nxt_);                                                                      \
    if (wave_has_rows) compute((cur_) + lane_off, nblk_);                                             \
  }
// Step t of a tail of R steps (t, R literals: straight-line code, no branches for the compiler's
// wait insertion to merge over): block kb0 + t, whose successor is in flight unless t + 1 == R.
#define MFMA_STEP_TAIL(t_, R_, cur_, nxt_, nblk_)                                                     \
  {                                                                                                   \
    if ((t_) + 1 < (R_)) wait_vmcnt<kLoads>(); else wait_vmcnt<0>();                                  \
    block_barrier();                                                                                  \
    if ((t_) + 2 < (R_)) MFMA_ISSUE(kb0 + (t_) + 2, nxt_);                                            \
    if (wave_has_rows) compute((cur_) + lane_off, nblk_);                                             \
  }
// The same with run-time bounds checks (one copy of the tail: fewer registers, but the compiler then
// waits for every LDS-DMA load, the just-issued ones included, before the step's LDS reads).
#define MFMA_STEP_TAIL_RT(kb_, cur_, nxt_, nblk_)                                                     \
  {                                                                                                   \
    const int kbs = (kb_);                                                                            \
    if (kbs + 1 < nkb) wait_vmcnt<kLoads>(); else wait_vmcnt<0>();                                    \
    block_barrier();                                                                                  \
    if (kbs + 2 < nkb) MFMA_ISSUE(kbs + 2, nxt_);                                                     \
    if (wave_has_rows) compute((cur_) + lane_off, nblk_);                                             \
  }
// K loop without a tail (partial tiles of the SwiGLU kernel): whole rounds of 3 steps; a step past
// the last block issues a surplus copy of the last block (an unconditional issue keeps the
// compiler's tracking of the stages intact) and computes nothing; the surplus loads land before
// the stages are reused.
#define MFMA_STEP_PAD(kb_, cur_, nxt_, nblk_)                                                         \
  {                                                                                                   \
    const int kbs = (kb_);                                                                            \
    wait_vmcnt<kLoads>();                                                                             \
    block_barrier();                                                                                  \
    MFMA_ISSUE(min(kbs + 2, nkb - 1), nxt_);                                                          \
    if (wave_has_rows && kbs < nkb) compute((cur_) + lane_off, nblk_);                                \
  }
#define MFMA_KLOOP_PAD(nblk_)                                                                         \
  {                                                                                                   \
    MFMA_ISSUE(0, smem0);                                                                             \
    MFMA_ISSUE(nkb > 1 ? 1 : 0, smem1);                                                               \
    for (int kb0 = 0; kb0 < nkb; kb0 += 3) {                                                          \
      MFMA_STEP_PAD(kb0, smem0, smem2, nblk_);                                                        \
      MFMA_STEP_PAD(kb0 + 1, smem1, smem0, nblk_);                                                    \
      MFMA_STEP_PAD(kb0 + 2, smem2, smem1, nblk_);                                                    \
    }                                                                                                 \
    wait_vmcnt<0>();                                                                                  \
  }
// K loop with a peeled tail (nkb steps).
#define MFMA_KLOOP(nblk_)                                                                             \
  {                                                                                                   \
    MFMA_ISSUE(0, smem0);                                                                             \
    MFMA_ISSUE(nkb > 1 ? 1 : 0, smem1);  /* unconditional (no branch before the loop); for nkb == 1  \
                                            a copy of block 0 that is never read */                   \
    int kb0 = 0;                                                                                      \
    for (; kb0 + 4 < nkb; kb0 += 3) {    /* every step here issues block kb + 2 < nkb */              \
      MFMA_STEP(kb0, smem0, smem2, nblk_);                                                            \
      MFMA_STEP(kb0 + 1, smem1, smem0, nblk_);                                                        \
      MFMA_STEP(kb0 + 2, smem2, smem1, nblk_);                                                        \
    }                                                                                                 \
    /* 2 to 4 blocks remain (1 when nkb == 1); kb0 is a multiple of 3.  The SwiGLU and 4-wave       \
       kernels keep the single run-time-checked copy (the straight-line ones push them past their     \
       register budget); the 8-wave plain kernels (the down GEMM's tail is 4 of 16 blocks) take the   \
       straight-line copies. */                                                                       \
    if constexpr (kExact || NW < 8) {                                                                 \
      MFMA_STEP_TAIL_RT(kb0, smem0, smem2, nblk_);                                                    \
      if (kb0 + 1 < nkb) MFMA_STEP_TAIL_RT(kb0 + 1, smem1, smem0, nblk_);                             \
      if (kb0 + 2 < nkb) MFMA_STEP_TAIL_RT(kb0 + 2, smem2, smem1, nblk_);                             \
      if (kb0 + 3 < nkb) MFMA_STEP_TAIL_RT(kb0 + 3, smem0, smem2, nblk_);                             \
    } else switch (nkb - kb0) {                                                                       \
      case 1:                                                                                         \
        MFMA_STEP_TAIL(0, 1, smem0, smem2, nblk_);                                                    \
        break;                                                                                        \
      case 2:                                                                                         \
        MFMA_STEP_TAIL(0, 2, smem0, smem2, nblk_);                                                    \
        MFMA_STEP_TAIL(1, 2, smem1, smem0, nblk_);                                                    \
        break;                                                                                        \
      case 3:                                                                                         \
        MFMA_STEP_TAIL(0, 3, smem0, smem2, nblk_);                                                    \
        MFMA_STEP_TAIL(1, 3, smem1, smem0, nblk_);                                                    \
        MFMA_STEP_TAIL(2, 3, smem2, smem1, nblk_);                                                    \
        break;                                                                                        \
      default:                                                                                        \
        MFMA_STEP_TAIL(0, 4, smem0, smem2, nblk_);                                                    \
        MFMA_STEP_TAIL(1, 4, smem1, smem0, nblk_);                                                    \
        MFMA_STEP_TAIL(2, 4, smem2, smem1, nblk_);                                                    \
        MFMA_STEP_TAIL(3, 4, smem0, smem2, nblk_);                                                    \
        break;                                                                                        \
    }                                                                                                 \
  }

  // One branch-free copy of the K loop per count of row blocks a wave computes (a branch per row
  // block made the compiler's wait insertion lose track of the LDS-DMA stages and wait for every
  // load once per unrolled iteration); a wave without rows runs the 1-block copy, compute off.  The
  // waves of a workgroup may run different copies, so every copy a workgroup can choose must pass
  // the same barriers: the loop form is chosen per tile.  SwiGLU kernel: full tiles run the loop
  // with the checked tail (nkb steps); partial tiles run padded copies (whole rounds of 3 steps),
  // since next to the checked tail any further copy of that loop again waited for every load.
  // Plain kernels: every copy has the straight-line tail.
  {
    const int nk = nmi < 1 ? 1 : nmi;
    if constexpr (kExact) {
      if (!partial) MFMA_KLOOP(MT)
      else if (nk >= MT) MFMA_KLOOP_PAD(MT)
      else if constexpr (MT == 4) {
        if (nk == 3) MFMA_KLOOP_PAD(3)
        else if (nk == 2) MFMA_KLOOP_PAD(2)
        else MFMA_KLOOP_PAD(1)
      } else if constexpr (MT == 2) {
        MFMA_KLOOP_PAD(1)
      }
    } else {
      if (nk >= MT) MFMA_KLOOP(MT)
      else if constexpr (MT == 4) {
        if (nk == 3) MFMA_KLOOP(3)
        else if (nk == 2) MFMA_KLOOP(2)
        else MFMA_KLOOP(1)
      } else if constexpr (MT == 2) {
        MFMA_KLOOP(1)
      }
    }
  }
#undef MFMA_KLOOP
#undef MFMA_KLOOP_PAD
#undef MFMA_STEP_PAD
#undef MFMA_STEP_TAIL_RT
#undef MFMA_STEP_TAIL
#undef MFMA_STEP
#undef MFMA_ISSUE

  void* const out = si ? s1.out : s0.out;
  float* const out_s = si ? s1.out_s : s0.out_s;
  const int ld_out = si ? s1.ld_out : s0.ld_out;
  const int32_t* const dst_row = si ? s1.dst_row : s0.dst_row;
  const float* const row_w = si ? s1.row_w : s0.row_w;
  // plain: lane holds rows wm*16*MT + 16 mi + 4q + i of the tile, columns nt*256 + wn*16*NTW + 16 f + r16;
  // SwiGLU (weights as the MFMA's first operand): lane holds row wm*16*MT + 16 mi + r16, h columns
  // nt*128 + wn*8*NTW + 16 j + 4q + i (gate f = j, up f = NTW/2 + j)
  if constexpr (EPI == kEpiSwiglu) {
    constexpr int H = NTW / 2;
    float h[MT][H][4];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int j = 0; j < H; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) h[mi][j][i] = swiglu(acc[mi][j][i], acc[mi][H + j][i]);
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      float mx = 0.0f;
#pragma unroll
      for (int j = 0; j < H; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(h[mi][j][i]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));             // the row's four quads
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (q == 0) red[wn][wm * 16 * MT + mi * 16 + r16] = mx;
    }
    __syncthreads();                                // also: every wave is past its last LDS stage read
    // one thread per row: the tile's amax, its scale and the scale's reciprocal (red[0][r] and
    // red[1][r] then hold sc and 1/sc; only this thread reads row r's partial maxima)
    if (tid < BM) {
      const int r = tid;
      float amax = red[0][r];
#pragma unroll
      for (int w2 = 1; w2 < WN; ++w2) amax = fmaxf(amax, red[w2][r]);
      const float sc = tile_scale(amax, (si ? s1.pow2_scales : s0.pow2_scales) != 0);
      red[0][r] = sc;
      red[1][r] = 1.0f / sc;                        // x * (1/sc) is within an ulp of x / sc (equal for power-of-two sc)
      if (m0 + r < m_end) out_s[(long)(m0 + r) * (half >> 7) + nt] = sc;
    }
    lds_barrier();
    uint8_t* stage = smem0;                         // BM x 128 codes
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      const int r = wm * 16 * MT + mi * 16 + r16;
      const float inv = red[1][r];
#pragma unroll
      for (int j = 0; j < H; ++j)
        *reinterpret_cast<uint32_t*>(stage + r * 128 + wn * 16 * H + 16 * j + 4 * q) =
            e4m3_encode4(h[mi][j][0] * inv, h[mi][j][1] * inv, h[mi][j][2] * inv, h[mi][j][3] * inv);
    }
    __syncthreads();
    for (int ci = tid; ci < BM * 8; ci += 64 * NW) {
      const int r = ci >> 3, c = ci & 7;
      if (m0 + r < m_end)
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(out) + (long)(m0 + r) * ld_out + nt * 128 + c * 16) =
            *reinterpret_cast<const u32x4*>(stage + r * 128 + c * 16);
    }
  } else if constexpr (EPI == kEpiScatter) {
    const int N = si ? s1.N : s0.N;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 16 * MT + mi * 16 + 4 * q + i;
        if (m >= m_end) continue;
        const long dst = dst_row ? (long)dst_row[m] : (long)m;
        const float wgt = row_w ? row_w[m] : 1.0f;
#pragma unroll
        for (int f = 0; f < NTW; ++f) {
          const int n = nt * 256 + wn * 16 * NTW + 16 * f + r16;
          if (n < N) atomicAdd(reinterpret_cast<float*>(out) + dst * ld_out + n, wgt * acc[mi][f][i]);
        }
      }
  } else {
    // Plain stores: each wave writes its 16*MT x 16*NTW fp32 tile to its own slice of the (now free)
    // stage arrays and reads it back by rows, so every lane stores 16 contiguous bytes (fp32) or 8
    // (bf16) and 16 lanes cover 256 contiguous bytes of a row: 4x fewer store instructions, and no
    // per-element address arithmetic.  Columns are XOR-swizzled by row bits 2-3 (the lane's quad),
    // so the four quads' writes of one fragment row fall on distinct LDS banks.
    constexpr int TR = 16 * MT, TC = 16 * NTW, TBYTES = TR * TC * 4, PER = STAGE / TBYTES;
    static_assert(3 * PER >= NW, "the wave tiles must fit the stage arrays");
    block_barrier();                              // every wave is past its last read of the stages
    uint8_t* const arr = wave / PER == 0 ? smem0 : (wave / PER == 1 ? smem1 : smem2);
    float* const wt = reinterpret_cast<float*>(arr + (wave % PER) * TBYTES);
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int f = 0; f < NTW; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mi * 16 + 4 * q + i, c = 16 * f + r16;
          wt[r * TC + (c ^ (((r >> 2) & 3) << 4))] = acc[mi][f][i];
        }
    const int N = si ? s1.N : s0.N;
    const int mrow0 = m0 + wm * TR, ncol0 = nt * 256 + wn * TC;
#pragma unroll
    for (int it = 0; it < TR * TC / 4 / 64; ++it) {
      const int t = it * 64 + lane, r = t / (TC / 4), c = (t % (TC / 4)) * 4;
      const float4 v = *reinterpret_cast<const float4*>(wt + r * TC + (c ^ (((r >> 2) & 3) << 4)));
      const int m = mrow0 + r, n = ncol0 + c;
      if (m < m_end && n < N) {
        if constexpr (EPI == kEpiF32) {
          // written once and read once, later, by the combine: a nontemporal store (V3 prefill
          // down GEMM 1.108 -> 1.085 ms)
          __builtin_nontemporal_store(v4f{v.x, v.y, v.z, v.w},
                                      reinterpret_cast<v4f*>(reinterpret_cast<float*>(out) + (long)m * ld_out + n));
        } else {
          uint2 o;
          o.x = (uint32_t)f32_to_bf16_rne(v.x) | ((uint32_t)f32_to_bf16_rne(v.y) << 16);
          o.y = (uint32_t)f32_to_bf16_rne(v.z) | ((uint32_t)f32_to_bf16_rne(v.w) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + (long)m * ld_out + n) = o;
        }
      }
    }
  }
}

template <int WM, int WN, int MT, int EPI>
static void launch_mfma_cfg(const GemmArgs& args, dim3 grid, hipStream_t st) {
  if (gemm_pow2(args)) mfma_gemm_kernel<WM, WN, MT, EPI, true><<<grid, 64 * WM * WN, 0, st>>>(args);
  else mfma_gemm_kernel<WM, WN, MT, EPI, false><<<grid, 64 * WM * WN, 0, st>>>(args);
}

// bm = rows per tile: 64 or 128.  The plain and SwiGLU epilogues run 8 waves with 64-column
// wave tiles (two waves per SIMD: one's LDS reads and VALU work overlap the other's MFMAs;
// measured 5-15% faster for the FP8 down GEMM than 4 waves with 128-column wave tiles, which
// need half the LDS reads per MFMA); the scatter epilogue runs 4 waves.
template <int MT>
static hipError_t launch_mfma(const GemmArgs& args, int epi, hipStream_t st) {
  const bool swiglu = epi == kEpiSwiglu;
  // workgroups per XCD: its static panels (at most ceil(panels / 8) of them) and an eighth of the
  // dynamic segment's items (upper bound: m tiles reserved x n tiles)
  const GemmSeg& S0 = args.seg[0];
  const GemmSeg& S1 = args.seg[1];
  const long ny0 = S0.m_tiles > 0 ? (swiglu ? S0.N / 256 : (S0.N + 255) / 256) : 0;
  const long ny1 = S1.m_tiles > 0 ? (swiglu ? S1.N / 256 : (S1.N + 255) / 256) : 0;
  const long panels = ((long)S0.m_tiles + kPanel - 1) / kPanel;
  const long per_xcd = (panels + 7) / 8 * kPanel * ny0 + ((long)S1.m_tiles * ny1 + 7) / 8;
  if (per_xcd == 0) return hipSuccess;
  const dim3 grid((unsigned)(8 * per_xcd));
  switch (epi) {
    case kEpiSwiglu:
      launch_mfma_cfg<2, 4, MT, kEpiSwiglu>(args, grid, st);
      break;
    case kEpiF32:
      launch_mfma_cfg<2, 4, MT, kEpiF32>(args, grid, st);
      break;
    case kEpiBf16:
      launch_mfma_cfg<2, 4, MT, kEpiBf16>(args, grid, st);
      break;
    default: launch_mfma_cfg<2, 2, MT, kEpiScatter>(args, grid, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmArgs& args, int epi, int bm, hipStream_t st) {
  switch (bm) {
    case 16: return launch_stream(args, epi, st, 1);
    case 32: return launch_stream(args, epi, st, 2);
    case 64: return launch_mfma<2>(args, epi, st);
    default: return launch_mfma<4>(args, epi, st);
  }
}

// Tile rows from the average group size (the host does not know the groups' sizes).  Measured
// on the V3 layer from T = 64 to 4096 tokens (per layer, ms): the weight-streaming kernel wins up
// to 10 rows per expert (T = 320: 1.99 against 2.04 for 64-row tiles) and loses from 11 (T = 352:
// 2.07 against 2.03; T = 512: 2.74 against 2.10), since its experts with more than 16 rows stream
// their weights once per 16-row tile; 64-row tiles beat 32-row ones everywhere (T = 1024: 2.28
// against 3.28 ms) and 128-row ones up to 56 rows per expert (T = 1536: 2.48 against 2.53;
// T = 2048, 64 rows: 3.0 against 2.75).  A single group (the dense layer) has exactly its rows,
// so 64-row tiles hold it up to 64.  The gate/up GEMM (SwiGLU epilogue) takes the 32-row streaming
// tiles from 11 to 18 rows: T = 352: 1.20 against 1.28 ms for the 64-row tiles, T = 512: 1.24
// against 1.30, T = 576: 1.28 against 1.30, T = 640: 1.32 against 1.31; the FP8 down GEMM ran
// slower on them at every size (T = 352: 0.72 against 0.66 ms) and keeps the 64-row tiles.
int gemm_pick_bm(long rows_upper, int groups, bool swiglu) {
  const long avg = groups > 0 ? rows_upper / groups : rows_upper;
  if (avg <= 10) return 16;
  if (swiglu && avg <= 18) return 32;
  if (avg <= (groups > 1 ? 56 : 64)) return 64;
  return 128;
}

}  // namespace moefp8
