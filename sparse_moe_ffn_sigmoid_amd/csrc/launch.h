// Host-side launchers of the gfx950 kernels (internal to libmoefp8).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moefp8 {

enum Epi { kEpiF32 = 0, kEpiBf16 = 1, kEpiSwiglu = 2, kEpiScatter = 3 };

// One segment of a grouped GEMM launch.  A static segment (offsets == nullptr)
// is one group of m_rows rows; a dynamic one reads its G+1 row offsets on the
// device.  Row m of group g multiplies B rows [0, N) of that group.
struct GemmSeg {
  const uint8_t* a_q;        // [*][K] e4m3
  const float* a_s;          // [*][K/128]
  const int32_t* a_gather;   // logical row -> source row, or nullptr
  const uint8_t* b_q;        // [G][N][K] in MFMA-fragment order (moe_pack_weights)
  const float* b_s;          // [G][N/128][K/128]
  long long b_stride;        // N*K
  long long bs_stride;       // (N/128)*(K/128)
  const int32_t* offsets;    // [G+1] on the device, or nullptr (static)
  int G;
  int m_rows;                // static segment rows
  int m_tiles;               // tiles reserved in the grid for this segment
  int N;
  int K;                     // % 128 == 0
  void* out;                 // epilogue output
  float* out_s;              // SwiGLU: scales [M][N/256]
  int ld_out;                // elements per output row
  const int32_t* dst_row;    // scatter: destination row per logical row (nullptr = identity)
  const float* row_w;        // scatter: weight per logical row (nullptr = 1)
  int pow2_scales;           // nonzero: every scale is a power of two (UE8M0): a_s and b_s enter through the
                             // MFMA's scale operands (FP8) or the bf16 conversion (exact path) instead of
                             // a per-block promotion, and the SwiGLU requantisation writes power-of-two scales
};

struct GemmArgs {
  GemmSeg seg[2];            // seg[0] static (may be empty), seg[1] dynamic (may be empty)
};

hipError_t launch_quant_1x128(const void* x, bool bf16, int rows, int cols, int ld_x, uint8_t* q, int ld_q, float* s,
                              bool pow2, hipStream_t st);
hipError_t launch_quant_128x128(const float* w, int rows, int cols, uint8_t* q, float* s, bool pow2, hipStream_t st);
hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps, int rows, int cols, int ld_x,
                                uint16_t* y, int ld_y, uint8_t* q, int ld_q, float* s, bool pow2, hipStream_t st);
hipError_t launch_bias_update(const int32_t* topk_idx, long n, int E, float gamma, float* bias, int32_t* counts,
                              hipStream_t st);
hipError_t launch_pack(const uint8_t* src, int G, int N, int K, uint8_t* dst, hipStream_t st);
// part: NULL, or a buffer of part_floats floats for partial logits (the K splits use it when it
// holds their T * E * splits floats; scores must then be 16-byte aligned).
// xq: NULL, or x's 1x128 quantisation outputs (row length D), written by the small-batch split's
// finishing kernel; only when router_small_split() holds for the same arguments.
struct RouterQuant {
  uint8_t* q;
  float* s;
  bool pow2;
};
bool router_small_split(int T, int E, int D, const float* part, size_t part_floats);
hipError_t launch_router(const uint16_t* x, const uint16_t* w, int T, int E, int D, float* scores, float* part,
                         size_t part_floats, const RouterQuant* xq, hipStream_t st);
hipError_t launch_route(const float* scores, const float* bias, int T, int E, int k, int G, int gk, int rule,
                        float routed_scale, int32_t* topk_idx, float* topk_w, hipStream_t st);
size_t permute_scratch_bytes(int n, int E);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets, int32_t* sorted_assign,
                          int32_t* assign_pos, int32_t* sorted_token, const float* topk_w, float* sorted_w,
                          int32_t* scratch, hipStream_t st);
hipError_t launch_gather_rows(const void* rows_in, int row_bytes, int n, int k, const int32_t* sorted_assign,
                              void* rows_out, hipStream_t st);
hipError_t launch_combine(const float* y, const int32_t* ap, const float* w, const float* shared, int T, int k, int d,
                          uint16_t* out, hipStream_t st);
hipError_t launch_unpermute(const void* y, const int32_t* ap, long n, int row_bytes, void* out, hipStream_t st);
hipError_t launch_cast_bf16(const float* in, long n, uint16_t* out, hipStream_t st);
hipError_t launch_fill_zero(float* p, long n, hipStream_t st);

// FP8 backward (backward.hip).
hipError_t launch_pad_offsets(const int32_t* offsets, int G, int32_t* padded, hipStream_t st);
hipError_t launch_quant_128x1_grouped(const void* x, bool bf16, int ld_x, const int32_t* offsets, int G,
                                      const int32_t* padded, int M_pad_max, int N, uint8_t* qt, int ld_q, float* st,
                                      bool pow2, hipStream_t s);
hipError_t launch_pack_transposed(const uint8_t* src, const float* s, int G, int N, int K, uint8_t* dst, float* s_t,
                                  hipStream_t st);
hipError_t launch_wgrad(const uint8_t* a_t, const float* a_ts, const uint8_t* b_t, const float* b_ts,
                        const int32_t* padded, int G, int Na, int Nb, int ld, float* out, bool pow2, hipStream_t st);

// Grouped block-scaled GEMM.  bm = rows per tile (16, 32, 64 or 128); the
// caller sets each segment's m_tiles for that bm.
hipError_t launch_grouped_gemm(const GemmArgs& args, int epi, int bm, hipStream_t st);
int gemm_pick_bm(long rows_upper, int groups, bool swiglu);

// Device-data checks (validate.hip).  Each runs on `st`, synchronises it and sets *first_bad to
// the smallest offending element index, or -1 when every element passes.
//   validate_range:   v[i] in [lo, hi) for i < n
//   validate_offsets: off[0..G] nondecreasing multiples of align, off[0] == first (first < 0:
//                     off[0] >= 0), off[G] <= last (== last when last_exact)
//   validate_rows:    idx[m] >= 0 for off[0] <= m < off[G] (off already validated; max_rows
//                     bounds off[G])
//   validate_finite:  v[i] neither NaN nor infinite for i < n
hipError_t validate_range(const int32_t* v, int n, int lo, int hi, hipStream_t st, long* first_bad);
hipError_t validate_offsets(const int32_t* off, int G, int first, int last, bool last_exact, int align, hipStream_t st,
                            long* first_bad);
hipError_t validate_rows(const int32_t* idx, const int32_t* off, int G, int max_rows, hipStream_t st, long* first_bad);
hipError_t validate_finite(const float* v, long n, hipStream_t st, long* first_bad);

}  // namespace moefp8
