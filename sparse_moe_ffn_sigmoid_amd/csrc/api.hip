// C ABI of libmoefp8: argument checks, workspace carve-up and kernel launches.
// Every entry point validates on the host before enqueueing anything and
// returns a status; launches are asynchronous on the caller's stream.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.h"
#include "moefp8.h"

using namespace moefp8;

// Workspace of moe_ffn_forward_noalloc: one array per GPU, allocated when the code object is
// loaded on that GPU and held until the process ends.  In host code the array's name is only a
// host-side stand-in: its device address comes from hipGetSymbolAddress, once per device, and
// only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return MOE_OK;
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

#define HIP_TRY(expr, what)                       \
  do {                                            \
    const int st_ = hip_check((expr), (what));    \
    if (st_ != MOE_OK) return st_;                \
  } while (0)

// MOEFP8_VALIDATE, read at each call: set to anything but "" or "0", the calls check the device
// data they would otherwise trust (validate.hip) before enqueueing their own kernels.
bool validation_on() {
  const char* e = std::getenv("MOEFP8_VALIDATE");
  return e && *e && std::strcmp(e, "0") != 0;
}

// One element of a device array, for the message of a failed check (the stream is synchronised).
long read_i32(const int32_t* p, long i) {
  int32_t v = 0;
  return hipMemcpy(&v, p + i, sizeof(v), hipMemcpyDeviceToHost) == hipSuccess ? (long)v : -999999999L;
}
double read_f32(const float* p, long i) {
  float v = 0.0f;
  return hipMemcpy(&v, p + i, sizeof(v), hipMemcpyDeviceToHost) == hipSuccess ? (double)v : 0.0;
}

// Runs a validate_* check (it sets bad_) and returns MOE_ERR_INVALID_DATA with the message when
// an element fails.
#define VALIDATE(check, ...)                                                   \
  do {                                                                         \
    long bad_ = -1;                                                            \
    HIP_TRY((check), "MOEFP8_VALIDATE check");                                 \
    if (bad_ >= 0) return fail(MOE_ERR_INVALID_DATA, "MOEFP8_VALIDATE: " __VA_ARGS__); \
  } while (0)

// Routing configuration checks shared by moe_route and moe_ffn_forward.
int check_route_cfg(const moe_cfg_t* c) {
  REQUIRE(c, MOE_ERR_INVALID_ARG, "cfg is NULL");
  REQUIRE(c->n_experts >= 1 && c->n_experts <= 1024, MOE_ERR_UNSUPPORTED_SHAPE, "n_experts %d not in [1, 1024]",
          c->n_experts);
  REQUIRE(c->n_group >= 1 && c->n_group <= 64, MOE_ERR_UNSUPPORTED_SHAPE, "n_group %d not in [1, 64]", c->n_group);
  REQUIRE(c->n_experts % c->n_group == 0, MOE_ERR_UNSUPPORTED_SHAPE, "n_experts %d %% n_group %d != 0", c->n_experts,
          c->n_group);
  REQUIRE(c->topk_group >= 1 && c->topk_group <= c->n_group, MOE_ERR_INVALID_ARG, "topk_group %d not in [1, %d]",
          c->topk_group, c->n_group);
  const int pool = c->topk_group * (c->n_experts / c->n_group);
  REQUIRE(c->top_k >= 1 && c->top_k <= pool && c->top_k <= 64, MOE_ERR_INVALID_ARG,
          "top_k %d not in [1, min(64, topk_group * n_experts / n_group = %d)]", c->top_k, pool);
  REQUIRE(c->group_score == MOE_GROUP_SCORE_TOP2_SUM || c->group_score == MOE_GROUP_SCORE_MAX, MOE_ERR_INVALID_ARG,
          "group_score %d unknown", c->group_score);
  return MOE_OK;
}

int check_layer_cfg(const moe_cfg_t* c) {
  REQUIRE(c, MOE_ERR_INVALID_ARG, "cfg is NULL");
  REQUIRE(c->scale_fmt == MOE_SCALE_F32 || c->scale_fmt == MOE_SCALE_UE8M0, MOE_ERR_INVALID_ARG,
          "scale_fmt %d unknown", c->scale_fmt);
  REQUIRE(c->norm_eps >= 0.0f && c->norm_eps < 3.0e38f, MOE_ERR_INVALID_ARG, "norm_eps %g not finite and >= 0",
          (double)c->norm_eps);
  REQUIRE(c->hidden > 0 && c->hidden % 128 == 0, MOE_ERR_UNSUPPORTED_SHAPE, "hidden %d not a positive multiple of 128",
          c->hidden);
  REQUIRE(c->n_shared == 0 || c->n_shared == 1, MOE_ERR_UNSUPPORTED_SHAPE, "n_shared %d not 0 or 1", c->n_shared);
  if (c->n_shared) {
    REQUIRE(c->inter_shared > 0 && c->inter_shared % 128 == 0, MOE_ERR_UNSUPPORTED_SHAPE,
            "inter_shared %d not a positive multiple of 128", c->inter_shared);
  }
  if (c->n_experts == 0) {
    REQUIRE(c->n_shared == 1, MOE_ERR_INVALID_ARG, "a dense layer (n_experts = 0) needs n_shared = 1");
    return MOE_OK;
  }
  const int st = check_route_cfg(c);
  if (st != MOE_OK) return st;
  REQUIRE(c->inter > 0 && c->inter % 128 == 0, MOE_ERR_UNSUPPORTED_SHAPE, "inter %d not a positive multiple of 128",
          c->inter);
  REQUIRE(c->n_experts % 16 == 0, MOE_ERR_UNSUPPORTED_SHAPE, "n_experts %d not a multiple of 16 (router tiles)",
          c->n_experts);
  return MOE_OK;
}

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

// Workspace layout of moe_ffn_forward (offsets from ws, 256-byte aligned).
struct FwdLayout {
  size_t x_norm, x_q, x_s, scores, topk_idx, topk_w, offsets, sorted_assign, assign_pos, sorted_token, perm_scratch,
      h_q, h_s, hs_q, hs_s, y_sorted, y_shared, total;
};

FwdLayout fwd_layout(int T, const moe_cfg_t* c) {
  FwdLayout L{};
  size_t p = 0;
  auto take = [&](size_t bytes) {
    const size_t at = p;
    p += align_up(bytes);
    return at;
  };
  const size_t t = (size_t)T, d = (size_t)c->hidden;
  const size_t E = (size_t)c->n_experts, k = (size_t)(c->n_experts ? c->top_k : 0);
  const size_t n = t * k;
  L.x_norm = take(t * d * 2);                    // bf16 rows after the optional RMSNorm
  L.x_q = take(t * d);
  L.x_s = take(t * (d / 128) * 4);
  L.scores = take(t * E * 4);
  L.topk_idx = take(n * 4);
  L.topk_w = take(n * 4);
  L.offsets = take((E + 1) * 4);
  L.sorted_assign = take(n * 4);
  L.assign_pos = take(n * 4);
  L.sorted_token = take(n * 4);
  L.perm_scratch = take(E ? permute_scratch_bytes((int)n, (int)E) : 0);
  const size_t w = E ? (size_t)c->inter : 0, ws = c->n_shared ? (size_t)c->inter_shared : 0;
  L.h_q = take(n * w);
  L.h_s = take(n * (w / 128) * 4);
  L.hs_q = take(t * ws);
  L.hs_s = take(t * (ws / 128) * 4);
  L.y_sorted = take(n * d * 4);
  L.y_shared = take(t * d * 4);
  L.total = p;
  return L;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first call per device).
int scratch_address(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_ERR_INVALID_ARG, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    REQUIRE(p != nullptr, MOE_ERR_HIP, "no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_INVALID_DATA: return "MOE_ERR_INVALID_DATA";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_validation_enabled(void) { return validation_on() ? 1 : 0; }

int fp8_quant_1x128(const void* x, int x_dtype, int rows, int cols, int ld_x, uint8_t* q, int ld_q, float* s,
                    int scale_fmt, void* stream) {
  REQUIRE(x_dtype == MOE_DTYPE_BF16 || x_dtype == MOE_DTYPE_F32, MOE_ERR_INVALID_ARG, "x_dtype %d not BF16/F32",
          x_dtype);
  REQUIRE(scale_fmt == MOE_SCALE_F32 || scale_fmt == MOE_SCALE_UE8M0, MOE_ERR_INVALID_ARG, "scale_fmt %d unknown",
          scale_fmt);
  REQUIRE(rows >= 0, MOE_ERR_INVALID_ARG, "rows %d < 0", rows);
  REQUIRE(cols > 0 && cols % 128 == 0, MOE_ERR_UNSUPPORTED_SHAPE, "cols %d not a positive multiple of 128", cols);
  REQUIRE(ld_x >= cols && ld_q >= cols, MOE_ERR_INVALID_ARG, "ld_x %d / ld_q %d smaller than cols %d", ld_x, ld_q,
          cols);
  if (rows == 0) return ok();
  REQUIRE(x && q && s, MOE_ERR_INVALID_ARG, "NULL pointer");
  const int esz = x_dtype == MOE_DTYPE_BF16 ? 2 : 4;
  REQUIRE(aligned(x, 16) && ((size_t)ld_x * esz) % 16 == 0, MOE_ERR_INVALID_ARG, "x rows not 16-byte aligned");
  REQUIRE(aligned(q, 16) && ld_q % 16 == 0 && aligned(s, 4), MOE_ERR_INVALID_ARG, "q/s not aligned");
  HIP_TRY(launch_quant_1x128(x, x_dtype == MOE_DTYPE_BF16, rows, cols, ld_x, q, ld_q, s, scale_fmt == MOE_SCALE_UE8M0,
                             (hipStream_t)stream),
          "fp8_quant_1x128");
  return ok();
}

int fp8_quant_128x128(const float* w, int rows, int cols, uint8_t* q, float* s, int scale_fmt, void* stream) {
  REQUIRE(scale_fmt == MOE_SCALE_F32 || scale_fmt == MOE_SCALE_UE8M0, MOE_ERR_INVALID_ARG, "scale_fmt %d unknown",
          scale_fmt);
  REQUIRE(rows >= 0 && cols >= 0, MOE_ERR_INVALID_ARG, "negative size");
  REQUIRE(rows % 128 == 0 && cols % 128 == 0, MOE_ERR_UNSUPPORTED_SHAPE, "rows %d / cols %d not multiples of 128",
          rows, cols);
  if (rows == 0 || cols == 0) return ok();
  REQUIRE(w && q && s, MOE_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned(w, 16) && aligned(q, 16) && aligned(s, 4), MOE_ERR_INVALID_ARG, "pointer not aligned");
  HIP_TRY(launch_quant_128x128(w, rows, cols, q, s, scale_fmt == MOE_SCALE_UE8M0, (hipStream_t)stream),
          "fp8_quant_128x128");
  return ok();
}

int fp8_rmsnorm_quant_1x128(const uint16_t* x, const uint16_t* gamma, float eps, int rows, int cols, int ld_x,
                            uint16_t* y, int ld_y, uint8_t* q, int ld_q, float* s, int scale_fmt, void* stream) {
  REQUIRE(scale_fmt == MOE_SCALE_F32 || scale_fmt == MOE_SCALE_UE8M0, MOE_ERR_INVALID_ARG, "scale_fmt %d unknown",
          scale_fmt);
  REQUIRE(rows >= 0, MOE_ERR_INVALID_ARG, "rows %d < 0", rows);
  REQUIRE(cols > 0 && cols % 128 == 0, MOE_ERR_UNSUPPORTED_SHAPE, "cols %d not a positive multiple of 128", cols);
  REQUIRE(eps >= 0.0f && eps < 3.0e38f, MOE_ERR_INVALID_ARG, "eps %g not finite and >= 0", (double)eps);
  REQUIRE(ld_x >= cols && ld_q >= cols && (!y || ld_y >= cols), MOE_ERR_INVALID_ARG,
          "leading dimensions smaller than cols %d", cols);
  if (rows == 0) return ok();
  REQUIRE(x && gamma && q && s, MOE_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned(x, 16) && ld_x % 8 == 0 && aligned(gamma, 16) && (!y || (aligned(y, 16) && ld_y % 8 == 0)),
          MOE_ERR_INVALID_ARG, "x / gamma / y rows not 16-byte aligned");
  REQUIRE(aligned(q, 16) && ld_q % 16 == 0 && aligned(s, 4), MOE_ERR_INVALID_ARG, "q/s not aligned");
  HIP_TRY(launch_rmsnorm_quant(x, gamma, eps, rows, cols, ld_x, y, ld_y, q, ld_q, s, scale_fmt == MOE_SCALE_UE8M0,
                               (hipStream_t)stream),
          "fp8_rmsnorm_quant_1x128");
  return ok();
}

int moe_bias_update(const int32_t* topk_idx, int T, int k, int E, float gamma, float* bias, int32_t* counts,
                    void* stream) {
  REQUIRE(T >= 0 && k >= 1, MOE_ERR_INVALID_ARG, "T %d, k %d", T, k);
  REQUIRE(E >= 1 && E <= 1024, MOE_ERR_UNSUPPORTED_SHAPE, "E %d not in [1, 1024]", E);
  REQUIRE((long)T * k <= (1l << 30), MOE_ERR_UNSUPPORTED_SHAPE, "T*k too large");
  REQUIRE(gamma == gamma && gamma > -3.0e38f && gamma < 3.0e38f, MOE_ERR_INVALID_ARG, "gamma not finite");
  REQUIRE(bias && (T == 0 || topk_idx), MOE_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned(bias, 4) && (!counts || aligned(counts, 4)) && (!topk_idx || aligned(topk_idx, 4)),
          MOE_ERR_INVALID_ARG, "pointer not aligned");
  HIP_TRY(launch_bias_update(topk_idx, (long)T * k, E, gamma, bias, counts, (hipStream_t)stream), "moe_bias_update");
  return ok();
}

int moe_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int T, const moe_cfg_t* cfg,
              float* scores, int flags, int32_t* topk_idx, float* topk_w, void* stream) {
  int st = check_route_cfg(cfg);
  if (st != MOE_OK) return st;
  REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "T %d < 0", T);
  REQUIRE((flags & ~MOE_ROUTE_SCORES_GIVEN) == 0, MOE_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (T == 0) return ok();
  REQUIRE(scores && topk_idx && topk_w, MOE_ERR_INVALID_ARG, "NULL scores/topk_idx/topk_w");
  const hipStream_t s = (hipStream_t)stream;
  if (validation_on()) {
    if (flags & MOE_ROUTE_SCORES_GIVEN)
      VALIDATE(validate_finite(scores, (long)T * cfg->n_experts, s, &bad_), "scores[%ld] = %g is not finite", bad_,
               read_f32(scores, bad_));
    if (bias)
      VALIDATE(validate_finite(bias, cfg->n_experts, s, &bad_), "bias[%ld] = %g is not finite", bad_,
               read_f32(bias, bad_));
  }
  if (!(flags & MOE_ROUTE_SCORES_GIVEN)) {
    REQUIRE(x && w_router, MOE_ERR_INVALID_ARG, "x and w_router are needed unless MOE_ROUTE_SCORES_GIVEN");
    REQUIRE(cfg->hidden > 0 && cfg->hidden % 128 == 0, MOE_ERR_UNSUPPORTED_SHAPE, "hidden %d not a multiple of 128",
            cfg->hidden);
    REQUIRE(cfg->n_experts % 16 == 0, MOE_ERR_UNSUPPORTED_SHAPE, "n_experts %d not a multiple of 16", cfg->n_experts);
    REQUIRE(aligned(x, 16) && aligned(w_router, 16), MOE_ERR_INVALID_ARG, "x / w_router not 16-byte aligned");
    HIP_TRY(launch_router(x, w_router, T, cfg->n_experts, cfg->hidden, scores, nullptr, 0, nullptr, s), "router");
  }
  HIP_TRY(launch_route(scores, bias, T, cfg->n_experts, cfg->top_k, cfg->n_group, cfg->topk_group, cfg->group_score,
                       cfg->routed_scale, topk_idx, topk_w, s),
          "moe_route");
  return ok();
}

size_t moe_permute_workspace_size(int T, int k, int E) {
  if (T < 0 || k < 1 || E < 1 || E > 1024 || (long)T * k > (1l << 30)) return 0;
  return align_up(permute_scratch_bytes(T * k, E));
}

int moe_permute(const int32_t* topk_idx, int T, int k, int E, int32_t* offsets, int32_t* sorted_assign,
                int32_t* assign_pos, const void* rows_in, int row_bytes, void* rows_out, void* ws, size_t ws_bytes,
                void* stream) {
  REQUIRE(T >= 0 && k >= 1 && E >= 1, MOE_ERR_INVALID_ARG, "T %d, k %d, E %d", T, k, E);
  REQUIRE(E <= 1024, MOE_ERR_UNSUPPORTED_SHAPE, "E %d > 1024", E);
  REQUIRE((long)T * k <= (1l << 30), MOE_ERR_UNSUPPORTED_SHAPE, "T*k too large");
  REQUIRE(offsets, MOE_ERR_INVALID_ARG, "offsets is NULL");
  REQUIRE((rows_in == nullptr) == (rows_out == nullptr), MOE_ERR_INVALID_ARG, "rows_in/rows_out: both or neither");
  if (rows_in) {
    REQUIRE(row_bytes > 0 && row_bytes % 16 == 0, MOE_ERR_INVALID_ARG, "row_bytes %d not a positive multiple of 16",
            row_bytes);
    REQUIRE(aligned(rows_in, 16) && aligned(rows_out, 16), MOE_ERR_INVALID_ARG, "rows not 16-byte aligned");
  }
  if (T > 0) REQUIRE(topk_idx && sorted_assign && assign_pos, MOE_ERR_INVALID_ARG, "NULL pointer");
  const size_t need = moe_permute_workspace_size(T, k, E);
  REQUIRE(need == 0 || (ws && ws_bytes >= need), MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  const hipStream_t s = (hipStream_t)stream;
  if (validation_on() && T > 0)
    VALIDATE(validate_range(topk_idx, T * k, 0, E, s, &bad_), "topk_idx[%ld] = %ld not in [0, %d)", bad_,
             read_i32(topk_idx, bad_), E);
  HIP_TRY(launch_permute(topk_idx, T, k, E, offsets, sorted_assign, assign_pos, nullptr, nullptr, nullptr,
                         reinterpret_cast<int32_t*>(ws), s),
          "moe_permute");
  if (rows_in) HIP_TRY(launch_gather_rows(rows_in, row_bytes, T * k, k, sorted_assign, rows_out, s), "gather rows");
  return ok();
}

int moe_unpermute(const void* y_sorted, int y_dtype, const int32_t* assign_pos, const float* topk_w,
                  const float* shared_y, int T, int k, int d, void* out, void* stream) {
  REQUIRE(T >= 0 && k >= 1 && d >= 1, MOE_ERR_INVALID_ARG, "T %d, k %d, d %d", T, k, d);
  REQUIRE(y_dtype == MOE_DTYPE_F32 || y_dtype == MOE_DTYPE_BF16 || y_dtype == MOE_DTYPE_U8, MOE_ERR_INVALID_ARG,
          "y_dtype %d unknown", y_dtype);
  REQUIRE(d % 4 == 0, MOE_ERR_UNSUPPORTED_SHAPE, "d %d not a multiple of 4", d);
  REQUIRE((long)T * k <= (1l << 30), MOE_ERR_UNSUPPORTED_SHAPE, "T*k too large");
  if (T == 0) return ok();
  REQUIRE(y_sorted && assign_pos && out, MOE_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned(y_sorted, 16) && aligned(out, 16) && (!shared_y || aligned(shared_y, 16)), MOE_ERR_INVALID_ARG,
          "pointer not 16-byte aligned");
  const hipStream_t s = (hipStream_t)stream;
  if (validation_on())
    VALIDATE(validate_range(assign_pos, T * k, 0, T * k, s, &bad_), "assign_pos[%ld] = %ld not in [0, %d)", bad_,
             read_i32(assign_pos, bad_), T * k);
  if (topk_w) {
    REQUIRE(y_dtype == MOE_DTYPE_F32, MOE_ERR_INVALID_ARG, "the weighted combine takes F32 rows");
    HIP_TRY(launch_combine(reinterpret_cast<const float*>(y_sorted), assign_pos, topk_w, shared_y, T, k, d,
                           reinterpret_cast<uint16_t*>(out), s),
            "moe_unpermute (combine)");
  } else {
    const int esz = y_dtype == MOE_DTYPE_F32 ? 4 : (y_dtype == MOE_DTYPE_BF16 ? 2 : 1);
    HIP_TRY(launch_unpermute(y_sorted, assign_pos, (long)T * k, d * esz, out, s), "moe_unpermute");
  }
  return ok();
}

int fp8_grouped_gemm_blockscaled(const uint8_t* a_q, const float* a_s, const int32_t* a_gather, const uint8_t* b_q,
                                 const float* b_s, const int32_t* offsets, int G, int M_max, int N, int K, int epilogue,
                                 const moe_epi_t* epi, void* out, void* stream) {
  REQUIRE(G >= 1 && G <= 1024, MOE_ERR_UNSUPPORTED_SHAPE, "G %d not in [1, 1024]", G);
  REQUIRE(M_max >= 0 && N > 0 && K > 0, MOE_ERR_INVALID_ARG, "M_max %d, N %d, K %d", M_max, N, K);
  REQUIRE(K % 128 == 0 && N % 128 == 0, MOE_ERR_UNSUPPORTED_SHAPE, "N %d / K %d not multiples of 128", N, K);
  REQUIRE(epilogue >= MOE_EPI_STORE_F32 && epilogue <= MOE_EPI_WEIGHTED_SCATTER_ADD, MOE_ERR_INVALID_ARG,
          "epilogue %d unknown", epilogue);
  if (epilogue == MOE_EPI_SWIGLU_QUANT)
    REQUIRE(N % 256 == 0 && epi && epi->h_s, MOE_ERR_INVALID_ARG, "SWIGLU_QUANT needs N %% 256 == 0 and epi->h_s");
  if (M_max == 0) return ok();
  REQUIRE(a_q && a_s && b_q && b_s && offsets && out, MOE_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned(a_q, 16) && aligned(b_q, 16) && aligned(out, 16), MOE_ERR_INVALID_ARG, "pointer not 16-byte aligned");
  if (validation_on()) {
    const hipStream_t s = (hipStream_t)stream;
    VALIDATE(validate_offsets(offsets, G, -1, M_max, false, 1, s, &bad_),
             "offsets[%ld] = %ld breaks 0 <= offsets[0] <= ... <= offsets[G] <= M_max = %d", bad_,
             read_i32(offsets, bad_), M_max);
    if (a_gather)
      VALIDATE(validate_rows(a_gather, offsets, G, M_max, s, &bad_), "a_gather[%ld] = %ld < 0", bad_,
               read_i32(a_gather, bad_));
    if (epilogue == MOE_EPI_WEIGHTED_SCATTER_ADD && epi && epi->dst_row)
      VALIDATE(validate_rows(epi->dst_row, offsets, G, M_max, s, &bad_), "epi->dst_row[%ld] = %ld < 0", bad_,
               read_i32(epi->dst_row, bad_));
  }
  GemmArgs args{};
  GemmSeg& sg = args.seg[1];
  const int bm = gemm_pick_bm(M_max, G, epilogue == MOE_EPI_SWIGLU_QUANT);
  sg.a_q = a_q;
  sg.a_s = a_s;
  sg.a_gather = a_gather;
  sg.b_q = b_q;
  sg.b_s = b_s;
  sg.b_stride = (long long)N * K;
  sg.bs_stride = (long long)(N / 128) * (K / 128);
  sg.offsets = offsets;
  sg.G = G;
  sg.m_tiles = (int)(((long)M_max + (long)G * (bm - 1)) / bm);
  sg.N = N;
  sg.K = K;
  sg.out = out;
  if (epi) {
    REQUIRE(epi->scale_fmt == MOE_SCALE_F32 || epi->scale_fmt == MOE_SCALE_UE8M0, MOE_ERR_INVALID_ARG,
            "epi->scale_fmt %d unknown", epi->scale_fmt);
    sg.pow2_scales = epi->scale_fmt == MOE_SCALE_UE8M0;
  }
  if (epilogue == MOE_EPI_SWIGLU_QUANT) {
    sg.out_s = epi->h_s;
    sg.ld_out = N / 2;
  } else {
    sg.ld_out = N;
  }
  if (epilogue == MOE_EPI_WEIGHTED_SCATTER_ADD && epi) {
    sg.dst_row = epi->dst_row;
    sg.row_w = epi->row_weight;
  }
  static const int kEpiMap[4] = {kEpiF32, kEpiBf16, kEpiSwiglu, kEpiScatter};
  HIP_TRY(launch_grouped_gemm(args, kEpiMap[epilogue], bm, (hipStream_t)stream), "fp8_grouped_gemm_blockscaled");
  return ok();
}

int moe_pack_weights(const uint8_t* src, int G, int N, int K, uint8_t* dst, void* stream) {
  REQUIRE(G >= 0 && N >= 0 && K >= 0, MOE_ERR_INVALID_ARG, "negative size");
  REQUIRE(N % 16 == 0 && K % 128 == 0, MOE_ERR_UNSUPPORTED_SHAPE, "N %d %% 16 or K %d %% 128 != 0", N, K);
  if ((long)G * N * K == 0) return ok();
  REQUIRE(src && dst && src != dst, MOE_ERR_INVALID_ARG, "NULL or aliased pointers");
  REQUIRE(aligned(src, 16) && aligned(dst, 16), MOE_ERR_INVALID_ARG, "pointer not 16-byte aligned");
  HIP_TRY(launch_pack(src, G, N, K, dst, (hipStream_t)stream), "moe_pack_weights");
  return ok();
}

size_t moe_padded_rows(int M, int G) {
  if (M < 0 || G < 1 || G > 1024) return 0;
  return ((size_t)(M + 127) / 128 + (size_t)G) * 128;
}

int fp8_quant_128x1_grouped(const void* x, int x_dtype, int M, int N, int ld_x, const int32_t* offsets, int G,
                            int32_t* padded_offsets, uint8_t* q_t, int ld_q, float* s_t, int scale_fmt, void* stream) {
  REQUIRE(x_dtype == MOE_DTYPE_BF16 || x_dtype == MOE_DTYPE_F32, MOE_ERR_INVALID_ARG, "x_dtype %d not BF16/F32",
          x_dtype);
  REQUIRE(scale_fmt == MOE_SCALE_F32 || scale_fmt == MOE_SCALE_UE8M0, MOE_ERR_INVALID_ARG, "scale_fmt %d unknown",
          scale_fmt);
  REQUIRE(G >= 1 && G <= 1024, MOE_ERR_UNSUPPORTED_SHAPE, "G %d not in [1, 1024]", G);
  REQUIRE(M >= 0 && M <= (1 << 30), MOE_ERR_INVALID_ARG, "M %d", M);
  REQUIRE(N > 0 && N % 128 == 0, MOE_ERR_UNSUPPORTED_SHAPE, "N %d not a positive multiple of 128", N);
  REQUIRE(ld_x >= N, MOE_ERR_INVALID_ARG, "ld_x %d < N %d", ld_x, N);
  const size_t mp = moe_padded_rows(M, G);
  REQUIRE(ld_q % 128 == 0 && (size_t)ld_q >= mp, MOE_ERR_INVALID_ARG,
          "ld_q %d: a multiple of 128 of at least moe_padded_rows(M, G) = %zu", ld_q, mp);
  REQUIRE(x && offsets && padded_offsets && q_t && s_t, MOE_ERR_INVALID_ARG, "NULL pointer");
  const int esz = x_dtype == MOE_DTYPE_BF16 ? 2 : 4;
  REQUIRE(aligned(x, 16) && ((size_t)ld_x * esz) % 16 == 0 && aligned(q_t, 16) && aligned(s_t, 4) &&
              aligned(offsets, 4) && aligned(padded_offsets, 4),
          MOE_ERR_INVALID_ARG, "pointer or leading dimension not aligned");
  const hipStream_t st = (hipStream_t)stream;
  if (validation_on())
    VALIDATE(validate_offsets(offsets, G, 0, M, true, 1, st, &bad_),
             "offsets[%ld] = %ld breaks 0 = offsets[0] <= ... <= offsets[G] = M = %d", bad_, read_i32(offsets, bad_),
             M);
  HIP_TRY(launch_pad_offsets(offsets, G, padded_offsets, st), "pad offsets");
  HIP_TRY(launch_quant_128x1_grouped(x, x_dtype == MOE_DTYPE_BF16, ld_x, offsets, G, padded_offsets, (int)mp, N, q_t,
                                     ld_q, s_t, scale_fmt == MOE_SCALE_UE8M0, st),
          "fp8_quant_128x1_grouped");
  return ok();
}

int moe_pack_weights_transposed(const uint8_t* w_q, const float* w_s, int G, int N, int K, uint8_t* wt_q, float* wt_s,
                                void* stream) {
  REQUIRE(G >= 0 && N >= 0 && K >= 0, MOE_ERR_INVALID_ARG, "negative size");
  REQUIRE(N % 128 == 0 && K % 128 == 0, MOE_ERR_UNSUPPORTED_SHAPE, "N %d / K %d not multiples of 128", N, K);
  if ((long)G * N * K == 0) return ok();
  REQUIRE(w_q && w_s && wt_q && wt_s && w_q != wt_q, MOE_ERR_INVALID_ARG, "NULL or aliased pointers");
  REQUIRE(aligned(w_q, 16) && aligned(wt_q, 16) && aligned(w_s, 4) && aligned(wt_s, 4), MOE_ERR_INVALID_ARG,
          "pointer not aligned");
  HIP_TRY(launch_pack_transposed(w_q, w_s, G, N, K, wt_q, wt_s, (hipStream_t)stream), "moe_pack_weights_transposed");
  return ok();
}

int fp8_grouped_gemm_wgrad(const uint8_t* a_t, const float* a_ts, const uint8_t* b_t, const float* b_ts,
                           const int32_t* padded_offsets, int G, int M, int Na, int Nb, int ld, float* out,
                           int scale_fmt, void* stream) {
  REQUIRE(scale_fmt == MOE_SCALE_F32 || scale_fmt == MOE_SCALE_UE8M0, MOE_ERR_INVALID_ARG, "scale_fmt %d unknown",
          scale_fmt);
  REQUIRE(G >= 1 && G <= 1024, MOE_ERR_UNSUPPORTED_SHAPE, "G %d not in [1, 1024]", G);
  REQUIRE(M >= 0 && M <= (1 << 30), MOE_ERR_INVALID_ARG, "M %d", M);
  REQUIRE(Na > 0 && Nb > 0 && Na % 128 == 0 && Nb % 128 == 0, MOE_ERR_UNSUPPORTED_SHAPE,
          "Na %d / Nb %d not positive multiples of 128", Na, Nb);
  const size_t mp = moe_padded_rows(M, G);
  REQUIRE(ld % 128 == 0 && (size_t)ld >= mp, MOE_ERR_INVALID_ARG,
          "ld %d: a multiple of 128 of at least moe_padded_rows(M, G) = %zu", ld, mp);
  REQUIRE(a_t && a_ts && b_t && b_ts && padded_offsets && out, MOE_ERR_INVALID_ARG, "NULL pointer");
  REQUIRE(aligned(a_t, 16) && aligned(b_t, 16) && aligned(out, 16) && aligned(a_ts, 4) && aligned(b_ts, 4),
          MOE_ERR_INVALID_ARG, "pointer not aligned");
  if (validation_on())
    VALIDATE(validate_offsets(padded_offsets, G, 0, (int)mp, false, 128, (hipStream_t)stream, &bad_),
             "padded_offsets[%ld] = %ld breaks 0 = padded[0] <= ... <= padded[G] <= moe_padded_rows(M, G) = %zu "
             "in multiples of 128", bad_, read_i32(padded_offsets, bad_), mp);
  HIP_TRY(launch_wgrad(a_t, a_ts, b_t, b_ts, padded_offsets, G, Na, Nb, ld, out, scale_fmt == MOE_SCALE_UE8M0,
                       (hipStream_t)stream),
          "fp8_grouped_gemm_wgrad");
  return ok();
}

size_t moe_ffn_workspace_size(int T, const moe_cfg_t* cfg) {
  if (T < 0 || check_layer_cfg(cfg) != MOE_OK) return 0;
  return fwd_layout(T, cfg).total;
}

int moe_ffn_forward(const uint16_t* x, int T, const moe_cfg_t* cfg, const moe_weights_t* w, void* ws,
                    size_t ws_bytes, uint16_t* out, float* scores, int32_t* topk_idx, float* topk_w, int flags,
                    void* stream) {
  return moe_ffn_forward_stages(x, T, cfg, w, ws, ws_bytes, out, scores, topk_idx, topk_w, flags, nullptr, 0, stream);
}

int moe_ffn_forward_noalloc(const uint16_t* x, int T, const moe_cfg_t* cfg, const moe_weights_t* w, uint16_t* out,
                            float* scores, int32_t* topk_idx, float* topk_w, int flags, void* stream) {
  int st = check_layer_cfg(cfg);
  if (st != MOE_OK) return st;
  REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "T %d < 0", T);
  const size_t need = fwd_layout(T, cfg).total;
  REQUIRE(need <= (size_t)MOE_NOALLOC_SCRATCH_BYTES, MOE_ERR_WORKSPACE,
          "T = %d needs %zu bytes of workspace; the static scratch holds %zu (use moe_ffn_forward with a "
          "caller workspace)", T, need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  if (T == 0) return moe_ffn_forward(x, T, cfg, w, nullptr, 0, out, scores, topk_idx, topk_w, flags, stream);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MOE_OK) return st;
  return moe_ffn_forward(x, T, cfg, w, ws, MOE_NOALLOC_SCRATCH_BYTES, out, scores, topk_idx, topk_w, flags, stream);
}

int moe_ffn_forward_stages(const uint16_t* x, int T, const moe_cfg_t* cfg, const moe_weights_t* w, void* ws,
                           size_t ws_bytes, uint16_t* out, float* scores, int32_t* topk_idx, float* topk_w, int flags,
                           void* const* events, int n_events, void* stream) {
  int st = check_layer_cfg(cfg);
  if (st != MOE_OK) return st;
  REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "T %d < 0", T);
  REQUIRE((flags & ~(MOE_ROUTE_SCORES_GIVEN | MOE_FWD_DETERMINISTIC)) == 0, MOE_ERR_INVALID_ARG, "unknown flags 0x%x",
          flags);
  REQUIRE((long)T * (cfg->n_experts ? cfg->top_k : 1) <= (1l << 30), MOE_ERR_UNSUPPORTED_SHAPE, "T too large");
  REQUIRE(n_events == 0 || (events && n_events == MOE_FWD_STAGE_EVENTS), MOE_ERR_INVALID_ARG,
          "n_events %d (0 or %d)", n_events, MOE_FWD_STAGE_EVENTS);
  if (T == 0) return ok();
  REQUIRE(x && out && w, MOE_ERR_INVALID_ARG, "NULL x / out / weights");
  REQUIRE(aligned(x, 16) && aligned(out, 16), MOE_ERR_INVALID_ARG, "x / out not 16-byte aligned");
  const bool routed = cfg->n_experts > 0;
  if (routed) {
    REQUIRE(w->w13_q && w->w13_s && w->w2_q && w->w2_s, MOE_ERR_INVALID_ARG, "NULL routed expert weights");
    if (flags & MOE_ROUTE_SCORES_GIVEN)
      REQUIRE(scores, MOE_ERR_INVALID_ARG, "MOE_ROUTE_SCORES_GIVEN needs scores");
    else
      REQUIRE(w->w_router, MOE_ERR_INVALID_ARG, "NULL router weights");
  }
  if (cfg->n_shared)
    REQUIRE(w->sh_w13_q && w->sh_w13_s && w->sh_w2_q && w->sh_w2_s, MOE_ERR_INVALID_ARG, "NULL shared weights");
  REQUIRE(!w->norm_w || aligned(w->norm_w, 16), MOE_ERR_INVALID_ARG, "norm_w not 16-byte aligned");
  const FwdLayout L = fwd_layout(T, cfg);
  REQUIRE(ws && aligned(ws, 256) && ws_bytes >= L.total, MOE_ERR_WORKSPACE,
          "workspace %zu bytes (needs %zu, 256-byte aligned)", ws_bytes, L.total);

  const hipStream_t s = (hipStream_t)stream;
  if (validation_on() && routed) {
    if (flags & MOE_ROUTE_SCORES_GIVEN)
      VALIDATE(validate_finite(scores, (long)T * cfg->n_experts, s, &bad_), "scores[%ld] = %g is not finite", bad_,
               read_f32(scores, bad_));
    if (w->bias)
      VALIDATE(validate_finite(w->bias, cfg->n_experts, s, &bad_), "bias[%ld] = %g is not finite", bad_,
               read_f32(w->bias, bad_));
  }
  auto mark = [&](int i) -> hipError_t {
    return n_events && events[i] ? hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), s) : hipSuccess;
  };
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  auto at = [&](size_t off) { return base + off; };
  const int d = cfg->hidden, E = cfg->n_experts, k = routed ? cfg->top_k : 0;
  const int W = cfg->inter, Ws = cfg->inter_shared;
  uint8_t* x_q = at(L.x_q);
  float* x_s = reinterpret_cast<float*>(at(L.x_s));
  const bool pow2 = cfg->scale_fmt == MOE_SCALE_UE8M0;
  const uint16_t* xin = x;                      // the rows the router reads
  const long n_assign = (long)T * k;
  float* sc = routed ? (scores ? scores : reinterpret_cast<float*>(at(L.scores))) : nullptr;
  const bool run_router = routed && !(flags & MOE_ROUTE_SCORES_GIVEN);
  // the router's partial logits (K split over workgroups) borrow the down GEMM's output rows, unused until then
  // (the split's last step stores the scores 16 bytes at a time: a caller's scores buffer must allow it)
  float* part = run_router && aligned(sc, 16) ? reinterpret_cast<float*>(at(L.y_sorted)) : nullptr;
  const size_t part_floats = (size_t)n_assign * (size_t)d;
  // small batches: x's quantisation rides in the router's finishing kernel (one launch less)
  const RouterQuant xq{x_q, x_s, pow2};
  const bool quant_in_router = !w->norm_w && run_router && router_small_split(T, E, d, part, part_floats);
  HIP_TRY(mark(0), "event");
  if (w->norm_w) {
    uint16_t* x_norm = reinterpret_cast<uint16_t*>(at(L.x_norm));
    HIP_TRY(launch_rmsnorm_quant(x, w->norm_w, cfg->norm_eps, T, d, d, x_norm, d, x_q, d, x_s, pow2, s),
            "RMSNorm + quantize x");
    xin = x_norm;
  } else if (!quant_in_router) {
    HIP_TRY(launch_quant_1x128(x, true, T, d, d, x_q, d, x_s, pow2, s), "quantize x");
  }
  HIP_TRY(mark(1), "event");

  int32_t* sorted_token = reinterpret_cast<int32_t*>(at(L.sorted_token));
  int32_t* assign_pos = reinterpret_cast<int32_t*>(at(L.assign_pos));
  int32_t* offsets = reinterpret_cast<int32_t*>(at(L.offsets));
  float* tw = topk_w ? topk_w : reinterpret_cast<float*>(at(L.topk_w));
  if (routed) {
    int32_t* ti = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(at(L.topk_idx));
    if (run_router)
      HIP_TRY(launch_router(xin, w->w_router, T, E, d, sc, part, part_floats, quant_in_router ? &xq : nullptr, s),
              "router");
    HIP_TRY(launch_route(sc, w->bias, T, E, k, cfg->n_group, cfg->topk_group, cfg->group_score, cfg->routed_scale, ti,
                         tw, s),
            "route");
    HIP_TRY(launch_permute(ti, T, k, E, offsets, reinterpret_cast<int32_t*>(at(L.sorted_assign)), assign_pos,
                           sorted_token, nullptr, nullptr,
                           reinterpret_cast<int32_t*>(at(L.perm_scratch)), s),
            "permute");
  }
  HIP_TRY(mark(2), "event");

  // gate/up GEMM with the SwiGLU + 1x128 requantisation epilogue
  uint8_t* h_q = at(L.h_q);
  float* h_s = reinterpret_cast<float*>(at(L.h_s));
  uint8_t* hs_q = at(L.hs_q);
  float* hs_s = reinterpret_cast<float*>(at(L.hs_s));
  // tile rows of the gate/up GEMM (bm) and of the down GEMM (bm_dn)
  const int bm = routed ? gemm_pick_bm(n_assign, E, true) : gemm_pick_bm(T, 1, true);
  const int bm_dn = routed ? gemm_pick_bm(n_assign, E, false) : gemm_pick_bm(T, 1, false);
  GemmArgs up{};
  if (cfg->n_shared) {
    GemmSeg& g0 = up.seg[0];
    g0.a_q = x_q;
    g0.a_s = x_s;
    g0.b_q = w->sh_w13_q;
    g0.b_s = w->sh_w13_s;
    g0.G = 1;
    g0.m_rows = T;
    g0.m_tiles = (T + bm - 1) / bm;
    g0.N = 2 * Ws;
    g0.K = d;
    g0.out = hs_q;
    g0.out_s = hs_s;
    g0.ld_out = Ws;
    g0.pow2_scales = pow2;
  }
  if (routed) {
    GemmSeg& g1 = up.seg[1];
    g1.a_q = x_q;
    g1.a_s = x_s;
    g1.a_gather = sorted_token;
    g1.b_q = w->w13_q;
    g1.b_s = w->w13_s;
    g1.b_stride = (long long)2 * W * d;
    g1.bs_stride = (long long)(2 * W / 128) * (d / 128);
    g1.offsets = offsets;
    g1.G = E;
    g1.m_tiles = (int)((n_assign + (long)E * (bm - 1)) / bm);
    g1.N = 2 * W;
    g1.K = d;
    g1.out = h_q;
    g1.out_s = h_s;
    g1.ld_out = W;
    g1.pow2_scales = pow2;
  }
  HIP_TRY(launch_grouped_gemm(up, kEpiSwiglu, bm, s), "gate/up GEMM");
  HIP_TRY(mark(3), "event");

  // down GEMM: routed rows in sorted order (fp32), then the slot-ordered combine.  (An fp32
  // atomic scatter-add of the weighted rows into one accumulator was measured slower at every
  // batch size, 5.67 vs 5.41 ms at the T = 4096 V3 layer, and is not bit-reproducible.)
  float* y_sorted = reinterpret_cast<float*>(at(L.y_sorted));
  float* y_shared = reinterpret_cast<float*>(at(L.y_shared));
  GemmArgs dn{};
  const int epi = routed ? kEpiF32 : kEpiBf16;  // dense layer: the shared MLP writes the output directly
  if (cfg->n_shared) {
    GemmSeg& g0 = dn.seg[0];
    g0.a_q = hs_q;
    g0.a_s = hs_s;
    g0.b_q = w->sh_w2_q;
    g0.b_s = w->sh_w2_s;
    g0.G = 1;
    g0.m_rows = T;
    g0.m_tiles = (T + bm_dn - 1) / bm_dn;
    g0.N = d;
    g0.K = Ws;
    g0.out = routed ? (void*)y_shared : (void*)out;
    g0.ld_out = d;
    g0.pow2_scales = pow2;
  }
  if (routed) {
    GemmSeg& g1 = dn.seg[1];
    g1.a_q = h_q;
    g1.a_s = h_s;
    g1.b_q = w->w2_q;
    g1.b_s = w->w2_s;
    g1.b_stride = (long long)d * W;
    g1.bs_stride = (long long)(d / 128) * (W / 128);
    g1.offsets = offsets;
    g1.G = E;
    g1.m_tiles = (int)((n_assign + (long)E * (bm_dn - 1)) / bm_dn);
    g1.N = d;
    g1.K = W;
    g1.out = y_sorted;
    g1.ld_out = d;
    g1.pow2_scales = pow2;
  }
  HIP_TRY(launch_grouped_gemm(dn, epi, bm_dn, s), "down GEMM");
  HIP_TRY(mark(4), "event");
  if (routed)
    HIP_TRY(launch_combine(y_sorted, assign_pos, tw, cfg->n_shared ? y_shared : nullptr, T, k, d, out, s), "combine");
  HIP_TRY(mark(5), "event");
  return ok();
}

}  // extern "C"
