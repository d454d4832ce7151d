// Device-side checks of the index, offset and score data that the C ABI's calls trust by default
// (switched on per call by the environment variable MOEFP8_VALIDATE).  Each check reads only the
// elements it is given, records the smallest offending element index in a per-device word, and
// the host reads that word back after synchronising the stream, before any of the call's own
// kernels is enqueued.
#include "launch.h"

namespace moefp8 {

// Smallest offending element index of the last check on this device (kNone: none).  Device code
// names it directly; the host reads it through hipMemcpyFromSymbolAsync.
static __device__ unsigned long long g_first_bad;
constexpr unsigned long long kNone = ~0ull;

namespace {

constexpr int kThreads = 256;

__global__ void validate_reset_kernel() { g_first_bad = kNone; }

__device__ __forceinline__ void flag(long i) { atomicMin(&g_first_bad, (unsigned long long)i); }

// v[i] in [lo, hi) for i < n
__global__ void check_range_kernel(const int32_t* __restrict__ v, int n, int lo, int hi) {
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) {
    const int x = v[i];
    if (x < lo || x >= hi) flag(i);
  }
}

// off[0..G]: off[0] == first (or >= 0 when first < 0), nondecreasing, every entry a multiple of
// align, off[G] <= last (== last when last_exact).
__global__ void check_offsets_kernel(const int32_t* __restrict__ off, int G, int first, int last, bool last_exact,
                                     int align) {
  for (int i = blockIdx.x * kThreads + threadIdx.x; i <= G; i += gridDim.x * kThreads) {
    const int x = off[i];
    bool ok = x % align == 0 && x >= 0;
    if (i == 0) ok = ok && (first < 0 || x == first);
    else ok = ok && x >= off[i - 1];
    if (i == G) ok = ok && (last_exact ? x == last : x <= last);
    if (!ok) flag(i);
  }
}

// idx[m] >= 0 for off[0] <= m < off[G] (off already checked)
__global__ void check_rows_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ off, int G) {
  const int m0 = off[0], n = off[G];
  for (int i = m0 + blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads)
    if (idx[i] < 0) flag(i);
}

// |v[i]| finite (no NaN, no infinity) for i < n
__global__ void check_finite_kernel(const float* __restrict__ v, long n) {
  for (long i = blockIdx.x * (long)kThreads + threadIdx.x; i < n; i += (long)gridDim.x * kThreads)
    if (!(fabsf(v[i]) <= 3.4028235e38f)) flag(i);
}

int grid_for(long n) {
  const long b = (n + kThreads - 1) / kThreads;
  return (int)(b < 1 ? 1 : (b > 2048 ? 2048 : b));
}

// Reads the check's result back (synchronising the stream): -1 when every element passed.
hipError_t fetch(hipStream_t s, long* first_bad) {
  unsigned long long v = kNone;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_first_bad), sizeof(v), 0, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  *first_bad = v == kNone ? -1 : (long)v;
  return hipSuccess;
}

}  // namespace

hipError_t validate_range(const int32_t* v, int n, int lo, int hi, hipStream_t s, long* first_bad) {
  *first_bad = -1;
  if (n <= 0) return hipSuccess;
  validate_reset_kernel<<<1, 1, 0, s>>>();
  check_range_kernel<<<grid_for(n), kThreads, 0, s>>>(v, n, lo, hi);
  return fetch(s, first_bad);
}

hipError_t validate_offsets(const int32_t* off, int G, int first, int last, bool last_exact, int align, hipStream_t s,
                            long* first_bad) {
  *first_bad = -1;
  validate_reset_kernel<<<1, 1, 0, s>>>();
  check_offsets_kernel<<<grid_for((long)G + 1), kThreads, 0, s>>>(off, G, first, last, last_exact, align);
  return fetch(s, first_bad);
}

hipError_t validate_rows(const int32_t* idx, const int32_t* off, int G, int max_rows, hipStream_t s, long* first_bad) {
  *first_bad = -1;
  validate_reset_kernel<<<1, 1, 0, s>>>();
  check_rows_kernel<<<grid_for(max_rows), kThreads, 0, s>>>(idx, off, G);
  return fetch(s, first_bad);
}

hipError_t validate_finite(const float* v, long n, hipStream_t s, long* first_bad) {
  *first_bad = -1;
  if (n <= 0) return hipSuccess;
  validate_reset_kernel<<<1, 1, 0, s>>>();
  check_finite_kernel<<<grid_for(n), kThreads, 0, s>>>(v, n);
  return fetch(s, first_bad);
}

}  // namespace moefp8
