// Checked mode: device-side checks of the values the draft, context and accept
// calls read from device memory (the caller's contract; those calls only
// clamp).  Each check kernel adds its violations to a report of kChecks
// (count, first index) pairs with device atomics; an init kernel resets the
// report first (a kernel rather than a memset, so the pair can sit in a
// captured graph).  Nothing here is on the draft / accept / inject path.
#include <hip/hip_runtime.h>

#include <climits>

#include "common.h"
#include "internal.h"

namespace dflash {

namespace {

constexpr int kChecks = DFLASH_CHECKS;

__global__ __launch_bounds__(64) void check_init_kernel(int32_t* __restrict__ report) {
  const int i = (int)threadIdx.x;
  if (i < kChecks) {
    report[2 * i] = 0;
    report[2 * i + 1] = INT_MAX;
  }
}

__device__ __forceinline__ void flag(int32_t* report, int rule, int index) {
  atomicAdd(report + 2 * rule, 1);
  atomicMin(report + 2 * rule + 1, index);
}

// One workgroup per request: anchor, length, fit of the block in a linear
// page-table row, and the page-table entries the pass reads (keys
// [lo, L + S): lo = L - context_window with a draft window, else 0; logical
// page p at entry p mod max_pages with a window (ring rows), else p).
__global__ __launch_bounds__(256) void check_draft_kernel(
    const int32_t* __restrict__ anchor, const int32_t* __restrict__ prefix_len,
    const int32_t* __restrict__ page_table, int max_pages, int max_prefix, int S, int P,
    int vocab, int64_t num_pages, int cwin, int32_t* __restrict__ report) {
  const int r = (int)blockIdx.x, tid = (int)threadIdx.x;
  const int L_raw = prefix_len[r];
  if (tid == 0) {
    const int a = anchor[r];
    if (a < 0 || a >= vocab) flag(report, 0, r);
    if (L_raw < 0 || L_raw > max_prefix) flag(report, 1, r);
    if (cwin == 0 && (int64_t)L_raw + S > (int64_t)max_pages * P) flag(report, 2, r);
  }
  // the entries the pass would read for this request (its length clamped to
  // the range the call accepts, so the loop stays bounded)
  const int L = L_raw < 0 ? 0 : (L_raw > max_prefix ? max_prefix : L_raw);
  const int lo = cwin > 0 ? (L - cwin > 0 ? L - cwin : 0) : 0;
  const int p0 = lo / P, p1 = (L + S - 1) / P;
  const int n = cwin > 0 ? (p1 - p0 + 1 < max_pages ? p1 - p0 + 1 : max_pages)
                         : ((p1 < max_pages - 1 ? p1 : max_pages - 1) - p0 + 1);
  for (int i = tid; i < n; i += (int)blockDim.x) {
    const int e = cwin > 0 ? (p0 + i) % max_pages : p0 + i;
    const int64_t page = page_table[(int64_t)r * max_pages + e];
    if (page < 0 || page >= num_pages) flag(report, 3, r * max_pages + e);
  }
}

// Live rows (t % rpr < valid[t / rpr], every row without valid): slot inside
// the pool, position >= 0; valid[r] inside [0, rpr].
__global__ __launch_bounds__(256) void check_context_kernel(
    const int32_t* __restrict__ positions, const int32_t* __restrict__ slots,
    const int32_t* __restrict__ valid, int n_req, int rpr, int64_t num_slots,
    int32_t* __restrict__ report) {
  const int64_t T = (int64_t)n_req * rpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < T; t += stride) {
    if (valid != nullptr && (int)(t % rpr) >= valid[t / rpr]) continue;
    const int64_t s = slots[t];
    if (s < 0 || s >= num_slots) flag(report, 0, (int)t);
    if (positions[t] < 0) flag(report, 1, (int)t);
  }
  if (valid != nullptr)
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < n_req; r += stride)
      if (valid[r] < 0 || valid[r] > rpr) flag(report, 2, (int)r);
}

// Candidate and posterior ids inside [0, vocab); prefix lengths >= 0.
__global__ __launch_bounds__(256) void check_accept_kernel(
    const int32_t* __restrict__ cand, const int32_t* __restrict__ post,
    const int32_t* __restrict__ prefix_len, int B, int S, int vocab,
    int32_t* __restrict__ report) {
  const int n = B * S, stride = (int)(gridDim.x * blockDim.x);
  for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += stride) {
    if (cand[i] < 0 || cand[i] >= vocab) flag(report, 0, i);
    if (post[i] < 0 || post[i] >= vocab) flag(report, 1, i);
  }
  for (int r = (int)(blockIdx.x * blockDim.x + threadIdx.x); r < B; r += stride)
    if (prefix_len[r] < 0) flag(report, 2, r);
}

unsigned grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (unsigned)(g < 1 ? 1 : (g > 1024 ? 1024 : g));
}

}  // namespace

hipError_t launch_check_draft(const int32_t* anchor, const int32_t* prefix_len,
                              const int32_t* page_table, int max_pages, int batch, int max_prefix,
                              int S, int P, int vocab, int64_t num_pages, int cwin,
                              int32_t* report, hipStream_t st) {
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, st, report);
  if (batch > 0)
    hipLaunchKernelGGL(check_draft_kernel, dim3((unsigned)batch), dim3(256), 0, st, anchor,
                       prefix_len, page_table, max_pages, max_prefix, S, P, vocab, num_pages,
                       cwin, report);
  return hipGetLastError();
}

hipError_t launch_check_context(const int32_t* positions, const int32_t* slots,
                                const int32_t* valid, int n_req, int rpr, int64_t num_slots,
                                int32_t* report, hipStream_t st) {
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, st, report);
  const int64_t T = (int64_t)n_req * rpr;
  if (T > 0)
    hipLaunchKernelGGL(check_context_kernel, dim3(grid_for(T)), dim3(256), 0, st, positions,
                       slots, valid, n_req, rpr, num_slots, report);
  return hipGetLastError();
}

hipError_t launch_check_accept(const int32_t* cand, const int32_t* post,
                               const int32_t* prefix_len, int B, int S, int vocab,
                               int32_t* report, hipStream_t st) {
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, st, report);
  if (B > 0)
    hipLaunchKernelGGL(check_accept_kernel, dim3(grid_for((int64_t)B * S)), dim3(256), 0, st,
                       cand, post, prefix_len, B, S, vocab, report);
  return hipGetLastError();
}

}  // namespace dflash
