// Cache-capacity reservation on the device ("Inside SGLang: DFlash and DFlash
// 2 Implementation", Step 2: reserve capacity before acceptance is known, a
// 2 x block_size page-aligned headroom; the overlap section: the next step
// plans from the lengths the GPU published).
//
// Run on the stream right after the accept step, the reservation reads the
// new_seq_len that step wrote: the next cycle's page table covers
// new_seq_len + 2 x block_size without a round trip to the host.  Physical
// pages come from a stack of free pages in device memory.  Requests are
// served in batch order, each popping the pages it lacks from the top of the
// stack; the first request whose shortfall the stack cannot cover (status 1)
// or whose row is too short (status 2) stops the pass for it and every later
// request.  One workgroup walks the batch in chunks of 256 requests with a
// block scan of the shortfalls, so the assignment is deterministic.
#include "common.h"
#include "internal.h"

namespace dflash {
namespace {

constexpr int kT = 256;

// Exclusive scan of one int per thread over the block (fixed order); total
// receives the sum.  tmp: kT / 64 ints of LDS.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  __syncthreads();
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int off = 0;
  total = 0;
  for (int w = 0; w < kT / 64; ++w) {
    if (w < wave) off += tmp[w];
    total += tmp[w];
  }
  return off + incl - v;
}

__device__ __forceinline__ int block_min(int v, int* tmp) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  int m = tmp[0];
  for (int w = 1; w < kT / 64; ++w) m = min(m, tmp[w]);
  return m;
}

__global__ __launch_bounds__(kT) void reserve_kernel(const int32_t* __restrict__ seq_len, int B,
                                                     int S, int P, int32_t* __restrict__ pt,
                                                     int max_pages, int32_t* __restrict__ n_pages,
                                                     const int32_t* __restrict__ free_pages,
                                                     int capacity, int32_t* free_count,
                                                     int32_t* status) {
  const int tid = threadIdx.x;
  __shared__ int tmp[kT / 64], tmp2[kT / 64];
  int top = min(max(free_count[0], 0), capacity);
  int st = 0;
  for (int base = 0; base < B && st == 0; base += kT) {
    const int r = base + tid;
    int need = 0, have = 0, shortfall = 0;
    bool bad_row = false;
    if (r < B) {
      need = (max(seq_len[r], 0) + 2 * S + P - 1) / P;
      have = min(max(n_pages[r], 0), max_pages);
      bad_row = need > max_pages;
      shortfall = bad_row ? 0 : max(0, need - have);
    }
    int total;
    const int excl = block_excl_scan(shortfall, tmp, total);
    // the first request of the chunk that cannot be served, in batch order
    const bool fail = r < B && (bad_row || excl + shortfall > top);
    const int first = block_min(fail ? r : 0x7fffffff, tmp2);
    const bool served = r < B && r < first;
    if (served) {
      for (int i = 0; i < shortfall; ++i)
        pt[(int64_t)r * max_pages + have + i] = free_pages[top - 1 - (excl + i)];
      n_pages[r] = have + shortfall;
    }
    // pages taken by the served prefix of the chunk
    int taken_total;
    block_excl_scan(served ? shortfall : 0, tmp, taken_total);
    top -= taken_total;
    if (first != 0x7fffffff) {
      // the failing request reports why (every thread reads the same value)
      const int fr = first;
      const int fneed = (max(seq_len[fr], 0) + 2 * S + P - 1) / P;
      st = fneed > max_pages ? 2 : 1;
    }
    __syncthreads();
  }
  if (tid == 0) {
    free_count[0] = top;
    status[0] = st;
  }
}

__global__ __launch_bounds__(kT) void release_kernel(const int32_t* __restrict__ mask, int B,
                                                     const int32_t* __restrict__ pt,
                                                     int max_pages, int32_t* __restrict__ n_pages,
                                                     int32_t* __restrict__ free_pages,
                                                     int capacity, int32_t* free_count) {
  const int tid = threadIdx.x;
  __shared__ int tmp[kT / 64];
  int top = min(max(free_count[0], 0), capacity);
  for (int base = 0; base < B; base += kT) {
    const int r = base + tid;
    const bool rel = r < B && mask[r] != 0;
    const int cnt = rel ? min(max(n_pages[r], 0), max_pages) : 0;
    int total;
    const int excl = block_excl_scan(cnt, tmp, total);
    if (rel) {
      for (int i = 0; i < cnt; ++i)
        if (top + excl + i < capacity)
          free_pages[top + excl + i] = pt[(int64_t)r * max_pages + i];
      n_pages[r] = 0;
    }
    top = min(top + total, capacity);
    __syncthreads();
  }
  if (tid == 0) free_count[0] = top;
}

// Relay of per-request decode state through request-pool slots ("Inside
// SGLang ...", section "Back in the scheduler: GPU continuation and CPU
// output": the relay is indexed by request-pool slots, so the batch can be
// filtered or merged between iterations).  One workgroup per batch row; the
// page-table row is copied with consecutive threads on consecutive entries.
// resolve: pool slot slots[b] -> batch row b (a slot outside the pool gives
// anchor 0, length 0, no pages and a row of -1); stash: batch row b -> pool
// slot slots[b] (a slot outside the pool is skipped).
__global__ __launch_bounds__(kT) void relay_resolve_kernel(
    const int32_t* __restrict__ slots, int capacity, int max_pages,
    const int32_t* __restrict__ p_anchor, const int32_t* __restrict__ p_len,
    const int32_t* __restrict__ p_pt, const int32_t* __restrict__ p_np,
    int32_t* __restrict__ anchor, int32_t* __restrict__ len, int32_t* __restrict__ pt,
    int32_t* __restrict__ np) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int s = slots[b];
  const bool ok = s >= 0 && s < capacity;
  if (tid == 0) {
    if (anchor != nullptr) anchor[b] = ok ? p_anchor[s] : 0;
    if (len != nullptr) len[b] = ok ? p_len[s] : 0;
    if (np != nullptr) np[b] = ok ? p_np[s] : 0;
  }
  if (pt != nullptr)
    for (int i = tid; i < max_pages; i += kT)
      pt[(int64_t)b * max_pages + i] = ok ? p_pt[(int64_t)s * max_pages + i] : -1;
}

__global__ __launch_bounds__(kT) void relay_stash_kernel(
    const int32_t* __restrict__ slots, int capacity, int max_pages,
    const int32_t* __restrict__ anchor, const int32_t* __restrict__ len,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ np,
    int32_t* __restrict__ p_anchor, int32_t* __restrict__ p_len, int32_t* __restrict__ p_pt,
    int32_t* __restrict__ p_np) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int s = slots[b];
  if (s < 0 || s >= capacity) return;
  if (tid == 0) {
    if (anchor != nullptr) p_anchor[s] = anchor[b];
    if (len != nullptr) p_len[s] = len[b];
    if (np != nullptr) p_np[s] = np[b];
  }
  if (pt != nullptr)
    for (int i = tid; i < max_pages; i += kT)
      p_pt[(int64_t)s * max_pages + i] = pt[(int64_t)b * max_pages + i];
}

}  // namespace

hipError_t launch_relay(bool stash, const int32_t* slots, int B, int capacity, int max_pages,
                        int32_t* p_anchor, int32_t* p_len, int32_t* p_pt, int32_t* p_np,
                        int32_t* anchor, int32_t* len, int32_t* pt, int32_t* np,
                        hipStream_t st) {
  if (stash)
    hipLaunchKernelGGL(relay_stash_kernel, dim3(B), dim3(kT), 0, st, slots, capacity, max_pages,
                       anchor, len, pt, np, p_anchor, p_len, p_pt, p_np);
  else
    hipLaunchKernelGGL(relay_resolve_kernel, dim3(B), dim3(kT), 0, st, slots, capacity,
                       max_pages, p_anchor, p_len, p_pt, p_np, anchor, len, pt, np);
  return hipGetLastError();
}

hipError_t launch_reserve(const int32_t* seq_len, int B, int S, int P, int32_t* pt, int max_pages,
                          int32_t* n_pages, const int32_t* free_pages, int capacity,
                          int32_t* free_count, int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(reserve_kernel, dim3(1), dim3(kT), 0, st, seq_len, B, S, P, pt, max_pages,
                     n_pages, free_pages, capacity, free_count, status);
  return hipGetLastError();
}

hipError_t launch_release(const int32_t* mask, int B, const int32_t* pt, int max_pages,
                          int32_t* n_pages, int32_t* free_pages, int capacity, int32_t* free_count,
                          hipStream_t st) {
  hipLaunchKernelGGL(release_kernel, dim3(1), dim3(kT), 0, st, mask, B, pt, max_pages, n_pages,
                     free_pages, capacity, free_count);
  return hipGetLastError();
}

}  // namespace dflash
