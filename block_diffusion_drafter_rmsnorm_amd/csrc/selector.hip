// DFlash 2 candidate selector ("Inside SGLang: DFlash and DFlash 2
// Implementation", section on DFlash 2: the selector replaces the argmax
// selection after the one backbone pass).
//
//   candidates: the K largest unary logits of each drafted row (descending,
//               ties to the lower id; NaN never wins), from the logits the
//               draft pass wrote;
//   lattice:    score(p, c) = U(c) + <A[p] * w_j, B[c]>, w_j = W_h y_j (the
//               final-normed row, projected by the streaming GEMM), for the
//               anchor (first position) or each candidate of the previous
//               position as predecessor p;
//   walk:       per request, position by position, the row of the chosen
//               predecessor: greedy first maximum or an inverse-CDF draw from
//               softmax(row / T); q_rows = that softmax.
//
// Kernels: topk_chunk_kernel (grid rows x chunks: a sorted register list per
// thread, then K rounds of block argmax over the lists' heads in LDS),
// topk_merge_kernel (one wave per row over the <= 64 chunk lists), and
// lattice_walk_kernel (one workgroup per request: every (position,
// predecessor, candidate) score in parallel, then the walk).
#include <math.h>

#include "common.cuh"
#include "internal.h"

namespace dflash {
namespace {

constexpr int kT = 256;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kNoIdx = 0x7fffffff;

// (value, index) order of the candidates: larger value first, then lower index
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

template <typename T> __device__ __forceinline__ float ldf(const T* p);
template <> __device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldf<bf16_t>(const bf16_t* p) {
  return bf16_to_f32(p->bits);
}

// Block-wide best (value, index) of one entry per thread; every thread gets it.
__device__ __forceinline__ void block_best(float& v, int& i, float* rv, int* ri) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(v, o, 64);
    const int oi = __shfl_xor(i, o, 64);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    rv[threadIdx.x >> 6] = v;
    ri[threadIdx.x >> 6] = i;
  }
  __syncthreads();
  v = rv[0];
  i = ri[0];
  for (int w = 1; w < kT / 64; ++w)
    if (better(rv[w], ri[w], v, i)) {
      v = rv[w];
      i = ri[w];
    }
}

// ---------------------------------------------------------------- top-K
template <typename T, int K>
__global__ __launch_bounds__(kT) void topk_chunk_kernel(const T* __restrict__ logits, int V,
                                                        int chunk, int n_chunks,
                                                        float* __restrict__ pv,
                                                        int* __restrict__ pi) {
  const int row = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const T* x = logits + (int64_t)row * V;
  const int c0 = c * chunk, c1 = min(V, c0 + chunk);
  float bv[K];
  int bi[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    bv[k] = kNegInf;
    bi[k] = kNoIdx;
  }
  for (int i = c0 + tid; i < c1; i += kT) {
    float cv = ldf(x + i);
    int ci = i;
    if (!better(cv, ci, bv[K - 1], bi[K - 1])) continue;
    // sorted insertion by compare-and-swap down the list (static indices)
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (better(cv, ci, bv[k], bi[k])) {
        const float tv = bv[k];
        const int ti = bi[k];
        bv[k] = cv;
        bi[k] = ci;
        cv = tv;
        ci = ti;
      }
  }
  __shared__ float lv[kT * K];
  __shared__ int li[kT * K];
  __shared__ float rv[kT / 64];
  __shared__ int ri[kT / 64];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    lv[tid * K + k] = bv[k];
    li[tid * K + k] = bi[k];
  }
  __syncthreads();
  int ptr = 0;
  float* ov = pv + ((int64_t)row * n_chunks + c) * K;
  int* oi = pi + ((int64_t)row * n_chunks + c) * K;
  for (int k = 0; k < K; ++k) {
    const float hv = ptr < K ? lv[tid * K + ptr] : kNegInf;
    const int hi = ptr < K ? li[tid * K + ptr] : kNoIdx;
    float v = hv;
    int i = hi;
    block_best(v, i, rv, ri);
    if (hi == i && i != kNoIdx) ++ptr;  // indices are unique: one thread advances
    if (tid == 0) {
      ov[k] = v;
      oi[k] = i;
    }
  }
}

// One wave per row: lane l holds chunk l's sorted list (n_chunks <= 64).
template <int K>
__global__ __launch_bounds__(64) void topk_merge_kernel(const float* __restrict__ pv,
                                                        const int* __restrict__ pi,
                                                        int n_chunks, int V,
                                                        int32_t* __restrict__ cand,
                                                        float* __restrict__ unary) {
  const int row = blockIdx.x, lane = threadIdx.x;
  __shared__ float lv[64 * K];
  __shared__ int li[64 * K];
  for (int e = lane; e < 64 * K; e += 64) {
    const int l = e / K;
    lv[e] = l < n_chunks ? pv[((int64_t)row * n_chunks + l) * K + e % K] : kNegInf;
    li[e] = l < n_chunks ? pi[((int64_t)row * n_chunks + l) * K + e % K] : kNoIdx;
  }
  __syncthreads();
  int ptr = 0;
  for (int k = 0; k < K; ++k) {
    const float hv = ptr < K ? lv[lane * K + ptr] : kNegInf;
    const int hi = ptr < K ? li[lane * K + ptr] : kNoIdx;
    float v = hv;
    int i = hi;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(v, o, 64);
      const int oi = __shfl_xor(i, o, 64);
      if (better(ov, oi, v, i)) {
        v = ov;
        i = oi;
      }
    }
    if (hi == i && i != kNoIdx) ++ptr;
    if (lane == 0) {
      cand[(int64_t)row * K + k] = (i >= 0 && i < V) ? i : 0;
      unary[(int64_t)row * K + k] = v;
    }
  }
}

// ---------------------------------------------------------------- lattice + walk
// grid (B); 256 threads.  J = S - 1 drafted positions, r = rank (multiple of 8).
template <typename T>
__global__ __launch_bounds__(kT) void lattice_walk_kernel(
    const int32_t* __restrict__ cand, const float* __restrict__ unary,
    const float* __restrict__ w, const T* __restrict__ A, const T* __restrict__ Bt,
    const int32_t* __restrict__ anchor, const float* __restrict__ uni, float temperature,
    int S, int K, int r, int V, int32_t* __restrict__ candidates, float* __restrict__ q_rows) {
  const int b = blockIdx.x, tid = threadIdx.x, J = S - 1;
  extern __shared__ float score[];  // [J][K][K]
  const int n = J * K * K;
  const int32_t* cb = cand + (int64_t)b * J * K;
  const float* ub = unary + (int64_t)b * J * K;
  const int a0 = min(max(anchor[b], 0), V - 1);
  for (int t = tid; t < n; t += kT) {
    const int j = t / (K * K), p = (t / K) % K, k = t % K;
    if (j == 0 && p > 0) {
      score[t] = kNegInf;  // the first position has one predecessor, the anchor
      continue;
    }
    const int pred = j == 0 ? a0 : min(max(cb[(j - 1) * K + p], 0), V - 1);
    const int c = min(max(cb[j * K + k], 0), V - 1);
    const T* ar = A + (int64_t)pred * r;
    const T* br = Bt + (int64_t)c * r;
    const float* wr = w + ((int64_t)b * J + j) * r;
    float s = 0.f;
    for (int e = 0; e < r; ++e) s += ldf(ar + e) * wr[e] * ldf(br + e);
    score[t] = ub[j * K + k] + s;
  }
  __syncthreads();
  if (tid != 0) return;
  const float invT = 1.0f / temperature;
  candidates[(int64_t)b * S] = anchor[b];
  int p = 0;
  for (int j = 0; j < J; ++j) {
    const float* row = score + (j * K + p) * K;
    float m = kNegInf;
    int best = 0;
    for (int k = 0; k < K; ++k)
      if (row[k] > m) {  // first maximum
        m = row[k];
        best = k;
      }
    const float mt = m * (uni ? invT : 1.f);
    float sum = 0.f;
    float* q = q_rows + ((int64_t)b * J + j) * K;
    for (int k = 0; k < K; ++k) {
      const float e = expf(row[k] * (uni ? invT : 1.f) - mt);
      q[k] = e;
      sum += e;
    }
    const float inv = 1.0f / sum;
    for (int k = 0; k < K; ++k) q[k] *= inv;
    int pick = best;
    if (uni) {
      const float x = uni[(int64_t)b * J + j];
      float cum = 0.f;
      pick = K - 1;
      for (int k = 0; k < K; ++k) {
        cum += q[k];
        if (cum > x) {
          pick = k;
          break;
        }
      }
    }
    candidates[(int64_t)b * S + 1 + j] = cb[j * K + pick];
    p = pick;
  }
}

template <int K>
hipError_t topk_launch(int dt, const void* logits, int rows, int V, const SelPlan& pl, float* pv,
                       int* pi, int32_t* cand, float* unary, hipStream_t st) {
  if (dt == DFLASH_BF16)
    hipLaunchKernelGGL((topk_chunk_kernel<bf16_t, K>), dim3(rows, pl.n_chunks), dim3(kT), 0, st,
                       static_cast<const bf16_t*>(logits), V, pl.chunk, pl.n_chunks, pv, pi);
  else
    hipLaunchKernelGGL((topk_chunk_kernel<float, K>), dim3(rows, pl.n_chunks), dim3(kT), 0, st,
                       static_cast<const float*>(logits), V, pl.chunk, pl.n_chunks, pv, pi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((topk_merge_kernel<K>), dim3(rows), dim3(64), 0, st, pv, pi, pl.n_chunks, V,
                     cand, unary);
  return hipGetLastError();
}

}  // namespace

SelPlan plan_selector(int rows, int V) {
  SelPlan pl{};
  int want = (1024 + rows - 1) / rows;
  want = want < 1 ? 1 : (want > 64 ? 64 : want);
  pl.chunk = ((V + want - 1) / want + 63) / 64 * 64;
  pl.n_chunks = (V + pl.chunk - 1) / pl.chunk;
  return pl;
}

hipError_t launch_topk(int dt, const void* logits, int rows, int V, int K, const SelPlan& pl,
                       float* pv, int* pi, int32_t* cand, float* unary, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  switch (K) {
    case 1: return topk_launch<1>(dt, logits, rows, V, pl, pv, pi, cand, unary, st);
    case 2: return topk_launch<2>(dt, logits, rows, V, pl, pv, pi, cand, unary, st);
    case 4: return topk_launch<4>(dt, logits, rows, V, pl, pv, pi, cand, unary, st);
    case 8: return topk_launch<8>(dt, logits, rows, V, pl, pv, pi, cand, unary, st);
    case 16: return topk_launch<16>(dt, logits, rows, V, pl, pv, pi, cand, unary, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_lattice_walk(int dt, const int32_t* cand, const float* unary, const float* w,
                               const void* A, const void* Bt, const int32_t* anchor,
                               const float* uni, float temperature, int B, int S, int K, int r,
                               int V, int32_t* candidates, float* q_rows, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  const size_t lds = sizeof(float) * (size_t)(S - 1) * K * K;
  if (dt == DFLASH_BF16)
    hipLaunchKernelGGL((lattice_walk_kernel<bf16_t>), dim3(B), dim3(kT), lds, st, cand, unary, w,
                       static_cast<const bf16_t*>(A), static_cast<const bf16_t*>(Bt), anchor, uni,
                       temperature, S, K, r, V, candidates, q_rows);
  else
    hipLaunchKernelGGL((lattice_walk_kernel<float>), dim3(B), dim3(kT), lds, st, cand, unary, w,
                       static_cast<const float*>(A), static_cast<const float*>(Bt), anchor, uni,
                       temperature, S, K, r, V, candidates, q_rows);
  return hipGetLastError();
}

}  // namespace dflash
