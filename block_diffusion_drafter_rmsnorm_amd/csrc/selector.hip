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
// Kernels: topk_chunk_kernel (grid rows x chunks of <= 8192 logits staged in
// LDS, K rounds of block argmax each strictly after the previous winner),
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
constexpr int kMaxChunk = 8192;  // logits of one top-K chunk (32 KB of LDS)

// (value, index) order of the candidates: larger value first, then lower index
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

template <typename T> __device__ __forceinline__ float ldf(const T* p);
template <> __device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldf<bf16_t>(const bf16_t* p) {
  return bf16_to_f32(p->bits);
}

// Eight consecutive values as fp32 (16-byte loads for bf16, two for fp32).
__device__ __forceinline__ void ld8(const bf16_t* p, float* v) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = __uint_as_float(u[k] << 16);
    v[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void ld8(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
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
// One workgroup per (row, chunk of at most kMaxChunk logits): the chunk is
// staged in LDS as fp32 (16-byte loads when VEC8: rows on 16-byte boundaries,
// V a multiple of 8), then K rounds each take the block's best element that
// comes strictly after the previous round's winner in the (value, index)
// order.  Every thread does the same work in every round (no divergent
// insertion); NaN is never taken.
template <typename T, int K, bool VEC8>
__global__ __launch_bounds__(kT) void topk_chunk_kernel(const T* __restrict__ logits, int V,
                                                        int chunk, int n_chunks,
                                                        float* __restrict__ pv,
                                                        int* __restrict__ pi) {
  const int row = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const T* x = logits + (int64_t)row * V;
  const int c0 = c * chunk, n = min(V, c0 + chunk) - c0;
  __shared__ float xs[kMaxChunk];
  __shared__ float rv[kT / 64];
  __shared__ int ri[kT / 64];
  if (VEC8) {
    for (int e = tid * 8; e < n; e += kT * 8) {
      float v[8];
      ld8(x + c0 + e, v);
#pragma unroll
      for (int u = 0; u < 8; ++u) xs[e + u] = v[u];
    }
  } else {
    for (int e = tid; e < n; e += kT) xs[e] = ldf(x + c0 + e);
  }
  __syncthreads();
  float prev_v = __builtin_huge_valf();
  int prev_i = -1;
  float* ov = pv + ((int64_t)row * n_chunks + c) * K;
  int* oi = pi + ((int64_t)row * n_chunks + c) * K;
  for (int k = 0; k < K; ++k) {
    float bv = kNegInf;
    int bi = kNoIdx;
    for (int e = tid; e < n; e += kT) {
      const float v = xs[e];
      const int i = c0 + e;
      if (better(prev_v, prev_i, v, i) && better(v, i, bv, bi)) {
        bv = v;
        bi = i;
      }
    }
    block_best(bv, bi, rv, ri);
    if (tid == 0) {
      ov[k] = bv;
      oi[k] = bi;
    }
    prev_v = bv;
    prev_i = bi;
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
template <typename T, int R>
__global__ __launch_bounds__(kT) void lattice_walk_kernel(
    const int32_t* __restrict__ cand, const float* __restrict__ unary,
    const float* __restrict__ w, const T* __restrict__ A, const T* __restrict__ Bt,
    const int32_t* __restrict__ anchor, const float* __restrict__ uni, float temperature,
    int S, int K, int V, int32_t* __restrict__ candidates, float* __restrict__ q_rows) {
  constexpr int r = R;
  const int b = blockIdx.x, tid = threadIdx.x, J = S - 1;
  extern __shared__ float score[];  // [J][K][K], then this request's w rows [J][r]
  const int n = J * K * K;
  float* ws = score + n;
  for (int e = tid; e < J * r; e += kT) ws[e] = w[(int64_t)b * J * r + e];
  __syncthreads();

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
    const float* wr = ws + j * r;
    // both rows' loads go out together (R / 8 of each), then the sum in order
    float av[R], bv[R];
#pragma unroll
    for (int e = 0; e < R; e += 8) {
      ld8(ar + e, av + e);
      ld8(br + e, bv + e);
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < R; ++e) s += av[e] * wr[e] * bv[e];
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

template <typename T, int K>
void topk_chunks(const void* logits, int rows, int V, const SelPlan& pl, float* pv, int* pi,
                 hipStream_t st) {
  const bool vec8 = V % 8 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0;
  const T* x = static_cast<const T*>(logits);
  if (vec8)
    hipLaunchKernelGGL((topk_chunk_kernel<T, K, true>), dim3(rows, pl.n_chunks), dim3(kT), 0, st,
                       x, V, pl.chunk, pl.n_chunks, pv, pi);
  else
    hipLaunchKernelGGL((topk_chunk_kernel<T, K, false>), dim3(rows, pl.n_chunks), dim3(kT), 0,
                       st, x, V, pl.chunk, pl.n_chunks, pv, pi);
}

template <int K>
hipError_t topk_launch(int dt, const void* logits, int rows, int V, const SelPlan& pl, float* pv,
                       int* pi, int32_t* cand, float* unary, hipStream_t st) {
  if (dt == DFLASH_BF16)
    topk_chunks<bf16_t, K>(logits, rows, V, pl, pv, pi, st);
  else
    topk_chunks<float, K>(logits, rows, V, pl, pv, pi, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((topk_merge_kernel<K>), dim3(rows), dim3(64), 0, st, pv, pi, pl.n_chunks, V,
                     cand, unary);
  return hipGetLastError();
}

}  // namespace

SelPlan plan_selector(int rows, int V) {
  SelPlan pl{};
  int want = (2048 + rows - 1) / rows;
  want = want < 1 ? 1 : (want > 64 ? 64 : want);
  pl.chunk = ((V + want - 1) / want + 63) / 64 * 64;
  if (pl.chunk > kMaxChunk) pl.chunk = kMaxChunk;  // V <= 64 * kMaxChunk keeps n_chunks <= 64
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

template <typename T, int R>
static void lattice_launch(const int32_t* cand, const float* unary, const float* w, const void* A,
                           const void* Bt, const int32_t* anchor, const float* uni,
                           float temperature, int B, int S, int K, int V, int32_t* candidates,
                           float* q_rows, hipStream_t st) {
  const size_t lds = sizeof(float) * ((size_t)(S - 1) * K * K + (size_t)(S - 1) * R);
  hipLaunchKernelGGL((lattice_walk_kernel<T, R>), dim3(B), dim3(kT), lds, st, cand, unary, w,
                     static_cast<const T*>(A), static_cast<const T*>(Bt), anchor, uni,
                     temperature, S, K, V, candidates, q_rows);
}

template <typename T>
static hipError_t lattice_rank(int r, const int32_t* cand, const float* unary, const float* w,
                               const void* A, const void* Bt, const int32_t* anchor,
                               const float* uni, float temperature, int B, int S, int K, int V,
                               int32_t* candidates, float* q_rows, hipStream_t st) {
  switch (r) {
    case 16: lattice_launch<T, 16>(cand, unary, w, A, Bt, anchor, uni, temperature, B, S, K, V,
                                   candidates, q_rows, st); break;
    case 32: lattice_launch<T, 32>(cand, unary, w, A, Bt, anchor, uni, temperature, B, S, K, V,
                                   candidates, q_rows, st); break;
    case 64: lattice_launch<T, 64>(cand, unary, w, A, Bt, anchor, uni, temperature, B, S, K, V,
                                   candidates, q_rows, st); break;
    case 128: lattice_launch<T, 128>(cand, unary, w, A, Bt, anchor, uni, temperature, B, S, K, V,
                                     candidates, q_rows, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lattice_walk(int dt, const int32_t* cand, const float* unary, const float* w,
                               const void* A, const void* Bt, const int32_t* anchor,
                               const float* uni, float temperature, int B, int S, int K, int r,
                               int V, int32_t* candidates, float* q_rows, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  if (dt == DFLASH_BF16)
    return lattice_rank<bf16_t>(r, cand, unary, w, A, Bt, anchor, uni, temperature, B, S, K, V,
                                candidates, q_rows, st);
  return lattice_rank<float>(r, cand, unary, w, A, Bt, anchor, uni, temperature, B, S, K, V,
                             candidates, q_rows, st);
}

}  // namespace dflash
