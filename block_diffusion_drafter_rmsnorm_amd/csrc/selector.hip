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
//               softmax(row / T); q_rows = the distribution the choice was
//               drawn from (that softmax, or one-hot on the greedy choice).
//
// Kernels: topk_tiles_kernel (one workgroup per row: only the 128-column
// tiles whose lm_head argmax partial reaches the K-th largest tile maximum can
// hold a candidate; their logits are searched by rounds of block argmax), and
// lattice_walk_kernel (one workgroup per request: every (position,
// predecessor, candidate) score in parallel, then the walk on one wave, a lane
// per candidate slot).
#include <math.h>

#include "common.h"
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

// ---------------------------------------------------------------- top-K
// Wave reductions on DPP moves (ALU latency, no LDS crossbar): quad
// permutations 1032 and 2301, the half-row and row mirrors combine each row of
// 16 lanes; row broadcasts of lanes 15 (into rows 1 and 3) and 31 (into rows
// 2 and 3) finish in lane 63, which readlane hands to every lane.  A lane a
// move leaves out keeps old.  Every lane of the wave must be active.
constexpr int kQuad1032 = 0xB1, kQuad2301 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;
constexpr int kBcast15 = 0x142, kBcast31 = 0x143, kRowShr = 0x110;

template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xf, false);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ void best_step(float& v, int& i) {
  const float ov = __int_as_float(dpp<CTRL, ROWS>(__float_as_int(v), __float_as_int(v)));
  const int oi = dpp<CTRL, ROWS>(i, i);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// Wave-wide best (value, index) in (value, lower index) order; every lane gets
// it.  Values must not be NaN (the order is then total, so any combining
// order gives the same result).
__device__ __forceinline__ void wave_best(float& v, int& i) {
  best_step<kQuad1032, 0xf>(v, i);
  best_step<kQuad2301, 0xf>(v, i);
  best_step<kHalfMirror, 0xf>(v, i);
  best_step<kMirror, 0xf>(v, i);
  best_step<kBcast15, 0xa>(v, i);
  best_step<kBcast31, 0xc>(v, i);
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float add_step(float s) {
  return s + __int_as_float(dpp<CTRL, ROWS>(0, __float_as_int(s)));
}

// Wave-wide sum in a fixed order; every lane gets it.
__device__ __forceinline__ float wave_sum(float s) {
  s = add_step<kQuad1032, 0xf>(s);
  s = add_step<kQuad2301, 0xf>(s);
  s = add_step<kHalfMirror, 0xf>(s);
  s = add_step<kMirror, 0xf>(s);
  s = add_step<kBcast15, 0xa>(s);
  s = add_step<kBcast31, 0xc>(s);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 63));
}

// Inclusive prefix sum over the 16 lanes of each row (row shifts by 1, 2, 4, 8;
// a lane whose source falls before its row adds 0).
__device__ __forceinline__ float row_incl_scan(float c) {
  c = add_step<kRowShr + 1, 0xf>(c);
  c = add_step<kRowShr + 2, 0xf>(c);
  c = add_step<kRowShr + 4, 0xf>(c);
  c = add_step<kRowShr + 8, 0xf>(c);
  return c;
}

// One workgroup per row, from the lm_head's per-128-column argmax partials.
// K tiles whose maxima all reach t hold K distinct logits >= t, so t bounds
// the row's K-th largest logit from below and only tiles whose maximum reaches
// t can hold a top-K logit, and only their logits that reach t.
//   t: each thread's largest tile maximum, ranked within its wave: the
//   lane maximum of rank K-1 bounds t from below (K distinct tiles reach it),
//   and the largest of the 4 waves' bounds selects the candidate tiles; when
//   they are at most 64, ranking them gives t exactly.
//   top-K: the logits of the qualifying tiles (16 per thread in registers, the
//   loads issued together) that reach t; when they are at most 64, one wave
//   ranks them and rank k is candidate k.
// Ranks count the entries before one in (value desc, index asc) order, so they
// are distinct and the result is the plain top-K with ties to the lower id.
// When a set is larger (ties over many tiles), the same result comes from K
// rounds of wave argmax (each strictly after the previous winner) over the
// tiles, then over batches of 32 qualifying tiles with a running list.
constexpr int kMaxTiles = 4096;  // 128-column tiles of a row (vocab <= 524288)

// The K best of one register array per lane (plus one extra entry), strictly
// after nothing, by K rounds of wave argmax; lane 0 writes round k to ov/oi.
template <int K, int N>
__device__ __forceinline__ void wave_topk(const float (&v)[N], const int (&ix)[N], float xv,
                                          int xi, float* ov, int* oi) {
  float pv = __builtin_huge_valf();
  int pi = -1;
  for (int k = 0; k < K; ++k) {
    float bv = kNegInf;
    int bi = kNoIdx;
    if (better(pv, pi, xv, xi)) {
      bv = xv;
      bi = xi;
    }
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (better(pv, pi, v[i], ix[i]) && better(v[i], ix[i], bv, bi)) {
        bv = v[i];
        bi = ix[i];
      }
    wave_best(bv, bi);
    if ((threadIdx.x & 63) == 0) {
      ov[k] = bv;
      oi[k] = bi;
    }
    pv = bv;
    pi = bi;
  }
}

// Rank of (v, i) among the n (value, index bits) entries of an LDS list.
// Reads go out 8 at a time: the list must hold n rounded up to 8 entries
// (the ones past n are not counted).
__device__ __forceinline__ int rank_in(const float2* list, int n, float v, int i) {
  int r = 0;
  for (int j0 = 0; j0 < n; j0 += 8) {
    float2 o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = list[j0 + u];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      r += (j0 + u < n && better(o[u].x, __float_as_int(o[u].y), v, i)) ? 1 : 0;
  }
  return r;
}

// This thread's offset for cnt entries in thread order, and the block total.
// All threads call it; it begins with a barrier (earlier readers of tmp are
// done) and ends with one (every count is in).
__device__ __forceinline__ int block_offset(int cnt, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  __syncthreads();
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int off = incl - cnt;
  total = 0;
  for (int w = 0; w < kT / 64; ++w) {
    if (w < wave) off += tmp[w];
    total += tmp[w];
  }
  return off;
}

template <typename T, int K>
__global__ __launch_bounds__(kT) void topk_tiles_kernel(const T* __restrict__ logits,
                                                        const float2* __restrict__ part, int V,
                                                        int n_tiles, int32_t* __restrict__ cand,
                                                        float* __restrict__ unary) {
  constexpr int NW = kT / 64;
  constexpr int TPT = kMaxTiles / kT;  // tile maxima per thread
  constexpr int TPB = 32;              // qualifying tiles per batch
  constexpr int EPT = TPB * 128 / kT;  // logits per thread per batch
  constexpr int kRankCap = 64;         // largest set ranked in one pass
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int qt[kMaxTiles];
  __shared__ float wv[NW * K];
  __shared__ int wi[NW * K];
  __shared__ float lv[K];
  __shared__ int li[K];
  __shared__ int wc[NW];
  __shared__ float2 cl[kT];  // lane maxima, then candidate tiles, then candidate logits
  __shared__ float2 bw[NW];
  // tile maxima: tile tid + i * kT in register i (never NaN: the partials map
  // NaN to -inf); absent tiles carry no index
  float tm[TPT];
  int ti[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int t = tid + i * kT;
    tm[i] = t < n_tiles ? part[(int64_t)row * n_tiles + t].x : kNegInf;
    ti[i] = t < n_tiles ? t : kNoIdx;
  }
  // lower bound of t: per wave, the lane maximum of rank K - 1
  float mv = kNegInf;
  int mi = kNoIdx;
#pragma unroll
  for (int i = 0; i < TPT; ++i)
    if (better(tm[i], ti[i], mv, mi)) {
      mv = tm[i];
      mi = ti[i];
    }
  cl[tid] = make_float2(mv, __int_as_float(mi));
  if (lane == 0) bw[wave] = make_float2(kNegInf, __int_as_float(kNoIdx));
  __syncthreads();
  if (mi != kNoIdx && rank_in(cl + wave * 64, 64, mv, mi) == K - 1)
    bw[wave] = make_float2(mv, __int_as_float(mi));
  __syncthreads();
  float lb = kNegInf;
  for (int w = 0; w < NW; ++w) lb = fmaxf(lb, bw[w].x);
  // candidate tiles (maxima >= lb): at least K of them
  int cnt0 = 0;
#pragma unroll
  for (int i = 0; i < TPT; ++i) cnt0 += (ti[i] != kNoIdx && tm[i] >= lb) ? 1 : 0;
  int nc;
  int off0 = block_offset(cnt0, wc, nc);
  if (nc <= kRankCap) {
#pragma unroll
    for (int i = 0; i < TPT; ++i)
      if (ti[i] != kNoIdx && tm[i] >= lb) cl[off0++] = make_float2(tm[i], __int_as_float(ti[i]));
  }
  __syncthreads();
  float thr;
  if (nc <= kRankCap) {
    // every wave ranks the candidates the same way: rank K - 1 is t (fewer
    // than K tiles: no bound, every tile qualifies)
    const float2 me = lane < nc ? cl[lane] : make_float2(kNegInf, __int_as_float(kNoIdx));
    const bool at = lane < nc && rank_in(cl, nc, me.x, __float_as_int(me.y)) == K - 1;
    const uint64_t hit = __ballot(at);
    thr = hit ? __shfl(me.x, __ffsll((unsigned long long)hit) - 1, 64) : kNegInf;
  } else {
    wave_topk<K>(tm, ti, kNegInf, kNoIdx, wv + wave * K, wi + wave * K);
    __syncthreads();
    // every wave merges the NW * K <= 64 entries (one per lane) the same way
    const float ev = lane < NW * K ? wv[lane] : kNegInf;
    const int ei = lane < NW * K ? wi[lane] : kNoIdx;
    float pv = __builtin_huge_valf();
    int pi = -1;
    for (int k = 0; k < K; ++k) {
      float bv = kNegInf;
      int bi = kNoIdx;
      if (better(pv, pi, ev, ei)) {
        bv = ev;
        bi = ei;
      }
      wave_best(bv, bi);
      pv = bv;
      pi = bi;
    }
    thr = pi == kNoIdx ? kNegInf : pv;  // fewer than K tiles: every tile qualifies
  }
  // qualifying tiles: a count per thread, a block scan, then each thread's own
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < TPT; ++i) cnt += (ti[i] != kNoIdx && tm[i] >= thr) ? 1 : 0;
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  __syncthreads();  // wv / wi are read above before the batches rewrite them
  if (lane == 63) wc[wave] = incl;
  __syncthreads();
  int off = incl - cnt, nq = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wave) off += wc[w];
    nq += wc[w];
  }
#pragma unroll
  for (int i = 0; i < TPT; ++i)
    if (ti[i] != kNoIdx && tm[i] >= thr) qt[off++] = ti[i];
  __syncthreads();
  // logit e = tid + i * kT of a batch of qualifying tiles is column (tid & 127)
  // of the batch's tile 2 i + (tid >> 7)
  if (nq <= TPB) {
    float v[EPT];
    int ix[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int slot = 2 * i + (tid >> 7);
      const int col = slot < nq ? qt[slot] * 128 + (tid & 127) : V;
      v[i] = col < V ? ldf(logits + (int64_t)row * V + col) : kNegInf;
      ix[i] = col < V ? col : kNoIdx;
    }
    // only logits that reach t can be among the K largest (NaN never does)
    int cnt1 = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) cnt1 += (ix[i] != kNoIdx && v[i] >= thr) ? 1 : 0;
    int ne;
    int off1 = block_offset(cnt1, wc, ne);
    if (ne <= kRankCap) {
#pragma unroll
      for (int i = 0; i < EPT; ++i)
        if (ix[i] != kNoIdx && v[i] >= thr) cl[off1++] = make_float2(v[i], __int_as_float(ix[i]));
      if (tid < K) {
        lv[tid] = kNegInf;
        li[tid] = kNoIdx;
      }
      __syncthreads();
      if (wave == 0 && lane < ne) {
        const float2 me = cl[lane];
        const int rk = rank_in(cl, ne, me.x, __float_as_int(me.y));
        if (rk < K) {
          lv[rk] = me.x;
          li[rk] = __float_as_int(me.y);
        }
      }
      __syncthreads();
      if (tid < K) {
        const int i = li[tid];
        cand[(int64_t)row * K + tid] = (i >= 0 && i < V) ? i : 0;
        unary[(int64_t)row * K + tid] = lv[tid];
      }
      return;
    }
  }
  // batches of at most 32 qualifying tiles with a running list
  int n_list = 0;
  for (int b0 = 0; b0 < nq; b0 += TPB) {
    const int nb = min(TPB, nq - b0);
    float v[EPT];
    int ix[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int slot = 2 * i + (tid >> 7);
      const int col = slot < nb ? qt[b0 + slot] * 128 + (tid & 127) : V;
      v[i] = col < V ? ldf(logits + (int64_t)row * V + col) : kNegInf;
      ix[i] = col < V ? col : kNoIdx;
    }
    const bool has_list = tid < K && tid < n_list;
    wave_topk<K>(v, ix, has_list ? lv[tid] : kNegInf, has_list ? li[tid] : kNoIdx,
                 wv + wave * K, wi + wave * K);
    __syncthreads();
    if (wave == 0) {  // merge the waves' lists (NW * K <= 64 entries, one per lane)
      const float ev = lane < NW * K ? wv[lane] : kNegInf;
      const int ei = lane < NW * K ? wi[lane] : kNoIdx;
      float pv = __builtin_huge_valf();
      int pi = -1;
      for (int k = 0; k < K; ++k) {
        float bv = kNegInf;
        int bi = kNoIdx;
        if (better(pv, pi, ev, ei)) {
          bv = ev;
          bi = ei;
        }
        wave_best(bv, bi);
        if (lane == 0) {
          lv[k] = bv;
          li[k] = bi;
        }
        pv = bv;
        pi = bi;
      }
    }
    n_list = K;
    __syncthreads();
  }
  if (tid < K) {
    const int i = li[tid];
    cand[(int64_t)row * K + tid] = (i >= 0 && i < V) ? i : 0;
    unary[(int64_t)row * K + tid] = lv[tid];
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
  // LDS: score [J][K][K], this request's w rows [J][r], its candidate ids
  // [J][K] and its uniforms [J] (the walk then reads no global memory)
  extern __shared__ float score[];
  const int n = J * K * K;
  float* ws = score + n;
  int* cb = reinterpret_cast<int*>(ws + J * r);
  float* us = reinterpret_cast<float*>(cb + J * K);
  for (int e = tid; e < J * r; e += kT) ws[e] = w[(int64_t)b * J * r + e];
  for (int e = tid; e < J * K; e += kT) cb[e] = cand[(int64_t)b * J * K + e];
  if (uni != nullptr)
    for (int e = tid; e < J; e += kT) us[e] = uni[(int64_t)b * J + e];
  __syncthreads();

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
  // the walk, on the first wave: lane k < K holds candidate slot k of the row
  if (tid >= 64) return;
  const int lane = tid;
  const float sc = uni ? 1.0f / temperature : 1.f;
  if (lane == 0) candidates[(int64_t)b * S] = anchor[b];
  int p = 0;
  for (int j = 0; j < J; ++j) {
    const float v = lane < K ? score[(j * K + p) * K + lane] : kNegInf;
    // greedy: the first maximum (NaN never wins)
    float m = v == v ? v : kNegInf;
    int best = lane < K ? lane : kNoIdx;
    wave_best(m, best);
    int pick = best;
    float q = lane == best ? 1.f : 0.f;  // greedy: all mass on the choice
    if (uni) {
      const float e = lane < K ? expf(v * sc - m * sc) : 0.f;
      q = e * (1.0f / wave_sum(e));
      // inverse CDF: the first slot whose running sum of q exceeds the draw
      const float x = us[j];
      const float c = row_incl_scan(q);  // K <= 16: the candidates sit in row 0
      const uint64_t hit = __ballot(lane < K && c > x);
      pick = hit ? __ffsll((unsigned long long)hit) - 1 : K - 1;
    }
    if (lane < K) q_rows[((int64_t)b * J + j) * K + lane] = q;
    if (lane == 0) candidates[(int64_t)b * S + 1 + j] = cb[j * K + pick];
    p = pick;
  }
}

template <int K>
hipError_t topk_launch(int dt, const void* logits, const float2* part, int rows, int V,
                       int32_t* cand, float* unary, hipStream_t st) {
  const int nt = logits_tiles(V);
  if (dt == DFLASH_BF16)
    hipLaunchKernelGGL((topk_tiles_kernel<bf16_t, K>), dim3(rows), dim3(kT), 0, st,
                       static_cast<const bf16_t*>(logits), part, V, nt, cand, unary);
  else
    hipLaunchKernelGGL((topk_tiles_kernel<float, K>), dim3(rows), dim3(kT), 0, st,
                       static_cast<const float*>(logits), part, V, nt, cand, unary);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(int dt, const void* logits, const float2* part, int rows, int V, int K,
                       int32_t* cand, float* unary, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  switch (K) {
    case 1: return topk_launch<1>(dt, logits, part, rows, V, cand, unary, st);
    case 2: return topk_launch<2>(dt, logits, part, rows, V, cand, unary, st);
    case 4: return topk_launch<4>(dt, logits, part, rows, V, cand, unary, st);
    case 8: return topk_launch<8>(dt, logits, part, rows, V, cand, unary, st);
    case 16: return topk_launch<16>(dt, logits, part, rows, V, cand, unary, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int R>
static void lattice_launch(const int32_t* cand, const float* unary, const float* w, const void* A,
                           const void* Bt, const int32_t* anchor, const float* uni,
                           float temperature, int B, int S, int K, int V, int32_t* candidates,
                           float* q_rows, hipStream_t st) {
  const size_t lds = sizeof(float) * ((size_t)(S - 1) * K * K + (size_t)(S - 1) * R) +
                     sizeof(int) * (size_t)(S - 1) * K + sizeof(float) * (size_t)(S - 1);
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
