// Rejection-sampling verify-accept ("Inside SGLang: DFlash and DFlash 2
// Implementation", the section on sampling with the proposal distribution the
// drafter used, and Step 6 for the emitted tokens and the commit).
//
// A drafted token y = d_{j+1} survives when u_j * q_j(y) < p_j(y), with
// p_j = softmax(target_logits[j] / T_t) and q_j = softmax(draft_logits[j] / T_d)
// (or the point mass on y for argmax drafts).  At the first rejection the
// correction token is drawn from [p_j - q_j]_+, after full acceptance the bonus
// from p_{S-1}; the draw is an inverse CDF at u_{S-1} * (total weight).
//
// Three kernels, all deterministic (every sum is taken in a fixed order):
//   1. spec_stats_kernel: one streaming pass over every target and draft row,
//      online (max, sum of exp2) per vocabulary chunk.  HBM-bound: this pass is
//      the only one that reads all the logits.
//   2. spec_walk_kernel: per request, the chunk partials are merged per row,
//      lanes take the S-1 decisions at once and a ballot finds the first
//      rejection; then every workgroup sums the weights of its chunk of the
//      row the token is drawn from.
//   3. spec_pick_kernel: per request, the chunk holding the draw; its weights
//      are staged in LDS with 16-byte loads, then a block-wide scan of
//      per-thread runs over LDS finds the token.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunk2 = 8192;  // logits per pick chunk (weights staged in 32 KB of LDS)
constexpr int kMaxStatsPartials = 4096;  // (2S - 1) * n_chunks1 per request, staged in LDS
constexpr float kNegInf = -__builtin_huge_valf();

// Walk result of one request, written by chunk 0 of the walk kernel.
struct SpecWalk {
  float mt, izt;  // max and 1 / sum(exp2((l - max) * ct)) of the target row drawn from
  float md, izd;  // the same for the draft row (mode 0)
  int a;          // accepted drafts
  int y;          // rejected draft token (mode 1)
  int mode;       // 0: [p - q]_+ with q from draft logits, 1: [p - point mass]_+, 2: p (bonus),
                  // 3: [p - q]_+ with q given as K (id, probability) pairs
  int pad;
};

template <typename T> __device__ __forceinline__ float ld1(const T* p);
template <> __device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld1<bf16_t>(const bf16_t* p) {
  return bf16_to_f32(p->bits);
}

// VEC consecutive logits as fp32 (16-byte loads when VEC > 1).
template <typename T, int VEC> struct VecLoad;
template <typename T> struct VecLoad<T, 1> {
  static __device__ __forceinline__ void run(const T* p, float* v) { v[0] = ld1(p); }
};
template <> struct VecLoad<bf16_t, 8> {
  static __device__ __forceinline__ void run(const bf16_t* p, float* v) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(u[k] << 16);
      v[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
    }
  }
};
template <> struct VecLoad<float, 4> {
  static __device__ __forceinline__ void run(const float* p, float* v) {
    const float4 w = *reinterpret_cast<const float4*>(p);
    v[0] = w.x;
    v[1] = w.y;
    v[2] = w.z;
    v[3] = w.w;
  }
};

// (m, s) with s = sum exp2((l - m) * sc): merge of two partials.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2, float sc) {
  if (m2 > m) {
    const float tm = m, ts = s;
    m = m2;
    s = s2;
    m2 = tm;
    s2 = ts;
  }
  if (m2 == kNegInf) return;
  s += s2 * exp2f((m2 - m) * sc);
}

// One vector of logits into the running (m, s).
template <int VEC>
__device__ __forceinline__ void lse_add(float& m, float& s, const float* v, float sc) {
  float mx = v[0];
#pragma unroll
  for (int k = 1; k < VEC; ++k) mx = fmaxf(mx, v[k]);
  if (mx > m) {
    s = (m == kNegInf) ? 0.f : s * exp2f((m - mx) * sc);
    m = mx;
  }
  if (m == kNegInf) return;
#pragma unroll
  for (int k = 0; k < VEC; ++k) s += exp2f((v[k] - m) * sc);
}

// A proposal given directly as K (id, probability) pairs per drafted row (the
// DFlash 2 selector's realised q rows); K == 0: absent.
struct SparseQ {
  const int32_t* ids;
  const float* probs;
  int K;
};

// Weight of token i in the row the final token is drawn from.  One function
// for the chunk sums and the pick so both evaluate the same expression; sid /
// sp hold the rejected row's K pairs (mode 3).
__device__ __forceinline__ float spec_weight(float lt, float ld, int i, const SpecWalk& w,
                                             float ct, float cd, const int* sid = nullptr,
                                             const float* sp = nullptr, int sk = 0) {
#pragma clang fp contract(off)
  const float pt = exp2f((lt - w.mt) * ct) * w.izt;
  if (w.mode == 2) return pt;
  if (w.mode == 1) return (i == w.y) ? fmaxf(pt - 1.f, 0.f) : pt;
  if (w.mode == 3) {
    float q = 0.f;
    for (int k = 0; k < sk; ++k) q += (sid[k] == i) ? sp[k] : 0.f;
    return fmaxf(pt - q, 0.f);
  }
  const float qt = exp2f((ld - w.md) * cd) * w.izd;
  return fmaxf(pt - qt, 0.f);
}
__device__ __forceinline__ float spec_p(float lt, const SpecWalk& w, float ct) {
#pragma clang fp contract(off)
  return exp2f((lt - w.mt) * ct) * w.izt;
}

// Deterministic block sum of 256 values (butterfly per wave, waves in order).
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

// ---------------------------------------------------------------- 1. stats
// grid (rows, n_chunks); rows = B*S target rows then B*(S-1) draft rows.
template <typename T, int VEC>
__global__ __launch_bounds__(kThreads) void spec_stats_kernel(const T* __restrict__ tl,
                                                              const T* __restrict__ dl, int n_t,
                                                              int V, int chunk, int n_chunks,
                                                              float ct, float cd,
                                                              float2* __restrict__ stats) {
  const int row = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const bool is_t = row < n_t;
  const T* base = is_t ? tl + (int64_t)row * V : dl + (int64_t)(row - n_t) * V;
  const float sc = is_t ? ct : cd;
  const int c0 = c * chunk, c1 = min(V, c0 + chunk);
  float m = kNegInf, s = 0.f;
  int i = c0 + tid * VEC;
  constexpr int STEP = kThreads * VEC;
  for (; i + 3 * STEP < c1; i += 4 * STEP) {  // four loads in flight per thread
    float v[4][VEC];
#pragma unroll
    for (int u = 0; u < 4; ++u) VecLoad<T, VEC>::run(base + i + u * STEP, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) lse_add<VEC>(m, s, v[u], sc);
  }
  for (; i < c1; i += STEP) {
    float v[VEC];
    VecLoad<T, VEC>::run(base + i, v);
    lse_add<VEC>(m, s, v, sc);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    lse_merge(m, s, m2, s2, sc);
  }
  __shared__ float2 red[kThreads / 64];
  if ((tid & 63) == 0) red[tid >> 6] = make_float2(m, s);
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kThreads / 64; ++w) lse_merge(m, s, red[w].x, red[w].y, sc);
    stats[(int64_t)row * n_chunks + c] = make_float2(m, s);
  }
}

// ---------------------------------------------------------------- 2. walk
// grid (B, n_chunks2).
template <typename T, int VEC>
__global__ __launch_bounds__(kThreads) void spec_walk_kernel(
    const int32_t* __restrict__ cand, const T* __restrict__ tl, const T* __restrict__ dl,
    const float* __restrict__ uni, const int32_t* __restrict__ prefix_len, int S, int V,
    const float2* __restrict__ stats, int n_chunks1, float ct, float cd, int chunk2,
    int n_chunks2, float2* __restrict__ csum, SpecWalk* __restrict__ walk, int32_t* accept_len,
    int32_t* commit_len, int32_t* out_tokens, int32_t* new_seq_len, SparseQ sq) {
  const int r = blockIdx.x, c = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int B = gridDim.x;
  const bool has_draft = dl != nullptr;
  __shared__ float2 st_t[64], st_d[64];  // (max, 1 / sum) per row of this request
  __shared__ SpecWalk sw;
  __shared__ float red[kThreads / 64];
  __shared__ float2 part[kMaxStatsPartials];

  // this request's stats partials into LDS in one coalesced pass (target rows
  // then draft rows, n_chunks1 per row), then one wave merges each row with a
  // fixed butterfly
  const int n_rows = has_draft ? 2 * S - 1 : S;
  {
    const float2* pt_ = stats + (int64_t)r * S * n_chunks1;
    const float2* pd_ = stats + ((int64_t)B * S + (int64_t)r * (S - 1)) * n_chunks1;
    const int nt = S * n_chunks1, nall = n_rows * n_chunks1;
    for (int k = tid; k < nall; k += kThreads) part[k] = (k < nt) ? pt_[k] : pd_[k - nt];
  }
  __syncthreads();
  for (int row = tid >> 6; row < n_rows; row += kThreads / 64) {
    const float sc = (row < S) ? ct : cd;
    float m = kNegInf, s = 0.f;
    if (lane < n_chunks1) {
      m = part[row * n_chunks1 + lane].x;
      s = part[row * n_chunks1 + lane].y;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
      lse_merge(m, s, m2, s2, sc);
    }
    if (lane == 0) {
      if (row < S)
        st_t[row] = make_float2(m, 1.f / s);
      else
        st_d[row - S] = make_float2(m, 1.f / s);
    }
  }
  __syncthreads();

  // the S-1 decisions at once; the first rejection ends the walk
  if (tid < 64) {
    bool reject = false;
    int y = 0;
    if (tid < S - 1) {
      y = min(max(cand[(int64_t)r * S + tid + 1], 0), V - 1);
      const float lt = ld1(tl + ((int64_t)r * S + tid) * V + y);
      float p, q = 1.f;
      {
#pragma clang fp contract(off)
        p = exp2f((lt - st_t[tid].x) * ct) * st_t[tid].y;
        if (has_draft) {
          const float ld = ld1(dl + ((int64_t)r * (S - 1) + tid) * V + y);
          q = exp2f((ld - st_d[tid].x) * cd) * st_d[tid].y;
        } else if (sq.K > 0) {
          const int64_t qr = ((int64_t)r * (S - 1) + tid) * sq.K;
          q = 0.f;
          for (int k = 0; k < sq.K; ++k) q += (sq.ids[qr + k] == y) ? sq.probs[qr + k] : 0.f;
        }
        reject = !(uni[(int64_t)r * S + tid] * q < p);
      }
    }
    const uint64_t mask = __ballot(reject);
    const int a = mask ? __builtin_ctzll(mask) : S - 1;
    if (tid == (a == S - 1 ? 0 : a)) {
      SpecWalk w;
      w.a = a;
      w.pad = 0;
      if (a == S - 1) {
        w.mode = 2;
        w.y = 0;
        w.mt = st_t[S - 1].x;
        w.izt = st_t[S - 1].y;
        w.md = 0.f;
        w.izd = 0.f;
      } else {
        w.mode = has_draft ? 0 : (sq.K > 0 ? 3 : 1);
        w.y = y;
        w.mt = st_t[a].x;
        w.izt = st_t[a].y;
        w.md = has_draft ? st_d[a].x : 0.f;
        w.izd = has_draft ? st_d[a].y : 0.f;
      }
      sw = w;
    }
  }
  __syncthreads();
  const SpecWalk w = sw;
  __shared__ int s_id[16];
  __shared__ float s_p[16];
  if (w.mode == 3 && tid < sq.K) {
    s_id[tid] = sq.ids[((int64_t)r * (S - 1) + w.a) * sq.K + tid];
    s_p[tid] = sq.probs[((int64_t)r * (S - 1) + w.a) * sq.K + tid];
  }
  __syncthreads();

  // weights of this chunk of the row the token is drawn from
  const int row_t = (w.mode == 2) ? S - 1 : w.a;
  const T* pt = tl + ((int64_t)r * S + row_t) * V;
  const T* pd = (w.mode == 0) ? dl + ((int64_t)r * (S - 1) + w.a) * V : nullptr;
  const int c0 = c * chunk2, c1 = min(V, c0 + chunk2);
  float sw_ = 0.f, sp = 0.f;
  for (int i = c0 + tid * VEC; i < c1; i += kThreads * VEC) {
    float vt[VEC], vd[VEC];
    VecLoad<T, VEC>::run(pt + i, vt);
    if (pd) {
      VecLoad<T, VEC>::run(pd + i, vd);
    } else {
#pragma unroll
      for (int k = 0; k < VEC; ++k) vd[k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
      sw_ += spec_weight(vt[k], vd[k], i + k, w, ct, cd, s_id, s_p, sq.K);
      sp += spec_p(vt[k], w, ct);
    }
  }
  sw_ = block_sum(sw_, red);
  sp = block_sum(sp, red);
  if (tid == 0) csum[(int64_t)r * n_chunks2 + c] = make_float2(sw_, sp);

  if (c == 0) {
    if (tid == 0) {
      walk[r] = w;
      accept_len[r] = w.a;
      commit_len[r] = w.a + 1;
      new_seq_len[r] = prefix_len[r] + w.a + 1;
    }
    if (tid < S && tid != w.a)
      out_tokens[(int64_t)r * S + tid] = (tid < w.a) ? cand[(int64_t)r * S + tid + 1] : 0;
  }
}

// ---------------------------------------------------------------- 3. pick
// Inclusive scan over the 64 lanes of a wave (fixed order).
__device__ __forceinline__ float wave_incl_scan(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// grid (B); 256 threads.
template <typename T, int VEC>
__global__ __launch_bounds__(kThreads) void spec_pick_kernel(
    const T* __restrict__ tl, const T* __restrict__ dl, const float* __restrict__ uni, int S,
    int V, float ct, float cd, int chunk2, int n_chunks2, const float2* __restrict__ csum,
    const SpecWalk* __restrict__ walk, int32_t* out_tokens, int32_t* next_anchor, SparseQ sq) {
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const SpecWalk w = walk[r];
  __shared__ float wl[kMaxChunk2];
  __shared__ int s_chunk, s_use_p;
  __shared__ float s_rem;
  __shared__ float wsum[kThreads / 64];
  __shared__ uint64_t wpos[kThreads / 64], wcross[kThreads / 64];
  __shared__ int s_tok;

  // chunk holding the draw (wave 0; n_chunks2 <= 64)
  if (tid < 64) {
    const float2 cs = (lane < n_chunks2) ? csum[(int64_t)r * n_chunks2 + lane]
                                         : make_float2(0.f, 0.f);
    const float tot_w = __shfl(wave_incl_scan(cs.x), 63, 64);
    const bool use_p = !(tot_w > 0.f);
    const float v = use_p ? cs.y : cs.x;
    const float incl = wave_incl_scan(v);
    const float tot = __shfl(incl, 63, 64);
    const float x = uni[(int64_t)r * S + S - 1] * tot;
    // ballots are wave-uniform: every lane finds the same chunk
    const uint64_t cross = __ballot(incl > x);
    const uint64_t pos = __ballot(v > 0.f);
    int ch;
    float rem;
    if (cross) {
      ch = __builtin_ctzll(cross);
      const float before = __shfl(incl, ch > 0 ? ch - 1 : 0, 64);  // chunks before ch
      rem = (ch > 0) ? x - before : x;
    } else {  // draw at the very top: the last chunk with weight, its last token
      ch = pos ? 63 - __builtin_clzll(pos) : 0;
      rem = __builtin_huge_valf();
    }
    if (lane == 0) {
      s_chunk = ch;
      s_use_p = use_p;
      s_rem = rem;
    }
  }
  __shared__ int s_id[16];
  __shared__ float s_p[16];
  if (w.mode == 3 && tid < sq.K) {
    s_id[tid] = sq.ids[((int64_t)r * (S - 1) + w.a) * sq.K + tid];
    s_p[tid] = sq.probs[((int64_t)r * (S - 1) + w.a) * sq.K + tid];
  }
  __syncthreads();
  const int ch = s_chunk;
  const bool use_p = s_use_p;
  const float rem = s_rem;

  // the chunk's weights into LDS (coalesced loads)
  const int row_t = (w.mode == 2) ? S - 1 : w.a;
  const T* pt = tl + ((int64_t)r * S + row_t) * V;
  const T* pd = (w.mode == 0) ? dl + ((int64_t)r * (S - 1) + w.a) * V : nullptr;
  const int c0 = ch * chunk2, c1 = min(V, c0 + chunk2);
  for (int i = c0 + tid * VEC; i < c1; i += kThreads * VEC) {
    float vt[VEC], vd[VEC];
    VecLoad<T, VEC>::run(pt + i, vt);
    if (pd) {
      VecLoad<T, VEC>::run(pd + i, vd);
    } else {
#pragma unroll
      for (int k = 0; k < VEC; ++k) vd[k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < VEC; ++k)
      wl[i - c0 + k] = use_p ? spec_p(vt[k], w, ct)
                             : spec_weight(vt[k], vd[k], i + k, w, ct, cd, s_id, s_p, sq.K);
  }
  __syncthreads();

  // per-thread contiguous runs of the chunk, scanned across the block
  const int n = c1 - c0;
  const int per = (n + kThreads - 1) / kThreads;
  const int r0 = min(n, tid * per), r1 = min(n, r0 + per);
  float s = 0.f;
  for (int i = r0; i < r1; ++i) s += wl[i];
  const float incl_w = wave_incl_scan(s);
  if (lane == 63) wsum[wv] = incl_w;
  const uint64_t posm = __ballot(s > 0.f);
  if (lane == 0) wpos[wv] = posm;
  __syncthreads();
  float off = 0.f;
  for (int k = 0; k < wv; ++k) off += wsum[k];
  const float incl = off + incl_w;
  const float prev = __shfl_up(incl_w, 1, 64);
  const float excl = (lane == 0) ? off : off + prev;
  const bool crosses = incl > rem && !(excl > rem);
  const uint64_t cm = __ballot(crosses);
  if (lane == 0) wcross[wv] = cm;
  if (tid == 0) s_tok = -1;
  __syncthreads();
  int owner = -1;
  bool last_positive = false;
  for (int k = 0; k < kThreads / 64 && owner < 0; ++k)
    if (wcross[k]) owner = 64 * k + __builtin_ctzll(wcross[k]);
  if (owner < 0) {  // no crossing (draw at the top): the last thread with weight
    last_positive = true;
    for (int k = kThreads / 64 - 1; k >= 0 && owner < 0; --k)
      if (wpos[k]) owner = 64 * k + 63 - __builtin_clzll(wpos[k]);
  }
  if (tid == owner) {
    int tok = -1, last = -1;
    float cum = excl;
    for (int i = r0; i < r1; ++i) {
      const float wi = wl[i];
      if (wi > 0.f) last = i;
      cum += wi;
      if (!last_positive && tok < 0 && cum > rem) tok = i;
    }
    s_tok = c0 + ((tok >= 0) ? tok : last);
  }
  __syncthreads();
  if (tid == 0) {
    const int tok = (s_tok >= c0) ? s_tok : 0;
    out_tokens[(int64_t)r * S + w.a] = tok;
    next_anchor[r] = tok;
  }
}

template <typename T, int VEC>
hipError_t spec_launch(const SparseQ& sq, const int32_t* cand, const void* tl_, const void* dl_,
                       const float* uni,
                       const int32_t* prefix_len, int B, int S, int V, float ct, float cd,
                       const SpecPlan& pl, void* ws, int32_t* accept_len, int32_t* commit_len,
                       int32_t* out_tokens, int32_t* next_anchor, int32_t* new_seq_len,
                       hipStream_t st) {
  const T* tl = static_cast<const T*>(tl_);
  const T* dl = static_cast<const T*>(dl_);
  char* p = static_cast<char*>(ws);
  float2* stats = reinterpret_cast<float2*>(p + pl.off_stats);
  float2* csum = reinterpret_cast<float2*>(p + pl.off_csum);
  SpecWalk* walk = reinterpret_cast<SpecWalk*>(p + pl.off_walk);
  hipLaunchKernelGGL((spec_stats_kernel<T, VEC>), dim3(pl.rows, pl.n_chunks1), dim3(kThreads), 0,
                     st, tl, dl, B * S, V, pl.chunk1, pl.n_chunks1, ct, cd, stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((spec_walk_kernel<T, VEC>), dim3(B, pl.n_chunks2), dim3(kThreads), 0, st,
                     cand, tl, dl, uni, prefix_len, S, V, stats, pl.n_chunks1, ct, cd, pl.chunk2,
                     pl.n_chunks2, csum, walk, accept_len, commit_len, out_tokens, new_seq_len, sq);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((spec_pick_kernel<T, VEC>), dim3(B), dim3(kThreads), 0, st, tl, dl, uni, S, V, ct,
                     cd, pl.chunk2, pl.n_chunks2, csum, walk, out_tokens, next_anchor, sq);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

SpecPlan plan_spec(int B, int S, int V, bool has_draft) {
  SpecPlan pl{};
  pl.rows = B * S + (has_draft ? B * (S - 1) : 0);
  // chunks are multiples of 64 logits (whole 16-byte vectors for either dtype)
  auto chunking = [&](int units, int target_wg, int& chunk, int& n) {
    int want = (target_wg + units - 1) / units;
    want = want < 1 ? 1 : (want > 64 ? 64 : want);
    chunk = (V + want - 1) / want;
    chunk = (chunk + 63) / 64 * 64;
    n = (V + chunk - 1) / chunk;
  };
  chunking(pl.rows, 2048, pl.chunk1, pl.n_chunks1);  // stats: ~2048 workgroups over all rows
  const int rows_per_req = has_draft ? 2 * S - 1 : S;
  while (pl.n_chunks1 > 1 && rows_per_req * pl.n_chunks1 > kMaxStatsPartials) {
    pl.chunk1 += 64;  // fewer, longer chunks until one request's partials fit in LDS
    pl.n_chunks1 = (V + pl.chunk1 - 1) / pl.chunk1;
  }
  chunking(B, 1024, pl.chunk2, pl.n_chunks2);        // weight sums: ~1024 over the batch
  if (pl.chunk2 > kMaxChunk2) {                      // the pick stages a chunk in LDS
    pl.chunk2 = kMaxChunk2;
    pl.n_chunks2 = (V + kMaxChunk2 - 1) / kMaxChunk2;  // <= 64 for V <= 64 * kMaxChunk2
  }
  size_t off = 0;
  pl.off_stats = off;
  off += align256(sizeof(float2) * (size_t)pl.rows * pl.n_chunks1);
  pl.off_csum = off;
  off += align256(sizeof(float2) * (size_t)B * pl.n_chunks2);
  pl.off_walk = off;
  off += align256(sizeof(SpecWalk) * (size_t)B);
  pl.bytes = off;
  return pl;
}

hipError_t launch_accept_sampling(int dt, int vec, const int32_t* cand, const void* tl,
                                  const void* dl, const int32_t* q_ids, const float* q_probs,
                                  int q_k, const float* uni, const int32_t* prefix_len, int B,
                                  int S, int V, float ct, float cd, const SpecPlan& pl, void* ws,
                                  int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens,
                                  int32_t* next_anchor, int32_t* new_seq_len, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  const SparseQ sq{q_ids, q_probs, q_ids != nullptr ? q_k : 0};
  if (dt == DFLASH_BF16) {
    if (vec > 1)
      return spec_launch<bf16_t, 8>(sq, cand, tl, dl, uni, prefix_len, B, S, V, ct, cd, pl, ws,
                                    accept_len, commit_len, out_tokens, next_anchor, new_seq_len,
                                    st);
    return spec_launch<bf16_t, 1>(sq, cand, tl, dl, uni, prefix_len, B, S, V, ct, cd, pl, ws,
                                  accept_len, commit_len, out_tokens, next_anchor, new_seq_len,
                                  st);
  }
  if (vec > 1)
    return spec_launch<float, 4>(sq, cand, tl, dl, uni, prefix_len, B, S, V, ct, cd, pl, ws,
                                 accept_len, commit_len, out_tokens, next_anchor, new_seq_len, st);
  return spec_launch<float, 1>(sq, cand, tl, dl, uni, prefix_len, B, S, V, ct, cd, pl, ws,
                               accept_len, commit_len, out_tokens, next_anchor, new_seq_len, st);
}

}  // namespace dflash
