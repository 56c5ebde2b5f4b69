// Small kernels of the draft/accept path: block preparation with the embedding
// gather and the RoPE table, row RMSNorm, the second argmax stage and greedy
// accept.
#include "common.h"
#include "internal.h"

namespace dflash {

__global__ void rope_table_kernel(const int32_t* __restrict__ pos, int rows, int D,
                                  double log_theta, float2* __restrict__ cs) {
  const int half = D / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * half) return;
  const int row = (int)(idx / half), i = (int)(idx % half);
  cs[idx] = rope_cs(pos[row], i, D, log_theta);
}

hipError_t launch_rope_table(const int32_t* positions, int rows, int D, float theta, float2* cs,
                             hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const int64_t n = (int64_t)rows * (D / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     positions, rows, D, log((double)theta), cs);
  return hipGetLastError();
}

// One workgroup per block row (r, j): ids / positions / slots, embedding
// gather into the fp32 residual stream with the row's sum of squares (for the
// first layer's input RMSNorm) and the row's RoPE table.
template <typename T>
__global__ __launch_bounds__(256) void block_prep_kernel(
    const T* __restrict__ embed, int V, int H, int S, int mask_id, int P, int D,
    double log_theta, const int32_t* __restrict__ anchor, const int32_t* __restrict__ prefix_len,
    const int32_t* __restrict__ pt, int max_pages, int32_t* block_ids, int32_t* positions,
    int32_t* slots, int32_t* candidates, float* __restrict__ x, float* __restrict__ ss, int n_ss,
    T* __restrict__ xg, int xg_blk, const T* __restrict__ g_first, float2* __restrict__ cs) {
  __shared__ float red[4];
  const int row = blockIdx.x, r = row / S, j = row % S, tid = threadIdx.x;
  int id = (j == 0) ? anchor[r] : mask_id;
  id = imin(imax(id, 0), V - 1);
  const int pos = prefix_len[r] + j;
  const int pidx = imax(pos / P, 0) % max_pages;  // the page table is a ring
  if (tid == 0) {
    if (block_ids != nullptr) block_ids[row] = (j == 0) ? anchor[r] : mask_id;
    positions[row] = pos;
    slots[row] = pt[(int64_t)r * max_pages + pidx] * P + pos % P;
    if (j == 0) candidates[(int64_t)r * S] = anchor[r];
  }
  // 8 consecutive columns per thread and pass: all loads of a pass issued
  // before any of its stores (H is a multiple of 32)
  const T* e = embed + (int64_t)id * H;
  float acc = 0.f;
  for (int c0 = tid * 8; c0 < H; c0 += 256 * 8) {
    Raw8<T> re, rg;
    re.load(e + c0);
    rg.load(g_first + c0);
    float v[8], g[8];
    re.to_f(v);
    rg.to_f(g);
    float* xo = x + (int64_t)row * H + c0;
    *reinterpret_cast<float4*>(xo) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(xo + 4) = make_float4(v[4], v[5], v[6], v[7]);
    T* go = xg + act_off(row, c0, H, xg_blk);  // 8 columns inside one 32-column block
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      go[i] = Num<T>::from_f(v[i] * g[i]);
      acc += v[i] * v[i];
    }
  }
  for (int i = tid; i < D / 2; i += 256) cs[(int64_t)row * (D / 2) + i] = rope_cs(pos, i, D, log_theta);
  acc = wave_sum(acc);
  if ((tid & 63) == 0) red[tid >> 6] = acc;
  __syncthreads();
  for (int t = tid; t < n_ss; t += 256)
    ss[(int64_t)row * n_ss + t] = (t == 0) ? (red[0] + red[1]) + (red[2] + red[3]) : 0.f;
}

hipError_t launch_block_prep(int dt, const dflash_config& c, const void* embed,
                             const int32_t* anchor, const int32_t* prefix_len,
                             const int32_t* page_table, int max_pages, int B, int32_t* block_ids,
                             int32_t* positions, int32_t* slots, int32_t* candidates, float* x,
                             float* ss, int n_ss, void* xg, int xg_blk, const void* g_first,
                             float2* cs, hipStream_t st) {
  const dim3 grid((unsigned)(B * c.block_size));
  const double lt = log((double)c.rope_theta);
  if (dt == DFLASH_BF16)
    hipLaunchKernelGGL(block_prep_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)embed,
                       c.vocab, c.hidden, c.block_size, c.mask_token_id, c.page_size, c.head_dim,
                       lt, anchor, prefix_len, page_table, max_pages, block_ids, positions, slots,
                       candidates, x, ss, n_ss, (bf16_t*)xg, xg_blk, (const bf16_t*)g_first, cs);
  else
    hipLaunchKernelGGL(block_prep_kernel<float>, grid, dim3(256), 0, st, (const float*)embed,
                       c.vocab, c.hidden, c.block_size, c.mask_token_id, c.page_size, c.head_dim,
                       lt, anchor, prefix_len, page_table, max_pages, block_ids, positions, slots,
                       candidates, x, ss, n_ss, (float*)xg, xg_blk, (const float*)g_first, cs);
  return hipGetLastError();
}

// Second argmax stage: one workgroup per logits row over the per-tile partials
// (value, first index); ties go to the lower index.  With S > 0 row m is block
// row (m / (S-1), 1 + m % (S-1)) of the [B, S] candidates; with S == 0 the id
// goes to out[m].
__global__ __launch_bounds__(256) void argmax_reduce_kernel(const float2* __restrict__ part,
                                                            int n_tiles, int S,
                                                            int32_t* __restrict__ candidates) {
  __shared__ float wv[4];
  __shared__ int wi[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float2* p = part + (int64_t)m * n_tiles;
  constexpr int U = 8;  // partials per thread and pass, all loaded before the compares
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int t0 = 0; t0 < n_tiles; t0 += 256 * U) {
    float2 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * 256 + tid;
      v[u] = t < n_tiles ? p[t] : make_float2(-INFINITY, __int_as_float(0x7fffffff));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pi = __float_as_int(v[u].y);
      if (v[u].x > best || (v[u].x == best && pi < bi)) {
        best = v[u].x;
        bi = pi;
      }
    }
  }
  // (value, lower index) is a total order: the reduction order does not matter
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > best || (ov == best && oi < bi)) {
      best = ov;
      bi = oi;
    }
  }
  if ((tid & 63) == 0) {
    wv[tid >> 6] = best;
    wi[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w)
      if (wv[w] > best || (wv[w] == best && wi[w] < bi)) {
        best = wv[w];
        bi = wi[w];
      }
    if (S > 0) {
      const int r = m / (S - 1), j = m % (S - 1);
      candidates[(int64_t)r * S + 1 + j] = bi;
    } else {
      candidates[m] = bi;
    }
  }
}

hipError_t launch_argmax_reduce(const float2* part, int M, int n_tiles, int S, int32_t* candidates,
                                hipStream_t st) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(M), dim3(256), 0, st, part, n_tiles, S,
                     candidates);
  return hipGetLastError();
}

// Greedy accept: one thread per request walks the block until the first
// mismatch between d_{a+1} and the target's choice after position a.
__global__ void accept_kernel(const int32_t* __restrict__ cand, const int32_t* __restrict__ post,
                              const int32_t* __restrict__ prefix_len, int B, int S,
                              int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens,
                              int32_t* next_anchor, int32_t* new_seq_len) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= B) return;
  const int32_t* c = cand + (int64_t)r * S;
  const int32_t* p = post + (int64_t)r * S;
  int a = 0;
  while (a < S - 1 && c[a + 1] == p[a]) ++a;
  int32_t* o = out_tokens + (int64_t)r * S;
  for (int j = 0; j < S; ++j) o[j] = (j < a) ? c[j + 1] : (j == a ? p[a] : 0);
  accept_len[r] = a;
  commit_len[r] = a + 1;
  next_anchor[r] = p[a];
  new_seq_len[r] = prefix_len[r] + a + 1;
}

hipError_t launch_accept(const int32_t* cand, const int32_t* post, const int32_t* prefix_len, int B,
                         int S, int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens,
                         int32_t* next_anchor, int32_t* new_seq_len, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(accept_kernel, dim3((B + 63) / 64), dim3(64), 0, st, cand, post, prefix_len,
                     B, S, accept_len, commit_len, out_tokens, next_anchor, new_seq_len);
  return hipGetLastError();
}

// ---- greedy accept from the target's logits ("Inside SGLang ...", Step 6:
// the target's choice after each block position is the argmax of its verify
// logits).  Row argmax in chunks of 16384 columns, one workgroup per (row,
// chunk): 256 threads x 8 runs of 8 consecutive columns (one 16-byte load per
// run of bf16, two of fp32; every load of the chunk issued before any compare,
// kept raw until then); NaN counts as -inf, ties go to the lower column.
// part[row * n_chunks + chunk] = (max, column bits).
template <typename T> struct ArgRuns {
  static constexpr int RUNS = 8;
  static constexpr int CHUNK = 256 * 8 * RUNS;  // columns per workgroup
};

__device__ __forceinline__ bool arg_better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void row_argmax_kernel(const T* __restrict__ x, int V,
                                                         int n_chunks, float2* __restrict__ part) {
  constexpr int RUNS = ArgRuns<T>::RUNS, CHUNK = ArgRuns<T>::CHUNK;
  __shared__ float rv[4];
  __shared__ int ri[4];
  const int row = blockIdx.x / n_chunks, ch = blockIdx.x % n_chunks, tid = threadIdx.x;
  const T* xr = x + (int64_t)row * V;
  const int c0 = ch * CHUNK;
  Raw8<T> raw[RUNS];
#pragma unroll
  for (int i = 0; i < RUNS; ++i) {
    const int col = c0 + (i * 256 + tid) * 8;
    if (VEC && col + 8 <= V) raw[i].load(xr + col);
  }
  float bv = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < RUNS; ++i) {
    const int col = c0 + (i * 256 + tid) * 8;
    float v[8];
    if (VEC && col + 8 <= V) {
      raw[i].to_f(v);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = col + k < V ? Num<T>::to_f(xr[col + k]) : -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float val = v[k] == v[k] ? v[k] : -INFINITY;
      if (col + k < V && arg_better(val, col + k, bv, bi)) {
        bv = val;
        bi = col + k;
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (arg_better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if ((tid & 63) == 0) {
    rv[tid >> 6] = bv;
    ri[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w)
      if (arg_better(rv[w], ri[w], bv, bi)) {
        bv = rv[w];
        bi = ri[w];
      }
    part[blockIdx.x] = make_float2(bv, __int_as_float(bi));
  }
}

// One wave per request: lane j < S merges row j's chunk partials in chunk
// order (the target's greedy token after position j); the first mismatch
// between d_{j+1} and that token (a ballot) ends the accepted prefix.
__global__ __launch_bounds__(64) void accept_logits_kernel(
    const int32_t* __restrict__ cand, const float2* __restrict__ part, int n_chunks,
    const int32_t* __restrict__ prefix_len, int S, int32_t* accept_len, int32_t* commit_len,
    int32_t* out_tokens, int32_t* next_anchor, int32_t* new_seq_len) {
  const int r = blockIdx.x, j = threadIdx.x;
  int post = 0;
  if (j < S) {
    const float2* p = part + ((int64_t)r * S + j) * n_chunks;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int c = 0; c < n_chunks; ++c) {
      const float2 q = p[c];
      if (arg_better(q.x, __float_as_int(q.y), bv, bi)) {
        bv = q.x;
        bi = __float_as_int(q.y);
      }
    }
    post = bi;
  }
  const int32_t* c = cand + (int64_t)r * S;
  const uint64_t mism = __ballot(j < S - 1 && c[j < S - 1 ? j + 1 : 0] != post);
  const int a = mism ? __ffsll((unsigned long long)mism) - 1 : S - 1;
  const int pa = __shfl(post, a, 64);
  if (j < S) out_tokens[(int64_t)r * S + j] = j < a ? c[j + 1] : (j == a ? pa : 0);
  if (j == 0) {
    accept_len[r] = a;
    commit_len[r] = a + 1;
    next_anchor[r] = pa;
    new_seq_len[r] = prefix_len[r] + a + 1;
  }
}

int accept_logits_chunks(int V) {
  return (V + ArgRuns<float>::CHUNK - 1) / ArgRuns<float>::CHUNK;
}

hipError_t launch_accept_logits(int dt, const void* logits, int V, bool vec, const int32_t* cand,
                                const int32_t* prefix_len, int B, int S, float2* part,
                                int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens,
                                int32_t* next_anchor, int32_t* new_seq_len, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  const int chunk = dt == DFLASH_BF16 ? ArgRuns<bf16_t>::CHUNK : ArgRuns<float>::CHUNK;
  const int nc = (V + chunk - 1) / chunk;
  const dim3 grid((unsigned)((int64_t)B * S * nc));
  if (dt == DFLASH_BF16) {
    const bf16_t* x = static_cast<const bf16_t*>(logits);
    if (vec) hipLaunchKernelGGL((row_argmax_kernel<bf16_t, true>), grid, dim3(256), 0, st, x, V, nc, part);
    else hipLaunchKernelGGL((row_argmax_kernel<bf16_t, false>), grid, dim3(256), 0, st, x, V, nc, part);
  } else {
    const float* x = static_cast<const float*>(logits);
    if (vec) hipLaunchKernelGGL((row_argmax_kernel<float, true>), grid, dim3(256), 0, st, x, V, nc, part);
    else hipLaunchKernelGGL((row_argmax_kernel<float, false>), grid, dim3(256), 0, st, x, V, nc, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_logits_kernel, dim3(B), dim3(64), 0, st, cand, part, nc, prefix_len, S,
                     accept_len, commit_len, out_tokens, next_anchor, new_seq_len);
  return hipGetLastError();
}

}  // namespace dflash
