// Weight-streaming MFMA GEMM for gfx950 with fused epilogues.
//
// C[M, Ncols] = A[M, K] * W[Ncols, K]^T, W row-major [out, in] (the layout of
// every projection of the draft model).  One workgroup (4 waves, 256 threads)
// owns a 16*MB x 128 output tile and one K range of a split-K decomposition;
// each wave owns 32 columns (two 16-column MFMA blocks) for all 16*MB rows,
// so every weight fragment a lane loads from HBM feeds MB MFMAs straight from
// registers.  A rows (the small activation matrix) come through L1/L2.
//
// After the K loop the fp32 tile is assembled in LDS (summing the split-K
// partials of the other workgroups in a fixed order when K is split, so the
// result is deterministic) and handed to an epilogue that sees whole rows of
// the 128-column tile: a full attention head for the q/k RMSNorm + RoPE of the
// QKV and K/V-injection epilogues, paired gate/up columns for SwiGLU, a
// 128-wide vocabulary slice for the argmax partials of lm_head.
#include "common.cuh"
#include "internal.h"

namespace dflash {

constexpr int BN = 128;      // output columns per workgroup tile
constexpr int LDT = BN + 4;  // LDS tile row stride in floats (bank-conflict padding)

GemmPlan plan_gemm(int M, int Ncols, int K) {
  GemmPlan p;
  p.MB = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.m_tiles = (M + 16 * p.MB - 1) / (16 * p.MB);
  p.n_tiles = (Ncols + BN - 1) / BN;
  int ks = 1;
  if (M <= 64) {
    // Split K so that the grid reaches ~512 workgroups.  The split depends on
    // (Ncols, K) only, so the same rows give the same bits at any M <= 64.
    ks = (512 + p.n_tiles - 1) / p.n_tiles;
    ks = ks < K / 256 ? ks : K / 256;
  } else {
    const int base = p.n_tiles * p.m_tiles;
    ks = (512 + base - 1) / base;
    ks = ks < K / 512 ? ks : K / 512;
  }
  if (ks < 1) ks = 1;
  int kc = (K + ks - 1) / ks;
  kc = (kc + 31) / 32 * 32;
  p.Kc = kc;
  p.KS = (K + kc - 1) / kc;
  return p;
}

size_t gemm_partial_floats(const GemmPlan& p) {
  if (p.KS <= 1) return 0;
  return (size_t)p.KS * p.m_tiles * p.n_tiles * 16 * p.MB * BN;
}

int logits_tiles(int V) { return (V + BN - 1) / BN; }

// ---------------------------------------------------------------- main kernel
template <typename T, int MB, class Epi>
__global__ __launch_bounds__(256) void gemm_stream(const T* __restrict__ A, int64_t lda, int M,
                                                   int K, int KS, int Kc, int m_tiles,
                                                   float* __restrict__ partial,
                                                   int* __restrict__ counters, Epi epi) {
  __shared__ float tile[16 * MB * LDT];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bid = blockIdx.x;
  const int ks = bid % KS;
  const int rest = bid / KS;
  const int mt = rest % m_tiles;
  const int nt = rest / m_tiles;
  const int m0 = mt * 16 * MB;
  const int k0 = ks * Kc;
  const int k1 = imin(K, k0 + Kc);
  const int r16 = lane & 15, g4 = lane >> 4;

  const T* bp[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) bp[nb] = epi.brow(nt, wave * 32 + nb * 16 + r16);
  const T* ap[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) ap[mb] = A + (int64_t)imin(m0 + mb * 16 + r16, M - 1) * lda;

  f32x4 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  int k = k0;
  // 64-wide steps: each lane reads 16 consecutive K elements per row (lanes
  // with the same l % 16 cover one contiguous 64-element span of that row).
  for (; k + 64 <= k1; k += 64) {
    const int kk = k + g4 * 16;
    Frag<T> b0[2], b1[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      load_frag(b0[nb], bp[nb] + kk);
      load_frag(b1[nb], bp[nb] + kk + 8);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      Frag<T> a0, a1;
      load_frag(a0, ap[mb] + kk);
      load_frag(a1, ap[mb] + kk + 8);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        mma(acc[mb][nb], a0, b0[nb]);
        mma(acc[mb][nb], a1, b1[nb]);
      }
    }
  }
  if (k < k1) {  // 32-wide tail
    const int kk = k + g4 * 8;
    Frag<T> b0[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) load_frag(b0[nb], bp[nb] + kk);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      Frag<T> a0;
      load_frag(a0, ap[mb] + kk);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) mma(acc[mb][nb], a0, b0[nb]);
    }
  }

  if (KS == 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          tile[(mb * 16 + g4 * 4 + i) * LDT + wave * 32 + nb * 16 + r16] = acc[mb][nb][i];
    __syncthreads();
    epi.apply(tile, 16 * MB, m0, M, nt, tid);
    return;
  }

  const int tile_elems = 16 * MB * BN;
  const int tix = nt * m_tiles + mt;
  float* base = partial + (int64_t)tix * KS * tile_elems;
  float* mine = base + (int64_t)ks * tile_elems;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mine[(mb * 16 + g4 * 4 + i) * BN + wave * 32 + nb * 16 + r16] = acc[mb][nb][i];
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&counters[tix], 1) == KS - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int idx = tid; idx < tile_elems; idx += 256) {
    float s = 0.f;
    for (int q = 0; q < KS; ++q) s += __builtin_nontemporal_load(base + (int64_t)q * tile_elems + idx);
    tile[(idx / BN) * LDT + idx % BN] = s;
  }
  if (tid == 0) counters[tix] = 0;
  __syncthreads();
  epi.apply(tile, 16 * MB, m0, M, nt, tid);
}

// ---------------------------------------------------------------- epilogues
template <typename T> struct EpiStoreF32 {
  const T* W; int N; int K; float* out; int ldo;
  __device__ const T* brow(int nt, int c) const {
    return W + (int64_t)imin(nt * BN + c, N - 1) * K;
  }
  __device__ void apply(const float* t, int rows, int m0, int M, int nt, int tid) const {
    for (int idx = tid; idx < rows * BN; idx += 256) {
      const int r = idx / BN, c = idx % BN, m = m0 + r, n = nt * BN + c;
      if (m < M && n < N) out[(int64_t)m * ldo + n] = t[r * LDT + c];
    }
  }
};

template <typename T> struct EpiResidual {
  const T* W; int N; int K; float* x;
  __device__ const T* brow(int nt, int c) const {
    return W + (int64_t)imin(nt * BN + c, N - 1) * K;
  }
  __device__ void apply(const float* t, int rows, int m0, int M, int nt, int tid) const {
    for (int idx = tid; idx < rows * BN; idx += 256) {
      const int r = idx / BN, c = idx % BN, m = m0 + r, n = nt * BN + c;
      if (m < M && n < N) x[(int64_t)m * N + n] += t[r * LDT + c];
    }
  }
};

// Tile columns 0..63 are gate rows nt*64.., columns 64..127 the matching up rows.
template <typename T> struct EpiSiluMul {
  const T* Wg; const T* Wu; int I; int K; T* act;
  __device__ const T* brow(int nt, int c) const {
    const int n = imin(nt * 64 + (c & 63), I - 1);
    return (c < 64 ? Wg : Wu) + (int64_t)n * K;
  }
  __device__ void apply(const float* t, int rows, int m0, int M, int nt, int tid) const {
    for (int idx = tid; idx < rows * 64; idx += 256) {
      const int r = idx / 64, c = idx % 64, m = m0 + r, n = nt * 64 + c;
      if (m < M && n < I) {
        const float g = t[r * LDT + c], u = t[r * LDT + 64 + c];
        act[(int64_t)m * I + n] = Num<T>::from_f(g / (1.0f + __expf(-g)) * u);
      }
    }
  }
};

// Per-head RMSNorm (gain g) followed by neox RoPE with the row's (cos, sin)
// table; lane i < D/2 owns the pair (i, i + D/2).  Returns the rotated pair.
template <typename T>
__device__ __forceinline__ void norm_rope_pair(float x0, float x1, int i, int D, bool active,
                                               const T* g, float eps, const float2* cs_row,
                                               float& o0, float& o1) {
  const float ss = wave_sum(active ? x0 * x0 + x1 * x1 : 0.f);
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
  if (!active) return;
  const float y0 = x0 * inv * Num<T>::to_f(g[i]);
  const float y1 = x1 * inv * Num<T>::to_f(g[i + D / 2]);
  const float2 c = cs_row[i];
  o0 = y0 * c.x - y1 * c.y;
  o1 = y1 * c.x + y0 * c.y;
}

template <typename T> struct EpiQKV {
  const T* W; int H; int nq, nkv, D; const T* qn; const T* kn; float eps;
  const float2* cs; T* q; T* k; T* v;
  __device__ const T* brow(int nt, int c) const {
    return W + (int64_t)imin(nt * BN + c, (nq + 2 * nkv) * D - 1) * H;
  }
  __device__ void apply(const float* t, int rows, int m0, int M, int nt, int tid) const {
    const int lane = tid & 63, wave = tid >> 6;
    const int HP = BN / D, half = D / 2;
    for (int item = wave; item < rows * HP; item += 4) {
      const int r = item / HP, hh = item % HP, m = m0 + r, gh = nt * HP + hh;
      if (m >= M || gh >= nq + 2 * nkv) continue;
      const bool act = lane < half;
      const float x0 = act ? t[r * LDT + hh * D + lane] : 0.f;
      const float x1 = act ? t[r * LDT + hh * D + lane + half] : 0.f;
      float o0 = x0, o1 = x1;
      T* dst;
      if (gh < nq) {
        norm_rope_pair<T>(x0, x1, lane, D, act, qn, eps, cs + (int64_t)m * half, o0, o1);
        dst = q + ((int64_t)m * nq + gh) * D;
      } else if (gh < nq + nkv) {
        norm_rope_pair<T>(x0, x1, lane, D, act, kn, eps, cs + (int64_t)m * half, o0, o1);
        dst = k + ((int64_t)m * nkv + (gh - nq)) * D;
      } else {
        dst = v + ((int64_t)m * nkv + (gh - nq - nkv)) * D;
      }
      if (act) {
        dst[lane] = Num<T>::from_f(o0);
        dst[lane + half] = Num<T>::from_f(o1);
      }
    }
  }
};

// Stacked K/V rows of every layer: column n -> layer n / (2 nkv D), then the
// k rows and v rows of that layer's w_qkv (which start after the nq*D q rows).
template <typename T, typename KT> struct EpiKVInject {
  KVTargets tg; int H; int n_layers, nq, nkv, D; float eps; const float2* cs;
  const int32_t* slots; const int32_t* valid; int rpr; int P; int64_t num_slots;
  __device__ const T* brow(int nt, int c) const {
    const int per = 2 * nkv * D;
    const int n = imin(nt * BN + c, n_layers * per - 1);
    const int l = n / per, w = n % per;
    return static_cast<const T*>(tg.w_qkv[l]) + (int64_t)(nq * D + w) * H;
  }
  __device__ void apply(const float* t, int rows, int m0, int M, int nt, int tid) const {
    const int lane = tid & 63, wave = tid >> 6;
    const int HP = BN / D, half = D / 2;
    for (int item = wave; item < rows * HP; item += 4) {
      const int r = item / HP, hh = item % HP, m = m0 + r, gh = nt * HP + hh;
      if (m >= M || gh >= n_layers * 2 * nkv) continue;
      if (valid != nullptr && (m % rpr) >= valid[m / rpr]) continue;
      const int l = gh / (2 * nkv), rem = gh % (2 * nkv);
      const bool is_v = rem >= nkv;
      const int head = rem % nkv;
      const bool act = lane < half;
      const float x0 = act ? t[r * LDT + hh * D + lane] : 0.f;
      const float x1 = act ? t[r * LDT + hh * D + lane + half] : 0.f;
      float o0 = x0, o1 = x1;
      if (!is_v)
        norm_rope_pair<T>(x0, x1, lane, D, act, static_cast<const T*>(tg.k_norm[l]), eps,
                          cs + (int64_t)m * half, o0, o1);
      const int64_t slot = slots[m];
      if (slot < 0 || slot >= num_slots) continue;  // outside the pool: never written
      const int64_t page = slot / P, off = slot % P;
      KT* dst = static_cast<KT*>(is_v ? tg.vc[l] : tg.kc[l]) + ((page * nkv + head) * P + off) * D;
      if (act) {
        dst[lane] = Num<KT>::from_f(o0);
        dst[lane + half] = Num<KT>::from_f(o1);
      }
    }
  }
};

// Logits of a 128-wide vocabulary slice: rounded to T (and stored when asked),
// then the (max, first index) of every row over the slice.
template <typename T> struct EpiLogits {
  const T* W; int V; int H; T* logits; float2* part; int n_tiles;
  __device__ const T* brow(int nt, int c) const {
    return W + (int64_t)imin(nt * BN + c, V - 1) * H;
  }
  __device__ void apply(const float* t, int rows, int m0, int M, int nt, int tid) const {
    const int lane = tid & 63, wave = tid >> 6;
    for (int r = wave; r < rows; r += 4) {
      const int m = m0 + r;
      if (m >= M) continue;
      float best = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = lane + 64 * h, n = nt * BN + c;
        if (n < V) {
          const T tv = Num<T>::from_f(t[r * LDT + c]);
          if (logits != nullptr) logits[(int64_t)m * V + n] = tv;
          float v = Num<T>::to_f(tv);
          if (!(v == v)) v = -INFINITY;
          if (v > best || (v == best && n < bi)) {
            best = v;
            bi = n;
          }
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > best || (ov == best && oi < bi)) {
          best = ov;
          bi = oi;
        }
      }
      if (lane == 0) part[(int64_t)m * n_tiles + nt] = make_float2(best, __int_as_float(bi));
    }
  }
};

// ---------------------------------------------------------------- launchers
template <typename T, class Epi>
static hipError_t run_gemm(const T* A, int64_t lda, int M, int K, int Ncols, const Epi& epi,
                           const GemmScratch& ws, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const GemmPlan p = plan_gemm(M, Ncols, K);
  if (p.KS > 1 && (gemm_partial_floats(p) > ws.partial_floats ||
                   p.n_tiles * p.m_tiles > ws.n_counters))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.n_tiles * p.m_tiles * p.KS));
  switch (p.MB) {
    case 1:
      hipLaunchKernelGGL((gemm_stream<T, 1, Epi>), grid, dim3(256), 0, st, A, lda, M, K, p.KS,
                         p.Kc, p.m_tiles, ws.partial, ws.counters, epi);
      break;
    case 2:
      hipLaunchKernelGGL((gemm_stream<T, 2, Epi>), grid, dim3(256), 0, st, A, lda, M, K, p.KS,
                         p.Kc, p.m_tiles, ws.partial, ws.counters, epi);
      break;
    default:
      hipLaunchKernelGGL((gemm_stream<T, 4, Epi>), grid, dim3(256), 0, st, A, lda, M, K, p.KS,
                         p.Kc, p.m_tiles, ws.partial, ws.counters, epi);
      break;
  }
  return hipGetLastError();
}

hipError_t gemm_store_f32(int dt, const void* A, int64_t lda, int M, int K, const void* W, int N,
                          float* out, const GemmScratch& ws, hipStream_t st) {
  if (dt == DFLASH_BF16) {
    EpiStoreF32<bf16_t> e{(const bf16_t*)W, N, K, out, N};
    return run_gemm((const bf16_t*)A, lda, M, K, N, e, ws, st);
  }
  EpiStoreF32<float> e{(const float*)W, N, K, out, N};
  return run_gemm((const float*)A, lda, M, K, N, e, ws, st);
}

hipError_t gemm_residual(int dt, const void* A, int M, int K, const void* W, int N, float* x,
                         const GemmScratch& ws, hipStream_t st) {
  if (dt == DFLASH_BF16) {
    EpiResidual<bf16_t> e{(const bf16_t*)W, N, K, x};
    return run_gemm((const bf16_t*)A, K, M, K, N, e, ws, st);
  }
  EpiResidual<float> e{(const float*)W, N, K, x};
  return run_gemm((const float*)A, K, M, K, N, e, ws, st);
}

hipError_t gemm_silu_mul(int dt, const void* A, int M, int K, const void* Wg, const void* Wu,
                         int I, void* act, const GemmScratch& ws, hipStream_t st) {
  const int ncols = ((I + 63) / 64) * BN;
  if (dt == DFLASH_BF16) {
    EpiSiluMul<bf16_t> e{(const bf16_t*)Wg, (const bf16_t*)Wu, I, K, (bf16_t*)act};
    return run_gemm((const bf16_t*)A, K, M, K, ncols, e, ws, st);
  }
  EpiSiluMul<float> e{(const float*)Wg, (const float*)Wu, I, K, (float*)act};
  return run_gemm((const float*)A, K, M, K, ncols, e, ws, st);
}

hipError_t gemm_qkv(int dt, const void* A, int M, int H, const void* Wqkv, const void* qn,
                    const void* kn, int nq, int nkv, int D, float eps, const float2* cs, void* q,
                    void* k, void* v, const GemmScratch& ws, hipStream_t st) {
  const int ncols = (nq + 2 * nkv) * D;
  if (dt == DFLASH_BF16) {
    EpiQKV<bf16_t> e{(const bf16_t*)Wqkv, H, nq, nkv, D, (const bf16_t*)qn, (const bf16_t*)kn,
                     eps, cs, (bf16_t*)q, (bf16_t*)k, (bf16_t*)v};
    return run_gemm((const bf16_t*)A, H, M, H, ncols, e, ws, st);
  }
  EpiQKV<float> e{(const float*)Wqkv, H, nq, nkv, D, (const float*)qn, (const float*)kn, eps, cs,
                  (float*)q, (float*)k, (float*)v};
  return run_gemm((const float*)A, H, M, H, ncols, e, ws, st);
}

hipError_t gemm_kv_inject(int dt, int kv_dt, const void* A, int M, int H, const KVTargets& t,
                          int n_layers, int nq, int nkv, int D, float eps, const float2* cs,
                          const int32_t* slots, const int32_t* valid_rows, int rows_per_req,
                          int page_size, int64_t num_pages, const GemmScratch& ws,
                          hipStream_t st) {
  const int64_t ns = num_pages * page_size;
  const int ncols = n_layers * 2 * nkv * D;
  if (dt == DFLASH_BF16) {
    const bf16_t* a = (const bf16_t*)A;
    if (kv_dt == DFLASH_FP8_E4M3) {
      EpiKVInject<bf16_t, fp8_t> e{t, H, n_layers, nq, nkv, D, eps, cs, slots, valid_rows,
                                   rows_per_req, page_size, ns};
      return run_gemm(a, H, M, H, ncols, e, ws, st);
    }
    EpiKVInject<bf16_t, bf16_t> e{t, H, n_layers, nq, nkv, D, eps, cs, slots, valid_rows,
                                  rows_per_req, page_size, ns};
    return run_gemm(a, H, M, H, ncols, e, ws, st);
  }
  EpiKVInject<float, float> e{t, H, n_layers, nq, nkv, D, eps, cs, slots, valid_rows,
                              rows_per_req, page_size, ns};
  return run_gemm((const float*)A, H, M, H, ncols, e, ws, st);
}

hipError_t gemm_logits(int dt, const void* A, int M, int H, const void* Wlm, int V, void* logits,
                       float2* part, const GemmScratch& ws, hipStream_t st) {
  const int nt = logits_tiles(V);
  if (dt == DFLASH_BF16) {
    EpiLogits<bf16_t> e{(const bf16_t*)Wlm, V, H, (bf16_t*)logits, part, nt};
    return run_gemm((const bf16_t*)A, H, M, H, V, e, ws, st);
  }
  EpiLogits<float> e{(const float*)Wlm, V, H, (float*)logits, part, nt};
  return run_gemm((const float*)A, H, M, H, V, e, ws, st);
}

}  // namespace dflash
