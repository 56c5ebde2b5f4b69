// Non-causal block attention over a paged context cache, split over the
// context keys (flash-decoding style) with a log-sum-exp combine.
//
// For one request r and kv head g the G = nq / nkv query heads of the S block
// rows form R = G * S <= 64 query rows (row rho = h_local * S + j); each of the
// 4 waves of a workgroup owns 16 of them.  A workgroup walks one range of
// context keys in 32-key tiles (each key's page looked up in the page table),
// staging K row-major and V transposed in LDS so that Q K^T and P V are both
// 16x16x32 bf16 MFMAs (8 fp32 MFMAs per K step for fp32 models), with an online
// softmax in the exp2 domain.  Split 0 also takes the S block keys, which every
// block row sees (no causal mask).  On a sliding layer context key i is visible
// to the row at logical position p iff p - i < W; the range starts at
// L - W + 1, the first key the anchor row can see.  fp8 caches are decoded to
// bf16 while staging.
#include "common.cuh"
#include "internal.h"

namespace dflash {

constexpr float LOG2E = 1.4426950408889634f;

AttnPlan plan_attention(int max_keys, int B, int nkv) {
  AttnPlan p;
  const int64_t work = (int64_t)max_keys * B * nkv;
  int chunk = (int)((work / 1024 + 31) / 32 * 32);
  if (chunk < 256) chunk = 256;
  p.chunk = chunk;
  p.n_splits = max_keys <= 0 ? 1 : (max_keys + chunk - 1) / chunk;
  return p;
}

struct AttnArgs {
  const void* q; const void* kb; const void* vb;  // block q [M, nq, D], k/v [M, nkv, D]
  const void* kc; const void* vc;                  // paged cache of this layer
  const int32_t* pt; int max_pages; int64_t num_pages;
  const int32_t* prefix_len; int max_prefix;
  int S, G, nq, nkv, P, window, chunk, n_splits;
  float scale_log2;
  float* o_part; float2* ml_part;
};

__device__ __forceinline__ void load8(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t* p, float* o) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xffffu));
    o[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
  }
}
__device__ __forceinline__ void load8(const fp8_t* p, float* o) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  const uint32_t w[2] = {u.x, u.y};
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = e4m3_to_f32((uint8_t)((w[i >> 2] >> (8 * (i & 3))) & 0xffu));
}

// Context-key range of request r on this layer and the number of splits it uses.
__device__ __forceinline__ void key_range(const AttnArgs& a, int r, int& L, int& lo, int& nvalid) {
  L = imin(imax(a.prefix_len[r], 0), imin(a.max_prefix, a.max_pages * a.P));
  lo = a.window > 0 ? imax(0, L - a.window + 1) : 0;
  nvalid = imax(1, (L - lo + a.chunk - 1) / a.chunk);
}

template <typename CT, typename KT, int D>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
  constexpr int KP = D + 8;   // K tile row stride (elements)
  constexpr int VP = 32 + 8;  // V^T and P row stride (elements)
  __shared__ CT Ks[32 * KP];
  __shared__ CT Vt[D * VP];
  __shared__ CT Ps[4 * 16 * VP];

  const int split = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  int L, lo, nvalid;
  key_range(a, r, L, lo, nvalid);
  if (split >= nvalid) return;
  const int kbeg = lo + split * a.chunk;
  const int kend = imin(L, kbeg + a.chunk);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int S = a.S, R = a.G * S;

  // Q fragments of this wave's 16 rows (A operand: row r16, K group g4).
  Frag<CT> qf[D / 32];
  {
    const int rho = imin(w * 16 + r16, R - 1);
    const int hl = rho / S, j = rho % S;
    const CT* qp = static_cast<const CT*>(a.q) + ((int64_t)(r * S + j) * a.nq + g * a.G + hl) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) load_frag(qf[ks], qp + ks * 32 + g4 * 8);
  }
  // logical position of the 4 accumulator rows this lane holds
  int qpos[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) qpos[i] = L + (imin(w * 16 + g4 * 4 + i, R - 1) % S);

  float mrow[4], lrow[4];
  f32x4 o[D / 16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mrow[i] = -INFINITY;
    lrow[i] = 0.f;
  }
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_ctx_tiles = (kend > kbeg) ? (kend - kbeg + 31) / 32 : 0;
  const int n_tiles = n_ctx_tiles + (split == 0 ? 1 : 0);
  for (int t = 0; t < n_tiles; ++t) {
    const bool is_blk = t == n_ctx_tiles;
    const int t0 = is_blk ? 0 : kbeg + t * 32;
    const int nk = is_blk ? S : imin(32, kend - t0);
    __syncthreads();
    for (int c = tid; c < 32 * (D / 8); c += 256) {
      const int kk = c / (D / 8), d0 = (c % (D / 8)) * 8;
      float kv[8], vv[8];
      if (kk < nk) {
        if (is_blk) {
          const int64_t off = ((int64_t)(r * S + kk) * a.nkv + g) * D + d0;
          load8(static_cast<const CT*>(a.kb) + off, kv);
          load8(static_cast<const CT*>(a.vb) + off, vv);
        } else {
          const int i = t0 + kk;
          int64_t page = a.pt[(int64_t)r * a.max_pages + i / a.P];
          page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
          const int64_t off = ((page * a.nkv + g) * a.P + i % a.P) * D + d0;
          load8(static_cast<const KT*>(a.kc) + off, kv);
          load8(static_cast<const KT*>(a.vc) + off, vv);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kv[e] = vv[e] = 0.f;
      }
      Frag<CT> kf;
      frag_from_f32(kf, kv);
      store_frag(&Ks[kk * KP + d0], kf);
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[(d0 + e) * VP + kk] = Num<CT>::from_f(vv[e]);
    }
    __syncthreads();

    f32x4 sacc[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      sacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        Frag<CT> kf;
        load_frag(kf, &Ks[(cb * 16 + r16) * KP + ks * 32 + g4 * 8]);
        mma(sacc[cb], qf[ks], kf);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int key = cb * 16 + r16;
        bool ok = key < nk;
        if (ok && !is_blk && a.window > 0) ok = (qpos[i] - (t0 + key)) < a.window;
        s[cb] = ok ? sacc[cb][i] * a.scale_log2 : -INFINITY;
      }
      const float mt = row16_max(fmaxf(s[0], s[1]));
      const float mn = fmaxf(mrow[i], mt);
      const float alpha = (mrow[i] == -INFINITY) ? 0.f : exp2f(mrow[i] - mn);
      float p[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) p[cb] = (s[cb] == -INFINITY) ? 0.f : exp2f(s[cb] - mn);
      lrow[i] = lrow[i] * alpha + row16_sum(p[0] + p[1]);
      mrow[i] = mn;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) o[nb][i] *= alpha;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        Ps[(w * 16 + g4 * 4 + i) * VP + cb * 16 + r16] = Num<CT>::from_f(p[cb]);
    }
    __syncthreads();
    Frag<CT> pf;
    load_frag(pf, &Ps[(w * 16 + r16) * VP + g4 * 8]);
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
      Frag<CT> vf;
      load_frag(vf, &Vt[(nb * 16 + r16) * VP + g4 * 8]);
      mma(o[nb], pf, vf);
    }
  }

  const int64_t base = ((int64_t)(r * a.nkv + g) * a.n_splits + split) * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rho = w * 16 + g4 * 4 + i;
    if (rho >= R) continue;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) a.o_part[(base + rho) * D + nb * 16 + r16] = o[nb][i];
    if (r16 == 0) a.ml_part[base + rho] = make_float2(mrow[i], lrow[i]);
  }
}

// Combine the splits of one query row: one wave per row.
template <typename CT, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, CT* __restrict__ out,
                                                           int B) {
  const int R = a.G * a.S;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= B * a.nkv * R) return;
  const int rho = row % R, g = (row / R) % a.nkv, r = row / (R * a.nkv);
  int L, lo, nvalid;
  key_range(a, r, L, lo, nvalid);
  const int64_t base = ((int64_t)(r * a.nkv + g) * a.n_splits) * 64 + rho;
  float M = -INFINITY;
  for (int s = 0; s < nvalid; ++s) M = fmaxf(M, a.ml_part[base + (int64_t)s * 64].x);
  float den = 0.f, acc[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) acc[e] = 0.f;
  for (int s = 0; s < nvalid; ++s) {
    const float2 ml = a.ml_part[base + (int64_t)s * 64];
    const float wgt = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
    den += wgt * ml.y;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) acc[e] += wgt * a.o_part[(base + (int64_t)s * 64) * D + lane + 64 * e];
  }
  const int hl = rho / a.S, j = rho % a.S;
  CT* dst = out + ((int64_t)(r * a.S + j) * a.nq + g * a.G + hl) * D;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) dst[lane + 64 * e] = Num<CT>::from_f(acc[e] / den);
}

template <typename CT, typename KT, int D>
static hipError_t run_attn(const AttnArgs& a, int B, void* out, hipStream_t st) {
  hipLaunchKernelGGL((attn_split_kernel<CT, KT, D>), dim3(a.n_splits, a.nkv, B), dim3(256), 0, st,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = B * a.nkv * a.G * a.S;
  hipLaunchKernelGGL((attn_combine_kernel<CT, D>), dim3((rows + 3) / 4), dim3(256), 0, st, a,
                     (CT*)out, B);
  return hipGetLastError();
}

hipError_t launch_attention(int dt, int kv_dt, int D, const void* q, const void* kb,
                             const void* vb, const void* kc, const void* vc,
                             const int32_t* page_table, int max_pages, int64_t num_pages,
                             const int32_t* prefix_len, int max_prefix, int B, int S, int nq, int nkv, int page_size,
                             int window, const AttnPlan& plan, float* o_part, float2* ml_part,
                             void* out, hipStream_t st) {
  AttnArgs a;
  a.q = q; a.kb = kb; a.vb = vb; a.kc = kc; a.vc = vc;
  a.pt = page_table; a.max_pages = max_pages; a.num_pages = num_pages;
  a.prefix_len = prefix_len; a.max_prefix = max_prefix;
  a.S = S; a.G = nq / nkv; a.nq = nq; a.nkv = nkv; a.P = page_size; a.window = window;
  a.chunk = plan.chunk; a.n_splits = plan.n_splits;
  a.scale_log2 = LOG2E / sqrtf((float)D);
  a.o_part = o_part; a.ml_part = ml_part;
  if (dt == DFLASH_F32) {
    if (D == 64) return run_attn<float, float, 64>(a, B, out, st);
    return run_attn<float, float, 128>(a, B, out, st);
  }
  if (kv_dt == DFLASH_FP8_E4M3) {
    if (D == 64) return run_attn<bf16_t, fp8_t, 64>(a, B, out, st);
    return run_attn<bf16_t, fp8_t, 128>(a, B, out, st);
  }
  if (D == 64) return run_attn<bf16_t, bf16_t, 64>(a, B, out, st);
  return run_attn<bf16_t, bf16_t, 128>(a, B, out, st);
}

}  // namespace dflash
