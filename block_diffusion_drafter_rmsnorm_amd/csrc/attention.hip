// Non-causal block attention over a paged context cache, split over the
// context keys (flash-decoding style) with a log-sum-exp combine.
//
// For one request r and kv head g the G = nq / nkv query heads of the S block
// rows form R = G * S <= 64 query rows (row rho = h_local * S + j).  One
// workgroup owns all of them for one range of context keys (wave w takes query
// rows 16w .. 16w+15; the four waves read the same K/V, so HBM sees each byte
// once per (request, kv head) and the repeats hit L1/L2).  Each wave walks the
// range in 32-key steps (two 16-key halves, each inside one cache page) and
// works in transposed form, which needs no LDS at all:
//   S^T = K Q^T      A operand = K rows straight from the page ([P][D] per
//                    page and head), B operand = Q^T held in registers;
//   O^T += V^T P^T   A operand = V^T rows straight from the page (V is stored
//                    [D][P] per page and head), B operand = P^T, which is
//                    exactly the S^T accumulator layout (the two operands only
//                    have to agree on the order of the 8 keys a lane holds).
// The online softmax runs per query column in the exp2 domain; the next step's
// K/V fragments are loaded while the current step computes.  Split 0 also
// takes the S block keys (every block row sees them: no causal mask), laid out
// by the QKV epilogue as one extra page.  On a sliding layer context key i is
// visible to the row at logical position p iff p - i < W; the range starts at
// L - W + 1 (rounded down to 32 keys, the extra keys masked).  fp8 caches are
// decoded to bf16 in registers.
#include "common.cuh"
#include "internal.h"

namespace dflash {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int kMaxChunk = 4096;                   // context keys per workgroup
constexpr int kMaxChunkPages = kMaxChunk / 16 + 8;  // page-table entries it can touch

AttnPlan plan_attention(int max_keys, int B, int nkv) {
  AttnPlan p;
  const int64_t base = (int64_t)B * nkv;
  const int64_t keys = (int64_t)max_keys + 32;
  const int64_t steps = (keys + 31) / 32 * base;  // 32-key steps over all (request, kv head)
  int64_t chunk;
  if (steps <= 2048) {
    // latency-bound (a short context or a small batch): one round of at most
    // 256 workgroups, one per CU, so that none waits for a second round
    const int64_t splits = base >= 256 ? 1 : 256 / base;
    chunk = ((keys + splits - 1) / splits + 31) / 32 * 32;
  } else {
    // about 1024 workgroups over the largest context: rounds balance ragged work
    chunk = (keys * base / 1024 + 31) / 32 * 32;
  }
  if (chunk < 128) chunk = 128;
  if (chunk > kMaxChunk) chunk = kMaxChunk;
  p.chunk = (int)chunk;
  p.n_splits = max_keys <= 0 ? 1 : (int)((max_keys + 31 + chunk - 1) / chunk);
  return p;
}

struct AttnArgs {
  const void* q;                       // [M, nq, D] block queries (after q-norm, RoPE)
  const void* kblk; const void* vblk;  // [B, nkv, 16, D] and [B, nkv, D, 16] block K / V^T
  const void* kc; const void* vc;      // paged cache of this layer: K [pages][nkv][P][D],
                                       // V [pages][nkv][D][P]
  const int32_t* pt; int max_pages; int64_t num_pages;
  const int32_t* prefix_len; int max_prefix;
  int S, G, nq, nkv, P, window, chunk, n_splits;
  float scale_log2;
  float* o_part; float2* ml_part;
};

// Context-key range of request r on this layer: keys [lo, L), walked from the
// 32-aligned a0 <= lo, and the number of splits it uses.
__device__ __forceinline__ void key_range(const AttnArgs& a, int r, int& L, int& lo, int& a0,
                                          int& nvalid) {
  L = imin(imax(a.prefix_len[r], 0), imin(a.max_prefix, a.max_pages * a.P));
  lo = a.window > 0 ? imax(0, L - a.window + 1) : 0;
  a0 = lo & ~31;
  nvalid = imax(1, (L - a0 + a.chunk - 1) / a.chunk);
}

// Fragments of one 32-key step: K rows for two 16-key halves x D/32 dim groups,
// V^T rows for D/16 dim blocks x two halves (4 keys each).
template <typename KT, int D> struct KVStep {
  Raw8<KT> k[2][D / 32];
  Raw4<KT> v[D / 16][2];
  __device__ __forceinline__ void load(const KT* kbase0, const KT* kbase1, const KT* vbase0,
                                       const KT* vbase1, int P, int r16, int g4) {
    const KT* kb[2] = {kbase0, kbase1};
    const KT* vb[2] = {vbase0, vbase1};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) k[h][ks].load(kb[h] + r16 * D + ks * 32 + g4 * 8);
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        v[db][h].load(vb[h] + (int64_t)(db * 16 + r16) * P + g4 * 4);
    }
  }
};

template <typename CT, typename KT, int D>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
  // physical pages of this workgroup's key range, read from the page table
  // once: the K/V loads of a step then depend on LDS only, so the next step's
  // loads go out while the current step computes
  __shared__ int pages[kMaxChunkPages];
  const int split = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int lane = threadIdx.x & 63, qb = threadIdx.x >> 6, r16 = lane & 15, g4 = lane >> 4;
  const int S = a.S, R = a.G * S;
  int L, lo, a0, nvalid;
  key_range(a, r, L, lo, a0, nvalid);
  if (split >= nvalid) {
    // no keys here: an empty partial, which the combine weighs zero
    const int64_t base = ((int64_t)(r * a.nkv + g) * a.n_splits + split) * 64;
    if (threadIdx.x < R) a.ml_part[base + threadIdx.x] = make_float2(-INFINITY, 0.f);
    return;
  }
  const int kbeg = a0 + split * a.chunk;
  const int kend = imin(L, kbeg + a.chunk);
  const int n_ctx = (kend > kbeg) ? (kend - kbeg + 31) / 32 : 0;
  const int pfirst = kbeg / a.P;
  if (n_ctx > 0) {
    const int npages = (kbeg + 32 * n_ctx - 1) / a.P - pfirst + 1;
    for (int i = threadIdx.x; i < npages; i += 256) {
      const int pi = imin(pfirst + i, a.max_pages - 1);
      const int64_t page = a.pt[(int64_t)r * a.max_pages + pi];
      pages[i] = (int)(page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page));
    }
  }
  __syncthreads();
  if (qb * 16 >= R) return;  // no barriers below: idle waves leave

  // Q^T (B operand): query r16 of this wave's block, dims ks*32 + g4*8 .. +8
  Frag<CT> qf[D / 32];
  int qpos;
  {
    const int rho = imin(qb * 16 + r16, R - 1);
    const int hl = rho / S, j = rho % S;
    const CT* qp = static_cast<const CT*>(a.q) + ((int64_t)(r * S + j) * a.nq + g * a.G + hl) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) load_frag(qf[ks], qp + ks * 32 + g4 * 8);
    qpos = L + j;
  }
  float mq = -INFINITY, lq = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const KT* kc = static_cast<const KT*>(a.kc);
  const KT* vc = static_cast<const KT*>(a.vc);
  auto page_of = [&](int key) -> int64_t { return pages[key / a.P - pfirst]; };
  auto load_ctx = [&](KVStep<KT, D>& st, int t0) {
    const KT *kb[2], *vb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key0 = t0 + 16 * h;
      const int64_t page = page_of(key0);
      const int off = key0 % a.P;
      kb[h] = kc + ((page * a.nkv + g) * a.P + off) * D;
      vb[h] = vc + (page * a.nkv + g) * (int64_t)D * a.P + off;
    }
    st.load(kb[0], kb[1], vb[0], vb[1], a.P, r16, g4);
  };

  // One 32-key step; key (16 h + 4 g4 + i) of the step is this lane's element
  // h * 4 + i of the S^T accumulators and of the V^T / P^T fragments.
  auto compute = [&](const auto& st, int t0, bool is_blk, int nk) {
    unsigned keep = 0, vis = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = 16 * h + 4 * g4 + i;
        const bool ok = is_blk ? (h == 0 && kk < nk) : (t0 + kk >= lo && t0 + kk < kend);
        bool v = ok;
        if (v && !is_blk && a.window > 0) v = (qpos - (t0 + kk)) < a.window;
        keep |= (ok ? 1u : 0u) << (h * 4 + i);
        vis |= (v ? 1u : 0u) << (h * 4 + i);
      }
    f32x4 sacc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sacc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        Frag<CT> kf;
        raw_to_frag(kf, st.k[h][ks]);
        mma(sacc[h], kf, qf[ks]);
      }
    }
    float s[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s[e] = ((vis >> e) & 1u) ? sacc[e >> 2][e & 3] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(mq, mx);
    const float alpha = (mq == -INFINITY) ? 0.f : exp2f(mq - mn);
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s[e] = (s[e] == -INFINITY) ? 0.f : exp2f(s[e] - mn);
      sum += s[e];
    }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    lq = lq * alpha + sum;
    mq = mn;
    Frag<CT> pf;
    frag_from_f32(pf, s);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      Frag<CT> vf;
      raw4x2_to_frag(vf, st.v[db][0], st.v[db][1], keep);  // keys past the range may hold garbage
      o[db] *= alpha;
      mma(o[db], vf, pf);
    }
  };

  if (n_ctx > 0) {
    KVStep<KT, D> s0, s1;
    load_ctx(s0, kbeg);
    int t = 0;
    for (; t + 2 <= n_ctx; t += 2) {
      load_ctx(s1, kbeg + (t + 1) * 32);
      compute(s0, kbeg + t * 32, false, 0);
      if (t + 2 < n_ctx) load_ctx(s0, kbeg + (t + 2) * 32);
      compute(s1, kbeg + (t + 1) * 32, false, 0);
    }
    if (t < n_ctx) compute(s0, kbeg + t * 32, false, 0);
  }
  if (split == 0) {
    // the block's own keys: one 16-key page of K and V^T in the block buffers
    KVStep<CT, D> sb;
    const CT* kb = static_cast<const CT*>(a.kblk) + (int64_t)(r * a.nkv + g) * 16 * D;
    const CT* vb = static_cast<const CT*>(a.vblk) + (int64_t)(r * a.nkv + g) * D * 16;
    sb.load(kb, kb, vb, vb, 16, r16, g4);
    compute(sb, 0, true, S);
  }

  // unnormalised O^T, and (m, l) per query row
  const int rho = qb * 16 + r16;
  if (rho < R) {
    const int64_t base = ((int64_t)(r * a.nkv + g) * a.n_splits + split) * 64;
    float* dst = a.o_part + (base + rho) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<float4*>(dst + db * 16 + g4 * 4) =
          make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
    if (g4 == 0) a.ml_part[base + rho] = make_float2(mq, lq);
  }
}

// Combine the splits of one query row: one wave per row.  Empty splits carry
// m = -inf and weigh zero (their O is never read).  Lane s holds split s's
// (m, l); the O loads of 16 splits go out together.
template <typename CT, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, CT* __restrict__ out,
                                                           int B) {
  const int R = a.G * a.S;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= B * a.nkv * R) return;
  const int rho = row % R, g = (row / R) % a.nkv, r = row / (R * a.nkv);
  const int64_t base = ((int64_t)(r * a.nkv + g) * a.n_splits) * 64 + rho;
  float M = -INFINITY;
  for (int s = lane; s < a.n_splits; s += 64) M = fmaxf(M, a.ml_part[base + (int64_t)s * 64].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  float den = 0.f, acc[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < a.n_splits; s0 += 64) {
    // this lane's split s0 + lane: its weight and weighted l
    float wl = 0.f, wm = 0.f;
    if (s0 + lane < a.n_splits) {
      const float2 ml = a.ml_part[base + (int64_t)(s0 + lane) * 64];
      wm = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
      wl = wm * ml.y;
    }
    const int ns = imin(64, a.n_splits - s0);
    for (int s1 = 0; s1 < ns; s1 += 16) {
      float v[16][D / 64];
      float w[16], l[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int src = (s1 + u) & 63;  // uniform across the wave
        w[u] = __shfl(wm, src, 64);
        l[u] = __shfl(wl, src, 64);
        if (s1 + u >= ns) w[u] = 0.f;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u)
#pragma unroll
        for (int e = 0; e < D / 64; ++e)
          v[u][e] = w[u] != 0.f
                        ? a.o_part[(base + (int64_t)(s0 + s1 + u) * 64) * D + lane + 64 * e]
                        : 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (w[u] != 0.f) {
          den += l[u];
#pragma unroll
          for (int e = 0; e < D / 64; ++e) acc[e] += w[u] * v[u][e];
        }
    }
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

hipError_t launch_attention(int dt, int kv_dt, int D, const void* q, const void* kblk,
                            const void* vblk, const void* kc, const void* vc,
                            const int32_t* page_table, int max_pages, int64_t num_pages,
                            const int32_t* prefix_len, int max_prefix, int B, int S, int nq,
                            int nkv, int page_size, int window, const AttnPlan& plan,
                            float* o_part, float2* ml_part, void* out, hipStream_t st) {
  AttnArgs a;
  a.q = q; a.kblk = kblk; a.vblk = vblk; a.kc = kc; a.vc = vc;
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
