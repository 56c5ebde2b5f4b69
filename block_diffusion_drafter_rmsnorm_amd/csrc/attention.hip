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
#include <type_traits>

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

// K/V of one 32-key step staged in LDS for the four waves, in fragment order
// (so every fragment read is one contiguous 512 B / 1 KB wave access):
//   K: [h][ks][lane][8]   record = K[key 16 h + l % 16][32 ks + 8 (l / 16) .. +8]
//   V: [db][h][lane][4]   record = V^T[dim 16 db + l % 16][keys 16 h + 4 (l / 16) .. +4]
// in the compute type CT (an fp8 cache is decoded once here, not per wave).
// A step is moved as 16-byte pieces of the cache: K pieces first (key fastest,
// so that a wave's LDS writes are conflict-free), then V (dim-major).
template <typename ST, int D> struct StepPieces {
  static constexpr int EPP = 16 / (int)sizeof(ST);          // elements per piece
  static constexpr int NK = 2 * 16 * D / EPP;               // K pieces (both halves)
  static constexpr int N = 2 * NK;                          // K and V pieces
  static constexpr int PPT = N / 256;                       // pieces per thread
};

// Store the EPP values of one piece (16 raw bytes of ST) at their fragment
// records, as 32-bit words (bf16 pairs or fp32).  K piece: key, first column
// col0; V^T piece: dim, first key key0; both within half h.
template <typename CT, typename ST, int D>
__device__ __forceinline__ void stage_piece(CT* stg, const uint4& raw, int q) {
  using SP = StepPieces<ST, D>;
  constexpr int EPP = SP::EPP;
  constexpr int NW = EPP * (int)sizeof(CT) / 4;  // words of the piece in CT
  uint32_t w[NW];
  if constexpr (std::is_same<ST, fp8_t>::value) {  // E4M3 -> bf16, exact
    const uint32_t r4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) e4m3x4_to_bf16x4(r4[i], w[2 * i], w[2 * i + 1]);
  } else {  // same type: the bits as they are
    w[0] = raw.x; w[1] = raw.y; w[2] = raw.z; w[3] = raw.w;
  }
  uint32_t* Ks = reinterpret_cast<uint32_t*>(stg);
  uint32_t* Vs = reinterpret_cast<uint32_t*>(stg + 32 * D);
  constexpr int RW8 = 8 * (int)sizeof(CT) / 4;  // words of a K record (8 elements)
  constexpr int RW4 = 4 * (int)sizeof(CT) / 4;  // words of a V record (4 elements)
  if (q < SP::NK) {
    // key fastest: the 16 lanes of a piece column write 16 consecutive records
    const int h = q / (16 * (D / EPP)), rem = q % (16 * (D / EPP));
    const int key = rem % 16, col0 = (rem / 16) * EPP;
#pragma unroll
    for (int i = 0; i < EPP; i += (EPP < 8 ? EPP : 8)) {
      const int col = col0 + i;
      const int ks = col / 32, g = (col % 32) / 8, within = col % 8;
      uint32_t* rec = Ks + ((h * (D / 32) + ks) * 64 + key + 16 * g) * RW8 +
                      within * (int)sizeof(CT) / 4;
      constexpr int n = (EPP < 8 ? EPP : 8) * (int)sizeof(CT) / 4;  // words written
      const int w0 = i * (int)sizeof(CT) / 4;
      if constexpr (n == 4) {
        *reinterpret_cast<uint4*>(rec) = make_uint4(w[w0], w[w0 + 1], w[w0 + 2], w[w0 + 3]);
      } else {
#pragma unroll
        for (int e = 0; e < n; e += 4)
          *reinterpret_cast<uint4*>(rec + e) = make_uint4(w[w0 + e], w[w0 + e + 1], w[w0 + e + 2], w[w0 + e + 3]);
      }
    }
  } else {
    const int qv = q - SP::NK;
    const int h = qv / (D * (16 / EPP)), rem = qv % (D * (16 / EPP));
    const int dim = rem / (16 / EPP), key0 = (rem % (16 / EPP)) * EPP;
#pragma unroll
    for (int i = 0; i < EPP; i += 4) {
      const int key = key0 + i;
      uint32_t* rec = Vs + (((dim / 16) * 2 + h) * 64 + dim % 16 + 16 * (key / 4)) * RW4;
      const int w0 = i * (int)sizeof(CT) / 4;
      if constexpr (RW4 == 2) *reinterpret_cast<uint2*>(rec) = make_uint2(w[w0], w[w0 + 1]);
      else *reinterpret_cast<uint4*>(rec) = make_uint4(w[w0], w[w0 + 1], w[w0 + 2], w[w0 + 3]);
    }
  }
}

// 16 bytes from global memory (a global, not a flat, load: flat loads count
// against the LDS wait counter, so the LDS barriers would wait for them)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload16(const void* p) {
  const u32x4_t v = *reinterpret_cast<const __attribute__((address_space(1))) u32x4_t*>(
      reinterpret_cast<uintptr_t>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Global address of piece q of a step whose K halves start at kp[h] (16 keys
// x D, row stride D) and V^T halves at vp[h] (D rows x 16 keys, row stride P).
template <typename ST, int D>
__device__ __forceinline__ const ST* piece_src(const ST* const* kp, const ST* const* vp, int P,
                                               int q) {
  using SP = StepPieces<ST, D>;
  constexpr int EPP = SP::EPP;
  if (q < SP::NK) {
    const int h = q / (16 * (D / EPP)), rem = q % (16 * (D / EPP));
    return kp[h] + (rem % 16) * D + (rem / 16) * EPP;
  }
  const int qv = q - SP::NK;
  const int h = qv / (D * (16 / EPP)), rem = qv % (D * (16 / EPP));
  return vp[h] + (int64_t)(rem / (16 / EPP)) * P + (rem % (16 / EPP)) * EPP;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses,
// not for its global loads in flight (a plain __syncthreads() waits for those
// too, which would drain the prefetch pipeline at every step).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename CT, typename KT, int D>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
  using SPK = StepPieces<KT, D>;
  using SPB = StepPieces<CT, D>;
  constexpr int STAGE = 64 * D;  // CT elements of one staged step
  __shared__ int pages[kMaxChunkPages];
  __shared__ __attribute__((aligned(16))) CT stg_s[2][STAGE];
  const int split = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, qb = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const int S = a.S, R = a.G * S;
  const bool qlive = qb * 16 < R;
  const int64_t base = ((int64_t)(r * a.nkv + g) * a.n_splits + split) * 64;

  // Work that does not depend on the prefix length goes first, so the memory
  // round trips overlap: the query loads, the block's own keys (split 0), the
  // prefix length, and on a full-attention layer (whose range starts at key
  // split * chunk) the page-table entries of the range.
  // Q^T (B operand): query r16 of this wave's block, dims ks*32 + g4*8 .. +8
  const int rho = imin(qb * 16 + r16, R - 1);
  const int jrow = rho % S;
  Frag<CT> qf[D / 32];
  {
    const int hl = rho / S;
    const CT* qp = static_cast<const CT*>(a.q) + ((int64_t)(r * S + jrow) * a.nq + g * a.G + hl) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) load_frag(qf[ks], qp + ks * 32 + g4 * 8);
  }
  uint4 rb[SPB::PPT];  // the block's own keys: one 16-key page (both halves point at it)
  if (split == 0) {
    const CT* kb = static_cast<const CT*>(a.kblk) + (int64_t)(r * a.nkv + g) * 16 * D;
    const CT* vb = static_cast<const CT*>(a.vblk) + (int64_t)(r * a.nkv + g) * D * 16;
    const CT* kp[2] = {kb, kb};
    const CT* vp[2] = {vb, vb};
#pragma unroll
    for (int u = 0; u < SPB::PPT; ++u)
      rb[u] = gload16(piece_src<CT, D>(kp, vp, 16, tid + 256 * u));
  }
  int pre = 0;
  if (a.window == 0 && tid < kMaxChunkPages)
    pre = a.pt[(int64_t)r * a.max_pages + imin((split * a.chunk) / a.P + tid, a.max_pages - 1)];
  int L, lo, a0, nvalid;
  key_range(a, r, L, lo, a0, nvalid);
  if (split >= nvalid) {
    // no keys here: an empty partial, which the combine weighs zero
    if (tid < R) a.ml_part[base + tid] = make_float2(-INFINITY, 0.f);
    return;
  }
  const int kbeg = a0 + split * a.chunk;
  const int kend = imin(L, kbeg + a.chunk);
  const int n_ctx = (kend > kbeg) ? (kend - kbeg + 31) / 32 : 0;
  const int pfirst = kbeg / a.P;
  if (n_ctx > 0) {
    const int npages = (kbeg + 32 * n_ctx - 1) / a.P - pfirst + 1;
    if (a.window == 0) {  // kbeg == split * chunk: the entries loaded above
      if (tid < npages)
        pages[tid] = pre < 0 ? 0 : (pre >= a.num_pages ? (int)(a.num_pages - 1) : pre);
      for (int i = tid + 256; i < npages; i += 256) {
        const int64_t page = a.pt[(int64_t)r * a.max_pages + imin(pfirst + i, a.max_pages - 1)];
        pages[i] = (int)(page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page));
      }
    } else {
      for (int i = tid; i < npages; i += 256) {
        const int64_t page = a.pt[(int64_t)r * a.max_pages + imin(pfirst + i, a.max_pages - 1)];
        pages[i] = (int)(page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page));
      }
    }
  }
  lds_barrier();

  const KT* kc = static_cast<const KT*>(a.kc);
  const KT* vc = static_cast<const KT*>(a.vc);
  // global loads of context step t (keys kbeg + 32 t ..) into a register set
  auto issue = [&](uint4 (&rr)[SPK::PPT], int t) {
    const KT *kp[2], *vp[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key0 = kbeg + 32 * t + 16 * h;
      const int64_t page = pages[key0 / a.P - pfirst];
      const int off = key0 % a.P;
      kp[h] = kc + ((page * a.nkv + g) * a.P + off) * D;
      vp[h] = vc + (page * a.nkv + g) * (int64_t)D * a.P + off;
    }
#pragma unroll
    for (int u = 0; u < SPK::PPT; ++u)
      rr[u] = gload16(piece_src<KT, D>(kp, vp, a.P, tid + 256 * u));
  };
  auto stage_ctx = [&](CT* stg, const uint4 (&rr)[SPK::PPT]) {
#pragma unroll
    for (int u = 0; u < SPK::PPT; ++u) stage_piece<CT, KT, D>(stg, rr[u], tid + 256 * u);
  };

  const int qpos = L + jrow;
  float mq = -INFINITY, lq = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One staged 32-key step; key (16 h + 4 g4 + i) of the step is this lane's
  // element h * 4 + i of the S^T accumulators and of the V^T / P^T fragments.
  auto compute = [&](const CT* stg, int t0, bool is_blk) {
    if (!qlive) return;
    const CT* Ks = stg;
    const CT* Vs = stg + 32 * D;
    // keys of the step inside [lo, kend) (the block: its first S keys); an
    // interior step has all 32 (the test is uniform across the wave)
    const bool full = is_blk ? false : (t0 >= lo && t0 + 32 <= kend);
    unsigned keep = 0xffu;
    if (!full) {
      keep = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = 16 * h + 4 * g4 + i;
          const bool ok = is_blk ? (h == 0 && kk < S) : (t0 + kk >= lo && t0 + kk < kend);
          keep |= (ok ? 1u : 0u) << (h * 4 + i);
        }
    }
    unsigned vis = keep;
    if (!is_blk && a.window > 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = 16 * (e >> 2) + 4 * g4 + (e & 3);
        if ((qpos - (t0 + kk)) >= a.window) vis &= ~(1u << e);
      }
    }
    const bool masked = !full || (!is_blk && a.window > 0);
    f32x4 sacc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sacc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        Frag<CT> kf;
        load_frag(kf, Ks + ((h * (D / 32) + ks) * 64 + lane) * 8);
        mma(sacc[h], kf, qf[ks]);
      }
    }
    Frag<CT> vf[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      load_frag_halves(vf[db], Vs + ((db * 2 + 0) * 64 + lane) * 4, Vs + ((db * 2 + 1) * 64 + lane) * 4);
    if (!full) {
      // keys outside the range (first and last steps only) are zeroed: their
      // memory may hold anything
#pragma unroll
      for (int db = 0; db < D / 16; ++db) frag_keep(vf[db], keep);
    }
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = sacc[e >> 2][e & 3] * a.scale_log2;
      if (masked && !((vis >> e) & 1u)) sv[e] = -INFINITY;
      mx = fmaxf(mx, sv[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // The reference maximum moves only when the step's maximum exceeds it by
    // more than 8 (log2 units): probabilities relative to it stay below 2^8,
    // and O and l are rescaled rarely.  The final O / l does not depend on the
    // reference (the combine and the split-level normalisation use m, l as a
    // pair).
    const float mold = mq;
    const bool move = __any(mx > mold + 8.f);
    const float mn = move ? fmaxf(mold, mx) : mold;
    // exp2 by the hardware instruction: exp2(-inf) = 0; the subtrahend is kept
    // finite so that a column with no visible key yet stays all zero
    const float msub = (mn == -INFINITY) ? 0.f : mn;
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = __builtin_amdgcn_exp2f(sv[e] - msub);
      sum += sv[e];
    }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    if (move) {
      const float alpha = __builtin_amdgcn_exp2f(mold - msub);
      lq *= alpha;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) o[db] *= alpha;
    }
    lq += sum;
    mq = mn;
    Frag<CT> pf;
    frag_from_f32(pf, sv);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) mma(o[db], vf[db], pf);
  };

  // context steps: loads four steps ahead in registers, LDS double buffer
  uint4 rr0[SPK::PPT], rr1[SPK::PPT], rr2[SPK::PPT], rr3[SPK::PPT], rr4[SPK::PPT];
  if (0 < n_ctx) issue(rr0, 0);
  if (1 < n_ctx) issue(rr1, 1);
  if (2 < n_ctx) issue(rr2, 2);
  if (3 < n_ctx) issue(rr3, 3);
  if (split == 0) {
#pragma unroll
    for (int u = 0; u < SPB::PPT; ++u) stage_piece<CT, CT, D>(stg_s[1], rb[u], tid + 256 * u);
    lds_barrier();
    compute(stg_s[1], 0, true);
  }
  if (n_ctx > 0) {
    stage_ctx(stg_s[0], rr0);
    lds_barrier();
    auto step = [&](int t, uint4 (&cur_next)[SPK::PPT], uint4 (&nxt)[SPK::PPT]) {
      // cur_next: the set that held step t - 1 (free now) -> step t + 4;
      // nxt: the set holding step t + 1
      if (t >= n_ctx) return;
      if (t + 4 < n_ctx) issue(cur_next, t + 4);
      compute(stg_s[t & 1], kbeg + 32 * t, false);
      if (t + 1 < n_ctx) stage_ctx(stg_s[(t + 1) & 1], nxt);
      lds_barrier();
    };
    for (int t0 = 0; t0 < n_ctx; t0 += 5) {
      step(t0, rr4, rr1);
      step(t0 + 1, rr0, rr2);
      step(t0 + 2, rr1, rr3);
      step(t0 + 3, rr2, rr4);
      step(t0 + 4, rr3, rr0);
    }
  }

  // unnormalised O^T, and (m, l) per query row
  if (qlive && qb * 16 + r16 < R) {
    float* dst = a.o_part + (base + qb * 16 + r16) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<float4*>(dst + db * 16 + g4 * 4) =
          make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
    if (g4 == 0) a.ml_part[base + qb * 16 + r16] = make_float2(mq, lq);
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
      // the O loads do not wait for the weights: an empty split's O (never
      // written, any bits) is dropped by the select below, not multiplied
#pragma unroll
      for (int u = 0; u < 16; ++u)
#pragma unroll
        for (int e = 0; e < D / 64; ++e)
          v[u][e] = s1 + u < ns
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
