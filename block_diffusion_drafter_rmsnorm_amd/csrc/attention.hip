// Non-causal block attention over a paged context cache, split over the
// context keys (flash-decoding style) with a log-sum-exp combine.
//
// For one request r and kv head g the G = nq / nkv query heads of the S block
// rows form R = G * S <= 64 query rows (row rho = h_local * S + j).  A
// workgroup owns all of them for a range of 32-key steps (wave w takes query
// rows 16w .. 16w+15); the four waves share each step's K/V through LDS, so
// HBM sees each byte once.  The products run in transposed form:
//   S^T = K Q^T      A operand = K rows of the step (K pages are [P][D] per
//                    page and head), B operand = Q^T held in registers;
//   O^T += V^T P^T   A operand = V^T rows (V pages are stored [D][P] per page
//                    and head), B operand = P^T, which is exactly the S^T
//                    accumulator layout (the two operands only have to agree
//                    on the order of the 8 keys a lane holds).
// The online softmax runs per query column in the exp2 domain.  The first
// unit of every (request, kv head) is the block's own S keys (every block row
// sees them: no causal mask), laid out by the QKV epilogue as one extra page.
// On a sliding layer context key i is visible to the row at logical position
// p iff p - i < W; the range starts at L - W + 1 (rounded down to 32 keys,
// the extra keys masked).  Two staging kernels: a bf16 cache, and an E4M3
// cache with head_dim 128, are copied straight from global memory into LDS
// (E4M3 steps then decoded once per workgroup, exactly, to bf16 in LDS);
// fp32 caches and head_dim 64 E4M3 ones go through registers (decoded once
// per workgroup on the way).
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace dflash {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int kMaxSteps = 128;                      // 32-key steps per workgroup (at most)
constexpr int kMaxChunkPages = kMaxSteps * 32 / 16 + 8;  // page-table entries it can touch
constexpr int kCUs = 256;                           // compute units the plan fills
constexpr int kDeepSteps = 8;                       // workgroup size of the deep pipeline

// Work partition (the split of flash decoding, cut by bytes).  A (request r,
// kv head g) pair -- a segment -- needs units_r = 1 + the number of 32-key
// context steps of r (unit 0 is the block's own keys).  Segments are laid
// end to end, request-major, into one sequence of U = nkv * sum_r units_r
// units, and workgroup w of the W in the grid takes the units
// [floor(w U / W), floor((w + 1) U / W)): every workgroup streams the same
// number of bytes whatever the mix of context lengths.  A workgroup whose
// range crosses segment boundaries takes its parts one after the other and
// writes one (O, m, l) partial per part, at slot w + s for segment s (the
// (w, s) pairs that meet form a staircase, so w + s is unique).  The range
// is cut on the device from the context lengths; the host knows only their
// maximum.  The dispatcher deals workgroup w to CU slot w mod 256, so W a
// multiple of 256 gives every CU the same load.
//   bf16 cache: when the job is small enough, at most one workgroup per CU
//   with all of its steps in flight at once (kDeepSteps LDS stages);
//   otherwise W = 768 (three per CU, 3 stages).  Other caches: 512.  W
//   grows (in multiples of 256) so that no range exceeds kMaxSteps units.
bool attn_uses_dma(int act_dtype, int kv_dtype, int head_dim) {
  return act_dtype == DFLASH_BF16 &&
         (kv_dtype == DFLASH_BF16 || (kv_dtype == DFLASH_FP8_E4M3 && head_dim == 128));
}

AttnPlan plan_attention(int max_keys, int B, int nkv, bool dma) {
  AttnPlan p;
  p.kps = 0;
  const int64_t units_max = 1 + ((int64_t)(max_keys > 0 ? max_keys : 0) + 31 + 31) / 32;
  const int64_t u_max = units_max * B * nkv;
  if (dma && (int64_t)B * nkv <= 16) {
    // Few segments (batch 1 or 2): kps >= 16 workgroups per segment, none
    // crossing a segment, at most 256 in all unless a part would exceed
    // kMaxSteps, and at least ~2 context steps each.  (With more segments the
    // byte-range partition at three workgroups per CU streams faster: 64
    // segments of 16384 keys took 120 us that way, 245 us aligned.)  The split is by the context length
    // the host bounds (max_prefix), so every workgroup knows its key range
    // before any length arrives (aligned kernel).
    const int segs = B * nkv;
    const int64_t ctx = units_max - 1;
    int64_t k = kCUs / segs;
    if (k > (ctx + 1) / 2) k = (ctx + 1) / 2;
    const int64_t kmin = (ctx + kMaxSteps - 2) / (kMaxSteps - 1);
    if (k < kmin) k = kmin;
    if (k < 1) k = 1;
    p.kps = (int)k;
    p.stages = kDeepSteps;
    p.n_launch = (int)(segs * k);
    p.n_partials = p.n_launch;
    p.fits = true;
    return p;
  }
  int64_t W;
  if (dma && u_max <= (int64_t)kDeepSteps * kCUs) {
    // at most one workgroup per CU, with at least ~5 steps each: fewer
    // would add (O, m, l) partials faster than they split the streaming
    p.stages = kDeepSteps;
    W = (u_max + 4) / 5;
    W = W < kCUs ? (W > 0 ? W : 1) : kCUs;
  } else {
    p.stages = dma ? 3 : 0;
    W = (int64_t)(dma ? 3 : 2) * kCUs;
  }
  const int64_t by_cap = (u_max + kMaxSteps - 1) / kMaxSteps;
  if (by_cap > W) W = (by_cap + kCUs - 1) / kCUs * kCUs;
  p.n_launch = (int)W;
  p.n_partials = (int)(W + (int64_t)B * nkv);
  p.fits = u_max < (1ll << 31) / 2;  // unit positions (and (x + 1) W) stay exact
  return p;
}

struct AttnArgs {
  const void* q;                       // [M, nq, D] block queries (after q-norm, RoPE)
  const void* kblk; const void* vblk;  // [B, nkv, 16, D] and [B, nkv, D, 16] block K / V^T
  const void* kc; const void* vc;      // paged cache of this layer: K [pages][nkv][P][D],
                                       // V [pages][nkv][D][P]
  const int32_t* pt; int max_pages; int64_t num_pages;
  const int32_t* prefix_len; int max_prefix;
  int B, S, G, nq, nkv, P, window, W;
  int cwin;                            // draft window: last cwin context keys (0: all)
  int kps;                             // aligned partition: workgroups per segment (0: by bytes)
  float scale_log2;
  float* o_part; float2* ml_part;  // per partial slot: [64 rows][D], [64 rows]
  int4* seg;                       // per request: (units before it per head, units, U, -)
  int o_blk;                       // the output [M, nq D] in the 16 x 32 blocks of act_off
};

// Inclusive prefix sum over a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Context length clamped as the kernels use it, the first context key any
// block query sees (sliding window: keys i > L - W; draft window: the last
// cwin keys), and the units of a request of that length.  Logical page q of a
// request lives in physical page page_table[q mod max_pages] (a ring: the
// identity when the table covers the whole prefix).
__device__ __forceinline__ int clamped_len(const AttnArgs& a, int r) {
  return imin(imax(a.prefix_len[r], 0), a.max_prefix);
}
__device__ __forceinline__ int key_lo(const AttnArgs& a, int L) {
  int lo = a.window > 0 ? L - a.window + 1 : 0;
  if (a.cwin > 0) lo = imax(lo, L - a.cwin);
  return imax(lo, 0);
}
__device__ __forceinline__ int units_of_len(const AttnArgs& a, int L) {
  const int lo = key_lo(a, L);
  const int a0 = lo & ~31;
  return 1 + (L > a0 ? (L - a0 + 31) / 32 : 0);
}

// The units of every request and the units before it.  With B <= 64 every
// wave holds them in registers, request i in lane i.  Otherwise thread tid
// owns requests tid * c .. tid * c + c - 1 and keeps only the units before
// its first one; find_segment reloads the lengths.  find_segment(x) returns
// the segment holding unit x of the sequence; all threads call it together
// (the large form uses LDS and barriers).
struct UnitTable {
  bool small;
  int c;
  int u, pre, L;  // small: this lane's request; large: pre = units before the thread's first
  int64_t U;      // units of the whole sequence
};
struct SegPos {
  int r, g, L;
  int units;       // units of the segment
  int64_t start;   // its first unit in the sequence
};
__device__ UnitTable unit_table(const AttnArgs& a, int* red) {
  UnitTable t;
  const int tid = threadIdx.x & 255, lane = tid & 63, wave = tid >> 6;
  t.small = a.B <= 64;
  if (t.small) {
    t.c = 1;
    t.L = lane < a.B ? clamped_len(a, lane) : 0;
    t.u = lane < a.B ? units_of_len(a, t.L) : 0;
    const int inc = wave_incl_scan(t.u, lane);
    t.pre = inc - t.u;
    t.U = (int64_t)__shfl(inc, 63, 64) * a.nkv;
    return t;
  }
  t.c = (a.B + 255) / 256;
  t.u = t.L = 0;
  int sum = 0;
  for (int i = 0; i < t.c; ++i)
    if (tid * t.c + i < a.B) sum += units_of_len(a, clamped_len(a, tid * t.c + i));
  const int inc = wave_incl_scan(sum, lane);
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    off += w < wave ? red[w] : 0;
    tot += red[w];
  }
  __syncthreads();
  t.pre = off + inc - sum;
  t.U = (int64_t)tot * a.nkv;
  return t;
}
__device__ SegPos find_segment(const AttnArgs& a, const UnitTable& t, int64_t x, int* red) {
  SegPos sp;
  const int tid = threadIdx.x & 255, lane = tid & 63;
  int64_t base;
  if (t.small) {
    const bool hit = lane < a.B && x >= (int64_t)t.pre * a.nkv &&
                     x < (int64_t)(t.pre + t.u) * a.nkv;
    const unsigned long long m = __ballot(hit);
    const int src = m ? __ffsll((long long)m) - 1 : 0;
    sp.r = src;
    sp.units = __shfl(t.u, src, 64);
    sp.L = __shfl(t.L, src, 64);
    base = (int64_t)__shfl(t.pre, src, 64) * a.nkv;
  } else {
    int pre = t.pre;
    for (int i = 0; i < t.c; ++i) {
      const int r = tid * t.c + i;
      if (r >= a.B) break;
      const int L = clamped_len(a, r), u = units_of_len(a, L);
      if (x >= (int64_t)pre * a.nkv && x < (int64_t)(pre + u) * a.nkv) {
        red[8] = r;
        red[9] = u;
        red[10] = pre;
        red[11] = L;
      }
      pre += u;
    }
    __syncthreads();
    sp.r = red[8];
    sp.units = red[9];
    sp.L = red[11];
    base = (int64_t)red[10] * a.nkv;
    __syncthreads();
  }
  sp.g = (int)((x - base) / imax(sp.units, 1));
  sp.start = base + (int64_t)sp.g * sp.units;
  return sp;
}
// The range of workgroup w: units [first, end) of the sequence.
__device__ __forceinline__ int64_t range_start(int64_t w, int64_t U, int W) { return w * U / W; }
// Workgroup whose range holds unit x.
__device__ __forceinline__ int range_owner(int64_t x, int64_t U, int W) {
  return (int)(((x + 1) * W - 1) / U);
}
// Workgroup 0 writes the table the combine reads: per request the units
// before it, its units, and U.
__device__ __forceinline__ void write_seg_table(const AttnArgs& a, const UnitTable& t) {
  if (blockIdx.x != 0) return;
  const int tid = threadIdx.x & 255;
  if (t.small) {
    if (tid < a.B) a.seg[tid] = make_int4(t.pre, t.u, (int)t.U, 0);
    return;
  }
  int pre = t.pre;
  for (int i = 0; i < t.c; ++i) {
    const int r = tid * t.c + i;
    if (r >= a.B) break;
    const int u = units_of_len(a, clamped_len(a, r));
    a.seg[r] = make_int4(pre, u, (int)t.U, 0);
    pre += u;
  }
}

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
  __shared__ int red[12];
  const int tid = threadIdx.x & 255, lane = tid & 63, qb = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
  const int S = a.S, R = a.G * S;
  const bool qlive = qb * 16 < R;
  const int rho = imin(qb * 16 + r16, R - 1);
  const int jrow = rho % S;
  const UnitTable tab = unit_table(a, red);
  write_seg_table(a, tab);
  const int64_t x_end = range_start((int64_t)blockIdx.x + 1, tab.U, a.W);
  for (int64_t x = range_start(blockIdx.x, tab.U, a.W); x < x_end;) {
  const SegPos sp = find_segment(a, tab, x, red);
  const int g = sp.g, r = sp.r, L = sp.L;
  const int u0 = (int)(x - sp.start);
  const int u1 = (int)((x_end < sp.start + sp.units ? x_end : sp.start + sp.units) - sp.start);
  const int64_t base = ((int64_t)blockIdx.x + r * a.nkv + g) * 64;  // partial slot w + s
  x = sp.start + u1;
  // Q^T (B operand): query r16 of this wave's block, dims ks*32 + g4*8 .. +8
  Frag<CT> qf[D / 32];
  {
    const int hl = rho / S;
    const CT* qp = static_cast<const CT*>(a.q) + ((int64_t)(r * S + jrow) * a.nq + g * a.G + hl) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) load_frag(qf[ks], qp + ks * 32 + g4 * 8);
  }
  // the block's own keys: one 16-key page (both halves point at it).  Every
  // part loads and stages it, only a segment's first uses it: a load whose
  // wait is conditional makes the compiler wait for all loads in flight later.
  uint4 rb[SPB::PPT];
  {
    const CT* kb = static_cast<const CT*>(a.kblk) + (int64_t)(r * a.nkv + g) * 16 * D;
    const CT* vb = static_cast<const CT*>(a.vblk) + (int64_t)(r * a.nkv + g) * D * 16;
    const CT* kp[2] = {kb, kb};
    const CT* vp[2] = {vb, vb};
#pragma unroll
    for (int u = 0; u < SPB::PPT; ++u)
      rb[u] = gload16(piece_src<CT, D>(kp, vp, 16, tid + 256 * u));
  }
  const int lo = key_lo(a, L);
  const int a0 = lo & ~31;
  const bool has_blk = u0 == 0;
  const int t_first = imax(u0 - 1, 0);             // first context step
  const int n_ctx = u1 - 1 - t_first;              // context steps of the part
  const int kbeg = a0 + 32 * t_first;
  const int kend = imin(L, kbeg + 32 * n_ctx);
  const int pfirst = kbeg / a.P;
  {
    // with no context keys (n_ctx == 0) the entries of step 0 are still
    // filled: the loads issued below read step 0 unconditionally
    const int npages = (kbeg + 32 * imax(n_ctx, 1) - 1) / a.P - pfirst + 1;
    for (int i = tid; i < npages; i += 256) {
      const int64_t page = a.pt[(int64_t)r * a.max_pages + (pfirst + i) % a.max_pages];
      pages[i] = (int)(page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page));
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

  // context steps: loads four steps ahead in registers, LDS double buffer.
  // Every step issues one step's loads and stages one set without a branch
  // (past the last step the loads repeat the last step's addresses and the
  // staged copy is never read): with conditional loads the compiler's wait
  // counting merges the paths and waits for every load in flight, which
  // drains the prefetch at each step.  Loop exits are the only branches.
  uint4 rr0[SPK::PPT], rr1[SPK::PPT], rr2[SPK::PPT], rr3[SPK::PPT], rr4[SPK::PPT];
  const int t_last = imax(n_ctx - 1, 0);
  issue(rr0, 0);
  issue(rr1, imin(1, t_last));
  issue(rr2, imin(2, t_last));
  issue(rr3, imin(3, t_last));
#pragma unroll
  for (int u = 0; u < SPB::PPT; ++u) stage_piece<CT, CT, D>(stg_s[1], rb[u], tid + 256 * u);
  lds_barrier();
  if (has_blk) compute(stg_s[1], 0, true);
  if (n_ctx > 0) {
    stage_ctx(stg_s[0], rr0);
    lds_barrier();
    // cur_next: the set that held step t - 1 (free now) -> step t + 4;
    // nxt: the set holding step t + 1
    auto step = [&](int t, uint4 (&cur_next)[SPK::PPT], uint4 (&nxt)[SPK::PPT]) {
      issue(cur_next, imin(t + 4, t_last));
      compute(stg_s[t & 1], kbeg + 32 * t, false);
      stage_ctx(stg_s[(t + 1) & 1], nxt);
      lds_barrier();
    };
    for (int t0 = 0;; t0 += 5) {
      step(t0, rr4, rr1);
      if (t0 + 1 > t_last) break;
      step(t0 + 1, rr0, rr2);
      if (t0 + 2 > t_last) break;
      step(t0 + 2, rr1, rr3);
      if (t0 + 3 > t_last) break;
      step(t0 + 3, rr2, rr4);
      if (t0 + 4 > t_last) break;
      step(t0 + 4, rr3, rr0);
      if (t0 + 5 > t_last) break;
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
  // the next part reuses the staging buffers and the page list
  __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bf16 cache: the K/V of a step go straight from global memory into LDS
// (global_load_lds_dwordx4, 64 lanes x 16 bytes per instruction), into NS
// stage buffers, NS - 1 steps ahead of the step being computed.  No register
// staging, so no register sets to rotate and no compiler-counted loads in the
// loop: the kernel waits for its own loads with explicit counts.
//
// Key order inside a 32-key step: for the K fragments of half h, row rho of
// the 16 x 32 A operand holds key 8 (rho / 4) + 4 h + rho % 4.  The S^T
// accumulator element i of half h in lane group g4 is then key 8 g4 + 4 h + i,
// so a lane's 8 scores are the 8 consecutive keys 8 g4 .. 8 g4 + 7, and its
// V^T fragment (A operand of O^T += V^T P^T, keys 8 g4 .. + 8 of one dim) is
// one 16-byte run of a V^T row: every fragment, K or V, is one 16-byte record
// per lane and one 1 KB DMA per wave.
//   LDS stage: K [kop = h * D/32 + ks][lane][8]   kop < D/16
//              V [db][lane][8]                     db  < D/16

// 16 bytes per lane from global memory into LDS at lds_wave_base + 16 lane.
// Inline asm: the compiler does not count these loads (it would otherwise wait
// for every one in flight before each LDS read); the kernel waits for them.
__device__ __forceinline__ void attn_dma16(const void* g, const void* lds_wave_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
  // m0 (the LDS base of the copy) is saved and restored inside the block, so
  // whatever the surrounding code keeps in m0 survives; the copy reads m0 when
  // it issues (the compiler's own code for these copies rewrites m0 right
  // after each one)
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(l)
      : "memory");
}
template <int N> __device__ __forceinline__ void attn_wait_vmcnt() {
  static_assert(N <= 63, "vmcnt holds 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait until at most `later` steps of DPW loads each are still in flight
// (later <= K).
template <int DPW, int K> __device__ __forceinline__ void attn_wait_steps(int later) {
  if constexpr (K <= 0) {
    attn_wait_vmcnt<0>();
  } else {
    if (later >= K) attn_wait_vmcnt<K * DPW>();
    else attn_wait_steps<DPW, K - 1>(later);
  }
}

// Exchanges with the lane 16 (32) apart, by the gfx950 row-swap instructions
// (VALU, no LDS round trip): permlane16_swap(x, x) returns x's rows as
// (0 0 2 2) and (1 1 3 3), permlane32_swap(x, x) its halves as (lo lo) and
// (hi hi); a lane takes the copy that is not its own.
__device__ __forceinline__ float lane_xor16(float x, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float((lane & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor32(float x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float((lane & 32) ? r[0] : r[1]);
}

// Cache element type of the direct-to-LDS kernels: K and V bytes of one
// 32-key step, and the LDS the staging takes (the ring; an fp8 cache also
// has one bf16 step buffer: the block's own keys, then each decoded step).
template <typename KT, int D, int NS> struct DmaStage {
  static constexpr bool F8 = std::is_same<KT, fp8_t>::value;
  static constexpr int BYTES = 64 * D * (int)sizeof(KT);      // K and V of one step
  static constexpr int BLK = F8 ? 64 * D * 2 : 0;              // the block's bf16 step
  static constexpr int LDS = NS * BYTES + BLK;
};

// One part of a segment on a bf16 or an E4M3 cache: the block's own keys
// (when blk) and n_ctx context steps from kbeg, staged NS deep straight from
// global memory into LDS, then this wave's unnormalised O^T and (m, l) per
// query row at partial slot `base`.  The page list (physical page of logical
// page pfirst + i in pages[i]) and Q are in place; every wave of the workgroup
// calls it.  `stg` is the DmaStage LDS of the workgroup.
//
// E4M3 cache (D = 128): a step's K and V bytes go to LDS as they lie in the
// cache (a wave copies one 1 KB K piece and one 1 KB V^T piece); each wave
// then decodes the two pieces it copied to bf16 (exact) into the bf16 step
// buffer, in the layout of a bf16 step, and after a barrier every wave reads
// its fragments from there: each code is converted once per workgroup rather
// than once per wave.  The block's own keys are bf16; they are copied first,
// into that buffer, and computed before the context steps.
template <int D, int NS, typename KT>
__device__ __forceinline__ void dma_part(const AttnArgs& a, int r, int g, int L, int lo, int blk,
                                         int n_ctx, int kbeg, int kend, int pfirst,
                                         const int* pages, char* stg,
                                         const Frag<bf16_t> (&qf)[D / 32], int64_t base) {
  using CT = bf16_t;
  using DS = DmaStage<KT, D, NS>;
  constexpr bool F8 = DS::F8;
  static_assert(!F8 || D == 128, "the E4M3 staging covers head_dim 128");
  constexpr int OPW = D / 64;                 // bf16: K (and V) copies per wave per step
  constexpr int DPW = F8 ? 2 : 2 * OPW;       // copies per wave per context step
  const int tid = threadIdx.x & 255, lane = tid & 63, wave = tid >> 6, r16 = lane & 15,
            g4 = lane >> 4;
  const int S = a.S, R = a.G * S;
  const bool qlive = wave * 16 < R;
  const int rho = imin(wave * 16 + r16, R - 1);
  const int jrow = rho % S;
  const KT* kc = static_cast<const KT*>(a.kc);
  const KT* vc = static_cast<const KT*>(a.vc);
  const CT* kblk = static_cast<const CT*>(a.kblk) + (int64_t)(r * a.nkv + g) * 16 * D;
  const CT* vblk = static_cast<const CT*>(a.vblk) + (int64_t)(r * a.nkv + g) * D * 16;
  // this lane's K row inside a half (key 8 (r16/4) + 4h + r16%4 of the step:
  // page half r16 / 8, row within it) and V^T key offset (page half g4 / 2)
  const int krow0 = (8 * (r16 >> 2) + (r16 & 3)) & 15;  // + 4 h
  const int khalf = r16 >> 3, vhalf = g4 >> 1, voff = 8 * (g4 & 1);
  char* const blkbuf = stg + NS * DS::BYTES;  // bf16 step buffer (E4M3 only)
  // bf16 step (the block's, or a context step of a bf16 cache) into `dst`:
  // K [kop = h * D/32 + ks][lane][8], V [db][lane][8]
  auto issue_bf16 = [&](CT* dst, const CT* const* kp, const CT* const* vp, int vstride) {
    const CT* kl = khalf ? kp[1] : kp[0];
    const CT* vl = vhalf ? vp[1] : vp[0];
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
      const int kop = wave * OPW + i, h = kop / (D / 32), ks = kop % (D / 32);
      attn_dma16(kl + (krow0 + 4 * h) * D + 32 * ks + 8 * g4, dst + kop * 512);
    }
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
      const int db = wave * OPW + i;
      attn_dma16(vl + (int64_t)(16 * db + r16) * vstride + voff, dst + 32 * D + db * 512);
    }
  };
  // the next context step (keys kbeg + 32 t ..) into ring slot `slot`.  E4M3: piece
  // kop = wave (score half h = wave / 2, dims 64 c .. with c = wave % 2)
  // holds, in lane l, 16 dims from 64 c + 16 g4 of step key 8 (r16 / 4) +
  // 4 h + r16 % 4 (page half r16 / 8, row krow0 + 4 h in it); piece vop =
  // wave holds, in lane l, the 16 keys of page half wave / 2 of dim 64 c + l
  // Steps are issued in order (t = 0, 1, ...): the page-list index and the
  // offset inside the page of the next step's first key advance by 32 keys
  // per call instead of being divided out (the page size is a multiple of 16,
  // so a 16-key half never straddles pages).
  int nx_pg = 0, nx_off = kbeg % a.P;  // kbeg's page is pages[0] (pfirst = kbeg / P)
  auto issue_ctx = [&](int slot) {
    char* dst = stg + slot * DS::BYTES;
    const KT* kp[2];
    const KT* vp[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t page = pages[nx_pg];
      kp[j] = kc + ((page * a.nkv + g) * a.P + nx_off) * D;
      vp[j] = vc + (page * a.nkv + g) * (int64_t)D * a.P + nx_off;
      nx_off += 16;
      if (nx_off == a.P) {
        nx_off = 0;
        ++nx_pg;
      }
    }
    if constexpr (F8) {
      const int h = wave >> 1, c = wave & 1;
      attn_dma16((khalf ? kp[1] : kp[0]) + (krow0 + 4 * h) * D + 64 * c + 16 * g4,
                 dst + wave * 1024);
      attn_dma16(vp[h] + (int64_t)(64 * c + lane) * a.P, dst + 4096 + wave * 1024);
    } else {
      issue_bf16(reinterpret_cast<CT*>(dst), reinterpret_cast<const CT* const*>(kp),
                 reinterpret_cast<const CT* const*>(vp), a.P);
    }
  };

  const int qpos = L + jrow;
  float mq = -INFINITY, lq = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one staged step: keys t0 + 8 g4 + e are this lane's elements e = 0..7.
  // kMasked (a compile-time tag) keeps the masks of the range edges, the
  // sliding window and the block's own keys; most steps need none, and with
  // the masks in the code the compiler computes them and selects on every step
  auto step = [&](const char* st, int t0, bool is_blk, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    // bf16 fragments at st, in the bf16 step layout
    const CT* Ks = reinterpret_cast<const CT*>(st);
    const CT* Vs = Ks + 32 * D;
    auto kfrag = [&](Frag<CT>& f, int h, int ks) {
      load_frag(f, Ks + ((h * (D / 32) + ks) * 64 + lane) * 8);
    };
    auto vfrag = [&](Frag<CT>& f, int db) { load_frag(f, Vs + (db * 64 + lane) * 8); };
    // keep: this lane's keys inside the step's range; vis: also visible to its
    // query row under the sliding window
    unsigned keep = 0xffu, vis = 0xffu;
    if constexpr (kMasked) {
      if (is_blk || t0 < lo || t0 + 32 > kend) {
        keep = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kk = 8 * g4 + e;
          const bool ok = is_blk ? (kk < S) : (t0 + kk >= lo && t0 + kk < kend);
          keep |= (ok ? 1u : 0u) << e;
        }
      }
      vis = keep;
      if (!is_blk && a.window > 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((qpos - (t0 + 8 * g4 + e)) >= a.window) vis &= ~(1u << e);
      }
    }
    f32x4 sacc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sacc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        Frag<CT> kf;
        kfrag(kf, h, ks);
        mma(sacc[h], kf, qf[ks]);
      }
    }
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = sacc[e >> 2][e & 3] * a.scale_log2;
      if constexpr (kMasked) {
        if (!((vis >> e) & 1u)) sv[e] = -INFINITY;
      }
      mx = fmaxf(mx, sv[e]);
    }
    mx = fmaxf(mx, lane_xor16(mx, lane));
    mx = fmaxf(mx, lane_xor32(mx, lane));
    // lazy reference maximum: it moves only when a step's maximum exceeds it
    // by more than 8 (log2 units), so probabilities stay below 2^8 and O, l
    // are rescaled rarely; O / l does not depend on the reference
    const float mold = mq;
    const bool move = __any(mx > mold + 8.f);
    const float mn = move ? fmaxf(mold, mx) : mold;
    const float msub = (mn == -INFINITY) ? 0.f : mn;
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = __builtin_amdgcn_exp2f(sv[e] - msub);
      sum += sv[e];
    }
    sum += lane_xor16(sum, lane);
    sum += lane_xor32(sum, lane);
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
    for (int db = 0; db < D / 16; ++db) {
      Frag<CT> vf;
      vfrag(vf, db);
      // keys outside the range (first and last steps only) are zeroed: their
      // memory may hold anything
      if constexpr (kMasked) frag_keep(vf, keep);
      mma(o[db], vf, pf);
    }
  };
  // a step needs no mask when its 32 keys lie inside the range and no sliding
  // window reaches them (the same for every lane: a scalar branch)
  auto compute = [&](const char* st, int t0, bool is_blk) {
    const bool plain = !is_blk && t0 >= lo && t0 + 32 <= kend &&
                       !(a.window > 0 && (L + S - 1) - t0 >= a.window);
    if (__builtin_amdgcn_readfirstlane(plain ? 1 : 0))
      step(st, t0, is_blk, std::false_type{});
    else
      step(st, t0, is_blk, std::true_type{});
  };

  if constexpr (F8) {
    // E4M3 step in ring slot `src` -> bf16 in blkbuf, in the bf16 step layout.
    // Each wave decodes the two pieces it copied (16 codes per lane each) and
    // writes them as two 8-element records.  K piece `wave` (h = wave / 2, c =
    // wave % 2), lane (r16, g4): dims 64 c + 16 g4 .. + 16 of its key row, i.e.
    // operand h * D/32 + 2 c + g4 / 2, records of lanes (r16, 2 (g4 % 2)) and
    // (r16, 2 (g4 % 2) + 1).  V^T piece `wave`, lane l: keys 16 h .. + 16 of
    // dim 64 c + l, i.e. operand 4 c + l / 16, records of lanes (l % 16, 2 h)
    // and (l % 16, 2 h + 1).
    auto decode_f8 = [&](const char* src) {
      CT* dst = reinterpret_cast<CT*>(blkbuf);
      const int h = wave >> 1, c = wave & 1;
      const uint4 kr = *reinterpret_cast<const uint4*>(src + wave * 1024 + lane * 16);
      const uint4 vr = *reinterpret_cast<const uint4*>(src + 4096 + wave * 1024 + lane * 16);
      Raw8<fp8_t> r[4];
      r[0].v = make_uint2(kr.x, kr.y);
      r[1].v = make_uint2(kr.z, kr.w);
      r[2].v = make_uint2(vr.x, vr.y);
      r[3].v = make_uint2(vr.z, vr.w);
      Frag<CT> f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) raw_to_frag<CT, fp8_t>(f[i], r[i]);
      const int kop = h * (D / 32) + 2 * c + (g4 >> 1), kg = 2 * (g4 & 1);
      const int vop = 4 * c + (lane >> 4), vr16 = lane & 15;
      *reinterpret_cast<uint4*>(dst + (kop * 64 + kg * 16 + r16) * 8) = f[0].v;
      *reinterpret_cast<uint4*>(dst + (kop * 64 + (kg + 1) * 16 + r16) * 8) = f[1].v;
      *reinterpret_cast<uint4*>(dst + 32 * D + (vop * 64 + 2 * h * 16 + vr16) * 8) = f[2].v;
      *reinterpret_cast<uint4*>(dst + 32 * D + (vop * 64 + (2 * h + 1) * 16 + vr16) * 8) = f[3].v;
    };
    // the block's keys first (4 bf16 copies per wave, older than every
    // context copy), then context steps 0 .. NS - 2 in flight
    const int n_pro = imin(NS - 1, n_ctx);
    if (blk) {
      const CT* kp[2] = {kblk, kblk};
      const CT* vp[2] = {vblk, vblk};
      issue_bf16(reinterpret_cast<CT*>(blkbuf), kp, vp, 16);
    }
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
      if (t < n_ctx) issue_ctx(t);
    if (blk) {
      attn_wait_steps<DPW, NS - 1>(n_pro);  // all but the context steps' copies
      lds_barrier();
      if (qlive) compute(blkbuf, 0, true);
    }
    for (int t = 0; t < n_ctx; ++t) {
      attn_wait_steps<DPW, NS - 2>(imin(NS - 2, n_ctx - 1 - t));
      // step t is in its slot; every wave has finished with blkbuf (the block
      // step or step t - 1) and with the slot of step t - 1
      lds_barrier();
      if (t + NS - 1 < n_ctx) issue_ctx((t + NS - 1) % NS);
      decode_f8(stg + (t % NS) * DS::BYTES);
      lds_barrier();
      if (qlive) compute(blkbuf, kbeg + 32 * t, false);
    }
  } else {
    // Steps: the block's own keys first (one 16-key page, both halves
    // pointing at it) when blk, then the context steps; steps s + 1 .. s +
    // NS - 1 in flight while step s computes
    const int n_seq = n_ctx + blk;
    auto issue = [&](int s) {
      if (s < blk) {
        const CT* kp[2] = {kblk, kblk};
        const CT* vp[2] = {vblk, vblk};
        issue_bf16(reinterpret_cast<CT*>(stg + (s % NS) * DS::BYTES), kp, vp, 16);
      } else {
        issue_ctx(s % NS);  // context step s - blk
      }
    };
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < n_seq) issue(s);
    for (int s = 0; s < n_seq; ++s) {
      // wait for this wave's copies of step s (those of later steps may stay
      // in flight), then for every wave's
      attn_wait_steps<DPW, NS - 2>(imin(NS - 2, n_seq - 1 - s));
      lds_barrier();
      // the buffer of step s - 1: every wave has finished with it
      if (s + NS - 1 < n_seq) issue(s + NS - 1);
      if (qlive) {
        const bool is_blk = s < blk;
        compute(stg + (s % NS) * DS::BYTES, is_blk ? 0 : kbeg + 32 * (s - blk), is_blk);
      }
    }
  }

  // unnormalised O^T, and (m, l) per query row
  if (qlive && wave * 16 + r16 < R) {
    float* dst = a.o_part + (base + wave * 16 + r16) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<float4*>(dst + db * 16 + g4 * 4) =
          make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
    if (g4 == 0) a.ml_part[base + wave * 16 + r16] = make_float2(mq, lq);
  }
}

template <int D, int NS, typename KT>
__global__ __launch_bounds__(256, NS <= 4 ? 3 : 1) void attn_dma_kernel(AttnArgs a) {
  using CT = bf16_t;
  __shared__ int pages[kMaxChunkPages];
  __shared__ __attribute__((aligned(1024))) char stg[DmaStage<KT, D, NS>::LDS];
  __shared__ int red[12];
  const int tid = threadIdx.x & 255, lane = tid & 63, wave = tid >> 6, r16 = lane & 15,
            g4 = lane >> 4;
  const int S = a.S, R = a.G * S;
  const int rho = imin(wave * 16 + r16, R - 1);
  const int jrow = rho % S;
  const UnitTable tab = unit_table(a, red);
  write_seg_table(a, tab);
  const int64_t x_end = range_start((int64_t)blockIdx.x + 1, tab.U, a.W);
  for (int64_t x = range_start(blockIdx.x, tab.U, a.W); x < x_end;) {
  const SegPos sp = find_segment(a, tab, x, red);
  const int g = sp.g, r = sp.r, L = sp.L;
  const int u0 = (int)(x - sp.start);
  const int u1 = (int)((x_end < sp.start + sp.units ? x_end : sp.start + sp.units) - sp.start);
  const int64_t base = ((int64_t)blockIdx.x + r * a.nkv + g) * 64;  // partial slot w + s
  x = sp.start + u1;
  // Q^T (B operand): query r16 of this wave's block, dims ks*32 + g4*8 .. +8
  Frag<CT> qf[D / 32];
  {
    const int hl = rho / S;
    const CT* qp = static_cast<const CT*>(a.q) + ((int64_t)(r * S + jrow) * a.nq + g * a.G + hl) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) load_frag(qf[ks], qp + ks * 32 + g4 * 8);
  }
  const int lo = key_lo(a, L);
  const int a0 = lo & ~31;
  const int blk = u0 == 0 ? 1 : 0;                 // the part starts with the block's keys
  const int t_first = imax(u0 - 1, 0);             // first context step
  const int n_ctx = u1 - 1 - t_first;              // context steps of the part
  const int kbeg = a0 + 32 * t_first;
  const int kend = imin(L, kbeg + 32 * n_ctx);
  const int pfirst = kbeg / a.P;
  if (n_ctx > 0) {
    const int npages = (kbeg + 32 * n_ctx - 1) / a.P - pfirst + 1;
    for (int i = tid; i < npages; i += 256) {
      const int64_t page = a.pt[(int64_t)r * a.max_pages + (pfirst + i) % a.max_pages];
      pages[i] = (int)(page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page));
    }
  }
  // every load the compiler issued (Q, page table) is complete from here on,
  // and it knows so: it does not wait again, behind the DMAs, before the
  // first use of Q
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  lds_barrier();

  dma_part<D, NS, KT>(a, r, g, L, lo, blk, n_ctx, kbeg, kend, pfirst, pages, stg, qf, base);
  // the next part reuses the stage buffers and the page list
  __syncthreads();
  }
}

// Aligned partition (few segments): workgroup w takes part w % kps of
// segment w / kps = (request r, kv head g): the segment's context steps are
// cut into kps equal parts (part 0 also takes the block's own keys), so no
// workgroup crosses a segment and each writes exactly one partial, at slot w.
// The cut is computed from max_prefix first, so the page-table entries of the
// part go out together with Q and the request's length; only when the length
// differs from max_prefix is the part recomputed and its page list reloaded.
struct PartGeom {
  int lo, blk, n_ctx, kbeg, kend, pfirst, npages;
};
__device__ __forceinline__ PartGeom part_geom(const AttnArgs& a, int L, int part) {
  PartGeom q;
  q.lo = key_lo(a, L);
  const int a0 = q.lo & ~31;
  const int steps = L > a0 ? (L - a0 + 31) / 32 : 0;
  const int t0 = (int)((int64_t)part * steps / a.kps);
  const int t1 = (int)((int64_t)(part + 1) * steps / a.kps);
  q.blk = part == 0 ? 1 : 0;
  q.n_ctx = t1 - t0;
  q.kbeg = a0 + 32 * t0;
  q.kend = imin(L, q.kbeg + 32 * q.n_ctx);
  q.pfirst = q.kbeg / a.P;
  q.npages = q.n_ctx > 0 ? (q.kbeg + 32 * q.n_ctx - 1) / a.P - q.pfirst + 1 : 0;
  return q;
}

template <int D, int NS, typename KT>
__global__ __launch_bounds__(256, 1) void attn_dma_aligned(AttnArgs a) {
  using CT = bf16_t;
  __shared__ int pages[kMaxChunkPages];
  __shared__ __attribute__((aligned(1024))) char stg[DmaStage<KT, D, NS>::LDS];
  const int tid = threadIdx.x & 255, lane = tid & 63, wave = tid >> 6, g4 = lane >> 4;
  const int S = a.S, R = a.G * S;
  const int rho = imin(wave * 16 + (lane & 15), R - 1);
  const int jrow = rho % S;
  const int seg = (int)blockIdx.x / a.kps, part = (int)blockIdx.x % a.kps;
  const int r = seg / a.nkv, g = seg % a.nkv;
  // the request's length, Q and the page entries of the part as if the
  // length were max_prefix, all in flight together
  const int L = clamped_len(a, r);
  Frag<CT> qf[D / 32];
  {
    const int hl = rho / S;
    const CT* qp = static_cast<const CT*>(a.q) + ((int64_t)(r * S + jrow) * a.nq + g * a.G + hl) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) load_frag(qf[ks], qp + ks * 32 + g4 * 8);
  }
  auto load_pages = [&](const PartGeom& q) {
    for (int i = tid; i < q.npages; i += 256) {
      const int64_t page = a.pt[(int64_t)r * a.max_pages + (q.pfirst + i) % a.max_pages];
      pages[i] = (int)(page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page));
    }
  };
  PartGeom q = part_geom(a, a.max_prefix, part);
  load_pages(q);
  if (L != a.max_prefix) {  // wave-uniform (one request per workgroup)
    q = part_geom(a, L, part);
    lds_barrier();          // every wave is done with the first list
    load_pages(q);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and the page list are in
  lds_barrier();
  dma_part<D, NS, KT>(a, r, g, L, q.lo, q.blk, q.n_ctx, q.kbeg, q.kend, q.pfirst, pages, stg, qf,
                      (int64_t)blockIdx.x * 64);
}

// Combine the partials of one query row: one wave per row.  A partial in
// which the row saw no key carries m = -inf and weighs zero (its O is never
// used).  Up to 32 partials at a time: lane s holds partial s's (m, l), and
// the O rows go out in one batch of float4 loads (D/4 lanes per partial, so a
// wave instruction covers 256 / D partials) at the same time as the (m, l)
// loads; the weights are applied once both are in.
template <typename CT, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, CT* __restrict__ out) {
  constexpr int LPP = D / 4;           // lanes per partial row
  constexpr int PPI = 64 / LPP;        // partials per load instruction
  constexpr int CH = 32;               // partials per chunk
  constexpr int NI = CH / PPI;         // load instructions for a chunk
  const int R = a.G * a.S;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= a.B * a.nkv * R) return;
  const int rho = row % R, g = (row / R) % a.nkv, r = row / (R * a.nkv);
  // the workgroups whose ranges meet segment s = (r, g): with the aligned
  // partition parts kps s .. kps s + kps - 1 (each at its own slot, every one
  // written); otherwise those of the byte ranges, workgroup w's at slot w + s
  int w_lo, n;
  int64_t U = 0;
  if (a.kps > 0) {
    w_lo = (r * a.nkv + g) * a.kps;
    n = a.kps;
  } else {
    const int4 sg = a.seg[r];
    U = sg.z;
    const int64_t s0 = ((int64_t)sg.x * a.nkv + (int64_t)g * sg.y);
    w_lo = range_owner(s0, U, a.W);
    n = range_owner(s0 + sg.y - 1, U, a.W) - w_lo + 1;
  }
  const int slot_off = a.kps > 0 ? 0 : r * a.nkv + g;
  auto prow = [&](int s) { return ((int64_t)w_lo + s + slot_off) * 64 + rho; };
  // with U < W some ranges are empty: those workgroups wrote nothing (with U
  // >= W consecutive starts floor(w U / W) differ by at least one, so every
  // range holds a unit and the 64-bit divisions below are skipped)
  auto has_range = [&](int s) {
    if (a.kps > 0 || U >= a.W) return true;
    const int64_t w = (int64_t)w_lo + s;
    return range_start(w + 1, U, a.W) > range_start(w, U, a.W);
  };
  const int sub = lane / LPP, d0 = (lane % LPP) * 4;
  float den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float mref = -INFINITY;  // reference of acc and den so far
  // one chunk of up to CH partials; NIC load instructions cover its O rows
  auto chunk = [&](auto nic_tag, int c0, int nc) {
    constexpr int NIC = decltype(nic_tag)::value;
    const bool mine = lane < nc && has_range(c0 + lane);
    float2 ml = make_float2(-INFINITY, 0.f);
    if (mine) ml = a.ml_part[prow(c0 + lane)];
    float4 v[NIC];
#pragma unroll
    for (int i = 0; i < NIC; ++i) {
      const int s = i * PPI + sub;
      v[i] = s < nc ? *reinterpret_cast<const float4*>(a.o_part + prow(c0 + s) * D + d0)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float mc = ml.x;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mc = fmaxf(mc, __shfl_xor(mc, o, 64));
    const float mn = fmaxf(mref, mc);
    if (mn == -INFINITY) return;  // nothing seen yet
    const float alpha = mref == -INFINITY ? 0.f : exp2f(mref - mn);
    acc.x *= alpha; acc.y *= alpha; acc.z *= alpha; acc.w *= alpha;
    den *= alpha;
    const float wm = ml.x == -INFINITY ? 0.f : exp2f(ml.x - mn);
    den += wave_sum(wm * ml.y);
#pragma unroll
    for (int i = 0; i < NIC; ++i) {
      const int s = i * PPI + sub;
      const float w = __shfl(wm, s & 63, 64);
      // an O with no key (any bits) is dropped, not multiplied
      if (s < nc && w != 0.f) {
        acc.x += w * v[i].x; acc.y += w * v[i].y; acc.z += w * v[i].z; acc.w += w * v[i].w;
      }
    }
    mref = mn;
  };
  for (int c0 = 0; c0 < n; c0 += CH) {
    const int nc = imin(CH, n - c0);
    if (nc <= 2 * PPI) chunk(std::integral_constant<int, 2>(), c0, nc);
    else if (nc <= 8 * PPI && 8 < NI) chunk(std::integral_constant<int, (8 < NI ? 8 : NI)>(), c0, nc);
    else chunk(std::integral_constant<int, NI>(), c0, nc);
  }
  // the PPI lane groups hold disjoint partials of the same dims
#pragma unroll
  for (int o = LPP; o < 64; o <<= 1) {
    acc.x += __shfl_xor(acc.x, o, 64);
    acc.y += __shfl_xor(acc.y, o, 64);
    acc.z += __shfl_xor(acc.z, o, 64);
    acc.w += __shfl_xor(acc.w, o, 64);
  }
  if (lane < LPP) {
    const int hl = rho / a.S, j = rho % a.S;
    // 4 columns inside one 32-column block
    CT* dst = out + act_off(r * a.S + j, (g * a.G + hl) * D + d0, (int64_t)a.nq * D, a.o_blk);
    const float inv = 1.0f / den;
    dst[0] = Num<CT>::from_f(acc.x * inv);
    dst[1] = Num<CT>::from_f(acc.y * inv);
    dst[2] = Num<CT>::from_f(acc.z * inv);
    dst[3] = Num<CT>::from_f(acc.w * inv);
  }
}

template <typename CT, typename KT, int D>
static hipError_t run_attn(const AttnArgs& a, const AttnPlan& plan, void* out, hipStream_t st) {
  const dim3 grid((unsigned)plan.n_launch);
  constexpr bool kDmaF8 = std::is_same<KT, fp8_t>::value && D == 128;
  if constexpr (std::is_same<CT, bf16_t>::value && (std::is_same<KT, bf16_t>::value || kDmaF8)) {
    // three workgroups per CU: 3 stages of a bf16 cache, 4 of an E4M3 one
    // (half the bytes per step) in the same LDS
    constexpr int NS3 = kDmaF8 ? 4 : 3;
    if (plan.kps > 0)
      hipLaunchKernelGGL((attn_dma_aligned<D, kDeepSteps, KT>), grid, dim3(256), 0, st, a);
    else if (plan.stages == kDeepSteps)
      hipLaunchKernelGGL((attn_dma_kernel<D, kDeepSteps, KT>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((attn_dma_kernel<D, NS3, KT>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((attn_split_kernel<CT, KT, D>), grid, dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = a.B * a.nkv * a.G * a.S;
  hipLaunchKernelGGL((attn_combine_kernel<CT, D>), dim3((rows + 3) / 4), dim3(256), 0, st, a,
                     (CT*)out);
  return hipGetLastError();
}

hipError_t launch_attention(int dt, int kv_dt, int D, const void* q, const void* kblk,
                            const void* vblk, const void* kc, const void* vc,
                            const int32_t* page_table, int max_pages, int64_t num_pages,
                            const int32_t* prefix_len, int max_prefix, int B, int S, int nq,
                            int nkv, int page_size, int window, int ctx_window,
                            const AttnPlan& plan,
                            float* o_part, float2* ml_part, int4* seg, void* out, int out_blk,
                            hipStream_t st) {
  const bool dma = attn_uses_dma(dt, kv_dt, D);
  if ((plan.stages != 0) != dma || !plan.fits) return hipErrorInvalidValue;
  AttnArgs a;
  a.q = q; a.kblk = kblk; a.vblk = vblk; a.kc = kc; a.vc = vc;
  a.pt = page_table; a.max_pages = max_pages; a.num_pages = num_pages;
  a.prefix_len = prefix_len; a.max_prefix = max_prefix;
  a.B = B; a.S = S; a.G = nq / nkv; a.nq = nq; a.nkv = nkv; a.P = page_size; a.window = window;
  a.cwin = ctx_window;
  a.kps = plan.kps;
  a.W = plan.n_launch;
  a.scale_log2 = LOG2E / sqrtf((float)D);
  a.o_part = o_part; a.ml_part = ml_part; a.seg = seg;
  a.o_blk = out_blk;
  if (dt == DFLASH_F32) {
    if (D == 64) return run_attn<float, float, 64>(a, plan, out, st);
    return run_attn<float, float, 128>(a, plan, out, st);
  }
  if (kv_dt == DFLASH_FP8_E4M3) {
    if (D == 64) return run_attn<bf16_t, fp8_t, 64>(a, plan, out, st);
    return run_attn<bf16_t, fp8_t, 128>(a, plan, out, st);
  }
  if (D == 64) return run_attn<bf16_t, bf16_t, 64>(a, plan, out, st);
  return run_attn<bf16_t, bf16_t, 128>(a, plan, out, st);
}

}  // namespace dflash
