// Weight-streaming MFMA GEMM for gfx950 with fused prologues and epilogues.
//
// C[M, Ncols] = A[M, K] * W[Ncols, K]^T with W[out, in] stored fragment-packed
// (pack_matrix): 16-row slabs, each a run of 32-column chunks, each chunk the
// 64 lane records of one MFMA B operand, so a wave's weight load is one
// contiguous 1 KB (bf16) and a wave streams its slab front to back.
// One workgroup (4 waves, 256 threads) owns a 16*MB x 128 output tile and one
// K range of a split-K decomposition; each wave owns two slabs (32 columns) for
// all 16*MB rows, so every weight fragment a lane loads from HBM feeds MB
// MFMAs straight from registers.  A rows (the small activation matrix) come
// through L1/L2 with the same K order as the packed records.
//
// RMSNorm is applied by linearity: rms(x) * g * W^T = rstd * ((x * g) W^T).  The
// producer of x (an epilogue) writes x * g_next rounded to T plus the row's
// sum of squares per 128-column tile; the consumer GEMM streams that as a plain
// A operand and scales each output row by rstd (sums of squares added in a
// fixed order) before any other epilogue math.
//
// After the K loop the fp32 tile is assembled in LDS (when K is split, a second
// kernel sums the split partials in a fixed order, so the result is
// deterministic and needs no cross-workgroup synchronisation) and handed to an
// epilogue that sees whole rows of the 128-column tile: a full attention head
// for the q/k RMSNorm + RoPE of the QKV and K/V-injection epilogues, paired
// gate/up columns for SwiGLU, a 128-wide vocabulary slice for the argmax
// partials of lm_head, the next RMSNorm's inputs.
#include "common.h"
#include "internal.h"

#include <type_traits>
#include <utility>

namespace dflash {

constexpr int BN = 128;      // output columns per workgroup tile
constexpr int LDT = BN + 4;  // LDS tile row stride in floats (bank-conflict padding)
constexpr int kChunkElems = 64 * 8;  // elements of one packed chunk (64 lane records of 8)

// Elements of one packed 16-row slab of a matrix with K columns.
__host__ __device__ __forceinline__ int64_t slab_elems(int K) {
  return (int64_t)(K / 32) * kChunkElems;
}

// The narrow QKV GEMM (its consumer adds K-range partials): target workgroup
// count, slabs per workgroup (and per wave), waves per workgroup.
constexpr int kQkvUnits = 768;  // target workgroups of the narrow QKV GEMM
constexpr int kQkvSlabs = 2;    // its slabs per workgroup (and per wave)
constexpr int kQkvWaves = 4;    // its waves per workgroup

GemmPlan plan_gemm(int M, int Ncols, int K, bool bf16, int narrow, int ksw) {
  GemmPlan p;
  p.rows = false;
  p.tall = false;
  p.NSL = p.NW = p.kw = 0;
  p.KSW = 1;
  // (128-column tiles: up to 32 rows, so the per-wave partial tiles fit in LDS)
  if (narrow > 0 && M <= (narrow == 8 ? 32 : 64)) {
    // narrow tiles: one or two slabs per workgroup (two for SwiGLU: a gate
    // slab and its up slab); the waves split K so that the grid holds ~4096+
    // waves (16 per workgroup when the groups are few, else 8; fp32: 8)
    p.rows = true;
    p.fat = p.big = false;
    p.NSL = narrow;
    p.MB = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    p.BM = 16 * p.MB;
    p.m_tiles = (M + p.BM - 1) / p.BM;
    p.n_tiles = (Ncols + 16 * p.NSL - 1) / (16 * p.NSL);
    // waves per workgroup: 16 when the tiles fit one round of 16 waves per CU
    // (4096 waves on the chip), else 8; the lm_head's 128-column tiles take 16
    // = 4 slab pairs x 4 K splits (measured faster than 8 = 4 x 2).  fp32: 8.
    if (!bf16) p.NW = 8;
    else if (p.NSL == 8) p.NW = 16;
    else if (ksw > 1) p.NW = kQkvWaves;  // the QKV store split over workgroups
    else if (p.NSL == 1) p.NW = p.n_tiles <= 256 ? 16 : 8;  // (narrow_rows: <= 8 x NW items)
    else p.NW = 8;  // (gate/up: 8 measured faster than 4)
    // K ranges across workgroups (ksw > 1 only for epilogues whose consumer
    // sums the partials): kw = the K of each range, a multiple of 64
    p.KSW = ksw > 1 ? ksw : 1;
    p.kw = ((K + p.KSW - 1) / p.KSW + 63) / 64 * 64;
    p.KS = 1;
    p.Kc = K;
    return p;
  }
  p.fat = bf16 && M > 64;
  p.big = false;
  if (p.fat && M > 192) {
    // 256 x 256 tiles, one 512-thread workgroup per CU (~6 TFLOP/s each,
    // several times the rate of gemm_fat's 256 x 128 tiles).  With fewer than
    // 128 tiles K is split so that the grid reaches (but stays within) the
    // 256 CUs, each split at least 512 deep; the split partials go through the
    // same reduce-and-epilogue kernel as gemm_fat's.  (With 128 rows or fewer
    // the 128-row tiles of gemm_fat waste less.)
    p.big = true;
    p.BM = 256;
    p.MB = 0;
    p.m_tiles = (M + 255) / 256;
    p.n_tiles = (Ncols + 255) / 256;
    const int tiles = p.m_tiles * p.n_tiles;
    int ks = tiles >= 128 ? 1 : 256 / tiles;
    ks = ks < K / 512 ? ks : K / 512;
    if (ks < 1) ks = 1;
    int kc = (K + ks - 1) / ks;
    kc = (kc + 31) / 32 * 32;
    p.Kc = kc;
    p.KS = (K + kc - 1) / kc;
    return p;
  }
  if (p.fat && M <= 128 && (Ncols + BN - 1) / BN >= 512) {
    // 65..128 rows and at least two 128-column tiles per CU (the lm_head):
    // gemm_tall, the whole K per workgroup.  (With fewer tiles, split K and
    // one workgroup per CU, gemm_fat's 128 x 128 tiles measured faster.)
    p.tall = true;
    p.BM = 128;
    p.MB = 0;
    p.m_tiles = 1;
    p.n_tiles = (Ncols + BN - 1) / BN;
    p.Kc = K;
    p.KS = 1;
    return p;
  }
  if (p.fat) {
    // LDS-tiled MFMA GEMM: 256 x 128 (or 128 x 128) tiles, K split until the
    // grid covers the 256 CUs
    p.BM = M > 128 ? 256 : 128;
    p.MB = 0;
    p.m_tiles = (M + p.BM - 1) / p.BM;
    p.n_tiles = (Ncols + BN - 1) / BN;
    const int base = p.m_tiles * p.n_tiles;
    int ks = base >= 256 ? 1 : (256 + base - 1) / base;
    ks = ks < K / 1024 ? ks : K / 1024;
    if (ks < 1) ks = 1;
    int kc = (K + ks - 1) / ks;
    kc = (kc + 63) / 64 * 64;
    p.Kc = kc;
    p.KS = (K + kc - 1) / kc;
    return p;
  }
  p.MB = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.BM = 16 * p.MB;
  p.m_tiles = (M + 16 * p.MB - 1) / (16 * p.MB);
  p.n_tiles = (Ncols + BN - 1) / BN;
  int ks = 1;
  if (M <= 64) {
    // Split K so that the grid reaches ~1024 workgroups (4 per CU: enough
    // weight loads in flight for the HBM rate).  The split depends on
    // (Ncols, K) only, so the same rows give the same bits at any M <= 64.
    ks = (1024 + p.n_tiles - 1) / p.n_tiles;
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
  // gemm_big's tiles are 256 wide: two 128-column partial tiles each
  const size_t n128 = p.big ? 2 * (size_t)p.n_tiles : (size_t)p.n_tiles;
  return (size_t)p.KS * p.m_tiles * n128 * p.BM * BN;
}

int logits_tiles(int V) { return (V + BN - 1) / BN; }

// K ranges of the narrow QKV GEMM across workgroups: enough that the
// workgroups come to ~kQkvUnits, at most 4.
int qkv_slabs() { return kQkvSlabs; }
int qkv_k_splits(int ncols) {
  const int slabs = (ncols + 15) / 16;
  int k = (kQkvUnits * kQkvSlabs + slabs - 1) / slabs;
  return k < 1 ? 1 : (k > 4 ? 4 : k);
}

// ---------------------------------------------------------------- A sources
// A rows as stored (T).  With S > 0 GEMM row m reads A row
// (m / (S-1)) * S + m % (S-1) + 1 (rows 1..S-1 of every block: lm_head skips
// the anchor row).
__host__ __device__ __forceinline__ int block_row(int m, int S) {
  return S > 0 ? (m / (S - 1)) * S + m % (S - 1) + 1 : m;
}

template <typename T> struct ASrcPlain {
  const T* A;
  int64_t lda;
  int S;
  int blk;  // A in the 16 x 32 blocks of act_off (lda = its width): streaming kernels only
  template <int MB> struct State {
    const T* p[MB];
  };
  template <int MB>
  __device__ __forceinline__ void setup(State<MB>& s, int m0, int M, int r16) const {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      s.p[mb] = A + act_off(block_row(imin(m0 + mb * 16 + r16, M - 1), S), 0, lda, blk);
  }
  // the 8 elements at column k of this lane's row (k mod 32 a multiple of 8):
  // column block k / 32 is 32 (row-major) or 512 (blocked) elements on
  template <int MB>
  __device__ __forceinline__ void load(Frag<T>& f, const State<MB>& s, int mb, int k) const {
    load_frag(f, s.p[mb] + (int64_t)(k >> 5) * (blk ? 512 : 32) + (k & 31));
  }
};

// A of a 16-row tile held in LDS in MFMA fragment order (the narrow kernel
// copies it there first): the fragment of columns 32 c .. 32 c + 31 at c * 512
// elements, lane l's 8 elements (row l mod 16, columns 32 c + 8 (l / 16) ..)
// at l * 8 of it, so every read is one contiguous 1 KB.
template <typename T> struct ASrcImg {
  const T* img;
  template <int MB> struct State {
    const T* p;
  };
  template <int MB>
  __device__ __forceinline__ void setup(State<MB>& s, int, int, int) const {
    s.p = img + (threadIdx.x & 63) * 8;
  }
  template <int MB>
  __device__ __forceinline__ void load(Frag<T>& f, const State<MB>& s, int, int k) const {
    load_frag(f, s.p + (k >> 5) * 512);
  }
};
// Columns of A that the LDS image of the narrow lm_head kernel holds at most
// (16 rows x 4096 bf16 = 128 KB, sharing LDS with the partial-tile buffer).
constexpr int kImgK = 4096;

// Per-row 1/rms from the sums of squares ss[row * n_ss + t] of a width-H row
// (ss == null: no scaling).  GEMM row m uses ss row block_row(m, S).
struct RowScale {
  const float* ss;
  int n_ss;
  int H;
  float eps;
  int S;
  // the values fill() computes, already computed for every GEMM row m (by
  // row_rstd_kernel, with fill() itself); nullable
  const float* pre;
  // 1/rms of the tile's rows m0 .. m0+rows-1 into out[] (LDS), one wave per row
  // (the row's partial sums spread over the lanes, all of a batch of G rows'
  // loads issued before any is summed; each lane adds its values in a fixed
  // order, then a fixed wave tree).  Called by all threads of the workgroup;
  // ends with a barrier.
  __device__ __forceinline__ void fill(float* out, int rows, int m0, int M, int tid) const {
    const int lane = tid & 63, wave = tid >> 6, nw = (int)(blockDim.x >> 6);
    if (pre != nullptr) {
      for (int r = tid; r < rows; r += (int)blockDim.x) out[r] = pre[imin(m0 + r, M - 1)];
      __syncthreads();
      return;
    }
    if (ss == nullptr) {
      for (int r = tid; r < rows; r += (int)blockDim.x) out[r] = 1.0f;
      __syncthreads();
      return;
    }
    if ((n_ss & 3) == 0 && n_ss <= 512) {
      // 16-byte loads: a row's <= 512 partials are one or two float4 per
      // lane; eight rows' loads go out together
      constexpr int G4 = 8;
      const int nq = n_ss > 256 ? 2 : 1;
      for (int r0 = wave; r0 < rows; r0 += nw * G4) {
        float4 v[G4][2];
#pragma unroll
        for (int u = 0; u < G4; ++u) {
          const int r = r0 + nw * u;
          const float* p = ss + (int64_t)block_row(imin(m0 + r, M - 1), S) * n_ss;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int t = 4 * (lane + 64 * q);
            v[u][q] = (r < rows && q < nq && t < n_ss) ? *reinterpret_cast<const float4*>(p + t)
                                                       : make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
#pragma unroll
        for (int u = 0; u < G4; ++u) {
          const int r = r0 + nw * u;
          if (r >= rows) break;
          const float acc = ((v[u][0].x + v[u][0].y) + (v[u][0].z + v[u][0].w)) +
                            ((v[u][1].x + v[u][1].y) + (v[u][1].z + v[u][1].w));
          const float inv = 1.0f / sqrtf(wave_sum(acc) / (float)H + eps);
          if (lane == 0) out[r] = inv;
        }
      }
      __syncthreads();
      return;
    }
    constexpr int G = 4;  // rows per wave batch
    constexpr int Q = 8;  // partials per lane held at once (n_ss <= 512 in one pass)
    for (int r0 = wave; r0 < rows; r0 += nw * G) {
      float v[G][Q];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int r = r0 + nw * u;
        const float* p = ss + (int64_t)block_row(imin(m0 + r, M - 1), S) * n_ss;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          const int t = lane + 64 * q;
          v[u][q] = (r < rows && t < n_ss) ? p[t] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int r = r0 + nw * u;
        if (r >= rows) break;
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < Q; ++q) acc += v[u][q];
        const float* p = ss + (int64_t)block_row(imin(m0 + r, M - 1), S) * n_ss;
        for (int t = lane + 64 * Q; t < n_ss; t += 64) acc += p[t];
        const float inv = 1.0f / sqrtf(wave_sum(acc) / (float)H + eps);
        if (lane == 0) out[r] = inv;
      }
    }
    __syncthreads();
  }
  // Rows first and first + step of a wave's rows (below): their partial sums
  // loaded into registers before the K loop, consumed after it (no wait in
  // between, so the loop's weight loads stay in flight).
  __device__ __forceinline__ void pre_rows(float (&v)[2][8], int rows, int m0, int M, int first,
                                           int step, int lane) const {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = first + step * u;
      const float* p = ss + (int64_t)block_row(imin(m0 + r, M - 1), S) * n_ss;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        v[u][q] = (ss != nullptr && r < rows && lane + 64 * q < n_ss) ? p[lane + 64 * q] : 0.f;
    }
  }
  __device__ __forceinline__ void finish_rows(const float (&v)[2][8], float* out, int rows,
                                              int m0, int M, int first, int step,
                                              int lane) const {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = first + step * u;
      if (r >= rows) break;
      float inv = 1.0f;
      if (ss != nullptr) {
        const float* p = ss + (int64_t)block_row(imin(m0 + r, M - 1), S) * n_ss;
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) acc += v[u][q];
        for (int t = lane + 64 * 8; t < n_ss; t += 64) acc += p[t];
        inv = 1.0f / sqrtf(wave_sum(acc) / (float)H + eps);
      }
      if (lane == 0) out[r] = inv;
    }
    // rows beyond two per wave
    fill_rows(out, rows, m0, M, first + 2 * step, step, lane);
  }
  // 1/rms of rows first, first + step, ... (< rows) into out[] (LDS), by the
  // calling wave alone and without a barrier (the caller's next barrier
  // publishes them).
  __device__ __forceinline__ void fill_rows(float* out, int rows, int m0, int M, int first,
                                            int step, int lane) const {
    constexpr int G = 4;  // rows whose loads go out together
    constexpr int Q = 8;
    for (int r0 = first; r0 < rows; r0 += step * G) {
      float v[G][Q];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int r = r0 + step * u;
        const float* p = ss + (int64_t)block_row(imin(m0 + r, M - 1), S) * n_ss;
#pragma unroll
        for (int q = 0; q < Q; ++q)
          v[u][q] = (ss != nullptr && r < rows && lane + 64 * q < n_ss) ? p[lane + 64 * q] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int r = r0 + step * u;
        if (r >= rows) break;
        float inv = 1.0f;
        if (ss != nullptr) {
          const float* p = ss + (int64_t)block_row(imin(m0 + r, M - 1), S) * n_ss;
          float acc = 0.f;
#pragma unroll
          for (int q = 0; q < Q; ++q) acc += v[u][q];
          for (int t = lane + 64 * Q; t < n_ss; t += 64) acc += p[t];
          inv = 1.0f / sqrtf(wave_sum(acc) / (float)H + eps);
        }
        if (lane == 0) out[r] = inv;
      }
    }
  }

};

// Values a narrow epilogue loads for its (up to) two items per thread before
// the K loop: the residual and the next norm's gain at the item's column, and
// the first 8 x 64 per-16-column sums of squares of (up to) two of the rows
// whose 1/rms this wave computes after the loop.
struct NarrowPre {
  float x[2];
  float g[2];
  float ss[2][8];
};

// 1/rms of the rows of the tile an epilogue works on: filled by the
// epilogue's prepare() (before the tile is complete where possible), read by
// its apply().
__device__ __forceinline__ float* row_scale_lds() {
  __shared__ float srs[128];
  return srs;
}

// Inputs of the next RMSNorm written by a producer epilogue: xg = x * g rounded
// to T (xg == null: nothing written).
template <typename T> struct NextNorm {
  T* xg;
  const T* g;
  int blk;  // xg in the 16 x 32 blocks of act_off
};

// 16 bytes per lane from global memory into LDS at (wave-uniform base) + 16 *
// lane.  Inline assembly, so the compiler's wait insertion does not treat the
// load as a pending LDS write before every LDS read (it would wait for all
// stages in flight); the kernel waits for its stages itself, before the
// barrier that precedes the reads.
__device__ __forceinline__ void dma16(const void* g, const void* lds_wave_base) {
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
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------- main kernel
// Fragments of one 64-wide K step (two 32-column chunks c, c+1): the lane's
// record of each chunk of its two slabs (B) and the matching 8 K elements
// 32 c + 8 (l / 16) .. of its A rows.  The K loop double-buffers steps in
// registers so the next step's weight loads are in flight during the MFMAs.
template <typename T, int MB, class ASrc, int NSL = 2> struct Step64 {
  Frag<T> a0[MB], a1[MB], b0[NSL], b1[NSL];
  __device__ __forceinline__ void load_b(const T* const* bp, int c) {
#pragma unroll
    for (int nb = 0; nb < NSL; ++nb) {
      load_frag(b0[nb], bp[nb] + (int64_t)c * kChunkElems);
      load_frag(b1[nb], bp[nb] + (int64_t)(c + 1) * kChunkElems);
    }
  }
  __device__ __forceinline__ void load_a(const ASrc& asrc,
                                         const typename ASrc::template State<MB>& as, int c,
                                         int g4) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      asrc.template load<MB>(a0[mb], as, mb, c * 32 + g4 * 8);
      asrc.template load<MB>(a1[mb], as, mb, c * 32 + 32 + g4 * 8);
    }
  }
  __device__ __forceinline__ void load(const ASrc& asrc, const typename ASrc::template State<MB>& as,
                                       const T* const* bp, int c, int g4) {
    load_b(bp, c);
    load_a(asrc, as, c, g4);
  }
  __device__ __forceinline__ void mma_into(f32x4 (&acc)[MB][NSL]) const {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NSL; ++nb) {
        mma(acc[mb][nb], a0[mb], b0[nb]);
        mma(acc[mb][nb], a1[mb], b1[nb]);
      }
  }
};

template <typename T, int MB, class ASrc, class Epi>
__global__ __launch_bounds__(256) void gemm_stream(ASrc asrc, int M, int K, int KS, int Kc,
                                                   int m_tiles, float* __restrict__ partial,
                                                   Epi epi) {
  __shared__ float tile[16 * MB * LDT];
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

  const T* bp[2];  // this lane's record in chunk 0 of the wave's two slabs
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) bp[nb] = epi.bslab(nt, wave * 2 + nb) + lane * 8;
  typename ASrc::template State<MB> as;
  asrc.template setup<MB>(as, m0, M, r16);

  f32x4 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  int c = k0 / 32;  // chunk index (k0, k1 are multiples of 32)
  if ((k1 - k0) & 32) {  // a single chunk first when the range is not a multiple of 64
    Frag<T> b0[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) load_frag(b0[nb], bp[nb] + (int64_t)c * kChunkElems);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      Frag<T> a0;
      asrc.template load<MB>(a0, as, mb, c * 32 + g4 * 8);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) mma(acc[mb][nb], a0, b0[nb]);
    }
    ++c;
  }
  // 64-wide steps through a ring of NB register buffers: NB - 1 steps of
  // weight loads stay in flight while a step's MFMAs run (buffer indices are
  // compile-time constants: step s lives in buf[s % NB])
  constexpr int NB = MB == 4 ? 3 : 4;
  const int n64 = (k1 / 32 - c) / 2;
  Step64<T, MB, ASrc> buf[NB];
#pragma unroll
  for (int b = 0; b < NB - 1; ++b)
    if (b < n64) buf[b].load(asrc, as, bp, c + 2 * b, g4);
  for (int i = 0; i < n64; i += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int st = i + b, nxt = st + NB - 1;
      if (st < n64) {
        if (nxt < n64) buf[(b + NB - 1) % NB].load(asrc, as, bp, c + 2 * nxt, g4);
        buf[b].mma_into(acc);
      }
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
    epi.prepare(16 * MB, m0, M, tid);
    epi.apply(tile, 16 * MB, m0, M, nt, tid);
    return;
  }
  // Split K: store this split's partial tile; gemm_splitk_reduce sums the
  // splits in a fixed order in the next kernel and runs the epilogue.
  const int tile_elems = 16 * MB * BN;
  float* mine = partial + ((int64_t)(nt * m_tiles + mt) * KS + ks) * tile_elems;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mine[(mb * 16 + g4 * 4 + i) * BN + wave * 32 + nb * 16 + r16] = acc[mb][nb][i];
}

// ---------------------------------------------------------------- narrow tiles
// Weight streaming for up to 64 rows with the K split inside the workgroup: a
// workgroup owns NSL packed slabs (16 NSL output columns, its column group g)
// over the whole K; its NW waves stream disjoint contiguous K ranges of all
// NSL slabs (wave w: [w kw, w kw + kw)), each into its own accumulators,
// through a ring of NB register buffers.  The NW partial tiles are then summed
// in LDS in wave order -- a fixed order, so the result does not depend on
// timing -- and the epilogue runs in the same kernel: no partial tiles in HBM
// and no second kernel.  The K ranges depend only on (Ncols, K), so a row's
// bits do not depend on how many rows share the call.
//
// Narrow epilogue interface: nslab(n0) = the packed slab holding output
// columns [n0, n0 + 16) of the epilogue's column space; nprepare() as
// prepare(); napply(tile, ldt, rows, m0, M, n0, ncols, tid) over columns
// [n0, n0 + ncols) with ncols a multiple of 16.
template <typename T, int MB, int NSL, int NSW, int NW, int NB, int MINW, class ASrc, class Epi,
          bool SA = false>
__global__ __launch_bounds__(NW * 64, MINW) void gemm_rows(ASrc asrc, int M, int K, int kq_len,
                                                           int ksw, int m_tiles, Epi epi_all) {
  constexpr int TR = 16 * MB, TC = 16 * NSL;
  constexpr int LDR = TC + 4;  // padded row of the summed tile (floats)
  constexpr int WC = 16 * NSW;  // columns of one wave's partial tile
  constexpr int NG = NSL / NSW;  // slab groups; wave = ks * NG + group
  constexpr int KSPL = NW / NG;  // K splits
  static_assert(NSL % NSW == 0 && NW % NG == 0, "waves cover slab groups x K splits");
  static_assert(!SA || (MB == 1 && sizeof(T) == 2), "the LDS image holds 16 bf16 rows");
  // SA: the tile's A rows copied once into an LDS image that every wave reads
  // (the NG waves of a K split would each load the same A fragments), sharing
  // LDS with the partial tiles, which are written only after every wave has
  // left the K loop
  constexpr int RED_BYTES = NW * TR * WC * 4, IMG_BYTES = SA ? 16 * kImgK * 2 : 0;
  __shared__ __attribute__((aligned(1024))) char lbuf[RED_BYTES > IMG_BYTES ? RED_BYTES : IMG_BYTES];
  float* const red = reinterpret_cast<float*>(lbuf);
  __shared__ float tile[TR * LDR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kq = (int)blockIdx.x % ksw, rest = (int)blockIdx.x / ksw;
  const int mt = rest % m_tiles, g = rest / m_tiles;
  const int m0 = mt * TR, n0 = g * TC;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int sg = wave % NG, ksp = wave / NG;
  // this workgroup's K range [kr0, kr1) (ksw > 1: one of ksw ranges, each
  // written as its own partial by the epilogue, for a consumer that sums them)
  const int kr0 = imin(K, kq * kq_len), kr1 = imin(K, kr0 + kq_len);
  const Epi epi = epi_all.nsplit(kq);

  // slab addresses from the kernel argument itself (nsplit changes outputs
  // only): a table indexed at run time stays in the argument segment rather
  // than in scratch memory under the workgroup's copy
  const T* bp[NSW];  // this lane's record in chunk 0 of each of the wave's slabs
#pragma unroll
  for (int s = 0; s < NSW; ++s) bp[s] = epi_all.nslab(n0 + 16 * (sg * NSW + s)) + lane * 8;
  if constexpr (SA) {
    // the image: the fragment of columns 32 c .. copied by wave c mod NW (lane
    // l: 16 bytes of row l mod 16 at column 32 c + 8 (l / 16)), every copy
    // issued before any weight load
    const int r = imin(m0 + (lane & 15), M - 1);
    const T* arow = asrc.A + act_off(block_row(r, asrc.S), 0, asrc.lda, asrc.blk) + (lane >> 4) * 8;
    const int64_t cstride = asrc.blk ? 512 : 32;
    for (int c = wave; c < K / 32; c += NW)
      dma16(arow + c * cstride, reinterpret_cast<T*>(lbuf) + c * 512);
  }
  auto src = [&]() {
    if constexpr (SA) return ASrcImg<T>{reinterpret_cast<const T*>(lbuf)};
    else return asrc;
  }();
  using AS = decltype(src);
  typename AS::template State<MB> as;
  src.template setup<MB>(as, m0, M, r16);

  f32x4 acc[MB][NSW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int s = 0; s < NSW; ++s) acc[mb][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The waves' K splits interleave by 64-wide step (split ksp takes steps
  // ksp, ksp + KSPL, ... of the range), so the waves of a slab group read one
  // contiguous run of the slabs at a time; an odd last 32-chunk goes to split 0.
  const int c0 = kr0 / 32;  // first chunk (kr0, kr1 are multiples of 32)
  const int steps = (kr1 - kr0) / 64;
  auto odd_chunk = [&]() {
    if (((kr1 - kr0) & 32) && ksp == 0) {  // the odd chunk
      const int c = kr1 / 32 - 1;
      Frag<T> b0[NSW];
#pragma unroll
      for (int s = 0; s < NSW; ++s) load_frag(b0[s], bp[s] + (int64_t)c * kChunkElems);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        Frag<T> a0;
        src.template load<MB>(a0, as, mb, c * 32 + g4 * 8);
#pragma unroll
        for (int s = 0; s < NSW; ++s) mma(acc[mb][s], a0, b0[s]);
      }
    }
  };
  if constexpr (!SA) odd_chunk();
  const int n64 = steps > ksp ? (steps - ksp + KSPL - 1) / KSPL : 0;
  auto chunk_of = [&](int st) { return c0 + 2 * (ksp + st * KSPL); };
  Step64<T, MB, AS, NSW> buf[NB];
  if constexpr (SA) {
    // the first steps' weight loads go out, then the wait for this lane's
    // image copies (older than those loads: at most their 2 NSW per step may
    // stay in flight) and the barrier that covers every wave's copies
#pragma unroll
    for (int b = 0; b < NB - 1; ++b)
      if (b < n64) buf[b].load_b(bp, chunk_of(b));
    static_assert(NB - 1 <= 2 && 2 * NSW * 2 <= 63, "waits below cover the prologue");
    const int in_flight = imin(NB - 1, n64);
    if (in_flight >= 2) wait_vmcnt<4 * NSW>();
    else if (in_flight == 1) wait_vmcnt<2 * NSW>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int b = 0; b < NB - 1; ++b)
      if (b < n64) buf[b].load_a(src, as, chunk_of(b), g4);
    odd_chunk();
  } else {
#pragma unroll
    for (int b = 0; b < NB - 1; ++b)
      if (b < n64) buf[b].load(src, as, bp, chunk_of(b), g4);
  }
  // while those loads are in flight: the loads of what the epilogue reads
  // (residual, gains) and of the sums of squares behind the row scales
  NarrowPre pre;
  epi.nfetch(pre, TR, m0, M, n0, TC, tid);
  epi.nrow_pre(pre, TR, m0, M, wave, NW, lane);
  for (int i = 0; i < n64; i += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int st = i + b, nxt = st + NB - 1;
      if (st < n64) {
        if (nxt < n64) buf[(b + NB - 1) % NB].load(src, as, bp, chunk_of(nxt), g4);
        buf[b].mma_into(acc);
      }
    }
  }
  // the row scales of the epilogue (one wave per row; published by the
  // barrier below), this wave's partial tile, then the sum over the K splits
  // in split order
  epi.nrow_fin(pre, row_scale_lds(), TR, m0, M, wave, NW, lane);
  if constexpr (SA) __syncthreads();  // every wave is done with the image
  float* mine = red + wave * (TR * WC);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int s = 0; s < NSW; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[(mb * 16 + g4 * 4 + i) * WC + s * 16 + r16] = acc[mb][s][i];
  __syncthreads();
  for (int e = tid; e < TR * TC; e += NW * 64) {
    const int r = e / TC, cc = e % TC, grp = cc / WC;
    const float* src = red + (grp * TR + r) * WC + cc % WC;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < KSPL; ++k) v += src[k * NG * TR * WC];
    tile[r * LDR + cc] = v;
  }
  __syncthreads();
  constexpr int J = (TR * NSL + 4 * NW - 1) / (4 * NW);  // epilogue items per thread
  epi.template napply<J>(tile, LDR, TR, m0, M, n0, TC, tid, pre);
}

// Row pass of a narrow epilogue: item (row r, 16-column group q) goes to a
// 16-lane group, lane i = column 16 q + i; every lane of a wave runs the same
// iterations (the 16-lane reductions are wave-uniform), J items per thread
// (rows x groups <= 4 x waves x J).  narrow_item() gives the thread's item j
// (the same for the prefetch before the K loop, which covers j < 2, and the
// pass after it).
// f(r, c, m, n, j) returns the value stored for tile (r, c) = output (m, n);
// its squares are summed per 16-column group into ss (nullable) and v *
// pre.g[j] (the next norm's gain at n) is written to xg.
struct NarrowItem {
  bool in;       // an item of the tile (the wave-uniform part of the bound)
  bool act;      // ... and inside the output
  int r, c, m, n;
};
__device__ __forceinline__ NarrowItem narrow_item(int j, int rows, int m0, int M, int n0,
                                                  int ncols, int N, int tid) {
  const int lane = tid & 63, wave = tid >> 6, nw = (int)(blockDim.x >> 6);
  const int ng = ncols / 16, items = rows * ng;
  const int b = wave * 4 + j * nw * 4, it = b + (lane >> 4);
  NarrowItem t;
  t.in = b < items;
  t.r = it / ng;
  t.c = (it % ng) * 16 + (lane & 15);
  t.m = m0 + t.r;
  t.n = n0 + t.c;
  t.act = it < items && t.m < M && t.n < N;
  return t;
}
template <int J, typename T, typename F>
__device__ __forceinline__ void narrow_rows(int rows, int m0, int M, int n0, int ncols, int N,
                                            int tid, float* ss, int n_ss, const NextNorm<T>& nn,
                                            const NarrowPre& pre, F&& f) {
  const int lane = tid & 63;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const NarrowItem t = narrow_item(j, rows, m0, M, n0, ncols, N, tid);
    if (!t.in) break;
    float v = 0.f;
    if (t.act) {
      v = f(t.r, t.c, t.m, t.n, j);
      if (nn.xg != nullptr) {
        // the gain prefetched for the first two items, loaded for later ones
        const float gj = j < 2 ? pre.g[j < 2 ? j : 0] : Num<T>::to_f(nn.g[t.n]);
        nn.xg[act_off(t.m, t.n, N, nn.blk)] = Num<T>::from_f(v * gj);
      }
    }
    if (ss != nullptr) {
      const float q = row16_sum(t.act ? v * v : 0.f);
      if ((lane & 15) == 0 && t.act) ss[(int64_t)t.m * n_ss + t.n / 16] = q;
    }
  }
}
// The next norm's gains (and with x != null the residual) at a thread's items.
template <typename T>
__device__ __forceinline__ void narrow_fetch(NarrowPre& pre, const float* x, const T* g, int rows,
                                             int m0, int M, int n0, int ncols, int N, int tid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const NarrowItem t = narrow_item(j, rows, m0, M, n0, ncols, N, tid);
    pre.x[j] = (x != nullptr && t.act) ? x[(int64_t)t.m * N + t.n] : 0.f;
    pre.g[j] = (g != nullptr && t.act) ? Num<T>::to_f(g[t.n]) : 0.f;
  }
}

// ---------------------------------------------------------------- tiled kernel
// LDS-tiled MFMA GEMM for M > 64 (bf16): a BM x 128 tile per workgroup, 4 waves
// in a 2 x 2 grid (each BM/2 x 64), K in 64-wide stages double-buffered in LDS
// (A rows padded to 144 bytes so the 16-row fragment reads are conflict-free;
// the B stage is the packed records as they lie in memory, read 1 KB per wave),
// the next stage's global loads in flight during the current stage's MFMAs.
// The grid keeps the M tiles of one column tile on one XCD (workgroup i runs on
// XCD i % 8), so the weight tile one of them fetched is still in that XCD's L2
// when the others read it.  Epilogue in 128-row halves through the staging LDS.
constexpr int FBK = 64;          // K per stage
constexpr int FLD = FBK + 8;     // LDS row stride (elements)
constexpr int FGM = 4;           // row tiles per group of the tile order

// Workgroups of a tiled launch: the tile count rounded up to a multiple of 8.
__host__ __forceinline__ int fat_grid(const GemmPlan& p) {
  return (p.KS * p.m_tiles * p.n_tiles + 7) / 8 * 8;
}

template <int BMt, class Epi>
__global__ __launch_bounds__(256) void gemm_fat(ASrcPlain<bf16_t> asrc, int M, int K, int KS,
                                                int Kc, int m_tiles, int n_tiles,
                                                float* __restrict__ partial, Epi epi) {
  constexpr int TM = BMt / 32;                         // 16-row blocks per wave
  constexpr int STAGE = BMt * FLD + BN * FBK;          // bf16 elements per stage
  constexpr int LDS_BYTES = 2 * STAGE * 2;
  constexpr int EPI_BYTES = 128 * LDT * 4;
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES > EPI_BYTES ? LDS_BYTES : EPI_BYTES];
  bf16_t* lds = reinterpret_cast<bf16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, r16 = lane & 15, g4 = lane >> 4;

  // Workgroup i is dispatched to XCD i % 8: give every XCD a contiguous range
  // of tiles, ordered (ks slowest) in groups of FGM row tiles, so the ~32
  // workgroups an XCD runs at once cover FGM row tiles x 32/FGM column tiles
  // and share both operands' stages in that XCD's L2.
  const int n_all = KS * m_tiles * n_tiles;
  const int per = (n_all + 7) / 8;
  const int t = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (t >= n_all) return;  // padding of the last XCD's range
  const int MN = m_tiles * n_tiles;
  const int ks = t / MN, r = t % MN;
  const int first = (r / (FGM * n_tiles)) * FGM;
  const int gsz = imin(m_tiles - first, FGM);
  const int within = r % (FGM * n_tiles);
  const int mt = first + within % gsz, nt = within / gsz;
  const int m0 = mt * BMt;
  const int k0 = ks * Kc, k1 = imin(K, k0 + Kc);

  // global -> register pieces of 16 B: A BMt x 64 (BMt*8 pieces); B the two
  // packed chunks of the stage for each of the tile's 8 slabs (1024 records)
  constexpr int ACH = BMt * 8 / 256, BCH = 1024 / 256;
  const bf16_t* ap[ACH];
  const bf16_t* bp[BCH];
  int acol[ACH];
#pragma unroll
  for (int u = 0; u < ACH; ++u) {
    const int c = tid + 256 * u, row = c / 8;
    acol[u] = (c % 8) * 8;
    ap[u] = asrc.A + (int64_t)block_row(imin(m0 + row, M - 1), asrc.S) * asrc.lda;
  }
#pragma unroll
  for (int u = 0; u < BCH; ++u) {
    const int rec = tid + 256 * u;  // slab rec / 128, chunk (rec / 64) % 2, lane rec % 64
    bp[u] = epi.bslab(nt, rec / 128) + ((rec / 64) % 2) * kChunkElems + (rec % 64) * 8;
  }
  uint4 ra[ACH], rb[BCH];
  auto gload = [&](int k) {
#pragma unroll
    for (int u = 0; u < ACH; ++u)
      ra[u] = (k + acol[u] < k1) ? *reinterpret_cast<const uint4*>(ap[u] + k + acol[u])
                                 : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < BCH; ++u)
      rb[u] = (k + ((tid + 256 * u) / 64) % 2 * 32 < k1)
                  ? *reinterpret_cast<const uint4*>(bp[u] + (int64_t)(k / 32) * kChunkElems)
                  : make_uint4(0, 0, 0, 0);
  };
  auto sstore = [&](int buf) {
    bf16_t* As = lds + buf * STAGE;
    bf16_t* Bs = As + BMt * FLD;
#pragma unroll
    for (int u = 0; u < ACH; ++u) {
      const int c = tid + 256 * u;
      *reinterpret_cast<uint4*>(As + (c / 8) * FLD + acol[u]) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < BCH; ++u)
      *reinterpret_cast<uint4*>(Bs + (tid + 256 * u) * 8) = rb[u];
  };

  f32x4 acc[TM][4];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_it = (k1 - k0 + FBK - 1) / FBK;
  if (n_it > 0) {
    gload(k0);
    sstore(0);
    __syncthreads();
    for (int it = 0; it < n_it; ++it) {
      const int buf = it & 1;
      if (it + 1 < n_it) gload(k0 + (it + 1) * FBK);
      const bf16_t* As = lds + buf * STAGE;
      const bf16_t* Bs = As + BMt * FLD;
#pragma unroll
      for (int kk = 0; kk < FBK / 32; ++kk) {
        Frag<bf16_t> bf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          load_frag(bf[j], Bs + ((wn * 4 + j) * 2 + kk) * kChunkElems + lane * 8);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          Frag<bf16_t> af;
          load_frag(af, As + (wm * (BMt / 2) + i * 16 + r16) * FLD + kk * 32 + g4 * 8);
#pragma unroll
          for (int j = 0; j < 4; ++j) mma(acc[i][j], af, bf[j]);
        }
      }
      if (it + 1 < n_it) sstore(buf ^ 1);
      __syncthreads();
    }
  }

  if (KS > 1) {
    // split partial tile [BMt][128] of this K range
    float* mine = partial + ((int64_t)(nt * m_tiles + mt) * KS + ks) * (BMt * BN);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          mine[(wm * (BMt / 2) + i * 16 + g4 * 4 + e) * BN + wn * 64 + j * 16 + r16] = acc[i][j][e];
    return;
  }
  float* tile = reinterpret_cast<float*>(smem);
  constexpr int HALVES = BMt / 128;
#pragma unroll
  for (int h = 0; h < HALVES; ++h) {
    // rows [128 h, 128 h + 128) of the tile: written by the waves that own them
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * (BMt / 2) + i * 16;   // tile row of this block
      if (row / 128 != h) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          tile[(row % 128 + g4 * 4 + e) * LDT + wn * 64 + j * 16 + r16] = acc[i][j][e];
    }
    __syncthreads();
    epi.prepare(128, m0 + 128 * h, M, tid);
    epi.apply(tile, 128, m0 + 128 * h, M, nt, tid);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- large tiles
// LDS-tiled MFMA GEMM for many rows (bf16, no split K): a 256 x 256 tile per
// workgroup of 8 waves (2 x 4, each 128 x 64), K in 32-wide stages that go
// from global memory straight into LDS (global_load_lds, 16 bytes per lane, so
// one wave instruction fills 1 KB: 16 A rows of 64 bytes, or one packed B
// chunk), a ring of 4 stages with 3 in flight and one barrier per stage.  The
// A rows of a stage are unpadded; a fragment read covers 1 KB contiguously.
// Same XCD-grouped tile order as gemm_fat; epilogue in 128 x 128 quarters.
constexpr int GB_STAGE = 256 * 32 + 256 * 32;  // bf16 elements: A [256][32], B [16 slabs][64][8]
constexpr int GB_NS = 4;

template <class Epi>
__global__ __launch_bounds__(512) void gemm_big(ASrcPlain<bf16_t> asrc, int M, int K, int m_tiles,
                                                int n_tiles, int n_tiles128, int KS, int Kc,
                                                float* __restrict__ partial, Epi epi) {
  constexpr int SMEM = 2 * 128 * LDT * 4 > GB_NS * GB_STAGE * 2 ? 2 * 128 * LDT * 4
                                                                 : GB_NS * GB_STAGE * 2;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  bf16_t* const st0 = reinterpret_cast<bf16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3, r16 = lane & 15, g4 = lane >> 4;
  // work item u = kb * tiles + t (K split slowest); XCD x (= workgroup id
  // mod 8) takes a contiguous range of items
  const int n_tile = m_tiles * n_tiles, n_all = n_tile * KS;
  const int per = (n_all + 7) / 8;
  const int u = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (u >= n_all) return;  // padding of the last XCD's range
  const int kb = u / n_tile, t = u % n_tile;
  const int k0 = kb * Kc, klen = imin(Kc, K - k0);
  const int first = (t / (FGM * n_tiles)) * FGM;
  const int gsz = imin(m_tiles - first, FGM);
  const int within = t % (FGM * n_tiles);
  const int mt = first + within % gsz, nt = within / gsz;
  const int m0 = mt * 256;
  // this wave's two A pieces (16 rows x 32 K; lane: row l / 4, 8 columns at
  // 8 (l % 4)) and two B slabs (slab s of the 256 columns: 128-column tile
  // 2 nt + s / 8, slab s % 8 of it)
  const bf16_t* ag[2];
  const bf16_t* bg[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int row = (wave * 2 + v) * 16 + lane / 4;
    ag[v] = asrc.A + (int64_t)block_row(imin(m0 + row, M - 1), asrc.S) * asrc.lda + (lane % 4) * 8 +
            k0;
    const int s = wave * 2 + v;
    bg[v] = epi.bslab(imin(2 * nt + s / 8, n_tiles128 - 1), s % 8) + lane * 8 +
            (int64_t)(k0 / 32) * kChunkElems;
  }
  auto issue = [&](bf16_t* stg, int c) {  // stage of K columns [32 c, 32 c + 32)
#pragma unroll
    for (int v = 0; v < 2; ++v) dma16(ag[v] + c * 32, stg + (wave * 2 + v) * 512);
#pragma unroll
    for (int v = 0; v < 2; ++v)
      dma16(bg[v] + (int64_t)c * kChunkElems, stg + 256 * 32 + (wave * 2 + v) * 512);
  };
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const bf16_t* stg) {
    Frag<bf16_t> bf[4], af[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) load_frag(bf[j], stg + 256 * 32 + (wn * 4 + j) * 512 + lane * 8);
    load_frag(af[0], stg + (wm * 128 + r16) * 32 + g4 * 8);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i + 1 < 8) load_frag(af[(i + 1) & 1], stg + (wm * 128 + (i + 1) * 16 + r16) * 32 + g4 * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) mma(acc[i][j], af[i & 1], bf[j]);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read,
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // then four MFMAs
    }
    __builtin_amdgcn_s_setprio(0);
  };
  const int n_it = klen / 32;
  bf16_t* const st1 = st0 + GB_STAGE;
  bf16_t* const st2 = st1 + GB_STAGE;
  bf16_t* const st3 = st2 + GB_STAGE;
  if (0 < n_it) issue(st0, 0);
  if (1 < n_it) issue(st1, 1);
  if (2 < n_it) issue(st2, 2);
  auto step = [&](int it, bf16_t* cur, bf16_t* nxt) {
    if (it >= n_it) return;
    // this lane's loads of stage it are done once at most those of the later
    // stages (4 per stage) are outstanding; the barrier then covers all lanes,
    // and also guarantees that every wave has finished reading stage it - 1,
    // whose buffer the next issue overwrites
    if (it + 2 < n_it) wait_vmcnt<8>();
    else if (it + 1 < n_it) wait_vmcnt<4>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (it + 3 < n_it) issue(nxt, it + 3);
    compute(cur);
  };
  for (int it0 = 0; it0 < n_it; it0 += 4) {
    step(it0, st0, st3);
    step(it0 + 1, st1, st0);
    step(it0 + 2, st2, st1);
    step(it0 + 3, st3, st2);
  }
  __syncthreads();
  float* tile0 = reinterpret_cast<float*>(smem);
  float* tile1 = tile0 + 128 * LDT;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // rows [128 h, 128 h + 128): waves (h, 0..1) hold columns 0..127, (h, 2..3) 128..255
    if (wm == h) {
      float* tl = (wn < 2 ? tile0 : tile1) + (wn & 1) * 64;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) tl[(i * 16 + g4 * 4 + e) * LDT + j * 16 + r16] = acc[i][j][e];
    }
    __syncthreads();
    if (KS == 1) {
      epi.prepare(128, m0 + 128 * h, M, tid);
      epi.apply(tile0, 128, m0 + 128 * h, M, 2 * nt, tid);
      epi.apply(tile1, 2 * nt + 1 < n_tiles128 ? 128 : 0, m0 + 128 * h, M, 2 * nt + 1, tid);
    } else {
      // split partial: rows [128 h, 128 h + 128) of the two 128-column tiles,
      // in the reduce kernel's layout [(nt128 * m_tiles + mt) * KS + kb][256][128]
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int n128 = 2 * nt + q;
        if (n128 >= n_tiles128) break;
        const float* src = q ? tile1 : tile0;
        float* dst = partial + ((int64_t)(n128 * m_tiles + mt) * KS + kb) * (256 * BN) +
                     (int64_t)(128 * h) * BN;
        for (int i = tid; i < 128 * BN / 4; i += 512) {
          const int r = i / (BN / 4), c = (i % (BN / 4)) * 4;
          *reinterpret_cast<float4*>(dst + r * BN + c) =
              make_float4(src[r * LDT + c], src[r * LDT + c + 1], src[r * LDT + c + 2],
                          src[r * LDT + c + 3]);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- tall tiles
// 65..128 rows (bf16) with many column tiles (the lm_head): every weight byte
// is used by at most 128 rows, so the kernel is bound by the weight stream.
// One 128 x 128 tile per workgroup (all rows, one 128-column tile) of 8 waves
// (2 x 4, each 64 x 32: 4 x 2 MFMA blocks), K in 32-wide stages copied
// straight into LDS as in gemm_big (a wave copies one 16-row A piece and one
// packed B slab: 2 KB of the stage's 16 KB), a ring of GT_NS stages with
// GT_NS - 1 in flight, one barrier per stage; the ring and the epilogue tile
// share 68 KB, so two workgroups run on a CU (48 KB of weights in flight per
// CU; a deeper ring with one workgroup per CU measured slower).  Column tiles
// run in the XCD-grouped order of the other tiled kernels, so the A rows stay
// in each XCD's L2.  K is whole (a multiple of 32, as every K here is).
constexpr int GT_NS = 4;
constexpr int GT_STAGE = 128 * 32 + 8 * kChunkElems;  // bf16: A [128][32], B [8 slabs][64][8]

// Wait until at most `later` stages of 2 copies per wave are in flight.
template <int K> __device__ __forceinline__ void gt_wait(int later) {
  if constexpr (K <= 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= K) wait_vmcnt<2 * K>();
    else gt_wait<K - 1>(later);
  }
}

template <class Epi>
__global__ __launch_bounds__(512) void gemm_tall(ASrcPlain<bf16_t> asrc, int M, int K, int n_tiles,
                                                 Epi epi) {
  constexpr int RING = GT_NS * GT_STAGE * 2, TILE = 128 * LDT * 4;
  constexpr int SMEM = RING > TILE ? RING : TILE;  // the epilogue tile reuses the ring
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  bf16_t* const ring = reinterpret_cast<bf16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3, r16 = lane & 15, g4 = lane >> 4;
  // XCD x (= workgroup id mod 8) takes a contiguous range of column tiles
  const int per = (n_tiles + 7) / 8;
  const int nt = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (nt >= n_tiles) return;  // padding of the last XCD's range
  // this wave's A piece (rows 16 wave .. + 16; lane: row l / 4, 8 columns at
  // 8 (l % 4); rows past M read row M - 1) and B slab (slab `wave` of tile nt)
  const bf16_t* ag = asrc.A +
                     (int64_t)block_row(imin(wave * 16 + lane / 4, M - 1), asrc.S) * asrc.lda +
                     (lane % 4) * 8;
  const bf16_t* bg = epi.bslab(nt, wave) + lane * 8;
  auto issue = [&](int c) {  // stage of K columns [32 c, 32 c + 32)
    bf16_t* stg = ring + (c % GT_NS) * GT_STAGE;
    dma16(ag + c * 32, stg + wave * 512);
    dma16(bg + (int64_t)c * kChunkElems, stg + 128 * 32 + wave * 512);
  };
  f32x4 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int n_it = K / 32;
#pragma unroll
  for (int c = 0; c < GT_NS - 1; ++c)
    if (c < n_it) issue(c);
  for (int it = 0; it < n_it; ++it) {
    // this lane's copies of stage it are done once at most those of the later
    // stages in flight remain; the barrier then covers every wave, and also
    // guarantees that every wave has finished reading stage it - 1, whose
    // buffer the next issue overwrites
    gt_wait<GT_NS - 2>(imin(GT_NS - 2, n_it - 1 - it));
    __builtin_amdgcn_s_barrier();
    if (it + GT_NS - 1 < n_it) issue(it + GT_NS - 1);
    const bf16_t* stg = ring + (it % GT_NS) * GT_STAGE;
    Frag<bf16_t> bf[2], af[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) load_frag(bf[j], stg + 128 * 32 + (wn * 2 + j) * 512 + lane * 8);
    load_frag(af[0], stg + (wm * 64 + r16) * 32 + g4 * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i + 1 < 4) load_frag(af[(i + 1) & 1], stg + (wm * 64 + (i + 1) * 16 + r16) * 32 + g4 * 8);
#pragma unroll
      for (int j = 0; j < 2; ++j) mma(acc[i][j], af[i & 1], bf[j]);
    }
  }
  __syncthreads();  // every wave is done with the ring: the tile takes its place
  float* tile = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        tile[(wm * 64 + i * 16 + g4 * 4 + e) * LDT + wn * 32 + j * 16 + r16] = acc[i][j][e];
  __syncthreads();
  epi.prepare(128, 0, M, tid);
  epi.apply(tile, 128, 0, M, nt, tid);
}

// Split-K reduction: one workgroup per 4 rows of a tile.  Thread t sums the
// splits q = t/128, t/128 + 2, ... of one float4 column (in split order, all
// loads issued before the adds); the two halves are then added in a fixed
// order, so the result does not depend on timing.
constexpr int RROWS = 4;

// An epilogue with kPrefetch has fetch(), which loads the inputs its apply()
// reads for one row per wave (rows <= the workgroup's waves), and apply_pre(),
// which takes them: the reduce issues fetch() while the partials are in flight.
template <class E, class = void> struct HasPrefetch {
  static constexpr bool value = false;
};
template <class E> struct HasPrefetch<E, decltype((void)E::kPrefetch)> {
  static constexpr bool value = E::kPrefetch;
};

template <int TROWS, class Epi>
__global__ __launch_bounds__(256) void gemm_splitk_reduce(int KS, int m_tiles, int M,
                                                          const float* __restrict__ partial,
                                                          Epi epi) {
  __shared__ float tile[RROWS * LDT];
  __shared__ float4 half1[RROWS * BN / 4];
  const int tid = threadIdx.x;
  constexpr int RB = TROWS / RROWS;  // row blocks per tile
  const int tix = blockIdx.x / RB, rb = blockIdx.x % RB;
  const int mt = tix % m_tiles, nt = tix / m_tiles;
  const int tile_elems = TROWS * BN;
  const int i4 = tid & 127, h = tid >> 7;
  const int row = i4 / (BN / 4), c = (i4 % (BN / 4)) * 4;
  const float* p = partial + (int64_t)tix * KS * tile_elems + (int64_t)(rb * RROWS + row) * BN + c;
  // the loads of (up to) the first 32 splits go out first; the epilogue's
  // own inputs (row scales, residual rows) are fetched while they are in flight
  constexpr int QB = 16;
  float4 v[QB];
#pragma unroll
  for (int u = 0; u < QB; ++u)
    v[u] = (h + 2 * u < KS) ? *reinterpret_cast<const float4*>(p + (int64_t)(h + 2 * u) * tile_elems)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
  epi.prepare(RROWS, mt * TROWS + rb * RROWS, M, tid);
  float pre[4];
  if constexpr (HasPrefetch<Epi>::value) epi.fetch(RROWS, mt * TROWS + rb * RROWS, M, nt, tid, pre);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < QB; ++u) {
    s.x += v[u].x;
    s.y += v[u].y;
    s.z += v[u].z;
    s.w += v[u].w;
  }
  for (int q = h + 2 * QB; q < KS; q += 2) {
    const float4 w = *reinterpret_cast<const float4*>(p + (int64_t)q * tile_elems);
    s.x += w.x;
    s.y += w.y;
    s.z += w.z;
    s.w += w.w;
  }
  if (h == 1) half1[i4] = s;
  __syncthreads();
  if (h == 0) {
    const float4 o = half1[i4];
    float* t = tile + row * LDT + c;
    t[0] = s.x + o.x;
    t[1] = s.y + o.y;
    t[2] = s.z + o.z;
    t[3] = s.w + o.w;
  }
  __syncthreads();
  if constexpr (HasPrefetch<Epi>::value)
    epi.apply_pre(tile, RROWS, mt * TROWS + rb * RROWS, M, nt, tid, pre);
  else
    epi.apply(tile, RROWS, mt * TROWS + rb * RROWS, M, nt, tid);
}

// ---------------------------------------------------------------- epilogues
// Epilogues run on every thread of the workgroup (any multiple of 64 threads).
// Row-wise pass over a [rows, 128] fp32 tile (one wave per row, two columns per
// lane); f returns the value stored for (row, col), whose squares are summed
// into the row's partial sum of squares over the tile when ss != null.
// gpre: the next norm's gains at the lane's two columns, already loaded (or null).
template <typename T, typename FL, typename F>
__device__ __forceinline__ void for_rows(int rows, int m0, int M, int nt, int N, int tid,
                                         float* ss, int n_ss, const NextNorm<T>& nn, FL&& in,
                                         F&& f, const float* gpre = nullptr) {
  const int lane = tid & 63, wave = tid >> 6, nw = (int)(blockDim.x >> 6);
  float gn[2] = {0.f, 0.f};  // the next norm's gain at this lane's two columns
  if (nn.xg != nullptr) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int n = nt * BN + lane + 64 * h;
      gn[h] = gpre != nullptr ? gpre[h] : (n < N ? Num<T>::to_f(nn.g[n]) : 0.f);
    }
  }
  // rows in groups of 4 per wave: the group's input loads go out before any
  // of its rows is finished
  constexpr int G = 4;
  for (int r0 = wave; r0 < rows; r0 += nw * G) {
    float iv[G][2];
#pragma unroll
    for (int u = 0; u < G; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = r0 + nw * u, m = m0 + r, n = nt * BN + lane + 64 * h;
        iv[u][h] = (r < rows && m < M && n < N) ? in(m, n) : 0.f;
      }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int r = r0 + nw * u, m = m0 + r;
      if (r >= rows) break;
      if (m >= M) continue;
      float sq[2] = {0.f, 0.f};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = lane + 64 * h, n = nt * BN + c;
        if (n < N) {
          const float v = f(r, c, m, n, iv[u][h]);
          sq[h] = v * v;
          if (nn.xg != nullptr) nn.xg[act_off(m, n, N, nn.blk)] = Num<T>::from_f(v * gn[h]);
        }
      }
      if (ss != nullptr) {
        // per 16-column group: lanes 16 q .. 16 q + 15 hold columns 16 q + i
        // (h = 0) and 64 + 16 q + i (h = 1) of the tile
        const float s0 = row16_sum(sq[0]), s1 = row16_sum(sq[1]);
        if ((lane & 15) == 0) {
          const int t0 = nt * (BN / 16) + (lane >> 4), t1 = t0 + 4;
          if (t0 < n_ss) ss[(int64_t)m * n_ss + t0] = s0;
          if (t1 < n_ss) ss[(int64_t)m * n_ss + t1] = s1;
        }
      }
    }
  }
}

template <typename T> struct EpiStoreF32 {
  const T* W; int N; int K; float* out; int ldo; float* ss; NextNorm<T> nn; RowScale rs;
  int64_t split_stride;  // elements between the partials of K ranges (gemm_rows ksw > 1)
  static constexpr int kNarrow = 1;
  static constexpr bool kRowScale = true;
  __device__ EpiStoreF32 nsplit(int kq) const {
    EpiStoreF32 e = *this;
    if (kq > 0) e.out += kq * split_stride;
    return e;
  }
  // rows of an RMSNorm-scaled A source are multiplied by 1/rms (1 for a plain source)
  __device__ void prepare(int rows, int m0, int M, int tid) const {
    rs.fill(row_scale_lds(), rows, m0, M, tid);
  }
  __device__ const T* bslab(int nt, int s) const {
    return W + (int64_t)(imin(nt * BN + 16 * s, N - 1) / 16) * slab_elems(K);
  }
  __device__ void apply(const float* t, int rows, int m0, int M, int nt, int tid) const {
    const float* srs = row_scale_lds();
    for_rows(rows, m0, M, nt, N, tid, ss, ss_tiles(N), nn, [&](int, int) { return 0.f; },
             [&](int r, int c, int m, int n, float) {
               const float v = t[r * LDT + c] * srs[r];
               if (out != nullptr) out[(int64_t)m * ldo + n] = v;
               return v;
             });
  }
  // narrow tiles (gemm_rows)
  __device__ const T* nslab(int n0) const {
    return W + (int64_t)(imin(n0, N - 1) / 16) * slab_elems(K);
  }
  __device__ void nrow_pre(NarrowPre& pre, int rows, int m0, int M, int wave, int nw,
                           int lane) const {
    rs.pre_rows(pre.ss, rows, m0, M, wave, nw, lane);
  }
  __device__ void nrow_fin(const NarrowPre& pre, float* srs, int rows, int m0, int M, int wave,
                           int nw, int lane) const {
    rs.finish_rows(pre.ss, srs, rows, m0, M, wave, nw, lane);
  }
  __device__ void nfetch(NarrowPre& pre, int rows, int m0, int M, int n0, int ncols,
                         int tid) const {
    narrow_fetch<T>(pre, nullptr, nn.xg != nullptr ? nn.g : nullptr, rows, m0, M, n0, ncols, N,
                    tid);
  }
  template <int J>
  __device__ void napply(const float* t, int ldt, int rows, int m0, int M, int n0, int ncols,
                         int tid, const NarrowPre& pre) const {
    const float* srs = row_scale_lds();
    narrow_rows<J>(rows, m0, M, n0, ncols, N, tid, ss, ss_tiles(N), nn, pre,
                   [&](int r, int c, int m, int n, int) {
                  const float v = t[r * ldt + c] * srs[r];
                  if (out != nullptr) out[(int64_t)m * ldo + n] = v;
                  return v;
                });
  }
};

// The QKV store of the narrow path: EpiStoreF32 on kQkvSlabs slabs per
// workgroup (its consumer adds the K-range partials).
template <typename T> struct EpiQKVStore : EpiStoreF32<T> {
  static constexpr int kNarrow = kQkvSlabs;
  __device__ EpiQKVStore nsplit(int kq) const {
    EpiQKVStore e = *this;
    if (kq > 0) e.out += kq * this->split_stride;
    return e;
  }
};

// Layers the narrow K/V store covers.
constexpr int kKVStoreLayers = DFLASH_MAX_LAYERS;

// The K/V store of an injection of <= 64 rows: EpiStoreF32 over the stacked
// K/V rows of every layer (column n of layer l = n / (2 nkv D) is row nq D +
// n % (2 nkv D) of that layer's w_qkv), on kQkvSlabs slabs per workgroup; its
// consumer adds the K-range partials and applies k_norm, RoPE and the cache
// write.
template <typename T> struct EpiKVStore : EpiStoreF32<T> {
  static constexpr int kNarrow = kQkvSlabs;
  int per;                     // 2 nkv D
  int qoff;                    // nq D
  const void* wl[kKVStoreLayers];  // the layers' w_qkv
  __device__ EpiKVStore nsplit(int kq) const {
    EpiKVStore e = *this;
    if (kq > 0) e.out += kq * this->split_stride;
    return e;
  }
  __device__ const T* nslab(int n0) const {
    const int n = imin(n0, this->N - 1), l = n / per, w = n % per;
    return static_cast<const T*>(wl[l]) + (int64_t)((qoff + w) / 16) * slab_elems(this->K);
  }
};

template <typename T> struct EpiResidual {
  const T* W; int N; int K; float* x; float* ss; NextNorm<T> nn;
  static constexpr int kNarrow = 1;
  static constexpr bool kRowScale = false;
  __device__ EpiResidual nsplit(int) const { return *this; }
  __device__ void prepare(int, int, int, int) const {}
  __device__ const T* bslab(int nt, int s) const {
    return W + (int64_t)(imin(nt * BN + 16 * s, N - 1) / 16) * slab_elems(K);
  }
  __device__ void apply(const float* t, int rows, int m0, int M, int nt, int tid) const {
    for_rows(rows, m0, M, nt, N, tid, ss, ss_tiles(N), nn,
             [&](int m, int n) { return x[(int64_t)m * N + n]; },
             [&](int r, int c, int m, int n, float res) {
               const float v = res + t[r * LDT + c];
               x[(int64_t)m * N + n] = v;
               return v;
             });
  }
  // narrow tiles (gemm_rows)
  __device__ const T* nslab(int n0) const {
    return W + (int64_t)(imin(n0, N - 1) / 16) * slab_elems(K);
  }
  __device__ void nrow_pre(NarrowPre&, int, int, int, int, int, int) const {}
  __device__ void nrow_fin(const NarrowPre&, float*, int, int, int, int, int, int) const {}
  __device__ void nfetch(NarrowPre& pre, int rows, int m0, int M, int n0, int ncols,
                         int tid) const {
    narrow_fetch<T>(pre, x, nn.xg != nullptr ? nn.g : nullptr, rows, m0, M, n0, ncols, N, tid);
  }
  template <int J>
  __device__ void napply(const float* t, int ldt, int rows, int m0, int M, int n0, int ncols,
                         int tid, const NarrowPre& pre) const {
    narrow_rows<J>(rows, m0, M, n0, ncols, N, tid, ss, ss_tiles(N), nn, pre,
                   [&](int r, int c, int m, int n, int j) {
                  // the residual prefetched for the first two items, loaded for later ones
                  const float res = j < 2 ? pre.x[j < 2 ? j : 0] : x[(int64_t)m * N + n];
                  const float v = res + t[r * ldt + c];
                  x[(int64_t)m * N + n] = v;
                  return v;
                });
  }
  // pre = the residual at row m0 + wave, columns nt * BN + lane (+ 64), then
  // the next norm's gains there (for_rows reads exactly these when rows <= waves)
  static constexpr bool kPrefetch = true;
  __device__ void fetch(int rows, int m0, int M, int nt, int tid, float (&pre)[4]) const {
    const int lane = tid & 63, wave = tid >> 6, m = m0 + wave;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int n = nt * BN + lane + 64 * h;
      pre[h] = (wave < rows && m < M && n < N) ? x[(int64_t)m * N + n] : 0.f;
      pre[2 + h] = (nn.xg != nullptr && n < N) ? Num<T>::to_f(nn.g[n]) : 0.f;
    }
  }
  __device__ void apply_pre(const float* t, int rows, int m0, int M, int nt, int tid,
                            const float (&pre)[4]) const {
    for_rows(rows, m0, M, nt, N, tid, ss, ss_tiles(N), nn,
             [&](int, int n) { return n - nt * BN >= 64 ? pre[1] : pre[0]; },
             [&](int r, int c, int m, int n, float res) {
               const float v = res + t[r * LDT + c];
               x[(int64_t)m * N + n] = v;
               return v;
             },
             pre + 2);
  }
};

// Tile columns 0..63 are gate rows nt*64.., columns 64..127 the matching up rows.
template <typename T> struct EpiSiluMul {
  const T* Wg; const T* Wu; int I; int K; T* act; RowScale rs;
  int blk;  // act in the 16 x 32 blocks of act_off
  static constexpr int kNarrow = 2;
  static constexpr bool kRowScale = true;
  __device__ EpiSiluMul nsplit(int) const { return *this; }
  __device__ void prepare(int rows, int m0, int M, int tid) const {
    rs.fill(row_scale_lds(), rows, m0, M, tid);
  }
  __device__ const T* bslab(int nt, int s) const {
    const int n = imin(nt * 64 + (16 * s & 63), I - 1);
    return (s < 4 ? Wg : Wu) + (int64_t)(n / 16) * slab_elems(K);
  }
  __device__ void apply(const float* t, int rows, int m0, int M, int nt, int tid) const {
    const float* srs = row_scale_lds();
    for (int idx = tid; idx < rows * 64; idx += (int)blockDim.x) {
      const int r = idx / 64, c = idx % 64, m = m0 + r, n = nt * 64 + c;
      if (m < M && n < I) {
        const float sc = srs[r];
        const float g = t[r * LDT + c] * sc, u = t[r * LDT + 64 + c] * sc;
        act[act_off(m, n, I, blk)] = Num<T>::from_f(g / (1.0f + __expf(-g)) * u);
      }
    }
  }
  // narrow tiles (gemm_rows): the column space is blocks of 32, [16 gate
  // rows | the 16 matching up rows] for output columns 16 b .. 16 b + 15
  __device__ const T* nslab(int n0) const {
    const int o = imin((n0 / 32) * 16, I - 1);
    return ((n0 & 16) ? Wu : Wg) + (int64_t)(o / 16) * slab_elems(K);
  }
  __device__ void nrow_pre(NarrowPre& pre, int rows, int m0, int M, int wave, int nw,
                           int lane) const {
    rs.pre_rows(pre.ss, rows, m0, M, wave, nw, lane);
  }
  __device__ void nrow_fin(const NarrowPre& pre, float* srs, int rows, int m0, int M, int wave,
                           int nw, int lane) const {
    rs.finish_rows(pre.ss, srs, rows, m0, M, wave, nw, lane);
  }
  __device__ void nfetch(NarrowPre&, int, int, int, int, int, int) const {}
  template <int J>
  __device__ void napply(const float* t, int ldt, int rows, int m0, int M, int n0, int ncols,
                         int tid, const NarrowPre&) const {
    const float* srs = row_scale_lds();
    const int half = ncols / 2;
    for (int idx = tid; idx < rows * half; idx += (int)blockDim.x) {
      const int r = idx / half, j = idx % half, pb = j / 16, i = j % 16;
      const int m = m0 + r, n = n0 / 2 + j;
      if (m < M && n < I) {
        const float sc = srs[r];
        const float g = t[r * ldt + 32 * pb + i] * sc, u = t[r * ldt + 32 * pb + 16 + i] * sc;
        act[act_off(m, n, I, blk)] = Num<T>::from_f(g / (1.0f + __expf(-g)) * u);
      }
    }
  }
};

// Per-head RMSNorm (gain g) followed by neox RoPE with the row's (cos, sin)
// table; lane i < D/2 owns the pair (i, i + D/2).  Returns the rotated pair.
template <typename T>
__device__ __forceinline__ void norm_rope_pair_c(float x0, float x1, int i, int D, bool active,
                                                 const T* g, float eps, float2 c, float& o0,
                                                 float& o1) {
  const float ss = wave_sum(active ? x0 * x0 + x1 * x1 : 0.f);
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
  if (!active) return;
  const float y0 = x0 * inv * Num<T>::to_f(g[i]);
  const float y1 = x1 * inv * Num<T>::to_f(g[i + D / 2]);
  o0 = y0 * c.x - y1 * c.y;
  o1 = y1 * c.x + y0 * c.y;
}
// ... with the pair's (cos, sin) from the row's table
template <typename T>
__device__ __forceinline__ void norm_rope_pair(float x0, float x1, int i, int D, bool active,
                                               const T* g, float eps, const float2* cs_row,
                                               float& o0, float& o1) {
  norm_rope_pair_c<T>(x0, x1, i, D, active, g, eps, active ? cs_row[i] : make_float2(1.f, 0.f),
                      o0, o1);
}

// q -> [M, nq, D]; the block's k and v -> one 16-key "page" per (request, kv
// head) in the attention kernel's cache layout: kblk [B][nkv][16][D] and
// vblk [B][nkv][D][16] (V transposed), block row j = m % S of request m / S.
template <typename T> struct EpiQKV {
  const T* W; int H; int nq, nkv, D; const T* qn; const T* kn; float eps;
  const float2* cs; T* q; T* k; T* v; RowScale rs; int S;
  __device__ void prepare(int rows, int m0, int M, int tid) const {
    rs.fill(row_scale_lds(), rows, m0, M, tid);
  }
  __device__ const T* bslab(int nt, int s) const {
    return W + (int64_t)(imin(nt * BN + 16 * s, (nq + 2 * nkv) * D - 1) / 16) * slab_elems(H);
  }
  __device__ void apply(const float* t, int rows, int m0, int M, int nt, int tid) const {
    const float* srs = row_scale_lds();
    const int lane = tid & 63, wave = tid >> 6;
    const int HP = BN / D, half = D / 2;
    for (int item = wave; item < rows * HP; item += (int)(blockDim.x >> 6)) {
      const int r = item / HP, hh = item % HP, m = m0 + r, gh = nt * HP + hh;
      if (m >= M || gh >= nq + 2 * nkv) continue;
      const bool act = lane < half;
      const float sc = srs[r];
      const float x0 = act ? t[r * LDT + hh * D + lane] * sc : 0.f;
      const float x1 = act ? t[r * LDT + hh * D + lane + half] * sc : 0.f;
      float o0 = x0, o1 = x1;
      const int rq = m / S, j = m % S;
      if (gh < nq) {
        norm_rope_pair<T>(x0, x1, lane, D, act, qn, eps, cs + (int64_t)m * half, o0, o1);
        T* dst = q + ((int64_t)m * nq + gh) * D;
        if (act) {
          dst[lane] = Num<T>::from_f(o0);
          dst[lane + half] = Num<T>::from_f(o1);
        }
      } else if (gh < nq + nkv) {
        norm_rope_pair<T>(x0, x1, lane, D, act, kn, eps, cs + (int64_t)m * half, o0, o1);
        T* dst = k + (((int64_t)rq * nkv + (gh - nq)) * 16 + j) * D;
        if (act) {
          dst[lane] = Num<T>::from_f(o0);
          dst[lane + half] = Num<T>::from_f(o1);
        }
      } else {
        T* dst = v + ((int64_t)rq * nkv + (gh - nq - nkv)) * D * 16 + j;
        if (act) {
          dst[(int64_t)lane * 16] = Num<T>::from_f(o0);
          dst[(int64_t)(lane + half) * 16] = Num<T>::from_f(o1);
        }
      }
    }
  }
};

// Stacked K/V rows of every layer: column n -> layer n / (2 nkv D), then the
// k rows and v rows of that layer's w_qkv (which start after the nq*D q rows).
// Sixteen consecutive values of one Vᵀ cache row (16 keys of one dim) stored
// as one contiguous run.
__device__ __forceinline__ void store_run16(bf16_t* dst, const float* v) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
  reinterpret_cast<uint4*>(dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
  reinterpret_cast<uint4*>(dst)[1] = make_uint4(w[4], w[5], w[6], w[7]);
}
__device__ __forceinline__ void store_run16(fp8_t* dst, const float* v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)f32_to_e4m3(v[4 * i]) | ((uint32_t)f32_to_e4m3(v[4 * i + 1]) << 8) |
           ((uint32_t)f32_to_e4m3(v[4 * i + 2]) << 16) | ((uint32_t)f32_to_e4m3(v[4 * i + 3]) << 24);
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void store_run16(float* dst, const float* v) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    reinterpret_cast<float4*>(dst)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

// Per 16-row block of an epilogue tile: 1 when all 16 rows are written to 16
// consecutive slots starting at a multiple of 16 (so within one page, whose
// size is a multiple of 16): their Vᵀ values then go out as contiguous runs.
__device__ __forceinline__ int* kv_block_flags() {
  __shared__ int f[8];
  return f;
}
// cache slot of each tile row, -1 when the row is not written
__device__ __forceinline__ int32_t* kv_row_slot() {
  __shared__ int32_t s[128];
  return s;
}

template <typename T, typename KT> struct EpiKVInject {
  KVTargets tg; int H; int n_layers, nq, nkv, D; float eps; const float2* cs;
  const int32_t* slots; const int32_t* valid; int rpr; int P; int64_t num_slots; RowScale rs;
  int64_t row0;  // grid row of GEMM row 0 (the chunk's first row): request (row0 + m) / rpr
  __device__ bool row_written(int m, int M) const {
    if (m >= M) return false;
    const int64_t t = row0 + m;
    if (valid != nullptr && (int)(t % rpr) >= valid[t / rpr]) return false;
    const int64_t slot = slots[m];
    return slot >= 0 && slot < num_slots;  // outside the pool: never written
  }
  __device__ void prepare(int rows, int m0, int M, int tid) const {
    // thread r checks row r against the first row of its 16-row block; a
    // block qualifies when all 16 lanes of its group agree (one ballot)
    if (rows >= 16 && tid < (rows & ~15)) {
      const int r = tid, m = m0 + r, mb = m0 + (r & ~15);
      const int32_t s0 = slots[imin(mb, M - 1)];
      const bool ok = row_written(m, M) && slots[m] == s0 + (r & 15) && (s0 % 16) == 0;
      const uint64_t b = __ballot(ok);
      if ((r & 15) == 0) kv_block_flags()[r / 16] = ((b >> (tid & 63 & ~15)) & 0xffffull) == 0xffffull;
    }
    if (tid < rows) kv_row_slot()[tid] = row_written(m0 + tid, M) ? slots[m0 + tid] : -1;
    rs.fill(row_scale_lds(), rows, m0, M, tid);  // ends with a barrier
  }
  __device__ const T* bslab(int nt, int s) const {
    const int per = 2 * nkv * D;
    const int n = imin(nt * BN + 16 * s, n_layers * per - 1);
    const int l = n / per, w = n % per;
    return static_cast<const T*>(tg.w_qkv[l]) + (int64_t)((nq * D + w) / 16) * slab_elems(H);
  }
  __device__ void apply(const float* t, int rows, int m0, int M, int nt, int tid) const {
    const float* srs = row_scale_lds();
    const int* bok = kv_block_flags();
    const int lane = tid & 63, wave = tid >> 6, nw = (int)(blockDim.x >> 6);
    const int HP = BN / D, half = D / 2, n_items = rows * HP;
    // k_norm gains of the tile's K heads (a tile holds HP <= 2 heads), loaded once
    float gk[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    for (int hh = 0; hh < HP; ++hh) {
      const int gh = nt * HP + hh;
      if (gh < n_layers * 2 * nkv && (gh % (2 * nkv)) < nkv && lane < half) {
        const T* g = static_cast<const T*>(tg.k_norm[gh / (2 * nkv)]);
        gk[hh][0] = Num<T>::to_f(g[lane]);
        gk[hh][1] = Num<T>::to_f(g[lane + half]);
      }
    }
    // V heads of 16-row blocks of consecutive page-aligned slots: one (block,
    // head) per wave, spread over the waves; lane = dimension, each writing a
    // 16-slot run of its V^T page row
    if (rows >= 16) {
      for (int bi = wave; bi < (rows / 16) * HP; bi += nw) {
        const int blk = bi / HP, hh = bi % HP, gh = nt * HP + hh, r = blk * 16;
        if (gh >= n_layers * 2 * nkv || (gh % (2 * nkv)) < nkv || !bok[blk]) continue;
        const int l = gh / (2 * nkv), head = gh % nkv;
        const int32_t s0 = kv_row_slot()[r];
        const int64_t page = s0 / P, off = s0 % P;
        KT* base = static_cast<KT*>(tg.vc[l]) + ((page * nkv + head) * D) * P + off;
        for (int d = lane; d < D; d += 64) {
          float v[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) v[i] = t[(r + i) * LDT + hh * D + d] * srs[r + i];
          store_run16(base + (int64_t)d * P, v);
        }
      }
    }
    constexpr int G = 4;  // items per wave whose loads go out together
    const int32_t* rsl = kv_row_slot();
    for (int ib = wave; ib < n_items; ib += nw * G) {
      int32_t sl[G];
      float2 c[G];
      int kind[G];  // 0 skip (or written with its 16-row block above), 1 K row, 2 V row
      // decisions from LDS, then the (cos, sin) loads of every K row of the
      // batch go out before any is used
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int item = ib + nw * u;
        const int r = item / HP, hh = item % HP, m = m0 + r, gh = nt * HP + hh;
        kind[u] = 0;
        sl[u] = -1;
        if (item >= n_items || m >= M || gh >= n_layers * 2 * nkv) continue;
        const bool is_v = (gh % (2 * nkv)) >= nkv;
        if (is_v && rows >= 16 && bok[r / 16]) continue;
        sl[u] = rsl[r];
        if (sl[u] >= 0) kind[u] = is_v ? 2 : 1;
      }
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int m = m0 + (ib + nw * u) / HP;
        c[u] = (kind[u] == 1 && lane < half) ? cs[(int64_t)m * half + lane] : make_float2(0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if (kind[u] == 0) continue;
        const int item = ib + nw * u;
        const int r = item / HP, hh = item % HP, gh = nt * HP + hh;
        const int l = gh / (2 * nkv), head = gh % nkv;
        const int64_t page = sl[u] / P, off = sl[u] % P;
        const bool act = lane < half;
        const float sc = srs[r];
        const float x0 = act ? t[r * LDT + hh * D + lane] * sc : 0.f;
        const float x1 = act ? t[r * LDT + hh * D + lane + half] * sc : 0.f;
        float o0 = x0, o1 = x1;
        if (kind[u] == 1) {
          // per-head RMSNorm (gain k_norm) and neox RoPE with the row's (cos, sin)
          const float ss = wave_sum(act ? x0 * x0 + x1 * x1 : 0.f);
          const float inv = 1.0f / sqrtf(ss / (float)D + eps);
          if (act) {
            const float y0 = x0 * inv * (hh ? gk[1][0] : gk[0][0]);
            const float y1 = x1 * inv * (hh ? gk[1][1] : gk[0][1]);
            o0 = y0 * c[u].x - y1 * c[u].y;
            o1 = y1 * c[u].x + y0 * c[u].y;
          }
        }
        if (!act) continue;
        if (kind[u] == 2) {  // V pages are stored transposed: [page][head][D][P]
          KT* dst = static_cast<KT*>(tg.vc[l]) + ((page * nkv + head) * D) * P + off;
          dst[(int64_t)lane * P] = Num<KT>::from_f(o0);
          dst[(int64_t)(lane + half) * P] = Num<KT>::from_f(o1);
        } else {             // K pages: [page][head][P][D]
          KT* dst = static_cast<KT*>(tg.kc[l]) + ((page * nkv + head) * P + off) * D;
          dst[lane] = Num<KT>::from_f(o0);
          dst[lane + half] = Num<KT>::from_f(o1);
        }
      }
    }
  }
};

// Logits of a 128-wide vocabulary slice: rounded to T (and stored when asked),
// then the (max, first index) of every row over the slice.
template <typename T> struct EpiLogits {
  const T* W; int V; int H; T* logits; float2* part; int n_tiles; RowScale rs;
  static constexpr int kNarrow = 8;  // 128-column tiles: one argmax partial each
  static constexpr bool kRowScale = true;
  __device__ EpiLogits nsplit(int) const { return *this; }
  __device__ const T* nslab(int n0) const {
    return W + (int64_t)(imin(n0, V - 1) / 16) * slab_elems(H);
  }
  __device__ void nrow_pre(NarrowPre& pre, int rows, int m0, int M, int wave, int nw,
                           int lane) const {
    rs.pre_rows(pre.ss, rows, m0, M, wave, nw, lane);
  }
  __device__ void nrow_fin(const NarrowPre& pre, float* srs, int rows, int m0, int M, int wave,
                           int nw, int lane) const {
    rs.finish_rows(pre.ss, srs, rows, m0, M, wave, nw, lane);
  }
  __device__ void nfetch(NarrowPre&, int, int, int, int, int, int) const {}
  template <int J>
  __device__ void napply(const float* t, int ldt, int rows, int m0, int M, int n0, int,
                         int tid, const NarrowPre&) const {
    apply_ld(t, ldt, rows, m0, M, n0 / BN, tid);
  }
  __device__ void prepare(int rows, int m0, int M, int tid) const {
    rs.fill(row_scale_lds(), rows, m0, M, tid);
  }
  __device__ const T* bslab(int nt, int s) const {
    return W + (int64_t)(imin(nt * BN + 16 * s, V - 1) / 16) * slab_elems(H);
  }
  __device__ void apply(const float* t, int rows, int m0, int M, int nt, int tid) const {
    apply_ld(t, LDT, rows, m0, M, nt, tid);
  }
  __device__ void apply_ld(const float* t, int ldt, int rows, int m0, int M, int nt,
                           int tid) const {
    const float* srs = row_scale_lds();
    const int lane = tid & 63, wave = tid >> 6;
    for (int r = wave; r < rows; r += (int)(blockDim.x >> 6)) {
      const int m = m0 + r;
      if (m >= M) continue;
      float best = -INFINITY;
      int bi = 0x7fffffff;
      const float sc = srs[r];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = lane + 64 * h, n = nt * BN + c;
        if (n < V) {
          const T tv = Num<T>::from_f(t[r * ldt + c] * sc);
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

// ---------------------------------------------------------------- packing
// Fragment-packed copy of a row-major [rows, cols] matrix: record i (8
// elements) of slab i / (64 cols/32), chunk (i / 64) % (cols/32), lane i % 64
// holds W[16 slab + lane % 16][32 chunk + 8 (lane / 16) + e], zero past the
// last row.  One thread per record; the writes are contiguous.
template <typename T>
__global__ __launch_bounds__(256) void pack_matrix_kernel(const T* __restrict__ src,
                                                          T* __restrict__ dst, int rows,
                                                          int cols, int64_t n_rec) {
  const int per_slab = (cols / 32) * 64;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_rec;
       i += (int64_t)gridDim.x * 256) {
    const int64_t slab = i / per_slab;
    const int rem = (int)(i % per_slab);
    const int l = rem % 64;
    const int64_t row = slab * 16 + (l & 15);
    const int col = (rem / 64) * 32 + (l >> 4) * 8;
    Frag<T> f;
    if (row < rows) load_frag(f, src + row * cols + col);
    else zero_frag(f);
    store_frag(dst + i * 8, f);
  }
}

size_t packed_matrix_elems(int rows, int cols) { return (size_t)((rows + 15) / 16) * 16 * cols; }

hipError_t pack_matrix(int dt, const void* src, void* dst, int rows, int cols, hipStream_t st) {
  const int64_t n_rec = (int64_t)packed_matrix_elems(rows, cols) / 8;
  const int64_t want = (n_rec + 255) / 256;
  const dim3 grid((unsigned)(want < 8192 ? want : 8192));
  if (dt == DFLASH_BF16)
    hipLaunchKernelGGL(pack_matrix_kernel<bf16_t>, grid, dim3(256), 0, st,
                       static_cast<const bf16_t*>(src), static_cast<bf16_t*>(dst), rows, cols,
                       n_rec);
  else
    hipLaunchKernelGGL(pack_matrix_kernel<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(src), static_cast<float*>(dst), rows, cols,
                       n_rec);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers
template <typename T, int MB, class AS, class Epi>
static void launch_mb(const AS& asrc, int M, int K, const GemmPlan& p, const Epi& epi,
                      float* partial, hipStream_t st) {
  const dim3 grid((unsigned)(p.n_tiles * p.m_tiles * p.KS));
  hipLaunchKernelGGL((gemm_stream<T, MB, AS, Epi>), grid, dim3(256), 0, st, asrc, M, K, p.KS,
                     p.Kc, p.m_tiles, partial, epi);
  if (p.KS > 1)
    hipLaunchKernelGGL((gemm_splitk_reduce<16 * MB, Epi>),
                       dim3((unsigned)(p.n_tiles * p.m_tiles * (16 * MB / RROWS))), dim3(256), 0,
                       st, p.KS, p.m_tiles, M, (const float*)partial, epi);
}

template <int BMt, class Epi>
static void launch_fat(const ASrcPlain<bf16_t>& asrc, int M, int K, const GemmPlan& p,
                       const Epi& epi, float* partial, hipStream_t st) {
  const dim3 grid((unsigned)fat_grid(p));
  hipLaunchKernelGGL((gemm_fat<BMt, Epi>), grid, dim3(256), 0, st, asrc, M, K, p.KS, p.Kc,
                     p.m_tiles, p.n_tiles, partial, epi);
  if (p.KS > 1)
    hipLaunchKernelGGL((gemm_splitk_reduce<BMt, Epi>),
                       dim3((unsigned)(p.n_tiles * p.m_tiles * (BMt / RROWS))), dim3(256), 0, st,
                       p.KS, p.m_tiles, M, (const float*)partial, epi);
}

template <class Epi>
static void launch_big(const ASrcPlain<bf16_t>& asrc, int M, int K, const GemmPlan& p,
                       int n_tiles128, const Epi& epi, float* partial, hipStream_t st) {
  const int grid = (p.m_tiles * p.n_tiles * p.KS + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_big<Epi>), dim3(grid), dim3(512), 0, st, asrc, M, K, p.m_tiles,
                     p.n_tiles, n_tiles128, p.KS, p.Kc, partial, epi);
  if (p.KS > 1)
    hipLaunchKernelGGL((gemm_splitk_reduce<256, Epi>),
                       dim3((unsigned)(n_tiles128 * p.m_tiles * (256 / RROWS))), dim3(256), 0, st,
                       p.KS, p.m_tiles, M, (const float*)partial, epi);
}

template <class Epi>
static void launch_tall(const ASrcPlain<bf16_t>& asrc, int M, int K, const GemmPlan& p,
                        const Epi& epi, hipStream_t st) {
  const int grid = (p.n_tiles + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_tall<Epi>), dim3(grid), dim3(512), 0, st, asrc, M, K, p.n_tiles, epi);
}

// Slabs per workgroup of an epilogue that runs on narrow tiles (0: it needs
// whole 128-column tiles).
template <class E, class = void> struct NarrowSlabs {
  static constexpr int value = 0;
};
template <class E> struct NarrowSlabs<E, decltype((void)E::kNarrow)> {
  static constexpr int value = E::kNarrow;
};

// Register ring depth and occupancy of gemm_rows: bf16 kernels are held to
// four waves per SIMD (<= 128 VGPRs: one 16-wave or two 8-wave workgroups per
// CU), fp32 ones to two; the ring takes what the accumulators and addresses
// leave.  (The second launch-bounds argument is the minimum waves per SIMD.)
template <typename T, int MB, int NSL, int NW, class AS, class Epi>
static void launch_rows_cfg(const AS& asrc, int M, int K, const GemmPlan& p, const Epi& epi,
                            hipStream_t st) {
  constexpr int NSW = NSL > 2 ? 2 : NSL;  // slabs per wave
  constexpr int STEP = (MB + NSW) * 2 * (sizeof(T) == 2 ? 4 : 8);
  // accumulators, addresses, indices, prefetch (+16 for the prefetched sums of
  // squares of an epilogue that applies a row scale)
  constexpr int FIXED = MB * NSW * 4 + 32 + (Epi::kRowScale ? 16 : 0);
  // four waves per SIMD where a two-step ring fits in 128 VGPRs (always for
  // 16-wave workgroups), else three (168)
  constexpr int MINW = sizeof(T) == 2 ? ((NW == 16 || 2 * STEP + FIXED <= 128) ? 4 : 3) : 2;
  constexpr int BUDGET = (MINW == 4 ? 128 : (MINW == 3 ? 168 : 256)) - FIXED;
  constexpr int NB0 = BUDGET / STEP;
  constexpr int NB = NB0 < 1 ? 1 : (NB0 > 6 ? 6 : NB0);
  const dim3 grid((unsigned)(p.n_tiles * p.m_tiles * p.KSW));
  // the lm_head's 16-wave workgroups at up to 16 rows: A through one LDS image
  // (its four slab-pair waves per K split would each load the same A)
  if constexpr (sizeof(T) == 2 && MB == 1 && NSL == 8 && NW == 16) {
    if (K <= kImgK && p.KSW == 1) {
      hipLaunchKernelGGL((gemm_rows<T, MB, NSL, NSW, NW, NB, MINW, AS, Epi, true>), grid,
                         dim3(NW * 64), 0, st, asrc, M, K, p.kw, p.KSW, p.m_tiles, epi);
      return;
    }
  }
  hipLaunchKernelGGL((gemm_rows<T, MB, NSL, NSW, NW, NB, MINW, AS, Epi>), grid, dim3(NW * 64), 0,
                     st, asrc, M, K, p.kw, p.KSW, p.m_tiles, epi);
}
template <typename T, int NSL, int NW, class AS, class Epi>
static void launch_rows_mb(const AS& asrc, int M, int K, const GemmPlan& p, const Epi& epi,
                           hipStream_t st) {
  if constexpr (NSL == 8) {  // up to 32 rows (plan_gemm)
    if (p.MB == 1) launch_rows_cfg<T, 1, NSL, NW>(asrc, M, K, p, epi, st);
    else launch_rows_cfg<T, 2, NSL, NW>(asrc, M, K, p, epi, st);
  } else {
    switch (p.MB) {
      case 1: launch_rows_cfg<T, 1, NSL, NW>(asrc, M, K, p, epi, st); return;
      case 2: launch_rows_cfg<T, 2, NSL, NW>(asrc, M, K, p, epi, st); return;
      default: launch_rows_cfg<T, 4, NSL, NW>(asrc, M, K, p, epi, st); return;
    }
  }
}
template <typename T, int NSL, class AS, class Epi>
static void launch_rows(const AS& asrc, int M, int K, const GemmPlan& p, const Epi& epi,
                        hipStream_t st) {
  if constexpr (sizeof(T) == 2 && NSL == 1) {
    if (p.NW == 16) return launch_rows_mb<T, NSL, 16>(asrc, M, K, p, epi, st);
  }
  if constexpr (sizeof(T) == 2 && NSL == 8) {
    if (p.NW == 16) return launch_rows_mb<T, NSL, 16>(asrc, M, K, p, epi, st);
  }
  if constexpr (sizeof(T) == 2 && NSL == 2) {
    if (p.NW == 4) return launch_rows_mb<T, NSL, 4>(asrc, M, K, p, epi, st);
  }
  launch_rows_mb<T, NSL, 8>(asrc, M, K, p, epi, st);
}

// 1/rms of GEMM rows [16 b, 16 b + 16) into out: RowScale::fill itself, so the
// values are the ones the tiles would compute.
constexpr int kRstdRows = 16;
__global__ __launch_bounds__(256) void row_rstd_kernel(RowScale rs, int M, float* __restrict__ out) {
  const int m0 = (int)blockIdx.x * kRstdRows, rows = imin(kRstdRows, M - m0);
  float* srs = row_scale_lds();
  rs.fill(srs, rows, m0, M, (int)threadIdx.x);  // ends with a barrier
  if ((int)threadIdx.x < rows) out[m0 + threadIdx.x] = srs[threadIdx.x];
}

template <class E, class = void> struct HasRowScale : std::false_type {};
template <class E>
struct HasRowScale<E, decltype((void)std::declval<const E&>().rs)> : std::true_type {};

template <typename T, class AS, class Epi>
static hipError_t run_gemm(const AS& asrc, int M, int K, int Ncols, const Epi& epi,
                           const GemmScratch& ws, hipStream_t st, int ksw = 1) {
  if (M <= 0) return hipSuccess;
  constexpr int NAR = NarrowSlabs<Epi>::value;
  const GemmPlan p = plan_gemm(M, Ncols, K, sizeof(T) == 2, NAR, ksw);
  if constexpr (NAR > 0) {
    if (p.rows) {
      launch_rows<T, NAR>(asrc, M, K, p, epi, st);
      return hipGetLastError();
    }
  }
  // tiled kernels: the row scales once per row, ahead of the GEMM, rather than
  // once per tile (each tile would re-read its rows' H / 16 sums of squares)
  if constexpr (HasRowScale<Epi>::value) {
    if (epi.rs.ss != nullptr && epi.rs.pre == nullptr && ws.rstd != nullptr &&
        (size_t)M <= ws.rstd_floats) {
      hipLaunchKernelGGL(row_rstd_kernel, dim3((unsigned)((M + kRstdRows - 1) / kRstdRows)),
                         dim3(256), 0, st, epi.rs, M, ws.rstd);
      Epi e = epi;
      e.rs.pre = ws.rstd;
      return run_gemm<T>(asrc, M, K, Ncols, e, ws, st, ksw);
    }
  }
  if (p.KS > 1 && gemm_partial_floats(p) > ws.partial_floats) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 2) {
    // the tiled kernels read A row-major (blocked A only below 65 rows)
    if ((p.big || p.tall || p.fat) && asrc.blk) return hipErrorInvalidValue;
    if (p.big) {
      launch_big(asrc, M, K, p, (Ncols + BN - 1) / BN, epi, ws.partial, st);
      return hipGetLastError();
    }
    if (p.tall) {
      launch_tall(asrc, M, K, p, epi, st);
      return hipGetLastError();
    }
    if (p.fat) {
      if (p.BM == 256) launch_fat<256>(asrc, M, K, p, epi, ws.partial, st);
      else launch_fat<128>(asrc, M, K, p, epi, ws.partial, st);
      return hipGetLastError();
    }
  }
  switch (p.MB) {
    case 1: launch_mb<T, 1>(asrc, M, K, p, epi, ws.partial, st); break;
    case 2: launch_mb<T, 2>(asrc, M, K, p, epi, ws.partial, st); break;
    default: launch_mb<T, 4>(asrc, M, K, p, epi, ws.partial, st); break;
  }
  return hipGetLastError();
}

template <typename T, class Epi>
static hipError_t run_any(const ASrc& a, int M, int K, int Ncols, const Epi& epi,
                          const GemmScratch& ws, hipStream_t st, int ksw = 1) {
  const ASrcPlain<T> s{static_cast<const T*>(a.a), a.lda, a.S_skip, a.blk};
  return run_gemm<T>(s, M, K, Ncols, epi, ws, st, ksw);
}

static RowScale row_scale(const ASrc& a) {
  return RowScale{a.ss, a.n_ss, a.H, a.eps, a.S_skip, nullptr};
}

hipError_t gemm_store_f32(int dt, const ASrc& a, int M, int K, const void* W, int N, float* out,
                          float* ss, void* xg, int xg_blk, const void* g_next,
                          const GemmScratch& ws, hipStream_t st) {
  if (dt == DFLASH_BF16) {
    EpiStoreF32<bf16_t> e{(const bf16_t*)W, N, K, out, N, ss,
                          NextNorm<bf16_t>{(bf16_t*)xg, (const bf16_t*)g_next, xg_blk},
                          row_scale(a)};
    return run_any<bf16_t>(a, M, K, N, e, ws, st);
  }
  EpiStoreF32<float> e{(const float*)W, N, K, out, N, ss,
                       NextNorm<float>{(float*)xg, (const float*)g_next, xg_blk}, row_scale(a)};
  return run_any<float>(a, M, K, N, e, ws, st);
}

hipError_t gemm_residual(int dt, const ASrc& a, int M, int K, const void* W, int N, float* x,
                         float* ss, void* xg, int xg_blk, const void* g_next,
                         const GemmScratch& ws, hipStream_t st) {
  if (dt == DFLASH_BF16) {
    EpiResidual<bf16_t> e{(const bf16_t*)W, N, K, x, ss,
                          NextNorm<bf16_t>{(bf16_t*)xg, (const bf16_t*)g_next, xg_blk}};
    return run_any<bf16_t>(a, M, K, N, e, ws, st);
  }
  EpiResidual<float> e{(const float*)W, N, K, x, ss,
                       NextNorm<float>{(float*)xg, (const float*)g_next, xg_blk}};
  return run_any<float>(a, M, K, N, e, ws, st);
}

hipError_t gemm_silu_mul(int dt, const ASrc& a, int M, int K, const void* Wg, const void* Wu,
                         int I, void* act, int act_blk, const GemmScratch& ws, hipStream_t st) {
  const int ncols = ((I + 63) / 64) * BN;
  if (dt == DFLASH_BF16) {
    EpiSiluMul<bf16_t> e{(const bf16_t*)Wg, (const bf16_t*)Wu, I, K, (bf16_t*)act, row_scale(a),
                         act_blk};
    return run_any<bf16_t>(a, M, K, ncols, e, ws, st);
  }
  EpiSiluMul<float> e{(const float*)Wg, (const float*)Wu, I, K, (float*)act, row_scale(a), act_blk};
  return run_any<float>(a, M, K, ncols, e, ws, st);
}

// Per-head q/k RMSNorm + RoPE of the block rows from the fp32 q/k/v the
// narrow QKV GEMM wrote (raw [M][(nq + 2 nkv) D], input RMSNorm applied), into
// the layouts attention reads: one wave per (row, head); the same arithmetic as
// EpiQKV on the same fp32 values.
template <typename T>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(
    const float* __restrict__ raw, int ksw, int M, int nq, int nkv, int D,
    const T* __restrict__ qn, const T* __restrict__ kn, float eps, const float2* __restrict__ cs,
    T* __restrict__ q, T* __restrict__ kblk, T* __restrict__ vblk, int S) {
  const int lane = threadIdx.x & 63, HH = nq + 2 * nkv, half = D / 2;
  const int item = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (item >= M * HH) return;  // wave-uniform
  const int m = item / HH, gh = item % HH, rq = m / S, j = m % S;
  const bool act = lane < half;
  // the ksw K-range partials of the GEMM, added in range order
  const int64_t pstride = (int64_t)M * HH * D;
  const float* src = raw + (int64_t)m * HH * D + (int64_t)gh * D;
  float p0[4], p1[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    p0[k] = (act && k < ksw) ? src[k * pstride + lane] : 0.f;
    p1[k] = (act && k < ksw) ? src[k * pstride + lane + half] : 0.f;
  }
  float x0 = p0[0], x1 = p1[0];
#pragma unroll
  for (int k = 1; k < 4; ++k) {
    x0 += p0[k];
    x1 += p1[k];
  }
  float o0 = x0, o1 = x1;
  if (gh < nq) {
    norm_rope_pair<T>(x0, x1, lane, D, act, qn, eps, cs + (int64_t)m * half, o0, o1);
    T* dst = q + ((int64_t)m * nq + gh) * D;
    if (act) {
      dst[lane] = Num<T>::from_f(o0);
      dst[lane + half] = Num<T>::from_f(o1);
    }
  } else if (gh < nq + nkv) {
    norm_rope_pair<T>(x0, x1, lane, D, act, kn, eps, cs + (int64_t)m * half, o0, o1);
    T* dst = kblk + (((int64_t)rq * nkv + (gh - nq)) * 16 + j) * D;
    if (act) {
      dst[lane] = Num<T>::from_f(o0);
      dst[lane + half] = Num<T>::from_f(o1);
    }
  } else {
    T* dst = vblk + ((int64_t)rq * nkv + (gh - nq - nkv)) * D * 16 + j;
    if (act) {
      dst[(int64_t)lane * 16] = Num<T>::from_f(o0);
      dst[(int64_t)(lane + half) * 16] = Num<T>::from_f(o1);
    }
  }
}

// K/V of an injection of <= 64 rows from the fp32 partials the narrow K/V
// store wrote (raw [ksw][M][Ly * 2 nkv * D], hidden_norm applied): one wave
// per (row, layer, K or V head).  The partials are added in range order; K
// heads get the layer's k_norm and RoPE; both are rounded to the cache type
// and written at the row's slot (K [page][head][P][D], V [page][head][D][P]).
// Rows past their request's valid prefix and slots outside the pool are not
// written.  The same arithmetic as EpiKVInject on the same fp32 values.
template <typename T, typename KT>
__global__ __launch_bounds__(256) void kv_norm_rope_store_kernel(
    const float* __restrict__ raw, int ksw, int M, int n_layers, int nkv, int D, KVTargets tg,
    float eps, const int32_t* __restrict__ positions, double log_theta,
    const int32_t* __restrict__ slots,
    const int32_t* __restrict__ valid, int rpr, int64_t row0, int P, int64_t num_slots) {
  const int lane = threadIdx.x & 63, HH = n_layers * 2 * nkv, half = D / 2;
  const int item = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (item >= M * HH) return;  // wave-uniform
  const int m = item / HH, gh = item % HH, l = gh / (2 * nkv), hk = gh % (2 * nkv);
  const int64_t t = row0 + m;
  if (valid != nullptr && (int)(t % rpr) >= valid[t / rpr]) return;
  const int64_t slot = slots[m];
  if (slot < 0 || slot >= num_slots) return;
  const bool act = lane < half;
  const int64_t pstride = (int64_t)M * HH * D;
  const float* src = raw + (int64_t)m * HH * D + (int64_t)gh * D;
  float p0[4], p1[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    p0[k] = (act && k < ksw) ? src[k * pstride + lane] : 0.f;
    p1[k] = (act && k < ksw) ? src[k * pstride + lane + half] : 0.f;
  }
  float x0 = p0[0], x1 = p1[0];
#pragma unroll
  for (int k = 1; k < 4; ++k) {
    x0 += p0[k];
    x1 += p1[k];
  }
  const int64_t page = slot / P, off = slot % P;
  if (hk < nkv) {
    // the row's (cos, sin) pair of this lane, formed here (the same function
    // the tiled path's table takes): no table kernel for a small injection
    float2 c = make_float2(1.f, 0.f);
    if (act) c = rope_cs(positions[m], lane, D, log_theta);
    float o0 = x0, o1 = x1;
    norm_rope_pair_c<T>(x0, x1, lane, D, act, static_cast<const T*>(tg.k_norm[l]), eps, c, o0, o1);
    KT* dst = static_cast<KT*>(tg.kc[l]) + ((page * nkv + hk) * P + off) * D;
    if (act) {
      dst[lane] = Num<KT>::from_f(o0);
      dst[lane + half] = Num<KT>::from_f(o1);
    }
  } else {
    KT* dst = static_cast<KT*>(tg.vc[l]) + ((page * nkv + (hk - nkv)) * D) * P + off;
    if (act) {
      dst[(int64_t)lane * P] = Num<KT>::from_f(x0);
      dst[(int64_t)(lane + half) * P] = Num<KT>::from_f(x1);
    }
  }
}

hipError_t gemm_qkv(int dt, const ASrc& a, int M, int H, const void* Wqkv, const void* qn,
                    const void* kn, int nq, int nkv, int D, float eps, const float2* cs, void* q,
                    void* k, void* v, int S, float* raw, const GemmScratch& ws, hipStream_t st) {
  const int ncols = (nq + 2 * nkv) * D;
  if (raw != nullptr && M <= 64) {
    // narrow GEMM into fp32 raw (input RMSNorm applied; K split over ksw
    // workgroups so that the CUs stream equal shares), then the per-head norms
    // and RoPE in a second small kernel that adds the partials: the GEMM needs
    // no whole heads
    const int ksw = qkv_k_splits(ncols);
    const int64_t pstride = (int64_t)M * ncols;
    const unsigned grid = (unsigned)((M * (nq + 2 * nkv) + 3) / 4);
    hipError_t e;
    if (dt == DFLASH_BF16) {
      EpiQKVStore<bf16_t> ep{{(const bf16_t*)Wqkv, ncols, H, raw, ncols, nullptr,
                              NextNorm<bf16_t>{nullptr, nullptr, 0}, row_scale(a), pstride}};
      if ((e = run_any<bf16_t>(a, M, H, ncols, ep, ws, st, ksw)) != hipSuccess) return e;
      hipLaunchKernelGGL(qk_norm_rope_kernel<bf16_t>, dim3(grid), dim3(256), 0, st, raw, ksw, M,
                         nq, nkv, D, (const bf16_t*)qn, (const bf16_t*)kn, eps, cs, (bf16_t*)q,
                         (bf16_t*)k, (bf16_t*)v, S);
    } else {
      EpiQKVStore<float> ep{{(const float*)Wqkv, ncols, H, raw, ncols, nullptr,
                             NextNorm<float>{nullptr, nullptr, 0}, row_scale(a), pstride}};
      if ((e = run_any<float>(a, M, H, ncols, ep, ws, st, ksw)) != hipSuccess) return e;
      hipLaunchKernelGGL(qk_norm_rope_kernel<float>, dim3(grid), dim3(256), 0, st, raw, ksw, M,
                         nq, nkv, D, (const float*)qn, (const float*)kn, eps, cs, (float*)q,
                         (float*)k, (float*)v, S);
    }
    return hipGetLastError();
  }
  if (dt == DFLASH_BF16) {
    EpiQKV<bf16_t> e{(const bf16_t*)Wqkv, H, nq, nkv, D, (const bf16_t*)qn, (const bf16_t*)kn,
                     eps, cs, (bf16_t*)q, (bf16_t*)k, (bf16_t*)v, row_scale(a), S};
    return run_any<bf16_t>(a, M, H, ncols, e, ws, st);
  }
  EpiQKV<float> e{(const float*)Wqkv, H, nq, nkv, D, (const float*)qn, (const float*)kn, eps, cs,
                  (float*)q, (float*)k, (float*)v, row_scale(a), S};
  return run_any<float>(a, M, H, ncols, e, ws, st);
}

template <typename T, typename KT>
static hipError_t kv_inject_narrow(const ASrc& a, int M, int H, const KVTargets& t, int n_layers,
                                   int nq, int nkv, int D, float eps, const int32_t* positions,
                                   double log_theta, const int32_t* slots, const int32_t* valid_rows,
                                   int rows_per_req, int64_t row0, int page_size, int64_t ns,
                                   float* raw, const GemmScratch& ws, hipStream_t st) {
  const int ncols = n_layers * 2 * nkv * D;
  const int ksw = qkv_k_splits(ncols);
  EpiKVStore<T> ep;
  static_cast<EpiStoreF32<T>&>(ep) =
      EpiStoreF32<T>{nullptr, ncols, H, raw, ncols, nullptr, NextNorm<T>{nullptr, nullptr},
                     row_scale(a), (int64_t)M * ncols};
  ep.per = 2 * nkv * D;
  ep.qoff = nq * D;
  for (int l = 0; l < kKVStoreLayers; ++l) ep.wl[l] = t.w_qkv[l];
  hipError_t e = run_any<T>(a, M, H, ncols, ep, ws, st, ksw);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((M * n_layers * 2 * nkv + 3) / 4);
  hipLaunchKernelGGL((kv_norm_rope_store_kernel<T, KT>), dim3(grid), dim3(256), 0, st, raw, ksw,
                     M, n_layers, nkv, D, t, eps, positions, log_theta, slots, valid_rows,
                     rows_per_req, row0, page_size, ns);
  return hipGetLastError();
}

bool kv_inject_is_narrow(int M, int n_layers, const float* raw) {
  return raw != nullptr && M <= 64 && n_layers <= kKVStoreLayers;
}

int kv_inject_raw_floats(int M, int n_layers, int nkv, int D) {
  if (M > 64 || n_layers > kKVStoreLayers) return 0;
  const int ncols = n_layers * 2 * nkv * D;
  return qkv_k_splits(ncols) * M * ncols;
}

hipError_t gemm_kv_inject(int dt, int kv_dt, const ASrc& a, int M, int H, const KVTargets& t,
                          int n_layers, int nq, int nkv, int D, float eps, const float2* cs,
                          const int32_t* positions, float rope_theta, const int32_t* slots,
                          const int32_t* valid_rows, int rows_per_req, int64_t row0,
                          int page_size, int64_t num_pages, float* raw, const GemmScratch& ws,
                          hipStream_t st) {
  const int64_t ns = num_pages * page_size;
  const int ncols = n_layers * 2 * nkv * D;
  if (kv_inject_is_narrow(M, n_layers, raw)) {
    // narrow K/V store into fp32 (K split over workgroups), then the norms,
    // RoPE (its (cos, sin) formed from the positions) and cache writes in a
    // small kernel that adds the partials
    const double lt = log((double)rope_theta);
    if (dt == DFLASH_BF16) {
      if (kv_dt == DFLASH_FP8_E4M3)
        return kv_inject_narrow<bf16_t, fp8_t>(a, M, H, t, n_layers, nq, nkv, D, eps, positions,
                                               lt, slots, valid_rows, rows_per_req, row0,
                                               page_size, ns, raw, ws, st);
      return kv_inject_narrow<bf16_t, bf16_t>(a, M, H, t, n_layers, nq, nkv, D, eps, positions,
                                              lt, slots, valid_rows, rows_per_req, row0,
                                              page_size, ns, raw, ws, st);
    }
    return kv_inject_narrow<float, float>(a, M, H, t, n_layers, nq, nkv, D, eps, positions, lt,
                                          slots, valid_rows, rows_per_req, row0, page_size, ns,
                                          raw, ws, st);
  }
  if (dt == DFLASH_BF16) {
    if (kv_dt == DFLASH_FP8_E4M3) {
      EpiKVInject<bf16_t, fp8_t> e{t, H, n_layers, nq, nkv, D, eps, cs, slots, valid_rows,
                                   rows_per_req, page_size, ns, row_scale(a), row0};
      return run_any<bf16_t>(a, M, H, ncols, e, ws, st);
    }
    EpiKVInject<bf16_t, bf16_t> e{t, H, n_layers, nq, nkv, D, eps, cs, slots, valid_rows,
                                  rows_per_req, page_size, ns, row_scale(a), row0};
    return run_any<bf16_t>(a, M, H, ncols, e, ws, st);
  }
  EpiKVInject<float, float> e{t, H, n_layers, nq, nkv, D, eps, cs, slots, valid_rows,
                              rows_per_req, page_size, ns, row_scale(a), row0};
  return run_any<float>(a, M, H, ncols, e, ws, st);
}

hipError_t gemm_logits(int dt, const ASrc& a, int M, int H, const void* Wlm, int V, void* logits,
                       float2* part, const GemmScratch& ws, hipStream_t st) {
  const int nt = logits_tiles(V);
  if (dt == DFLASH_BF16) {
    EpiLogits<bf16_t> e{(const bf16_t*)Wlm, V, H, (bf16_t*)logits, part, nt, row_scale(a)};
    return run_any<bf16_t>(a, M, H, V, e, ws, st);
  }
  EpiLogits<float> e{(const float*)Wlm, V, H, (float*)logits, part, nt, row_scale(a)};
  return run_any<float>(a, M, H, V, e, ws, st);
}

}  // namespace dflash
