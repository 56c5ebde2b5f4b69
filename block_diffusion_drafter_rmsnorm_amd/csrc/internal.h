// Host-side interface between the C ABI layer and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dflash.h"

namespace dflash {

// Split-K scratch of the weight-streaming GEMM: fp32 partial tiles, summed in
// a fixed order by a second kernel that runs the epilogue.
struct GemmScratch {
  float* partial;
  size_t partial_floats;
  // 1/rms of each row of a row-scaled GEMM of more than 64 rows, computed once
  // before the GEMM instead of by every tile (nullable: the tiles compute it)
  float* rstd = nullptr;
  size_t rstd_floats = 0;
};

// Launch geometry of a GEMM C[M, Ncols] = A[M, K] W^T: the weight-streaming
// kernel (M <= 64, or fp32) or the LDS-tiled kernel (bf16, M > 64).
struct GemmPlan {
  bool rows;     // narrow tiles, K split inside the workgroup (gemm_rows; M <= 64)
  int NSL;       //   packed 16-column slabs per workgroup (1 or 2)
  int NW;        //   waves per workgroup (8 or 16), each streaming kw of K
  int kw;       //   K of each workgroup's range (a multiple of 64)
  int KSW;       //   K ranges across workgroups (1 unless the caller adds partials)
  bool fat;      // LDS-tiled kernel
  bool big;      // 256 x 256 tiles, no split K (n_tiles counts 256 columns)
  bool tall;     // 65..128 rows: one 128 x 128 tile per column tile, deep copy ring
  int BM;        // rows per tile (16 MB for the streaming kernel; 128 or 256)
  int MB;        // 16-row blocks per workgroup tile of the streaming kernel (1, 2, 4)
  int m_tiles;   // ceil(M / BM)
  int n_tiles;   // ceil(Ncols / 128)
  int KS;        // split-K factor
  int Kc;        // K elements per split
};
// narrow: slabs per workgroup when the epilogue runs on narrow tiles (1 for
// store and residual, 2 for SwiGLU's gate/up pairs; 0: it needs 128-column
// tiles), so that up to 64 rows take gemm_rows (no split-K partials)
// ksw: K ranges across workgroups, each written as its own partial (narrow
// epilogues whose consumer adds them: the QKV store)
GemmPlan plan_gemm(int M, int Ncols, int K, bool bf16, int narrow = 0, int ksw = 1);
// K ranges of the narrow QKV GEMM (its fp32 output holds that many partials)
int qkv_k_splits(int ncols);
int qkv_slabs();  // slabs per workgroup of the narrow QKV GEMM
size_t gemm_partial_floats(const GemmPlan& p);

struct KVTargets {
  const void* w_qkv[DFLASH_MAX_LAYERS];
  const void* k_norm[DFLASH_MAX_LAYERS];
  void* kc[DFLASH_MAX_LAYERS];
  void* vc[DFLASH_MAX_LAYERS];
};

// A operand of a GEMM: rows of T with row stride lda, or (blk = 1) in the
// 16 x 32 blocks of act_off (common.h) with lda the row width; blocked A goes
// only to calls of at most 64 rows (the narrow and streaming kernels).  S_skip
// > 0 maps GEMM row m to A row (m / (S-1)) * S + m % (S-1) + 1.  When ss !=
// null the A rows are x * g of an RMSNorm and each output row is scaled by
// 1/rms(x), from the sums of squares ss[row * n_ss + t] of columns [16 t, 16 t
// + 16) of x (width H).
struct ASrc {
  const void* a;
  int64_t lda;
  const float* ss;
  int n_ss;
  int H;
  float eps;
  int S_skip;
  int blk;
};
inline ASrc asrc_plain(const void* a, int64_t lda, int S_skip = 0, int blk = 0) {
  return ASrc{a, lda, nullptr, 0, 0, 0.f, S_skip, blk};
}
inline ASrc asrc_normed(const void* xg, int H, const float* ss, float eps, int S_skip = 0,
                        int blk = 0) {
  return ASrc{xg, H, ss, (H + 15) / 16, H, eps, S_skip, blk};
}
// Whether a call of M rows keeps its activations (the GEMMs' A operands) in
// 16 x 32 blocks, and the rows such a matrix takes.
inline int act_blocked(int64_t M) { return M <= 64 ? 1 : 0; }
inline int64_t act_rows(int64_t M) { return act_blocked(M) ? (M + 15) / 16 * 16 : M; }
// 16-column groups of a row: the granularity of the row sums of squares (one
// packed weight slab of output columns, the narrowest tile a GEMM writes)
__host__ __device__ inline int ss_tiles(int H) { return (H + 15) / 16; }

// y = A W^T: out[M, N] fp32 (nullable), per-128-column row sums of squares of y
// into ss (nullable) and xg = y * g_next rounded to the act dtype (nullable;
// in 16 x 32 blocks when xg_blk)
// Fragment-packed weight layout read by every GEMM (see gemm.hip).
size_t packed_matrix_elems(int rows, int cols);
hipError_t pack_matrix(int dt, const void* src, void* dst, int rows, int cols, hipStream_t st);

hipError_t gemm_store_f32(int dt, const ASrc& a, int M, int K, const void* W, int N, float* out,
                          float* ss, void* xg, int xg_blk, const void* g_next,
                          const GemmScratch& ws, hipStream_t st);
// x[M, N] += A W^T (x fp32, ld N), then ss / xg of the new x as above
hipError_t gemm_residual(int dt, const ASrc& a, int M, int K, const void* W, int N, float* x,
                         float* ss, void* xg, int xg_blk, const void* g_next,
                         const GemmScratch& ws, hipStream_t st);
// act[M, I] = silu(A Wg^T) * (A Wu^T) (in 16 x 32 blocks when act_blk)
hipError_t gemm_silu_mul(int dt, const ASrc& a, int M, int K, const void* Wg, const void* Wu,
                         int I, void* act, int act_blk, const GemmScratch& ws, hipStream_t st);
// q/k/v of the block rows with per-head RMSNorm + RoPE on q and k; q -> [M, nq, D],
// k -> kblk [B][nkv][16][D], v -> vblk [B][nkv][D][16] (block row j = m % S).
// raw (nullable, [M][(nq + 2 nkv) D] fp32): with M <= 64 the GEMM runs on
// narrow tiles into raw and a second kernel applies the per-head norms.
hipError_t gemm_qkv(int dt, const ASrc& a, int M, int H, const void* Wqkv, const void* qn,
                    const void* kn, int nq, int nkv, int D, float eps, const float2* cs, void* q,
                    void* kblk, void* vblk, int S, float* raw, const GemmScratch& ws,
                    hipStream_t st);
// stacked K/V of all layers for context rows -> paged cache.  GEMM row m is
// row row0 + m of the [n_req, rows_per_req] grid (valid_rows indexed by grid
// request; slots by GEMM row).
// raw (nullable): fp32 scratch of kv_inject_raw_floats(M, ...) floats; with it
// and M <= 64 (kv_inject_is_narrow) the K/V GEMM is the narrow store plus a
// norm/RoPE/write kernel, which forms each row's RoPE (cos, sin) from
// positions[m] and rope_theta; the tiled path reads them from the table cs
// [M][D/2] (launch_rope_table), which the narrow path does not read.
bool kv_inject_is_narrow(int M, int n_layers, const float* raw);
hipError_t gemm_kv_inject(int dt, int kv_dt, const ASrc& a, int M, int H, const KVTargets& t,
                          int n_layers, int nq, int nkv, int D, float eps, const float2* cs,
                          const int32_t* positions, float rope_theta, const int32_t* slots,
                          const int32_t* valid_rows, int rows_per_req, int64_t row0,
                          int page_size, int64_t num_pages, float* raw, const GemmScratch& ws,
                          hipStream_t st);
int kv_inject_raw_floats(int M, int n_layers, int nkv, int D);
// logits[M, V] (nullable) and per-tile argmax partials (value, index) [M, n_tiles]
hipError_t gemm_logits(int dt, const ASrc& a, int M, int H, const void* Wlm, int V, void* logits,
                       float2* part, const GemmScratch& ws, hipStream_t st);
int logits_tiles(int V);

// ---- elementwise / small kernels
// block ids / positions / slots, the embedding rows into x (fp32) with their
// sums of squares (ss[row * n_ss] = total, the other n_ss - 1 entries zero),
// xg = x * g_first rounded to the act dtype (in 16 x 32 blocks when xg_blk),
// and the RoPE table of the block rows
hipError_t launch_block_prep(int dt, const dflash_config& c, const void* embed,
                             const int32_t* anchor, const int32_t* prefix_len,
                             const int32_t* page_table, int max_pages, int B, int32_t* block_ids,
                             int32_t* positions, int32_t* slots, int32_t* candidates, float* x,
                             float* ss, int n_ss, void* xg, int xg_blk, const void* g_first,
                             float2* cs, hipStream_t st);
hipError_t launch_rope_table(const int32_t* positions, int rows, int D, float theta, float2* cs,
                             hipStream_t st);
hipError_t launch_argmax_reduce(const float2* part, int M, int n_tiles, int S, int32_t* candidates,
                                hipStream_t st);
hipError_t launch_accept(const int32_t* cand, const int32_t* post, const int32_t* prefix_len, int B,
                         int S, int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens,
                         int32_t* next_anchor, int32_t* new_seq_len, hipStream_t st);
// greedy accept from target logits [B, S, V] (dt F32 or BF16): chunked row
// argmax into part [B * S * accept_logits_chunks(V)], then the accept; vec:
// every run of 8 columns starts on a 16-byte boundary (V % 8 == 0 and an
// aligned base)
int accept_logits_chunks(int V);
hipError_t launch_accept_logits(int dt, const void* logits, int V, bool vec, const int32_t* cand,
                                const int32_t* prefix_len, int B, int S, float2* part,
                                int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens,
                                int32_t* next_anchor, int32_t* new_seq_len, hipStream_t st);

// ---- rejection-sampling verify (sampling.hip)
// Vocabulary chunking and workspace layout: stats partials (max, sum) per
// row and chunk, weight sums (residual, p) per request and chunk, walk records.
struct SpecPlan {
  int rows;                  // B*S target rows (+ B*(S-1) draft rows)
  int chunk1, n_chunks1;     // chunking of the statistics pass
  int chunk2, n_chunks2;     // chunking of the weight sums and the pick (<= 64)
  size_t off_stats, off_csum, off_walk, bytes;
};
SpecPlan plan_spec(int B, int S, int V, bool has_draft);
// vec: 8 (bf16) / 4 (f32) for 16-byte loads, else 1; ct, cd = log2(e) / temperature
// q_ids / q_probs (nullable, [B, S-1, q_k]): the proposal given as q_k (id,
// probability) pairs per drafted row instead of draft logits or a point mass
hipError_t launch_accept_sampling(int dt, int vec, const int32_t* cand, const void* tl,
                                  const void* dl, const int32_t* q_ids, const float* q_probs,
                                  int q_k, const float* uni, const int32_t* prefix_len, int B,
                                  int S, int V, float ct, float cd, const SpecPlan& pl, void* ws,
                                  int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens,
                                  int32_t* next_anchor, int32_t* new_seq_len, hipStream_t st);

// ---- cache reservation (reserve.hip)
// checked mode (check.hip): reset `report`, then add each rule's violations
hipError_t launch_check_draft(const int32_t* anchor, const int32_t* prefix_len,
                              const int32_t* page_table, int max_pages, int batch, int max_prefix,
                              int S, int P, int vocab, int64_t num_pages, int cwin,
                              int32_t* report, hipStream_t st);
hipError_t launch_check_context(const int32_t* positions, const int32_t* slots,
                                const int32_t* valid, int n_req, int rpr, int64_t num_slots,
                                int32_t* report, hipStream_t st);
hipError_t launch_check_accept(const int32_t* cand, const int32_t* post,
                               const int32_t* prefix_len, int B, int S, int vocab,
                               int32_t* report, hipStream_t st);

hipError_t launch_reserve(const int32_t* seq_len, int B, int S, int P, int32_t* pt, int max_pages,
                          int32_t* n_pages, const int32_t* free_pages, int capacity,
                          int32_t* free_count, int32_t* status, hipStream_t st);
// request-pool relay: stash = batch rows -> pool slots, else pool slots -> batch
// rows; any of the four fields may be NULL on both sides (not copied)
hipError_t launch_relay(bool stash, const int32_t* slots, int B, int capacity, int max_pages,
                        int32_t* p_anchor, int32_t* p_len, int32_t* p_pt, int32_t* p_np,
                        int32_t* anchor, int32_t* len, int32_t* pt, int32_t* np,
                        hipStream_t st);
hipError_t launch_release(const int32_t* mask, int B, const int32_t* pt, int max_pages,
                          int32_t* n_pages, int32_t* free_pages, int capacity, int32_t* free_count,
                          hipStream_t st);

// ---- DFlash 2 candidate selector (selector.hip)
// top-K (K in {1, 2, 4, 8, 16}) of rows x V logits (act dtype) from the
// lm_head's per-128-column argmax partials part [rows][ceil(V / 128)]:
// cand [rows][K] ids, unary [rows][K] values
hipError_t launch_topk(int dt, const void* logits, const float2* part, int rows, int V, int K,
                       int32_t* cand, float* unary, hipStream_t st);
// lattice of every (position, predecessor, candidate) and the walk: candidates
// [B, S] = anchor + chosen tokens, q_rows [B, S-1, K]; uni nullable (greedy)
hipError_t launch_lattice_walk(int dt, const int32_t* cand, const float* unary, const float* w,
                               const void* A, const void* Bt, const int32_t* anchor,
                               const float* uni, float temperature, int B, int S, int K, int r,
                               int V, int32_t* candidates, float* q_rows, hipStream_t st);

// ---- attention
struct AttnPlan {
  int stages;      // LDS stages of the bf16-cache kernel (0: the register-staged kernel)
  int n_launch;    // workgroups W (a multiple of 256)
  int n_partials;  // (O, m, l) partial slots: W + B * nkv
  bool fits;       // the unit count fits the kernels' 32-bit bookkeeping
  int kps;         // aligned partition (few segments): workgroups per segment; 0: by bytes
};
// max_keys: the most context keys a request sees on the layer; dma: the cache
// and compute types are bf16 (the direct-to-LDS kernel runs).
AttnPlan plan_attention(int max_keys, int B, int nkv, bool dma);
// Whether block attention stages the cache straight into LDS (bf16 compute on
// a bf16 cache, or on an E4M3 cache with head_dim 128).
bool attn_uses_dma(int act_dtype, int kv_dtype, int head_dim);
hipError_t launch_attention(int dt, int kv_dt, int D, const void* q, const void* kblk,
                            const void* vblk,
                            const void* kc, const void* vc, const int32_t* page_table,
                            int max_pages, int64_t num_pages, const int32_t* prefix_len,
                            int max_prefix, int B,
                            int S, int nq, int nkv, int page_size, int window, int ctx_window,
                            const AttnPlan& plan,
                            float* o_part, float2* ml_part, int4* seg, void* out, int out_blk,
                            hipStream_t st);

// Record msg as the calling thread's last error (dflash_last_error) and return s.
dflash_status set_error(dflash_status s, const char* msg);

}  // namespace dflash
