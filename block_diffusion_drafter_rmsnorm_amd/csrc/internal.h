// Host-side interface between the C ABI layer and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dflash.h"

namespace dflash {

// Split-K scratch of the weight-streaming GEMM: fp32 partial tiles plus one
// arrival counter per output tile (counters are zero between launches: the
// last arriving workgroup of a tile resets its counter).
struct GemmScratch {
  float* partial;
  size_t partial_floats;
  int* counters;
  int n_counters;
};

// Launch geometry of the weight-streaming GEMM C[M, Ncols] = A[M, K] W^T.
struct GemmPlan {
  int MB;        // 16-row blocks per workgroup tile (1, 2, 4 or 8)
  int m_tiles;   // ceil(M / (16 MB))
  int n_tiles;   // ceil(Ncols / 128)
  int KS;        // split-K factor
  int Kc;        // K elements per split (multiple of 32)
};
GemmPlan plan_gemm(int M, int Ncols, int K);
size_t gemm_partial_floats(const GemmPlan& p);

struct KVTargets {
  const void* w_qkv[DFLASH_MAX_LAYERS];
  const void* k_norm[DFLASH_MAX_LAYERS];
  void* kc[DFLASH_MAX_LAYERS];
  void* vc[DFLASH_MAX_LAYERS];
};

// fc: out[M, N] (fp32) = A[M, K] W[N, K]^T
hipError_t gemm_store_f32(int dt, const void* A, int64_t lda, int M, int K, const void* W, int N,
                          float* out, const GemmScratch& ws, hipStream_t st);
// x[M, N] += A[M, K] W[N, K]^T   (x fp32, ld N)
hipError_t gemm_residual(int dt, const void* A, int M, int K, const void* W, int N, float* x,
                         const GemmScratch& ws, hipStream_t st);
// act[M, I] = silu(A Wg^T) * (A Wu^T)
hipError_t gemm_silu_mul(int dt, const void* A, int M, int K, const void* Wg, const void* Wu,
                         int I, void* act, const GemmScratch& ws, hipStream_t st);
// q/k/v of the block rows with per-head RMSNorm + RoPE on q and k
hipError_t gemm_qkv(int dt, const void* A, int M, int H, const void* Wqkv, const void* qn,
                    const void* kn, int nq, int nkv, int D, float eps, const float2* cs,
                    void* q, void* k, void* v, const GemmScratch& ws, hipStream_t st);
// stacked K/V of all layers for context rows -> paged cache
hipError_t gemm_kv_inject(int dt, int kv_dt, const void* A, int M, int H, const KVTargets& t,
                          int n_layers, int nq, int nkv, int D, float eps, const float2* cs,
                          const int32_t* slots, const int32_t* valid_rows, int rows_per_req,
                          int page_size, int64_t num_pages, const GemmScratch& ws,
                          hipStream_t st);
// logits[M, V] (nullable) and per-tile argmax partials (value, index) [M, n_tiles]
hipError_t gemm_logits(int dt, const void* A, int M, int H, const void* Wlm, int V, void* logits,
                       float2* part, const GemmScratch& ws, hipStream_t st);
int logits_tiles(int V);

// ---- elementwise / small kernels
hipError_t launch_zero_i32(int* p, int n, hipStream_t st);
hipError_t launch_block_prep(int dt, const dflash_config& c, const void* embed,
                             const int32_t* anchor, const int32_t* prefix_len,
                             const int32_t* page_table, int max_pages, int B, int32_t* block_ids,
                             int32_t* positions, int32_t* slots, int32_t* candidates, float* x,
                             float2* cs, hipStream_t st);
hipError_t launch_rope_table(const int32_t* positions, int rows, int D, float theta, float2* cs,
                             hipStream_t st);
// out[m] = rms(in[src(m)]) * g; src(m) = m when S == 0, else the block row
// m / (S-1) * S + m % (S-1) + 1 (rows 1..S-1 of every block).
hipError_t launch_rmsnorm(int dt, const float* in, int M, int H, const void* g, float eps,
                          void* out, int S_skip_anchor, hipStream_t st);
hipError_t launch_argmax_reduce(const float2* part, int M, int n_tiles, int S, int32_t* candidates,
                                hipStream_t st);
hipError_t launch_accept(const int32_t* cand, const int32_t* post, const int32_t* prefix_len, int B,
                         int S, int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens,
                         int32_t* next_anchor, int32_t* new_seq_len, hipStream_t st);

// ---- attention
struct AttnPlan {
  int chunk;      // context keys per split
  int n_splits;   // grid splits per (request, kv head)
};
AttnPlan plan_attention(int max_keys, int B, int nkv);
hipError_t launch_attention(int dt, int kv_dt, int D, const void* q, const void* kb, const void* vb,
                            const void* kc, const void* vc, const int32_t* page_table,
                            int max_pages, int64_t num_pages, const int32_t* prefix_len,
                            int max_prefix, int B,
                            int S, int nq, int nkv, int page_size, int window, const AttnPlan& plan,
                            float* o_part, float2* ml_part, void* out, hipStream_t st);

}  // namespace dflash
