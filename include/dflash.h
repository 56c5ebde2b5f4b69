/*
 * dflash.h - C ABI of the DFlash draft-and-accept hot path on MI355X (gfx950).
 *
 * The library computes the three steps that one speculative-decoding cycle
 * of a DFlash block-diffusion drafter runs on the GPU:
 *   dflash_project_context  context injection (target features -> draft K/V cache)
 *   dflash_draft_block      one non-causal draft pass over [anchor, MASK x (S-1)]
 *   dflash_draft_block_selector  the same pass with the DFlash 2 candidate selector
 *   dflash_draft_block_noalloc   the draft pass on a fixed in-library scratch array
 *   dflash_accept           greedy verify-accept, commit and logical crop
 *   dflash_accept_sampling  rejection-sampling verify-accept and commit
 *   dflash_accept_sampling_sparse  the same with the selector's sparse q rows
 *   dflash_reserve_pages / dflash_release_pages  page reservation on the device
 *   dflash_relay_resolve / dflash_relay_stash  decode state by request-pool slot
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is DEVICE memory unless its name starts with
 *     host_.  The caller owns every buffer (weights, cache, page table,
 *     inputs, outputs, workspace); the library never allocates or frees
 *     device memory and keeps no state between calls (one exception:
 *     dflash_draft_block_noalloc's fixed scratch array, below).
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream).  Results are ready when the stream is.
 *   - Failures come back as a dflash_status; nothing throws across the ABI.
 *     The library checks what the host can see (null pointers, sizes, dtype
 *     and shape support, workspace size).  Device-resident values (token ids
 *     < vocab, slots inside the pool, prefix + block inside the page table)
 *     are the caller's contract; kernels clamp indices so that a violation
 *     produces wrong values, never an out-of-bounds access.
 *     dflash_last_error() returns a message for the last failure on the
 *     calling thread.
 *   - Integer tensors are int32.  Token embeddings are row-major [V, H].  The
 *     projection matrices (fc, w_qkv, w_o, w_gate, w_up, w_down, lm_head) are
 *     passed fragment-packed: dflash_pack_matrix turns a row-major [out, in]
 *     matrix (y = x W^T) into that layout once, when the weights are loaded.
 *   - Calls that share a workspace must be ordered on one stream.  A
 *     workspace must be 16-byte aligned (DFLASH_EINVAL otherwise).
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_MAX_LAYERS 16

typedef enum {
  DFLASH_OK = 0,
  DFLASH_EINVAL = -1,        /* null pointer, negative or inconsistent size        */
  DFLASH_EUNSUPPORTED = -2,  /* configuration outside what the kernels implement   */
  DFLASH_EWORKSPACE = -3,    /* workspace smaller than dflash_*_workspace_bytes()  */
  DFLASH_EHIP = -4           /* a HIP runtime call failed (launch error)           */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1, DFLASH_FP8_E4M3 = 2 } dflash_dtype;

/*
 * Draft model description (the draft checkpoint's config: block size, mask
 * token id, layer types with their sliding window, head counts and head_dim;
 * CSDN DFlash article, the Kimi-K2.6-DFlash config sample).
 * Supported: head_dim 64 or 128; n_q_heads a multiple of n_kv_heads; page_size a
 * multiple of 16;
 * (n_q_heads / n_kv_heads) * block_size <= 64; block_size 2..16;
 * hidden, feat_dim, inter and n_q_heads*head_dim multiples of 32; inter a
 * multiple of 64; act_dtype F32 or BF16; kv_dtype F32, BF16 or FP8_E4M3
 * (FP8 and BF16 caches need act_dtype BF16; an F32 cache needs F32).
 */
typedef struct {
  int32_t hidden;          /* H: draft hidden size                                 */
  int32_t n_layers;        /* draft decoder layers (<= DFLASH_MAX_LAYERS)          */
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;        /* D                                                    */
  int32_t inter;           /* SwiGLU intermediate size                             */
  int32_t vocab;           /* target vocabulary (shared embedding and lm_head)     */
  int32_t feat_dim;        /* F: width of the concatenated target-layer features   */
  int32_t block_size;      /* S: anchor + S-1 MASK positions                       */
  int32_t mask_token_id;
  int32_t page_size;       /* tokens per cache page                                */
  int32_t sliding_window[DFLASH_MAX_LAYERS]; /* per layer; 0 = full attention      */
  float rms_eps;
  float rope_theta;        /* neox (rotate-half) RoPE over the whole head_dim      */
  int32_t act_dtype;       /* dflash_dtype of weights, features and logits         */
  int32_t kv_dtype;        /* dflash_dtype of the draft K/V cache                  */
  int32_t context_window;  /* draft window: the draft pass reads only the last      */
                           /* context_window committed rows on every layer (0: all) */
} dflash_config;

/* Weights of one draft decoder layer, all of dtype act_dtype; the matrices
 * fragment-packed (dflash_pack_matrix), shapes given as the row-major [out, in]. */
typedef struct {
  const void* in_norm;     /* [H]                                                  */
  const void* w_qkv;       /* [(nq + 2 nkv) * D, H]: q rows, then k rows, v rows   */
  const void* q_norm;      /* [D] per-head RMSNorm gain for q                      */
  const void* k_norm;      /* [D] per-head RMSNorm gain for k (block and context)  */
  const void* w_o;         /* [H, nq * D]                                          */
  const void* post_norm;   /* [H]                                                  */
  const void* w_gate;      /* [inter, H]                                           */
  const void* w_up;        /* [inter, H]                                           */
  const void* w_down;      /* [H, inter]                                           */
} dflash_layer_weights;

typedef struct {
  const void* embed;       /* [V, H] the target's token embedding                 */
  const void* lm_head;     /* [V, H] the target's lm_head (packed)                 */
  const void* fc;          /* [H, F] fuses the concatenated target features (packed) */
  const void* hidden_norm; /* [H] RMSNorm gain after fc                            */
  const void* final_norm;  /* [H]                                                  */
  dflash_layer_weights layer[DFLASH_MAX_LAYERS];
} dflash_weights;

/*
 * Paged draft K/V cache.  For layer l, k[l] and v[l] each hold num_pages pages
 * in kv_dtype.  K pages are [num_pages][n_kv_heads][page_size][head_dim]; V
 * pages are stored transposed, [num_pages][n_kv_heads][head_dim][page_size],
 * so that attention reads both as matrix-core operands straight from memory.
 * Physical slot s lives at page s / page_size, offset s % page_size.
 */
typedef struct {
  void* k[DFLASH_MAX_LAYERS];
  void* v[DFLASH_MAX_LAYERS];
  int64_t num_pages;
} dflash_kv_cache;

/*
 * Fragment-packed weight layout.  The draft model's projections and the
 * target's lm_head ("Inside SGLang: DFlash and DFlash 2 Implementation", the
 * draft model structure; CSDN DFlash article, the fc / hidden_norm and decoder
 * layer description) are the operands the GEMMs stream from HBM once per
 * pass.  For a row-major [rows, cols] matrix W (cols a multiple of 32) the
 * packed matrix holds ceil(rows / 16) slabs of 16 rows; slab s holds cols / 32
 * chunks; chunk c holds 64 records; record l holds the 8 elements
 *   W[16 s + l % 16][32 c + 8 (l / 16) + e],  e = 0..7
 * (zero for rows >= rows).  A record is the part of one matrix-core operand
 * that one lane supplies, so a wavefront reads a chunk as one contiguous
 * 1 KB (bf16) and streams a slab front to back.
 *   dflash_packed_matrix_bytes  bytes of the packed copy (0 on invalid
 *                               arguments): ceil(rows / 16) * 16 * cols * elem
 *   dflash_pack_matrix          writes the packed copy of src [rows, cols]
 *                               (dtype F32 or BF16) to dst; src and dst must not
 *                               overlap, both 16-byte aligned; asynchronous on
 *                               `stream`.
 */
size_t dflash_packed_matrix_bytes(int32_t rows, int32_t cols, int32_t dtype);
dflash_status dflash_pack_matrix(const void* src, void* dst, int32_t rows, int32_t cols,
                                 int32_t dtype, void* stream);

/* Workspace sizes in bytes (host functions; 0 on invalid arguments). */
size_t dflash_context_workspace_bytes(const dflash_config* cfg, int64_t rows);
size_t dflash_draft_workspace_bytes(const dflash_config* cfg, int32_t batch,
                                    int32_t max_prefix_len);

/*
 * (1) Context injection ("Inside SGLang: DFlash and DFlash 2 Implementation",
 * Step 1 and Step 7; CSDN DFlash article, the draft model's target_hidden path
 * and the fused_kv_materialize section).
 *
 * Row t of `feats` holds the concatenated hidden states of the selected target
 * layers for one token.  The call computes c = RMSNorm(feats_t W_fc^T;
 * hidden_norm) and, for every draft layer l, K = RoPE(k_norm_l(c W_k,l^T),
 * positions[t]) and V = c W_v,l^T (W_k,l and W_v,l are the k and v rows of
 * layer l's w_qkv), rounds both to kv_dtype (round to nearest even; FP8
 * saturates at +-448) and stores them at cache slot slots[t].
 *
 * The rows form a dense grid of n_req requests x rows_per_req rows
 * (row t = r * rows_per_req + j).  valid_rows (nullable, [n_req]) makes the
 * write prefix-valid: row j of request r is written only if j < valid_rows[r]
 * (the committed verify rows; pass the commit_len written by dflash_accept).
 * NULL writes every row (prefill).
 *
 *   feats       [n_req * rows_per_req, F] act_dtype, row stride feat_row_stride
 *               elements (>= F, a multiple of 8)
 *   positions   [n_req * rows_per_req] logical token positions (RoPE)
 *   slots       [n_req * rows_per_req] physical cache slots
 *   workspace   >= dflash_context_workspace_bytes(cfg, n_req * rows_per_req)
 * Rows with j >= valid_rows[r] are never read beyond their feature row.
 */
dflash_status dflash_project_context(const dflash_config* cfg, const dflash_weights* w,
                                     const dflash_kv_cache* cache, const void* feats,
                                     int64_t feat_row_stride, const int32_t* positions,
                                     const int32_t* slots, const int32_t* valid_rows,
                                     int32_t n_req, int32_t rows_per_req, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * (2) One draft pass ("Inside SGLang ...", Step 3 and Step 4; CSDN DFlash
 * article, draft model predict and SGLang flow step 7).
 *
 * For request r with committed prefix L_r = prefix_len[r] and anchor token
 * anchor[r] the block is ids = [anchor, MASK x (S-1)] at logical positions
 * L_r .. L_r+S-1 and cache slots page_table[r][(pos / P) mod max_pages] * P +
 * pos % P: the page table is read as a ring, the identity when it covers the
 * whole prefix.  With a draft window N (cfg->context_window) the context keys
 * are those at positions [L_r - N, L_r) on every layer (also bounded by a
 * sliding window), so the table needs only the pages that the window and the
 * block span ("Inside SGLang ...", section "Who owns what?": windowed drafting
 * keeps a private compact mapping); the caller keeps those positions'
 * slots distinct (N + S + P - 1 <= max_pages * P suffices) and injects the
 * committed rows at the slots this call returns.
 * x = embed[ids]; each layer applies q/k/v projection with per-head q/k
 * RMSNorm and RoPE, attention of the S block queries over the cached context
 * keys 0..L_r-1 (on a sliding layer with window W only keys i with
 * pos - i < W) plus all S block keys with no causal mask, o-projection and
 * residual, then RMSNorm + SwiGLU MLP + residual (pre-norm layers).  The
 * final RMSNorm of rows 1..S-1 goes through lm_head; the argmax (first index
 * among equal maxima, taken on the logits as rounded to act_dtype) is the
 * draft token.  The block's own K/V are not stored.
 *
 *   anchor, prefix_len  [batch]
 *   page_table          [batch, max_pages], read as a ring; every entry the
 *                       window and the block reach (logical pages up to
 *                       (L_r + S - 1) / P, mod max_pages) must be a valid page
 *   max_prefix_len      host upper bound of every prefix_len[r] (sizes the
 *                       split-KV grid; larger prefixes are truncated to it)
 *   block_ids           nullable [batch, S] out: [anchor, MASK, ...]
 *   positions, slots    [batch, S] out: logical positions and cache slots of the
 *                       block rows (the slots the committed rows are later
 *                       injected into)
 *   candidates          [batch, S] out: [anchor, d_1 .. d_{S-1}]
 *   logits              nullable [batch, S-1, V] act_dtype out
 *   workspace           >= dflash_draft_workspace_bytes(cfg, batch, max_prefix_len)
 */
dflash_status dflash_draft_block(const dflash_config* cfg, const dflash_weights* w,
                                 const dflash_kv_cache* cache, const int32_t* anchor,
                                 const int32_t* prefix_len, const int32_t* page_table,
                                 int32_t max_pages, int32_t batch, int32_t max_prefix_len,
                                 int32_t* block_ids, int32_t* positions, int32_t* slots,
                                 int32_t* candidates, void* logits, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * (2-noalloc) dflash_draft_block for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, kernels and results as dflash_draft_block
 * except that the workspace is a fixed device array inside the library
 * (dflash_draft_block_noalloc_limit() bytes, 64 MiB; one copy per GPU, held
 * until the process ends).  The caller still passes every input and output.
 *   - A call whose dflash_draft_workspace_bytes(cfg, batch, max_prefix_len)
 *     exceeds the limit returns DFLASH_EWORKSPACE before any HIP call.
 *   - The first call on a device looks up that device's copy of the array
 *     (the current device, hipGetDevice); nothing is allocated, then or later.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (different streams, or threads) race and give wrong
 *     results.  Calls ordered on one stream are safe.  Nothing in the array
 *     needs to start at zero: each call writes every scratch value it reads.
 */
size_t dflash_draft_block_noalloc_limit(void);
dflash_status dflash_draft_block_noalloc(const dflash_config* cfg, const dflash_weights* w,
                                         const dflash_kv_cache* cache, const int32_t* anchor,
                                         const int32_t* prefix_len, const int32_t* page_table,
                                         int32_t max_pages, int32_t batch, int32_t max_prefix_len,
                                         int32_t* block_ids, int32_t* positions, int32_t* slots,
                                         int32_t* candidates, void* logits, void* stream);

/*
 * (3) Greedy verify-accept and commit ("Inside SGLang ...", Step 6 and Step 7;
 * CSDN DFlash article, the z-lab verify step and SGLang flow steps 7-9).
 *
 * candidates[r] = [anchor, d_1 .. d_{S-1}]; posterior[r, j] = the target's
 * greedy token after reading candidates[r, j].  accept_len = length of the
 * longest prefix with d_{j+1} == posterior[j]; commit_len = accept_len + 1;
 * out_tokens[r] = d_1 .. d_a, posterior[a], then zeros; next_anchor =
 * posterior[a]; new_seq_len = prefix_len + commit_len (the logical crop).
 *   candidates, posterior, out_tokens  [batch, block_size]
 *   prefix_len, accept_len, commit_len, next_anchor, new_seq_len  [batch]
 * Bit-exact integer work; no workspace.
 */
dflash_status dflash_accept(const int32_t* candidates, const int32_t* posterior,
                            const int32_t* prefix_len, int32_t batch, int32_t block_size,
                            int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens,
                            int32_t* next_anchor, int32_t* new_seq_len, void* stream);

/*
 * (3a) Greedy verify-accept reading the target's logits ("Inside SGLang ...",
 * Step 6: the verify forward's logits give the target's greedy choice after
 * each block position): posterior[r, j] = the first index among the largest
 * values of target_logits[r, j] (a NaN logit never wins), then exactly
 * dflash_accept.  The argmax runs on the GPU in chunks of 16384 columns.
 *   candidates     [batch, block_size]
 *   target_logits  [batch, block_size, vocab] logits_dtype (F32 or BF16)
 *   prefix_len and the outputs as dflash_accept
 *   workspace      >= dflash_accept_logits_workspace_bytes(batch, block_size,
 *                  vocab), 16-byte aligned
 * Bit-exact integer results; block_size 2..64; vocab <= 524288.
 */
size_t dflash_accept_logits_workspace_bytes(int32_t batch, int32_t block_size, int32_t vocab);
dflash_status dflash_accept_logits(const int32_t* candidates, const void* target_logits,
                                   int32_t logits_dtype, int32_t vocab,
                                   const int32_t* prefix_len, int32_t batch, int32_t block_size,
                                   int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens,
                                   int32_t* next_anchor, int32_t* new_seq_len, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * (3') Rejection-sampling verify-accept and commit ("Inside SGLang ...", the
 * section on sampling with the proposal distribution the drafter used, and
 * Step 6 for the outputs; CSDN DFlash article, SGLang flow step 7: non-greedy
 * requests take a speculative-sampling verify).
 *
 * p_j = softmax(target_logits[r, j] / target_temperature) is the target's
 * distribution after reading candidates[r, j]; q_j = softmax(draft_logits[r, j]
 * / draft_temperature), or, when draft_logits is NULL (argmax drafts), the
 * point mass on d_{j+1}.  Walking j = 0 .. S-2, d_{j+1} survives when
 * uniforms[r, j] * q_j(d_{j+1}) < p_j(d_{j+1}); at the first rejection (a = j)
 * the token is drawn from [p_j - q_j]_+, after full acceptance (a = S-1) from
 * p_{S-1}.  The draw is an inverse CDF: the smallest token t whose running sum
 * of weights exceeds uniforms[r, S-1] * (sum of the weights); a residual with
 * no mass falls back to p_j; a draw past the last running sum takes the last
 * token with weight.  Outputs as dflash_accept: accept_len = a, commit_len =
 * a + 1, out_tokens = d_1 .. d_a, the drawn token, then zeros; next_anchor =
 * the drawn token; new_seq_len = prefix_len + commit_len.
 *
 *   candidates     [batch, block_size]      [anchor, d_1 .. d_{S-1}], ids < vocab
 *   target_logits  [batch, block_size, vocab] logits_dtype
 *   draft_logits   nullable [batch, block_size - 1, vocab] logits_dtype (the
 *                  layout dflash_draft_block writes)
 *   uniforms       [batch, block_size] f32 draws in [0, 1), supplied by the caller
 *   prefix_len     [batch]
 *   workspace      >= dflash_accept_sampling_workspace_bytes(batch, block_size,
 *                  vocab, draft_logits != NULL), 16-byte aligned
 * Arithmetic is fp32 with fixed-order sums (deterministic).  block_size 2..64;
 * vocab <= 524288; logits_dtype F32 or BF16; temperatures finite and > 0 (draft_temperature is
 * read only with draft_logits).  NaN or +inf logits give unspecified tokens.
 */
size_t dflash_accept_sampling_workspace_bytes(int32_t batch, int32_t block_size, int32_t vocab,
                                              int32_t has_draft_logits);
dflash_status dflash_accept_sampling(const int32_t* candidates, const void* target_logits,
                                     const void* draft_logits, int32_t logits_dtype,
                                     int32_t vocab, float target_temperature,
                                     float draft_temperature, const float* uniforms,
                                     const int32_t* prefix_len, int32_t batch,
                                     int32_t block_size, int32_t* accept_len,
                                     int32_t* commit_len, int32_t* out_tokens,
                                     int32_t* next_anchor, int32_t* new_seq_len, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * (3'') Rejection-sampling verify with the proposal given as q_k (id,
 * probability) pairs per drafted row: the DFlash 2 selector's cand_ids and
 * q_rows ("Inside SGLang ...", section on sampling with the proposal
 * distribution the walk used: the selector's q rows, not the unary
 * distribution).  q_j(t) = the probability paired with t in row j (0 for a
 * token not listed); everything else as dflash_accept_sampling.
 *   q_ids    [batch, block_size - 1, q_k] int32;  q_probs [batch, block_size - 1, q_k] f32
 *   workspace >= dflash_accept_sampling_workspace_bytes(batch, block_size, vocab, 0)
 * q_k 1..16.
 */
dflash_status dflash_accept_sampling_sparse(
    const int32_t* candidates, const void* target_logits, int32_t logits_dtype, int32_t vocab,
    float target_temperature, const int32_t* q_ids, const float* q_probs, int32_t q_k,
    const float* uniforms, const int32_t* prefix_len, int32_t batch, int32_t block_size,
    int32_t* accept_len, int32_t* commit_len, int32_t* out_tokens, int32_t* next_anchor,
    int32_t* new_seq_len, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Cache reservation before acceptance is known ("Inside SGLang ...", Step 2:
 * a 2 x block_size page-aligned headroom beyond the committed prefix;
 * allocation is not acceptance; the overlap section and the Spec V2 PR: the
 * next step plans from the lengths the GPU published).  Enqueued after
 * dflash_accept on the same stream, it reads the new_seq_len that call wrote.
 *
 * For each request r in batch order: need = ceil((seq_len[r] + 2 * block_size)
 * / page_size) pages; the pages it lacks (need - n_pages[r]) are popped from
 * the top of the free stack (free_pages[free_count - 1], then below) and
 * appended to page_table[r] from entry n_pages[r]; n_pages[r] = need.  The
 * first request whose shortfall exceeds the stack (status 1) or whose need
 * exceeds max_pages (status 2) is left as it is, and so is every later one.
 *   seq_len     [batch]   committed lengths (device)
 *   page_table  [batch, max_pages]; n_pages [batch]: pages each row holds
 *   free_pages  [free_capacity] stack of free physical pages; free_count [1]
 *   status      [1] out: 0 served, 1 out of pages, 2 row too short
 * Rows are linear (logical page i in entry i): a request read through a draft
 * window keeps a fixed ring of pages (dflash_draft_block) and is not passed
 * here, since its need grows past any ring (status 2).
 * Reservations never shrink or move a page.  dflash_release_pages pushes the
 * pages of every request with mask[r] != 0 back (batch order, row order) and
 * sets its n_pages to 0.  Deterministic; one workgroup; no workspace.
 */
dflash_status dflash_reserve_pages(const int32_t* seq_len, int32_t batch, int32_t block_size,
                                   int32_t page_size, int32_t* page_table, int32_t max_pages,
                                   int32_t* n_pages, const int32_t* free_pages,
                                   int32_t free_capacity, int32_t* free_count, int32_t* status,
                                   void* stream);
dflash_status dflash_release_pages(const int32_t* mask, int32_t batch, const int32_t* page_table,
                                   int32_t max_pages, int32_t* n_pages, int32_t* free_pages,
                                   int32_t free_capacity, int32_t* free_count, void* stream);

/*
 * Relay of per-request decode state through a request pool ("Inside SGLang
 * ...", section "Back in the scheduler: GPU continuation and CPU output":
 * before the worker, the previous iteration's anchor and lengths are gathered
 * for the current request rows; after it, the lengths and the next anchor are
 * stashed; the relay is indexed by request-pool slots, so the batch can be
 * filtered or merged between iterations without the old row order).
 *
 * The pool holds, per slot, the request's next anchor, committed length, and
 * its page-table row with the count of pages it holds (the reservation
 * travels with the request).  A batch is req_slots[batch]: distinct pool
 * slots, in the order of the batch rows (device memory, so the next
 * iteration's composition can be written without a host round trip).
 *   dflash_relay_resolve  batch row b <- pool slot req_slots[b]: anchor,
 *                         prefix_len, page_table[b, :], n_pages (a slot
 *                         outside [0, capacity) gives 0, 0, a row of -1, 0)
 *   dflash_relay_stash    pool slot req_slots[b] <- batch row b: next_anchor,
 *                         new_seq_len, page_table[b, :], n_pages (a slot
 *                         outside the pool is skipped; every other slot is
 *                         left as it is)
 * Typical cycle, all on one stream: resolve -> dflash_draft_block -> accept
 * -> dflash_reserve_pages (on the batch rows) -> stash -> dflash_project_context
 * of the committed rows.  Batch-side page_table rows have the pool's
 * max_pages entries.  Each of the four fields is copied when both its pool
 * array and its batch array are non-NULL and skipped when both are NULL
 * (DFLASH_EINVAL otherwise).  Duplicate slots in one stash are the caller's
 * error (unspecified which row lands).  Bit-exact integer copies; no workspace.
 */
typedef struct {
  int32_t* anchor;      /* [capacity] next anchor                                */
  int32_t* seq_len;     /* [capacity] committed length                           */
  int32_t* page_table;  /* [capacity, max_pages] physical pages in logical order */
  int32_t* n_pages;     /* [capacity] pages held                                 */
  int32_t capacity;
  int32_t max_pages;
} dflash_request_pool;
dflash_status dflash_relay_resolve(const dflash_request_pool* pool, const int32_t* req_slots,
                                   int32_t batch, int32_t* anchor, int32_t* prefix_len,
                                   int32_t* page_table, int32_t* n_pages, void* stream);
dflash_status dflash_relay_stash(const dflash_request_pool* pool, const int32_t* req_slots,
                                 int32_t batch, const int32_t* next_anchor,
                                 const int32_t* new_seq_len, const int32_t* page_table,
                                 const int32_t* n_pages, void* stream);

/*
 * (2') One draft pass with the DFlash 2 candidate selector in place of the
 * argmax ("Inside SGLang ...", section on DFlash 2: candidates, lattice, walk).
 *
 * Runs dflash_draft_block's backbone and lm_head, then, per drafted row j
 * (block rows 1..S-1): the top_k tokens by logit (descending, ties to the
 * lower id; NaN never wins) -> cand_ids[b, j, :] with their logits U; the
 * lattice score(p, c) = U(c) + <a[p] * (w_h y_j), b[c]> for every predecessor
 * p (the anchor for j = 0, else each candidate of row j - 1) and candidate c,
 * y_j the row after the final RMSNorm; and the walk: from the anchor's row,
 * the chosen candidate's row at the next position, taking the first maximum
 * (uniforms NULL) or the smallest candidate whose running sum of
 * softmax(row / temperature) exceeds uniforms[b, j].  q_rows[b, j, :] is
 * the distribution the choice was drawn from: softmax(row / temperature) of
 * the row walked when sampling, one-hot on the chosen slot when greedy (the
 * proposal of a greedy walk is a point mass), so either feeds
 * dflash_accept_sampling_sparse as it is;
 * candidates[b] = [anchor, chosen tokens].  The selector weights' values,
 * top_k and rank are the caller's (the pages give none).
 *
 *   sel->a, sel->b  [vocab, rank] act_dtype;  sel->w_h [rank, hidden]
 *                   fragment-packed (dflash_pack_matrix)
 *   cand_ids        [batch, S-1, top_k] out;  q_rows [batch, S-1, top_k] f32 out
 *   uniforms        nullable [batch, S-1] f32 draws in [0, 1)
 *   logits          nullable [batch, S-1, vocab] out (kept in the workspace
 *                   when NULL)
 *   workspace       >= dflash_selector_workspace_bytes(cfg, sel, batch,
 *                   max_prefix_len)
 * top_k in {1, 2, 4, 8, 16}, rank in {16, 32, 64, 128}, vocab <= 524288; other
 * arguments as
 * dflash_draft_block.
 */
typedef struct {
  const void* a;    /* [vocab, rank] predecessor table                         */
  const void* b;    /* [vocab, rank] successor table                           */
  const void* w_h;  /* [rank, hidden] projection of the hidden row, packed      */
  int32_t rank;
  int32_t top_k;
} dflash_selector;
size_t dflash_selector_workspace_bytes(const dflash_config* cfg, const dflash_selector* sel,
                                       int32_t batch, int32_t max_prefix_len);
dflash_status dflash_draft_block_selector(
    const dflash_config* cfg, const dflash_weights* w, const dflash_kv_cache* cache,
    const dflash_selector* sel, const int32_t* anchor, const int32_t* prefix_len,
    const int32_t* page_table, int32_t max_pages, int32_t batch, int32_t max_prefix_len,
    int32_t* block_ids, int32_t* positions, int32_t* slots, int32_t* candidates,
    int32_t* cand_ids, float* q_rows, const float* uniforms, float temperature, void* logits,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The draft-token selection step alone ("Inside SGLang ...", Step 4: the target
 * lm_head over the final draft hidden rows, then argmax): logits = hidden
 * lm_head^T rounded to act_dtype, ids = argmax per row (first index among
 * equal maxima).  dflash_draft_block runs the same kernels on its rows
 * 1..S-1; this entry point serves callers that hold the normalised rows.
 *   lm_head    [V, H] fragment-packed (dflash_pack_matrix)
 *   hidden     [rows, H] act_dtype (already through the final RMSNorm)
 *   logits     nullable [rows, V] act_dtype out
 *   ids        [rows] out
 *   workspace  >= dflash_lm_head_workspace_bytes(cfg, rows)
 */
size_t dflash_lm_head_workspace_bytes(const dflash_config* cfg, int32_t rows);
dflash_status dflash_lm_head_argmax(const dflash_config* cfg, const void* lm_head,
                                    const void* hidden, int32_t rows, void* logits, int32_t* ids,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Checked mode (tests and debugging; not for the serving loop).  The calls
 * above check what the host sees; the values they read from device memory
 * are the caller's contract, which their kernels only clamp.  These calls
 * check that contract on the device: each launches two small kernels on
 * `stream` that write `report` (device memory, 2 * DFLASH_CHECKS int32:
 * per rule k, report[2k] = the number of violations and report[2k+1] = the
 * smallest index among them, INT32_MAX when there is none) and reads nothing
 * back, so the caller synchronises and reads the report.  Rules without a
 * meaning for a call report 0, INT32_MAX.  No other call runs them.
 *
 * dflash_check_draft_inputs, for dflash_draft_block's arguments (indices r =
 * batch row):
 *   0  anchor[r] outside [0, vocab)
 *   1  prefix_len[r] outside [0, max_prefix_len]
 *   2  without a draft window (context_window 0): prefix_len[r] + block_size
 *      > max_pages * page_size (the block does not fit the page-table row)
 *   3  a page-table entry the pass reads outside [0, num_pages): the entries
 *      of the logical pages holding keys [lo, prefix_len[r] + block_size),
 *      lo = max(0, prefix_len[r] - context_window) with a draft window (a
 *      ring row: logical page p at entry p mod max_pages) and 0 without one
 *      (entries below max_pages); prefix_len[r] clamped to [0,
 *      max_prefix_len] for this rule; index r * max_pages + entry
 * dflash_check_context_inputs, for dflash_project_context's (indices t = row,
 * r = request; a live row is one with t mod rows_per_req < valid_rows[t /
 * rows_per_req], every row when valid_rows is NULL):
 *   0  a live row's slot outside [0, num_pages * page_size)
 *   1  a live row's position < 0
 *   2  valid_rows[r] outside [0, rows_per_req]
 * dflash_check_accept_inputs, for dflash_accept's (indices i = r *
 * block_size + j, r):
 *   0  candidates[i] outside [0, vocab)
 *   1  posterior[i] outside [0, vocab)
 *   2  prefix_len[r] < 0
 * Errors: DFLASH_EINVAL for NULL pointers (valid_rows may be NULL), negative
 * sizes, or indices that would not fit an int32 (batch * max_pages, n_req *
 * rows_per_req, batch * block_size above 2^31 - 1); DFLASH_EHIP for a launch
 * failure.
 */
#define DFLASH_CHECKS 4
dflash_status dflash_check_draft_inputs(const dflash_config* cfg, const dflash_kv_cache* cache,
                                        const int32_t* anchor, const int32_t* prefix_len,
                                        const int32_t* page_table, int32_t max_pages,
                                        int32_t batch, int32_t max_prefix_len, int32_t* report,
                                        void* stream);
dflash_status dflash_check_context_inputs(const dflash_config* cfg, const dflash_kv_cache* cache,
                                          const int32_t* positions, const int32_t* slots,
                                          const int32_t* valid_rows, int32_t n_req,
                                          int32_t rows_per_req, int32_t* report, void* stream);
dflash_status dflash_check_accept_inputs(const int32_t* candidates, const int32_t* posterior,
                                         const int32_t* prefix_len, int32_t batch,
                                         int32_t block_size, int32_t vocab, int32_t* report,
                                         void* stream);

const char* dflash_status_string(dflash_status s);
const char* dflash_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
