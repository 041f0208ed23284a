/* dflash.h -- C ABI of the DFlash draft hot path on MI355X (gfx950).
 *
 * DFlash ("DFlash: Block Diffusion for Flash Speculative Decoding"; the paper
 * is arXiv 2602.06036) speculates a block of tokens with a small drafter that
 * reads the target model's hidden states.  One speculative cycle (summary
 * page, "Putting It Together", steps 2-4) is three calls here:
 *
 *   dflash_inject_ctx    fuse the target features of new context tokens and
 *                        append their per-layer K/V to the draft cache
 *   dflash_draft_block   one parallel forward over [anchor, mask, ..., mask]
 *                        -> proposed block
 *   dflash_verify_greedy compare the block with the target's argmax tokens
 *                        -> accepted length and output tokens
 *
 * Conventions for every call:
 *   - Pointers are DEVICE memory unless marked [host].  The caller owns all
 *     memory (weights, KV pages, page table, context lengths, workspace,
 *     outputs); the library allocates nothing in these calls.
 *   - Matrices are row-major [out][in].  Element type is the model dtype
 *     (DFLASH_BF16: raw bf16 bits; DFLASH_F32: float) unless stated.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL is the default stream).  No call synchronises except
 *     dflash_device_error and dflash_profile_read.
 *   - Return value: DFLASH_OK or a negative dflash_status.  Host-checkable
 *     problems (null pointers, shapes, dtype, sizes, workspace too small) are
 *     reported before anything is launched; dflash_last_error() gives the
 *     message.  Problems only the device can see (a page index outside the
 *     pool, a position beyond the page table, an anchor outside the vocab)
 *     set a sticky device error word and the offending reads/writes are
 *     skipped; dflash_device_error() reads it.
 *   - Calls that share a model, cache or workspace and overlap in time race;
 *     order them on one stream.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH_OK = 0,
  DFLASH_E_INVAL = -1,    /* null pointer or out-of-range scalar argument */
  DFLASH_E_SHAPE = -2,    /* dimensions the kernels do not support */
  DFLASH_E_DTYPE = -3,    /* unknown or mismatched element type */
  DFLASH_E_CAPACITY = -4, /* workspace / batch / block larger than provisioned */
  DFLASH_E_HIP = -5,      /* a HIP runtime call failed */
  DFLASH_E_DEVICE = -6    /* the device error word was set (see below) */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Device error word bits (dflash_device_error). */
#define DFLASH_DEVERR_PAGE 1u     /* page-table entry outside [0, n_pages) */
#define DFLASH_DEVERR_POS 2u      /* position beyond max_pages_per_seq*page_size */
#define DFLASH_DEVERR_TOKEN 4u    /* anchor token outside [0, vocab) (row uses token 0) */
#define DFLASH_DEVERR_XCD 8u      /* a split-K reduction ran on a chiplet that could not see
                                     all partial sums (workgroups were not placed round-robin
                                     over the 8 XCDs); the call's results are unreliable */

#define DFLASH_MAX_LAYERS 16
#define DFLASH_MAX_BLOCK 16
#define DFLASH_STATE_BYTES 16384

/* Drafter dimensions.  Constraints checked at model creation:
 *   hidden % 4 == 0 and hidden <= 8192, head_dim in {64, 128},
 *   n_q_heads % n_kv_heads == 0, n_q_heads / n_kv_heads <= 8,
 *   n_target_feats >= 1, 1 <= max_block <= DFLASH_MAX_BLOCK, page_size == 16,
 *   0 <= mask_token_id < vocab, n_layers <= DFLASH_MAX_LAYERS;
 *   bf16 models also need hidden, intermediate and n_q_heads * head_dim to
 *   be multiples of 256. */
typedef struct {
  int32_t hidden;          /* D */
  int32_t n_layers;        /* draft layers (5 for the Qwen3-8B-shaped drafter) */
  int32_t n_q_heads;       /* Hq */
  int32_t n_kv_heads;      /* Hkv */
  int32_t head_dim;        /* dh */
  int32_t intermediate;    /* SwiGLU width I */
  int32_t vocab;           /* V, shared with the target's embedding and LM head */
  int32_t n_target_feats;  /* m: target layers fused per token (5) */
  int32_t max_block;       /* largest block size (anchor included) */
  int32_t mask_token_id;   /* token id of the mask positions */
  int32_t page_size;       /* tokens per KV page (16) */
  int32_t dtype;           /* dflash_dtype of weights, activations and cache */
  float rope_theta;        /* rotary base (1e6) */
  float rms_eps;           /* RMSNorm epsilon (1e-6) */
} dflash_config;

/* Per-layer weights, device pointers in the model dtype:
 *   attn_norm, mlp_norm [D]; wq [Hq*dh][D]; wk, wv [Hkv*dh][D];
 *   wo [D][Hq*dh]; w_gate, w_up [I][D]; w_down [D][I]. */
typedef struct {
  const void* attn_norm;
  const void* wq;
  const void* wk;
  const void* wv;
  const void* wo;
  const void* mlp_norm;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
} dflash_layer_weights;

/* fc_w [D][m*D] is W_c, the context projection (summary page, "Target Hidden
 * States Supply the Missing Context"; paper §7.3), with gain fc_norm [D].
 * embed and lm_head [V][D] are the target's (frozen, shared; paper §4.2
 * "Shared embedding and LM head"); they may alias.  final_norm [D]. */
typedef struct {
  const void* fc_w;
  const void* fc_norm;
  const void* embed;
  const void* lm_head;
  const void* final_norm;
  dflash_layer_weights layer[DFLASH_MAX_LAYERS];
} dflash_weights;

/* Paged draft KV cache: the injected target context of every draft layer
 * (paper §4.1: the projected features are stored in the draft model's KV
 * cache and reused across drafting iterations).  Block K/V are never stored.
 *   pages      [n_layers][n_pages][2 (K, V)][n_kv_heads][page_size * head_dim]:
 *              the K half of a page is [page_size][head_dim] (token-major),
 *              the V half is [head_dim][page_size] (dimension-major), so
 *              that attention streams both as contiguous blocks
 *   page_table [batch][max_pages_per_seq]: page of tokens
 *              [i*page_size, (i+1)*page_size) of each sequence
 *   ctx_lens   [batch]: tokens already in the cache per sequence; K is
 *              stored after rotary embedding at its absolute position. */
typedef struct {
  void* pages;
  int32_t n_pages;
  int32_t max_pages_per_seq;
  const int32_t* page_table;
  int32_t* ctx_lens;
} dflash_kv;

typedef struct dflash_model dflash_model;   /* opaque host handle */

/* Create a model handle.  cfg and w are [host] structs; the weight pointers
 * are device pointers the caller keeps alive for the handle's lifetime.
 * state: device buffer of DFLASH_STATE_BYTES bytes owned by the caller (it
 * holds the sticky device error word, the LM-head argmax slots and the
 * arrival counters of the split-K reductions, which every call leaves at
 * zero, and the workgroup placement the last split-K launch observed); it is
 * cleared here
 * (synchronously).  The handle binds to the device current at creation.
 * Calls that share a handle must be ordered (one stream, or streams joined
 * by events): concurrent calls on one handle race on its counters. */
int dflash_model_create(const dflash_config* cfg, const dflash_weights* w, void* state,
                        dflash_model** out /* [host] */);
void dflash_model_destroy(dflash_model* model);

/* Bytes of workspace the three calls need for at most max_batch sequences,
 * blocks of at most max_block positions, at most max_new_tokens tokens per
 * inject call, and page tables of at most max_pages_per_seq entries.
 * Returns 0 for invalid arguments. */
size_t dflash_workspace_bytes(const dflash_model* model, int32_t max_batch, int32_t max_block,
                              int32_t max_new_tokens, int32_t max_pages_per_seq);

/* Packed weights (bf16 models).  The products with at most 64 rows (block
 * rows of up to 4 sequences, or up to 64 injected tokens) stream their
 * weights faster from a copy in matrix-core tile order: for each product,
 * its rows in the order the kernel walks them, padded to a multiple of 64,
 * cut into 16-row x 32-column tiles of 1 KB whose 16-byte pieces sit in the
 * order of the lanes that consume them, stored [64-row group][32-column
 * block][16-row group]; every weight load of a wave reads 1 KB of contiguous
 * memory and the four waves of a workgroup read 4 adjacent KB.
 *   dflash_packed_weight_bytes: size of that copy (0 for fp32 models).
 *   dflash_pack_weights: fills `packed` [device, caller-owned, 256-byte
 *     aligned, >= dflash_packed_weight_bytes] from the model's weights on
 *     `stream` and makes the model use it from then on; calls on other
 *     streams must be ordered after the packing.  The caller keeps the
 *     buffer alive for the handle's lifetime, and the original weights too
 *     (the other paths read them).  Returns DFLASH_E_DTYPE for fp32 models,
 *     DFLASH_E_CAPACITY if `bytes` is too small. */
size_t dflash_packed_weight_bytes(const dflash_model* model);
int dflash_pack_weights(dflash_model* model, void* packed, size_t bytes, void* stream);

/* Context injection (summary page: "Target Hidden States Supply the Missing
 * Context", eq. H_t = RMSNorm(W_c [H^(l1); ...; H^(lm)]), and "Per-Layer K/V
 * Injection Prevents Context Dilution", K_i = [W_i^K H_t; ...],
 * V_i = [W_i^V H_t; ...]; paper §4.1 and §7.3).
 *   target_hidden [n_tok][m*D]: the new tokens' target features, per token
 *                 the m selected layers concatenated shallow to deep; the
 *                 tokens of sequence b are rows cu_new[b] .. cu_new[b+1]-1
 *   cu_new        [batch+1] device prefix sums of new tokens per sequence,
 *                 cu_new[0] = 0, cu_new[batch] = n_tok
 *   n_tok         [host] total new tokens (grid sizing; 0 is a no-op)
 * For token i of sequence b, position p = ctx_lens[b] + i:
 *   c = RMSNorm(W_c f) and, for every layer l, K = RoPE(W_K^l c, p),
 *   V = W_V^l c are written to page page_table[b][p / page_size], slot
 *   p % page_size; afterwards ctx_lens[b] += cu_new[b+1] - cu_new[b]. */
int dflash_inject_ctx(const dflash_model* model, const dflash_kv* kv, const void* target_hidden,
                      const int32_t* cu_new, int32_t batch, int32_t n_tok, void* workspace,
                      size_t ws_bytes, void* stream);

/* Single-pass block draft (summary page: "Block Diffusion Makes Draft Cost
 * Nearly Independent of Block Length" and "Putting It Together", step 3;
 * paper §3.2 and §4.1 "Parallel diffusion drafting").
 *   anchor       [batch] the clean anchor token of each sequence
 *   block_size   gamma, 1..max_block, positions in the block incl. the anchor
 *   block_tokens [batch][gamma] out: [anchor, d_1, ..., d_{gamma-1}],
 *                d_j = lowest-index argmax of the logits of row j
 *   logits       [batch][gamma][V] fp32 out, or NULL
 * Row j of sequence b holds token (j == 0 ? anchor : mask_token_id) at
 * position ctx_lens[b] + j; its attention sees the sequence's ctx_lens[b]
 * cached keys and all gamma block keys (bidirectional, no mask inside the
 * block).  The cache and ctx_lens are read only. */
int dflash_draft_block(const dflash_model* model, const dflash_kv* kv, const int32_t* anchor,
                       int32_t batch, int32_t block_size, int32_t* block_tokens, float* logits,
                       void* workspace, size_t ws_bytes, void* stream);

/* Bytes of the scratch array behind dflash_draft_block_noalloc, per GPU. */
#define DFLASH_NOALLOC_SCRATCH_BYTES (48u << 20)

/* dflash_draft_block for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same draft and the same results, with no workspace
 * argument: its scratch is a static device array of
 * DFLASH_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends (dflash_model_create locates its device's copy).
 * The call allocates nothing and never records profiling events.
 *   - DFLASH_E_CAPACITY (before any launch) when the call needs more scratch
 *     than that (its need is at most dflash_workspace_bytes(model, batch,
 *     block_size, 0, kv->max_pages_per_seq) bytes).  Batch 1 at block 16 on a drafter of
 *     hidden 4096, 32 query heads and SwiGLU width 12288 fits with a page
 *     table of up to 8192 pages (131072 context tokens).
 *   - DFLASH_E_INVAL when the current device is not the model's;
 *     DFLASH_E_HIP when the array could not be located on it.
 * All calls on one GPU share the array and it keeps the last call's
 * contents: calls that overlap in time on one GPU race (order them on one
 * stream).  Each call writes every scratch byte before it reads it, so
 * nothing needs clearing between calls.  Other arguments as
 * dflash_draft_block. */
int dflash_draft_block_noalloc(const dflash_model* model, const dflash_kv* kv,
                               const int32_t* anchor, int32_t batch, int32_t block_size,
                               int32_t* block_tokens, float* logits, void* stream);

/* Greedy verification (summary page: "The Target Verifier Remains the
 * Correctness Anchor" -- at temperature 0 the acceptance rule
 * min(1, p_t/p_d) accepts a proposal exactly when it is the target's argmax;
 * paper §3.1 for the accepted length).
 *   block_tokens  [batch][gamma]: [anchor, d_1, ..., d_{gamma-1}]
 *   target_logits [batch][gamma][vocab] in logits_dtype: row j is the
 *                 target's scores for the token after block[0..j]
 *   accept_len    [batch] out: tau = n + 1, n = longest prefix with
 *                 block[j] == T_{j-1} for j = 1..n, T_j = lowest-index
 *                 argmax of row j
 *   out_tokens    [batch][gamma] out: block[1..n], T_n, then -1
 *   target_argmax [batch][gamma] out (T_j), or NULL
 *   workspace     at least dflash_verify_greedy_workspace_bytes(batch,
 *                 block_size, vocab) = 8 * batch * block_size *
 *                 ceil(vocab / 8192) bytes (one argmax key per row and
 *                 8192-column chunk; covered by dflash_workspace_bytes for
 *                 the model's vocabulary).  Nothing in it needs clearing.
 * Limits: block_size <= 1024 (DFLASH_E_CAPACITY). */
size_t dflash_verify_greedy_workspace_bytes(int32_t batch, int32_t block_size, int32_t vocab);
int dflash_verify_greedy(const int32_t* block_tokens, const void* target_logits,
                         int32_t logits_dtype, int32_t batch, int32_t block_size, int32_t vocab,
                         int32_t* accept_len, int32_t* out_tokens, int32_t* target_argmax,
                         void* workspace, size_t ws_bytes, void* stream);

/* Sampled block draft: dflash_draft_block with each proposal drawn from
 * the drafter's distribution instead of taken as its argmax (the lossless
 * rule of the summary page's section "The Target Verifier Remains the
 * Correctness Anchor" checks proposals drawn from p_d).  The draw is
 * Gumbel-max at temperature 1:
 *   d_j = lowest-index argmax over v of logits[b][j][v] + g(seed, b, j, v),
 *   g = -log(-log(w)), w = (2 * (z >> 41) + 1) / 2^24, z the n-th output of
 *   SplitMix64 started at `seed` (Steele, Lea and Flood 2014) with
 *   n = (b << 40 | j << 32 | v) + 1, evaluated in fp32.
 * The noise depends only on (seed, b, j, v): pass a fresh seed per call.
 *   logits [batch][gamma][V] fp32 out, required (the verifier needs p_d).
 * Everything else as dflash_draft_block; DFLASH_E_INVAL for NULL logits. */
int dflash_draft_block_sampled(const dflash_model* model, const dflash_kv* kv,
                               const int32_t* anchor, int32_t batch, int32_t block_size,
                               uint64_t seed, int32_t* block_tokens, float* logits,
                               void* workspace, size_t ws_bytes, void* stream);

/* Lossless (stochastic) verification of a sampled block (summary page,
 * section "The Target Verifier Remains the Correctness Anchor": proposal
 * x_k is kept with probability min(1, p_t(x_k) / p_d(x_k)); the first
 * rejection is corrected from the residual distribution and the rest of
 * the block dropped; a block kept whole earns a bonus token).
 *   block_tokens  [batch][gamma]: [anchor, x_1, ..., x_{gamma-1}]
 *   draft_logits  [batch][gamma][vocab] fp32: row k gives p_d of x_k (row 0
 *                 is not read), as written by dflash_draft_block_sampled
 *   target_logits [batch][gamma][vocab] in logits_dtype: row j gives p_t of
 *                 the token after block[0..j]
 *   uniforms      [batch][gamma] fp32 in [0, 1): uniforms[b][k] decides x_k,
 *                 uniforms[b][0] draws the correction or the bonus token
 * p_d and p_t are softmax rows at temperature 1; every decision is the
 * one their fp64 values give (fp32 normalisers decide where the margin is
 * wide, fp64 ones everywhere else).  x_k
 * (k = 1, 2, ...) is kept while u_k * p_d[k](x_k) < p_t[k-1](x_k); a token
 * outside [0, vocab) is never kept.  At the first rejection k:
 * accept_len = k and out_tokens = [x_1 .. x_{k-1}, r, -1 ...] with r drawn
 * from max(0, p_t[k-1] - p_d[k]) (from p_t[k-1] when that has no mass);
 * with no rejection accept_len = gamma and the last token is drawn from
 * p_t[gamma-1].  A draw from weights w with uniform u is the smallest token
 * v whose running sum of w exceeds u * sum(w).
 *   workspace  device, 16-byte aligned, at least
 *              dflash_verify_stochastic_workspace_bytes(batch, gamma, vocab)
 *              = 16 * (ceil(vocab / 4096) * (4 * batch * gamma + 256 * batch)
 *                + batch)
 * Limits: gamma <= 64 and batch * gamma <= 65535 (DFLASH_E_CAPACITY).
 * Inputs are read only; rows of NaN logits give unspecified tokens. */
size_t dflash_verify_stochastic_workspace_bytes(int32_t batch, int32_t block_size, int32_t vocab);
int dflash_verify_stochastic(const int32_t* block_tokens, const float* draft_logits,
                             const void* target_logits, int32_t logits_dtype,
                             const float* uniforms, int32_t batch, int32_t block_size,
                             int32_t vocab, int32_t* accept_len, int32_t* out_tokens,
                             void* workspace, size_t ws_bytes, void* stream);

/* Packed multi-block forward (summary page: "Training Rehearses the Same
 * Masked Blocks Used at Runtime", Figure 4; paper §4.2 "Random sampling of
 * masked blocks") with the position-decayed loss (summary page: "Early
 * Positions Receive More Learning Budget"; paper §4.2 eq. 1).  Forward
 * only.  n_blocks blocks of one sequence run in one pass: block b holds
 * [anchors[b], mask, ..., mask] at positions anchor_pos[b] + j, and its rows
 * see the context keys [0, anchor_pos[b]) and the keys of their own block,
 * nothing of the other blocks.
 *   ctx         the sequence's context: page_table [1][max_pages_per_seq],
 *               ctx_lens [1] = tokens in the cache (read only)
 *   anchors     [n_blocks] clean anchor tokens
 *   anchor_pos  [n_blocks] anchor positions, each in [0, ctx_lens[0]]
 *               (else DFLASH_DEVERR_POS and the nearest bound is used)
 *   targets     [n_blocks][block_size] true tokens (column 0 unused), or
 *               NULL for no loss
 *   decay       the loss weights' constant: w_k = exp(-(k-1)/decay) for the
 *               predicted positions k = 1 .. block_size-1
 *   logits      [n_blocks][block_size][V] fp32 out (required)
 *   block_tokens [n_blocks][block_size] out (anchor, then argmax), or NULL
 *   block_loss  [n_blocks] fp32 out: sum_k w_k CE_k / sum_k w_k, CE_k =
 *               logsumexp(logits_k) - logits_k[target_k]; or NULL
 *   loss        [1] fp32 out: mean of the block losses; or NULL
 * A target outside [0, V) gives NaN for its block and sets
 * DFLASH_DEVERR_TOKEN.  workspace: at least dflash_packed_workspace_bytes
 * for this many blocks, block size and page-table width. */
size_t dflash_packed_workspace_bytes(const dflash_model* model, int32_t max_blocks,
                                     int32_t max_block, int32_t max_pages_per_seq);
int dflash_packed_forward(const dflash_model* model, const dflash_kv* ctx, const int32_t* anchors,
                          const int32_t* anchor_pos, int32_t n_blocks, int32_t block_size,
                          const int32_t* targets, float decay, float* logits,
                          int32_t* block_tokens, float* block_loss, float* loss,
                          void* workspace, size_t ws_bytes, void* stream);

/* Autoregressive drafting with the same drafter (paper §5.5.5, DFlash-AR:
 * K/V injection, autoregressive drafting; summary page "Block Diffusion
 * Makes Draft Cost Nearly Independent of Block Length": one forward pass per
 * proposed token).  For i = 1 .. block_size-1, pass i runs the drafter over
 * the tokens [anchor, d_1, ..., d_{i-1}] at positions ctx_lens[b] + j with a
 * causal mask inside them (row j sees the cached context and rows 0..j),
 * and d_i is the lowest-index argmax of the pass's last row.  Each pass
 * recomputes all its rows.
 *   block_tokens [batch][block_size] out: [anchor, d_1, ..., d_{block_size-1}]
 *                (also the passes' input, so it must not alias anchor)
 *   logits       [batch][block_size-1][V] fp32 out, or NULL: the last
 *                pass's rows; row j gives the scores that chose d_{j+1}
 *                (equal to pass j+1's last row, the mask being causal)
 *   workspace    at least dflash_ar_workspace_bytes(model, batch, block_size,
 *                max_pages_per_seq)
 * The cache and ctx_lens are read only. */
size_t dflash_ar_workspace_bytes(const dflash_model* model, int32_t max_batch, int32_t max_block,
                                 int32_t max_pages_per_seq);
int dflash_draft_block_ar(const dflash_model* model, const dflash_kv* kv, const int32_t* anchor,
                          int32_t batch, int32_t block_size, int32_t* block_tokens, float* logits,
                          void* workspace, size_t ws_bytes, void* stream);

/* Message for the last non-OK status returned on this thread. */
const char* dflash_last_error(void);

/* Synchronise `stream`, then read and clear the model's device error word
 * into *code [host] (a mask of DFLASH_DEVERR_*).  Returns DFLASH_OK,
 * DFLASH_E_DEVICE if the word was non-zero, or DFLASH_E_HIP. */
int dflash_device_error(const dflash_model* model, void* stream, int32_t* code);

/* Timing of the LM-head kernel of dflash_draft_block (the largest single
 * launch of the draft step).  While enabled, each draft call records a HIP
 * event pair on its stream around that launch.  Enabling creates 256 pairs
 * up front, so up to 256 timed calls between reads create no event (more
 * create pairs on demand).  dflash_profile_read waits for the recorded
 * events, returns the summed milliseconds and the number of launches timed
 * since the last reset, and returns their pairs to the pool. */
int dflash_profile_enable(dflash_model* model, int32_t on);
int dflash_profile_read(dflash_model* model, double* total_ms /* [host] */,
                        int64_t* count /* [host] */, int32_t reset);

/* Counter calibration (a measurement aid, not part of the method): stream
 * `bytes` of device memory at src with the LM head's load pattern (16-byte
 * non-temporal loads, each workgroup one contiguous run, a wave 1 KB of
 * contiguous memory per load instruction) and write one 16-byte checksum per
 * workgroup to out [workgroups].  The bytes read are known exactly, so a
 * hardware byte counter read over this call gives its scale for that
 * pattern.  bytes: a positive multiple of 16; workgroups: 1..65535.
 * DFLASH_E_INVAL otherwise or for null pointers. */
int dflash_read_calibration(const void* src, size_t bytes, void* out, int32_t workgroups,
                            void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
