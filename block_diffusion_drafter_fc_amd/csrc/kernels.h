// kernels.h -- launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// A virtual weight matrix [N][K] made of up to 32 row-stacked pieces (for
// example [W_Q; W_K; W_V]).  Piece s holds rows [row_end[s-1], row_end[s]);
// every boundary is a multiple of 16.
#define WSEG_MAX 32
struct WSeg {
  const void* ptr[WSEG_MAX];
  int32_t row_end[WSEG_MAX];
  int32_t n;
};

enum GemmKind { GEMM_F32 = 0, GEMM_SKINNY = 1, GEMM_TILED = 2, GEMM_BIG = 3 };

// Sampled drafting: the LM head's row argmax becomes a Gumbel-max draw over
// logit + gumbel_noise(seed, row / gamma, row % gamma, column).
struct DrawArgs {
  int on;
  int gamma;
  unsigned long long seed;
};

struct GemmPlan {
  int kind;
  int mt;      // skinny: 16-row tiles of M per wave (1, 2 or 4)
  int nt;      // skinny: 16-column tiles of N per wave
  int unroll;  // skinny: 32-wide K steps per loop iteration
  int waves;   // waves per workgroup (skinny: K split inside the group)
  int splits;  // workgroups along K; partial sums go to separate slices
  int kpw;     // K columns per wave (skinny) or per split (tiled)
};

// Choose the kernel and its split of K for out = A[M][K] * W[N][K]^T.
// argmax: the product feeds the fused row-argmax (no K split across groups).
GemmPlan plan_gemm(bool bf16, int M, int N, int K, bool argmax);

// Run the plan.  A: fp32 [M][lda] for fp32 models; bf16 [M][lda] for bf16
// models, with Alo the lo plane of a split activation (or null when A is an
// exact bf16 input).  Without `best`: part[s][M][N] (fp32) receives the
// partial product of split s.  With `best` (argmax mode, splits == 1):
// best[g][row] receives the argmax key of row `row` over the columns of
// group g (gemm_argmax_groups groups), and logits[M][N] receives the fp32
// products when non-null.
int gemm_argmax_groups(const GemmPlan& p, int N);
hipError_t launch_gemm(const GemmPlan& p, bool bf16, const void* A, const void* Alo, int lda,
                       int M, const WSeg& w, int N, int K, float* part, uint64_t* best,
                       float* logits, hipStream_t stream, const DrawArgs& draw = DrawArgs{});
// gate/up product with the SwiGLU in its epilogue: w = [W_gate; W_up] (I
// rows each), two activation planes, h = silu(A W_gate^T) * (A W_up^T) as
// split planes [M][I].  Only for plans gemm_swiglu_ok accepts (the large
// product, one K split, 192-column tiles).
bool gemm_swiglu_ok(const GemmPlan& p, int I);
hipError_t launch_gemm_swiglu(const GemmPlan& p, const void* A, const void* Alo, int lda, int M,
                              const WSeg& w, int I, int K, void* h, size_t h_plane,
                              hipStream_t stream);

// ---- skinny product with fused epilogues (bf16 models, M <= 64) -----------
// Activation source of the product.
enum SkinnyA {
  SA_SPLIT = 0,  // A: hi plane, A + a_plane: lo plane (transient fp32 activations)
  SA_BF16 = 1,   // A: exact bf16 input (target hidden states)
  SA_NORM = 2,   // A: fp32 rows x[M][lda]; the product uses RMSNorm(x) * gain,
                 // with the row sums of squares taken from ss_in[ss_tiles][M]
  SA_NORM1 = 3,  // as SA_NORM, but the normalised rows are rounded to bf16 and
                 // staged as one plane (the fused context of an injection)
};
// What happens to the product.  Except for SO_PART and SO_ARGMAX, the K
// splits of one output tile run on one XCD and the last to finish reduces
// the fp32 partials (in split order) and applies the epilogue.
enum SkinnyOut {
  SO_PART = 0,     // leave the partial slices part[S][M][N]
  SO_ARGMAX = 1,   // row argmax keys per 64-column group (S == 1)
  SO_QKV = 2,      // per head: RoPE on q and k; q -> split planes, k and v -> fp32
  SO_SWIGLU = 3,   // columns [gate | up] -> h = silu(gate) * up, split planes
  SO_RESID = 4,    // x += product; ss_out[tile][row] = sum over the tile of x^2
  SO_STORE_SS = 5, // x = product;  ss_out[tile][row] as above
  SO_KV = 6,       // per head of [K^0 | V^0 | K^1 | ...]: RoPE on K at the token's
                   // position, store into the paged cache
};

struct SkinnyArgs {
  // activations
  const void* A;
  size_t a_plane;          // SA_SPLIT: elements from the hi plane to the lo plane
  int lda, M;
  const float* ss_in;      // SA_NORM
  int ss_tiles;
  const void* gain;        // SA_NORM: [K] bf16
  float eps;
  // weights and shape
  WSeg w;
  const uint16_t* packed;  // the same weights in MFMA tile order (launch_pack), or null
  int N, K;
  // split-K bookkeeping
  float* part;             // [S][M][N]
  unsigned long long* ctr; // one arrival counter per output tile, zero between launches
  uint32_t* err;
  // workgroup -> XCD rotation seen by the previous split-K launch (read), and
  // the word this launch's workgroup 0 records what it sees in (or both null)
  const uint32_t* qhint_rd;
  uint32_t* qhint_wr;
  // SO_ARGMAX: row argmax keys merged into amax[8 XCDs][64] (zero between
  // launches); the last workgroup writes block_tokens[M] (row r = b*gamma + j:
  // anchor[b] for j == 0, else the argmax column) and re-zeroes amax and actr
  unsigned long long* amax;
  unsigned long long* actr;
  // packed weights: a counter (zero between launches) from which workgroups
  // take further column groups dynamically, or null for static runs
  unsigned int* wctr;
  // SO_KV: a launch-wide count of finished tiles (zero between launches);
  // the workgroup that finishes the last tile advances ctx_lens by the new
  // tokens (cu_new).  Null: the caller advances ctx_lens itself.
  unsigned int* kvdone;
  int32_t* ctx_lens_rw;   // the same lengths, written by that advance
  const int32_t* anchor;   // null: row 0 also gets its argmax
  int32_t* block_tokens;
  float* logits;           // [M][N] or null
  DrawArgs draw;           // SO_ARGMAX: draw instead of argmax (draw.gamma = gamma)
  // SO_QKV
  void* q;
  size_t q_plane;
  float* kb;
  float* vb;
  int gamma, Hq, Hkv, dh;
  const int32_t* ctx_lens;
  float theta;
  const float* rope;       // SO_QKV / SO_KV: (cos, sin) [M][dh/2][2] at each row's position
  // SO_STORE_SS side job (inject): rope_out[rope_rows][dh/2][2] at the
  // positions of the new tokens (cu_new, ctx_lens before the advance)
  float* rope_out;
  int rope_rows;
  // SO_SWIGLU (N == 2 I; weight rows [gate; up])
  void* h;
  size_t h_plane;
  int I;
  // SO_RESID / SO_STORE_SS
  float* x;
  float* ss_out;           // [N/64][M]
  // SO_KV
  void* pages;
  const int32_t* cu_new;
  int batch;
  const int32_t* page_table;
  int max_pages, n_pages, page_size;
};
// K split and tiling of a fused skinny product.
GemmPlan plan_skinny(int M, int N, int K, int out, int dh);
// Output tiles of a fused skinny product (the counters it uses), or -1 if
// the shape does not fit the epilogue.
int skinny_tiles(int out, int N, int dh, int I);
hipError_t launch_skinny(const GemmPlan& p, int asrc, int out, const SkinnyArgs& a,
                         hipStream_t stream);
// Weights of one fused product in MFMA tile order: the product's virtual rows
// (swiglu_I > 0: gate/up 64-row groups interleaved) padded to a multiple of
// 64, 16 x 32 tiles of 1 KB with lane l holding row l % 16, columns 8 (l / 16)
// .. + 7 of the tile, ordered [64-row group][32-column block][16-row group].
// packed_elems(N, K) bf16 elements.
size_t packed_elems(int N, int K);
hipError_t launch_pack(const WSeg& w, int N, int K, int swiglu_I, uint16_t* out,
                       hipStream_t stream);

// ---- attention ------------------------------------------------------------
struct AttnPlan {
  int chunk;          // context keys per workgroup (multiple of 32)
  int n_ctx_splits;   // workgroups along the context; one more handles the block
};
AttnPlan plan_attention(int batch, int n_kv_heads, int max_pages, int page_size);

struct AttnArgs {
  const void* q;        // [M][Hq][dh]: fp32, or the hi plane of a split (bf16 models)
  size_t q_plane;       // elements from the hi plane to the lo plane
  const void* k;        // [M][Hkv][dh] fp32: block keys of this layer
  const void* v;        // [M][Hkv][dh] fp32
  const void* pages;    // cache base
  int n_pages, max_pages, page_size;
  const int32_t* page_table;
  const int32_t* ctx_lens;
  int batch, gamma, Hq, Hkv, dh, layer;
  float* part_o;        // [n_ctx_splits+1][B][Hq][gamma][dh]
  float* part_ml;       // [n_ctx_splits+1][B][Hq][gamma][2]  (max in log2 units, sum)
  uint32_t* err;
  int causal;           // 1: block query j sees block keys 0..j only
};
hipError_t launch_attention(bool bf16, const AttnArgs& a, const AttnPlan& p, hipStream_t stream);
hipError_t launch_attn_combine(bool bf16, const float* part_o, const float* part_ml, int n_parts,
                               int batch, int gamma, int Hq, int dh, void* o, size_t o_plane,
                               hipStream_t stream);

// ---- element-wise and row kernels -----------------------------------------
// ss non-null: write the row sums of squares ss[M] instead of y.
// rope non-null: also write rope[M][dh/2][2] = (cos, sin) of the rotary
// angles at the position ctx_lens[b] + j of row r = b*gamma + j.
// tokens non-null: row r = b*gamma + j takes tokens[b*tok_stride + j]
// instead of (j == 0 ? anchor[b] : mask_id).
hipError_t launch_embed(bool bf16, const int32_t* anchor, int batch, int gamma, int mask_id,
                        int vocab, const void* embed, int D, float* x, const void* g, float eps,
                        void* y, size_t y_plane, float* ss, float* rope, const int32_t* ctx_lens,
                        int dh, float theta, uint32_t* err, hipStream_t stream,
                        const int32_t* tokens = nullptr, int tok_stride = 0);
// Outputs named y, q, h, c are transient activations: fp32 for fp32 models,
// split hi/lo bf16 planes for bf16 models (the lo plane starts *_plane
// elements after the hi plane).
hipError_t launch_rmsnorm(bool bf16, const float* x, int M, int D, const void* g, float eps,
                          void* y, size_t y_plane, hipStream_t stream);
hipError_t launch_residual_norm(bool bf16, float* x, const float* part, int splits, int M, int D,
                                const void* g, float eps, void* y, size_t y_plane,
                                hipStream_t stream);
// rope: the call's table [M][dh/2] of (cos, sin) pairs (launch_embed writes it)
hipError_t launch_qkv_epilogue(bool bf16, const float* part, int splits, int M, int Hq,
                               int Hkv, int dh, const float* rope, void* q, size_t q_plane,
                               float* k, float* v, hipStream_t stream);
hipError_t launch_swiglu(bool bf16, const float* part, int splits, int M, int I, void* h,
                         size_t h_plane, hipStream_t stream);
// block_tokens[r] = r % gamma == 0 && anchor ? anchor[r / gamma] : column of
// the largest key of row r over best[0..groups)[r].
hipError_t launch_argmax_finalize(const uint64_t* best, int groups, const int32_t* anchor,
                                  int batch, int gamma, int32_t* block_tokens, hipStream_t stream);
// c[n][D] = RMSNorm of the summed fc partials, in the model dtype (bf16
// models: one rounded plane, the precision the context is held in).
hipError_t launch_inject_norm(bool bf16, const float* part, int splits, int n, int D, const void* g,
                              float eps, void* c, hipStream_t stream);
hipError_t launch_inject_scatter(bool bf16, const float* part, int splits, int n_tok,
                                 const int32_t* cu_new, int batch, const int32_t* ctx_lens,
                                 const int32_t* page_table, int max_pages, int n_pages,
                                 int page_size, void* pages, int n_layers, int Hkv, int dh,
                                 float theta, uint32_t* err, hipStream_t stream);
hipError_t launch_advance_ctx(int32_t* ctx_lens, const int32_t* cu_new, int batch,
                              hipStream_t stream);
// Greedy verification: target columns per argmax workgroup, the largest
// block it takes, and its workspace (one key per row and column chunk).
constexpr int kVerifyChunk = 8192;
constexpr int kVerifyMaxBlock = 1024;
size_t verify_greedy_workspace(int batch, int gamma, int vocab);
hipError_t launch_verify(bool bf16, const int32_t* block_tokens, const void* target, int batch,
                         int gamma, int vocab, uint64_t* best, int32_t* accept_len,
                         int32_t* out_tokens, int32_t* target_argmax, hipStream_t stream);
hipError_t launch_clear_word(uint32_t* word, hipStream_t stream);

// ---- lossless verification of sampled blocks ------------------------------
constexpr int kMaxVerifyBlock = 64;
// Workspace of launch_verify_sampled: 16 * (ceil(vocab / 4096) *
// (4 * batch * gamma + 256 * batch) + batch) bytes, 16-byte aligned.
size_t verify_sampled_ws_bytes(int batch, int gamma, int vocab);
// draft [batch][gamma][vocab] fp32 (row 0 unused), target [batch][gamma][vocab]
// (bf16 or fp32), uniforms [batch][gamma]; writes accept_len [batch] and
// out_tokens [batch][gamma] (-1 past the accepted length).
hipError_t launch_verify_sampled(bool bf16, const int32_t* block_tokens, const void* target,
                                 const float* draft, const float* uniforms, int batch, int gamma,
                                 int vocab, void* workspace, int32_t* accept_len,
                                 int32_t* out_tokens, hipStream_t stream);

// ---- packed multi-block forward -------------------------------------------
// table[b][p] = page_row[p] for b < n_blocks; lens[b] = anchor_pos[b]
// (DFLASH_DEVERR_POS and clamped to [0, ctx_len[0]] when outside).
hipError_t launch_packed_setup(const int32_t* page_row, int max_pages, const int32_t* ctx_len,
                               const int32_t* anchor_pos, int n_blocks, int32_t* table,
                               int32_t* lens, uint32_t* err, hipStream_t stream);
// Weighted cross-entropy of packed blocks: ce [n_blocks][gamma-1] fp64
// scratch; block_loss [n_blocks] and loss [1] fp32 outputs (either may be
// null).
hipError_t launch_block_loss(const float* logits, const int32_t* targets, int n_blocks, int gamma,
                             int vocab, double decay, double* ce, float* block_loss, float* loss,
                             uint32_t* err, hipStream_t stream);

// ---- autoregressive drafting (DFlash-AR) ----------------------------------
// block[b][0] = anchor[b]; after pass i, block[b][i] = pass_tokens[b*i + i-1].
hipError_t launch_ar_seed(const int32_t* anchor, int batch, int gamma, int32_t* block,
                          hipStream_t stream);
hipError_t launch_ar_pick(const int32_t* pass_tokens, int batch, int i, int gamma, int32_t* block,
                          hipStream_t stream);

// ---- counter calibration ---------------------------------------------------
// Stream `bytes` (a multiple of 16) of device memory with 16-byte
// non-temporal loads, one contiguous run per workgroup; out[workgroups]
// receives one 16-byte checksum per workgroup.
hipError_t launch_read_calibration(const void* src, size_t bytes, void* out, int workgroups,
                                   hipStream_t stream);
