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

enum GemmKind { GEMM_F32 = 0, GEMM_SKINNY = 1, GEMM_TILED = 2 };

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
                       float* logits, hipStream_t stream);

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
};
hipError_t launch_attention(bool bf16, const AttnArgs& a, const AttnPlan& p, hipStream_t stream);
hipError_t launch_attn_combine(bool bf16, const float* part_o, const float* part_ml, int n_parts,
                               int batch, int gamma, int Hq, int dh, void* o, size_t o_plane,
                               hipStream_t stream);

// ---- element-wise and row kernels -----------------------------------------
hipError_t launch_embed(bool bf16, const int32_t* anchor, int batch, int gamma, int mask_id,
                        int vocab, const void* embed, int D, float* x, const void* g, float eps,
                        void* y, size_t y_plane, uint32_t* err, hipStream_t stream);
// Outputs named y, q, h, c are transient activations: fp32 for fp32 models,
// split hi/lo bf16 planes for bf16 models (the lo plane starts *_plane
// elements after the hi plane).
hipError_t launch_rmsnorm(bool bf16, const float* x, int M, int D, const void* g, float eps,
                          void* y, size_t y_plane, hipStream_t stream);
hipError_t launch_residual_norm(bool bf16, float* x, const float* part, int splits, int M, int D,
                                const void* g, float eps, void* y, size_t y_plane,
                                hipStream_t stream);
hipError_t launch_qkv_epilogue(bool bf16, const float* part, int splits, int M, int gamma, int Hq,
                               int Hkv, int dh, const int32_t* ctx_lens, float theta, void* q,
                               size_t q_plane, float* k, float* v, hipStream_t stream);
hipError_t launch_swiglu(bool bf16, const float* part, int splits, int M, int I, void* h,
                         size_t h_plane, hipStream_t stream);
// block_tokens[r] = r % gamma == 0 ? anchor[r / gamma] : column of the
// largest key of row r over best[0..groups)[r].
hipError_t launch_argmax_finalize(const uint64_t* best, int groups, const int32_t* anchor,
                                  int batch, int gamma, int32_t* block_tokens, hipStream_t stream);
hipError_t launch_inject_norm(bool bf16, const float* part, int splits, int n, int D, const void* g,
                              float eps, void* c, size_t c_plane, hipStream_t stream);
hipError_t launch_inject_scatter(bool bf16, const float* part, int splits, int n_tok,
                                 const int32_t* cu_new, int batch, const int32_t* ctx_lens,
                                 const int32_t* page_table, int max_pages, int n_pages,
                                 int page_size, void* pages, int n_layers, int Hkv, int dh,
                                 float theta, uint32_t* err, hipStream_t stream);
hipError_t launch_advance_ctx(int32_t* ctx_lens, const int32_t* cu_new, int batch,
                              hipStream_t stream);
hipError_t launch_verify(bool bf16, const int32_t* block_tokens, const void* target, int batch,
                         int gamma, int vocab, uint64_t* best, int32_t* accept_len,
                         int32_t* out_tokens, int32_t* target_argmax, hipStream_t stream);
hipError_t launch_clear_word(uint32_t* word, hipStream_t stream);
