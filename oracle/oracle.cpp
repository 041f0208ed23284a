// oracle.cpp -- plain, slow CPU model of the DFlash draft step, its context
// injection and greedy verification.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
// call this file; only the tests, the package smoke check and the CPU
// baseline leg of the benchmark do.  It shares no code, header, table or
// helper with the HIP library: the two are written separately so that one
// can check the other.
//
// Every sum is accumulated in double, in the natural index order, one output
// at a time.  OpenMP only spreads independent outputs over threads; it never
// changes the order of the additions inside one output.
//
// Precision.  Weights, the target's hidden states and the draft K/V cache are
// stored in the model dtype.  In bf16 mode the method rounds (to nearest,
// ties to even) the two context activations the paper sizes at two bytes per
// element: the fused context c = RMSNorm(W_c f), the fc's output, and the
// context keys and values stored in the cache (paper §7.3, "KV Injection
// Mechanism and Memory Overhead": the projection's output at batch 1 and
// 2048 tokens is counted at 8 MB, i.e. D = 2048 values of 2 bytes per token).
// Every transient value of a draft pass -- norms, q/k/v of the block,
// attention weights and outputs, the SwiGLU product, the residual stream,
// the logits -- stays in double: the pages say nothing of their precision.
// In fp32 mode nothing is rounded.
//
// Sources (titles of the pages the method is described on):
//   [S] "DFlash: Block Diffusion for Flash Speculative Decoding", the
//       framework summary page (zhongzhoutan-coder.github.io).
//   [P] the DFlash paper text, arXiv 2602.06036.
// Readings the pages leave open (layer internals, RoPE, tie rule, ...) are
// noted at each function.
//
// Parity status of each function: pinned by tests/test_oracle_pins.py unless
// marked otherwise.

#include <omp.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <cstdlib>
#include <vector>
#include <algorithm>

extern "C" {

// ---------------------------------------------------------------------------
// Dimensions and weights (the oracle's own description; mirrored in
// oracle/__init__.py).
typedef struct {
  int32_t hidden;        // D
  int32_t n_layers;      // draft layers
  int32_t n_q_heads;     // Hq
  int32_t n_kv_heads;    // Hkv
  int32_t head_dim;      // dh
  int32_t inter;         // SwiGLU width I
  int32_t vocab;         // V
  int32_t n_feats;       // number of fused target layers (5 on the pages)
  int32_t bf16;          // 1: bf16 storage + rounding points; 0: fp32, no rounding
  int32_t pad_;
  double rope_theta;
  double eps;
} oracle_dims;

#define ORACLE_MAX_LAYERS 32
typedef struct {
  const void* fc_w;        // [D][n_feats*D]
  const void* fc_norm;     // [D]
  const void* embed;       // [V][D]
  const void* lm_head;     // [V][D]
  const void* final_norm;  // [D]
  const void* attn_norm[ORACLE_MAX_LAYERS];  // [D]
  const void* wq[ORACLE_MAX_LAYERS];         // [Hq*dh][D]
  const void* wk[ORACLE_MAX_LAYERS];         // [Hkv*dh][D]
  const void* wv[ORACLE_MAX_LAYERS];         // [Hkv*dh][D]
  const void* wo[ORACLE_MAX_LAYERS];         // [D][Hq*dh]
  const void* mlp_norm[ORACLE_MAX_LAYERS];   // [D]
  const void* w_gate[ORACLE_MAX_LAYERS];     // [I][D]
  const void* w_up[ORACLE_MAX_LAYERS];       // [I][D]
  const void* w_down[ORACLE_MAX_LAYERS];     // [D][I]
} oracle_weights;

// ---------------------------------------------------------------------------
// Scalar helpers.

// Exact value of a bf16 bit pattern.
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// Round a double to the nearest bf16 value (8 significant bits, exponent
// range of fp32), ties to even.  Written from the definition: split x into
// m * 2^e with m in [0.5, 1), keep 8 bits of m with round-half-even.
double oracle_round_bf16(double x) {
  if (x == 0.0 || !std::isfinite(x)) return x;
  int e;
  double m = std::frexp(x, &e);          // x = m * 2^e, 0.5 <= |m| < 1
  // bf16 keeps 8 significant bits for normal numbers; below 2^-126 the
  // quantum stays at 2^-133.
  int bits = 8;
  if (e - 1 < -126) bits = 8 - (-126 - (e - 1));
  if (bits < 0) return std::copysign(0.0, x);
  double scaled = std::ldexp(m, bits);   // exact
  double r = std::nearbyint(scaled);     // default mode: ties to even
  return std::ldexp(r, e - bits);
}

static inline double rnd(const oracle_dims* d, double x) {
  return d->bf16 ? oracle_round_bf16(x) : x;
}

// Element i of an array stored as bf16 bits (bf16 != 0) or fp32.
static inline double ld(const void* p, size_t i, int bf16) {
  if (bf16) return bf16_bits_to_double(((const uint16_t*)p)[i]);
  return (double)((const float*)p)[i];
}

// y[j][n] = sum_k W[n][k] * x[j][k]   (W row-major [N][K], x [R][K], y [R][N])
static void matvec_rows(const void* W, int bf16, int N, int K,
                        const double* x, int R, double* y) {
  #pragma omp parallel
  {
    std::vector<double> wrow((size_t)K);
    #pragma omp for schedule(static)
    for (int n = 0; n < N; ++n) {
      for (int k = 0; k < K; ++k) wrow[k] = ld(W, (size_t)n * K + k, bf16);
      for (int j = 0; j < R; ++j) {
        const double* xj = x + (size_t)j * K;
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += wrow[k] * xj[k];
        y[(size_t)j * N + n] = acc;
      }
    }
  }
}

// RMSNorm: out_i = x_i / sqrt(mean_i(x_i^2) + eps) * g_i.
// The pages name RMSNorm for the context fusion ([S] "Target Hidden States
// Supply the Missing Context", eq. for H_t; [P] §7.3); the draft layers are
// read as pre-norm blocks with RMSNorm gains (a reading: the pages do not
// print the layer internals).
void oracle_rmsnorm(const double* x, int n, const void* g, int g_bf16,
                    double eps, double* out) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / std::sqrt(ss / (double)n + eps);
  for (int i = 0; i < n; ++i) out[i] = x[i] * inv * ld(g, i, g_bf16);
}

// Rotary embedding, rotate-half form, applied in place to `heads` vectors of
// length dh stored back to back, all at position pos.  The angle for pair i
// (i < dh/2) is pos * theta^(-2i/dh), computed in double.  (The pages do not
// mention the positional encoding; the drafter is read as a Qwen3-style
// decoder, which uses this form with theta = 1e6.)
void oracle_rope(double* x, int heads, int dh, double pos, double theta) {
  int half = dh / 2;
  for (int h = 0; h < heads; ++h) {
    double* v = x + (size_t)h * dh;
    for (int i = 0; i < half; ++i) {
      double inv = std::pow(theta, -2.0 * (double)i / (double)dh);
      double phi = pos * inv;
      double c = std::cos(phi), s = std::sin(phi);
      double a = v[i], b = v[i + half];
      v[i] = a * c - b * s;
      v[i + half] = b * c + a * s;
    }
  }
}

static double silu(double a) { return a / (1.0 + std::exp(-a)); }

// SwiGLU MLP on R rows (a reading: the pages do not print the layer; the
// drafter is taken as a Qwen3-style decoder layer):
// out = W_down( silu(W_gate z) * W_up z ).  z: [R][D], out: [R][D].
void oracle_swiglu(const void* w_gate, const void* w_up, const void* w_down, int bf16,
                   int D, int I, const double* z, int R, double* out) {
  std::vector<double> g((size_t)R * I), u((size_t)R * I), hh((size_t)R * I);
  matvec_rows(w_gate, bf16, I, D, z, R, g.data());
  matvec_rows(w_up, bf16, I, D, z, R, u.data());
  for (size_t i = 0; i < (size_t)R * I; ++i) hh[i] = silu(g[i]) * u[i];
  matvec_rows(w_down, bf16, D, I, hh.data(), R, out);
}

// Lowest index among the maxima of row[0..n).
int oracle_argmax(const double* row, int n) {
  int best = 0;
  for (int i = 1; i < n; ++i)
    if (row[i] > row[best]) best = i;
  return best;
}

// ---------------------------------------------------------------------------
// Dense masked attention, brute force.  q: [nq][dh], k, v: [nk][dh],
// visible: [nq][nk] (nonzero = query may see key).  Scores are q.k/sqrt(dh);
// the softmax runs over the visible keys only.  o: [nq][dh].
// A query with no visible key gets o = 0.
void oracle_attention_dense(const double* q, int nq, const double* k,
                            const double* v, int nk, int dh,
                            const uint8_t* visible, double* o) {
  double scale = 1.0 / std::sqrt((double)dh);
  std::vector<double> s((size_t)nk);
  for (int i = 0; i < nq; ++i) {
    double mx = -INFINITY;
    for (int r = 0; r < nk; ++r) {
      if (!visible[(size_t)i * nk + r]) { s[r] = -INFINITY; continue; }
      double acc = 0.0;
      for (int t = 0; t < dh; ++t) acc += q[(size_t)i * dh + t] * k[(size_t)r * dh + t];
      s[r] = acc * scale;
      if (s[r] > mx) mx = s[r];
    }
    double* oi = o + (size_t)i * dh;
    for (int t = 0; t < dh; ++t) oi[t] = 0.0;
    if (mx == -INFINITY) continue;
    double den = 0.0;
    for (int r = 0; r < nk; ++r) {
      double p = (s[r] == -INFINITY) ? 0.0 : std::exp(s[r] - mx);
      s[r] = p;
      den += p;
    }
    for (int r = 0; r < nk; ++r) {
      if (s[r] == 0.0) continue;
      double w = s[r] / den;
      for (int t = 0; t < dh; ++t) oi[t] += w * v[(size_t)r * dh + t];
    }
  }
}

// ---------------------------------------------------------------------------
// Context injection for one token ([S] "Target Hidden States Supply the
// Missing Context" eq. H_t and "Per-Layer K/V Injection Prevents Context
// Dilution" eq. K_i, V_i; [P] §4.1 "Conditioning via KV injection" and §7.3):
//   f = [h^(1); ...; h^(m)]   (the m target features, shallow to deep)
//   c = RMSNorm(W_c f)        (no bias; gain fc_norm)
//   for each draft layer l:  k_l = RoPE(W_K^l c, pos),  v_l = W_V^l c
// The same c feeds every layer; no per-layer norm is applied to it, and c
// bypasses the query, output, attention update and MLP paths.
//
// hidden: [n_tok][n_feats*D] (bf16 bits or fp32 per dims->bf16)
// pos:    [n_tok] absolute positions
// out_k, out_v: [n_tok][n_layers][Hkv][dh] doubles: the stored values, rounded
//         to bf16 in bf16 mode
void oracle_inject(const oracle_dims* d, const oracle_weights* w,
                   const void* hidden, const int32_t* pos, int n_tok,
                   double* out_k, double* out_v) {
  const int D = d->hidden, F = d->n_feats * D, Hkv = d->n_kv_heads, dh = d->head_dim;
  const int NL = d->n_layers, KV = Hkv * dh;
  std::vector<double> f((size_t)n_tok * F), u((size_t)n_tok * D), c((size_t)n_tok * D);
  for (size_t i = 0; i < (size_t)n_tok * F; ++i) f[i] = ld(hidden, i, d->bf16);
  matvec_rows(w->fc_w, d->bf16, D, F, f.data(), n_tok, u.data());
  for (int t = 0; t < n_tok; ++t) {
    oracle_rmsnorm(&u[(size_t)t * D], D, w->fc_norm, d->bf16, d->eps, &c[(size_t)t * D]);
  }
  // c is held in the model dtype (bf16: rounded), like the cache it feeds
  for (size_t i = 0; i < (size_t)n_tok * D; ++i) c[i] = rnd(d, c[i]);
  std::vector<double> kk((size_t)n_tok * KV), vv((size_t)n_tok * KV);
  for (int l = 0; l < NL; ++l) {
    matvec_rows(w->wk[l], d->bf16, KV, D, c.data(), n_tok, kk.data());
    matvec_rows(w->wv[l], d->bf16, KV, D, c.data(), n_tok, vv.data());
    for (int t = 0; t < n_tok; ++t) {
      double* kt = &kk[(size_t)t * KV];
      oracle_rope(kt, Hkv, dh, (double)pos[t], d->rope_theta);
      for (int i = 0; i < KV; ++i) {
        size_t o = (((size_t)t * NL + l) * KV) + i;
        out_k[o] = rnd(d, kt[i]);
        out_v[o] = rnd(d, vv[(size_t)t * KV + i]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Forward pass of R block rows through the draft layers, with attention over
// [context keys 0..Lc) ++ [the R rows' own keys], restricted by `visible`.
//
//   tokens[R], pos[R]:   the rows' token ids and absolute positions
//   ctx_k, ctx_v:        [n_layers][Lbuf][Hkv][dh] (bf16 bits or fp32);
//                        only the first Lc entries of each layer are read
//   visible:             [R][Lc + R]
//   logits (out):        [R][V]
//
// Layer internals (reading: the pages only fix the K/V injection; the
// drafter is a pre-norm Qwen3-style decoder layer with RMSNorm and SwiGLU):
//   y = RMSNorm(x); q,k = RoPE(W_Q y), RoPE(W_K y); v = W_V y
//   x += W_O Attn(q, [ctx_k; k], [ctx_v; v])      (GQA: head h uses kv head
//                                                   h / (Hq/Hkv))
//   z = RMSNorm(x); x += W_down(silu(W_gate z) * W_up z)
//   logits = W_lm RMSNorm(x)      (shared LM head, [S] "Early Positions
//                                  Receive More Learning Budget"; [P] §4.2)
void oracle_forward(const oracle_dims* d, const oracle_weights* w,
                    const int32_t* tokens, const int32_t* pos, int R,
                    const void* ctx_k, const void* ctx_v, int Lc, int Lbuf,
                    const uint8_t* visible, double* logits) {
  const int D = d->hidden, Hq = d->n_q_heads, Hkv = d->n_kv_heads, dh = d->head_dim;
  const int I = d->inter, V = d->vocab, NL = d->n_layers;
  (void)V;
  const int QD = Hq * dh, KV = Hkv * dh, group = Hq / Hkv, NK = Lc + R;
  std::vector<double> x((size_t)R * D), y((size_t)R * D);
  for (int j = 0; j < R; ++j)
    for (int i = 0; i < D; ++i)
      x[(size_t)j * D + i] = ld(w->embed, (size_t)tokens[j] * D + i, d->bf16);

  std::vector<double> q((size_t)R * QD), k((size_t)R * KV), v((size_t)R * KV);
  std::vector<double> o((size_t)R * QD), t1((size_t)R * D);

  for (int l = 0; l < NL; ++l) {
    for (int j = 0; j < R; ++j) {
      oracle_rmsnorm(&x[(size_t)j * D], D, w->attn_norm[l], d->bf16, d->eps, &y[(size_t)j * D]);
    }
    matvec_rows(w->wq[l], d->bf16, QD, D, y.data(), R, q.data());
    matvec_rows(w->wk[l], d->bf16, KV, D, y.data(), R, k.data());
    matvec_rows(w->wv[l], d->bf16, KV, D, y.data(), R, v.data());
    for (int j = 0; j < R; ++j) {
      oracle_rope(&q[(size_t)j * QD], Hq, dh, (double)pos[j], d->rope_theta);
      oracle_rope(&k[(size_t)j * KV], Hkv, dh, (double)pos[j], d->rope_theta);
    }

    // Heads are independent; threads take whole heads, each with its own
    // buffers, so every head's arithmetic is the same as in a serial loop.
    #pragma omp parallel
    {
      std::vector<double> qh((size_t)R * dh), kh((size_t)NK * dh), vh((size_t)NK * dh);
      std::vector<double> oh((size_t)R * dh);
      #pragma omp for schedule(dynamic, 1)
      for (int h = 0; h < Hq; ++h) {
        int kvh = h / group;
        for (int r = 0; r < Lc; ++r)
          for (int t = 0; t < dh; ++t) {
            size_t src = (((size_t)l * Lbuf + r) * Hkv + kvh) * dh + t;
            kh[(size_t)r * dh + t] = ld(ctx_k, src, d->bf16);
            vh[(size_t)r * dh + t] = ld(ctx_v, src, d->bf16);
          }
        for (int r = 0; r < R; ++r)
          for (int t = 0; t < dh; ++t) {
            kh[(size_t)(Lc + r) * dh + t] = k[(size_t)r * KV + kvh * dh + t];
            vh[(size_t)(Lc + r) * dh + t] = v[(size_t)r * KV + kvh * dh + t];
          }
        for (int j = 0; j < R; ++j)
          for (int t = 0; t < dh; ++t) qh[(size_t)j * dh + t] = q[(size_t)j * QD + h * dh + t];
        oracle_attention_dense(qh.data(), R, kh.data(), vh.data(), NK, dh, visible, oh.data());
        for (int j = 0; j < R; ++j)
          for (int t = 0; t < dh; ++t) o[(size_t)j * QD + h * dh + t] = oh[(size_t)j * dh + t];
      }
    }
    matvec_rows(w->wo[l], d->bf16, D, QD, o.data(), R, t1.data());
    for (size_t i = 0; i < (size_t)R * D; ++i) x[i] += t1[i];

    for (int j = 0; j < R; ++j) {
      oracle_rmsnorm(&x[(size_t)j * D], D, w->mlp_norm[l], d->bf16, d->eps, &y[(size_t)j * D]);
    }
    oracle_swiglu(w->w_gate[l], w->w_up[l], w->w_down[l], d->bf16, D, I, y.data(), R, t1.data());
    for (size_t i = 0; i < (size_t)R * D; ++i) x[i] += t1[i];
  }
  for (int j = 0; j < R; ++j) {
    oracle_rmsnorm(&x[(size_t)j * D], D, w->final_norm, d->bf16, d->eps, &y[(size_t)j * D]);
  }
  matvec_rows(w->lm_head, d->bf16, V, D, y.data(), R, logits);
}

// ---------------------------------------------------------------------------
// Single-pass block draft for one sequence ([S] "Block Diffusion Makes Draft
// Cost Nearly Independent of Block Length" and the cycle table in "Putting It
// Together", step 3; [P] §4.1 "Parallel diffusion drafting").
//   ctx_k, ctx_v:  [n_layers][Lbuf][Hkv][dh]; entries L..Lbuf-1 are never read
//   tokens[gamma]: t_0 = the clean anchor, t_j = the mask token for j >= 1
//                  (passed in explicitly so tests can perturb single rows)
//   Row j sits at position L + j and sees all L context keys plus every
//   block key (bidirectional inside the block, no causal mask).
//   logits[gamma][V] (out); block[gamma] (out): block[0] = t_0,
//   block[j] = lowest-index argmax of logits[j] for j >= 1 (row j predicts
//   the token at its own position).
void oracle_draft(const oracle_dims* d, const oracle_weights* w,
                  const void* ctx_k, const void* ctx_v, int L, int Lbuf,
                  const int32_t* tokens, int gamma,
                  double* logits, int32_t* block) {
  std::vector<int32_t> pos((size_t)gamma);
  for (int j = 0; j < gamma; ++j) pos[j] = L + j;
  std::vector<uint8_t> vis((size_t)gamma * (L + gamma), 1);
  oracle_forward(d, w, tokens, pos.data(), gamma, ctx_k, ctx_v, L, Lbuf, vis.data(), logits);
  block[0] = tokens[0];
  for (int j = 1; j < gamma; ++j) block[j] = oracle_argmax(logits + (size_t)j * d->vocab, d->vocab);
}

// Packed multi-block forward (the training layout of [S] "Training Rehearses
// the Same Masked Blocks Used at Runtime", Figure 4; [P] §4.2 "Random
// sampling of masked blocks"): n_blocks blocks of gamma rows share one pass.
// Block b starts at anchor position anchors_pos[b]; its rows see context
// keys [0, anchors_pos[b]) and the keys of their own block only.
//   tokens: [n_blocks][gamma]; logits: [n_blocks*gamma][V]
void oracle_draft_packed(const oracle_dims* d, const oracle_weights* w,
                         const void* ctx_k, const void* ctx_v, int Lc,
                         const int32_t* tokens, const int32_t* anchors_pos,
                         int n_blocks, int gamma, double* logits) {
  int R = n_blocks * gamma, NK = Lc + R;
  std::vector<int32_t> pos((size_t)R);
  std::vector<uint8_t> vis((size_t)R * NK, 0);
  for (int b = 0; b < n_blocks; ++b)
    for (int j = 0; j < gamma; ++j) {
      int row = b * gamma + j;
      pos[row] = anchors_pos[b] + j;
      for (int r = 0; r < anchors_pos[b] && r < Lc; ++r) vis[(size_t)row * NK + r] = 1;
      for (int jj = 0; jj < gamma; ++jj) vis[(size_t)row * NK + Lc + b * gamma + jj] = 1;
    }
  oracle_forward(d, w, tokens, pos.data(), R, ctx_k, ctx_v, Lc, Lc, vis.data(), logits);
}

// ---------------------------------------------------------------------------
// Greedy verification of one block ([S] "The Target Verifier Remains the
// Correctness Anchor": acceptance rule min(1, p_t/p_d) and its worked
// example; cycle table step 4; [P] §3.1 for tau in [1, gamma+1]).
// At temperature 0 the target distribution is one-hot at its argmax T_j, so
// the rule accepts a proposal exactly when it equals T_j.
//   block[gamma]:      [anchor, d_1, ..., d_{gamma-1}]
//   target[gamma][V]:  row j = the target's scores for the token after
//                      block[0..j] (bf16 bits or fp32 per tgt_bf16)
//   T_j = lowest-index argmax of row j (compared in the scores' own values)
//   n   = length of the longest prefix with block[j] == T_{j-1}, j = 1..n
//   tau = n + 1;  out = [block[1..n], T_n, -1, ...]
int oracle_verify(const int32_t* block, const void* target, int tgt_bf16,
                  int gamma, int V, int32_t* out_tokens, int32_t* out_T) {
  std::vector<double> row((size_t)V);
  for (int j = 0; j < gamma; ++j) {
    for (int i = 0; i < V; ++i) row[i] = ld(target, (size_t)j * V + i, tgt_bf16);
    out_T[j] = oracle_argmax(row.data(), V);
  }
  int n = 0;
  while (n < gamma - 1 && block[n + 1] == out_T[n]) ++n;
  for (int j = 0; j < gamma; ++j) out_tokens[j] = -1;
  for (int j = 0; j < n; ++j) out_tokens[j] = block[j + 1];
  out_tokens[n] = out_T[n];
  return n + 1;
}

// ---------------------------------------------------------------------------
// Position-decayed loss weights ([S] "Early Positions Receive More Learning
// Budget"; [P] §4.2 eq. 1 and §7.1 for the decay constants):
// w_k = exp(-(k-1)/gamma_decay), k = 1..K; k = 1 is the first predicted
// position after the anchor.
void oracle_loss_weights(double gamma_decay, int K, double* w) {
  for (int k = 1; k <= K; ++k) w[k - 1] = std::exp(-(double)(k - 1) / gamma_decay);
}

// Weighted token cross-entropy over K predicted positions:
// sum_k w_k * CE_k / sum_k w_k with CE_k = logsumexp(logits_k) - logits_k[target_k].
// (The pages say only that the weight multiplies the token-level
// cross-entropy; the normalisation by sum w_k is a reading.)
double oracle_weighted_ce(const double* logits, const int32_t* targets,
                          const double* w, int K, int V) {
  double num = 0.0, den = 0.0;
  for (int k = 0; k < K; ++k) {
    const double* lk = logits + (size_t)k * V;
    double mx = lk[0];
    for (int i = 1; i < V; ++i) mx = std::max(mx, lk[i]);
    double s = 0.0;
    for (int i = 0; i < V; ++i) s += std::exp(lk[i] - mx);
    double ce = mx + std::log(s) - lk[targets[k]];
    num += w[k] * ce;
    den += w[k];
  }
  return num / den;
}

// ---------------------------------------------------------------------------
// Threads (timing harness only; no arithmetic): the OpenMP team size the
// parallel loops above use.  Results do not depend on it.
int oracle_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { if (n >= 1) omp_set_num_threads(n); }

}  // extern "C"
