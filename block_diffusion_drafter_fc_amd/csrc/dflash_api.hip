// dflash_api.hip -- the C ABI declared in include/dflash.h: argument checks,
// workspace layout and the launch sequence of each call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <utility>
#include <vector>

#include "dflash.h"
#include "kernels.h"

// Scratch of dflash_draft_block_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes its name as an
// address (on the host it is only a stand-in symbol): dflash_model_create
// looks up the copy of its device with hipGetSymbolAddress and the entry
// point uses that pointer.
static __device__ __align__(256) unsigned char scratch[DFLASH_NOALLOC_SCRATCH_BYTES];

struct dflash_model {
  dflash_config cfg;
  dflash_weights w;
  uint32_t* err;   // device error word (in the caller's state buffer)
  unsigned long long* ctr;   // split-K arrival counters (same buffer, zero between calls)
  unsigned long long* amax;  // LM-head argmax slots and their counter (same buffer)
  unsigned long long* actr;
  unsigned int* wctr;        // LM-head group counter (same buffer, zero between calls)
  unsigned int* kvdone;      // inject K/V launch: finished tiles (same buffer, zero between calls)
  uint32_t* qhint;           // two words: workgroup -> XCD rotation seen by split-K launches
  mutable uint32_t hint_seq; // split-K launches so far: selects the word a launch reads
  const uint16_t* packed;    // weights in MFMA tile order (dflash_pack_weights), or null
  int device;
  bool bf16;
  bool prof_on;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending, pool;
  double prof_ms;
  int64_t prof_count;
};

namespace {

thread_local std::string g_err;

// Device address of `scratch` on each GPU (null until resolved).
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// Resolve the scratch array's address on device `dev`, which must be the
// current device.  Done once per device; a failure leaves the slot null and
// is retried by the next model creation on that device.
void resolve_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices || g_scratch[dev].load() != nullptr) return;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p != nullptr)
    g_scratch[dev].store(p);
  else
    (void)hipGetLastError();   // leave no error behind for the caller's next call
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIPCHK(expr)                                                                     \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess) return fail(DFLASH_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Dims {
  int D, QD, KVD, I, V, NL, Hq, Hkv, dh, F;
};
Dims dims_of(const dflash_config& c) {
  Dims d;
  d.D = c.hidden;
  d.Hq = c.n_q_heads;
  d.Hkv = c.n_kv_heads;
  d.dh = c.head_dim;
  d.QD = c.n_q_heads * c.head_dim;
  d.KVD = c.n_kv_heads * c.head_dim;
  d.I = c.intermediate;
  d.V = c.vocab;
  d.NL = c.n_layers;
  d.F = c.n_target_feats * c.hidden;
  return d;
}

// Partial-slice floats of a plain product with at most M rows: the split
// count depends on M (whole rounds of workgroups), so S * M * N is not
// monotone in M; the workspace covers every row count up to M.
// The split counts depend on M only through the 128-row tile counts, so
// the maximum is reached at M itself, at 255 or at a multiple of 128.
size_t part_floats(bool bf16, int M, int N, int K) {
  size_t best = 0;
  auto at = [&](int m) {
    const GemmPlan p = plan_gemm(bf16, m, N, K, false);
    best = std::max(best, (size_t)p.splits * m * N);
  };
  at(M);
  if (M > 64) {
    if (M >= 255) at(255);
    for (int m = 128; m < M; m += 128) at(m);
  }
  return best;
}

// State buffer: the error word; at 128 two words holding the workgroup ->
// XCD rotation observed by split-K launches (each launch reads one and writes
// the other, so all workgroups of a launch read the same value); then the
// LM-head argmax slots [8 XCDs][64 rows], their arrival counter, (64 bytes
// further) the LM head's column-group counter and (64 more) the inject K/V
// launch's count of finished tiles; then one arrival counter per
// output tile of a fused product.  Every call leaves the slots and counters
// at zero.
constexpr size_t kQhintOffset = 128;
constexpr size_t kProfPool = 256;   // LM-head timing event pairs created by profile_enable
constexpr size_t kAmaxOffset = 256;
constexpr size_t kActrOffset = kAmaxOffset + 8 * 64 * 8;
constexpr size_t kCtrOffset = kActrOffset + 256;
constexpr int kMaxCounters = (int)((DFLASH_STATE_BYTES - kCtrOffset) / 8);

// bf16 models with at most 64 product rows run the fused skinny products
// (epilogues inside the product kernels); larger M and fp32 models run the
// plain products followed by separate epilogue kernels.
bool use_fused(const dflash_model* m, int M) {
  if (!m->bf16 || M > 64) return false;
  const dflash_config& c = m->cfg;
  const int qkv = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  const int kvn = 2 * c.n_layers * c.n_kv_heads * c.head_dim;
  const int tiles[] = {skinny_tiles(SO_QKV, qkv, c.head_dim, c.intermediate),
                       skinny_tiles(SO_SWIGLU, 2 * c.intermediate, c.head_dim, c.intermediate),
                       skinny_tiles(SO_RESID, c.hidden, c.head_dim, c.intermediate),
                       skinny_tiles(SO_KV, kvn, c.head_dim, c.intermediate)};
  for (int t : tiles)
    if (t < 0 || t > kMaxCounters) return false;
  return true;
}

// Launch a fused product.  Split-K launches alternate between the two hint
// words: launch n reads word n mod 2 (written by launch n - 1) and its
// workgroup 0 writes word (n + 1) mod 2, which no workgroup of launch n reads.
hipError_t run_skinny(const dflash_model* m, const GemmPlan& p, int asrc, int out, SkinnyArgs a,
                      hipStream_t st) {
  if (out != SO_ARGMAX) {
    const uint32_t r = m->hint_seq & 1u;
    a.qhint_rd = m->qhint + r;
    a.qhint_wr = m->qhint + (r ^ 1u);
    ++m->hint_seq;
  }
  return launch_skinny(p, asrc, out, a, st);
}

size_t skinny_part_floats(int M, int N, int K, int out, int dh) {
  const GemmPlan p = plan_skinny(M, N, K, out, dh);
  return (size_t)p.splits * M * N;
}

// Weight matrices of the fused products, as row-stacked segments.
WSeg seg1(const void* p, int rows) {
  WSeg w{};
  w.ptr[0] = p;
  w.row_end[0] = rows;
  w.n = 1;
  return w;
}
WSeg wseg_qkv(const dflash_model* m, int l) {
  const Dims d = dims_of(m->cfg);
  const dflash_layer_weights& W = m->w.layer[l];
  WSeg w{};
  w.ptr[0] = W.wq;
  w.ptr[1] = W.wk;
  w.ptr[2] = W.wv;
  w.row_end[0] = d.QD;
  w.row_end[1] = d.QD + d.KVD;
  w.row_end[2] = d.QD + 2 * d.KVD;
  w.n = 3;
  return w;
}
WSeg wseg_gu(const dflash_model* m, int l) {
  const Dims d = dims_of(m->cfg);
  WSeg w{};
  w.ptr[0] = m->w.layer[l].w_gate;
  w.ptr[1] = m->w.layer[l].w_up;
  w.row_end[0] = d.I;
  w.row_end[1] = 2 * d.I;
  w.n = 2;
  return w;
}
WSeg wseg_kv(const dflash_model* m) {   // [W_K^0; W_V^0; W_K^1; ...]
  const Dims d = dims_of(m->cfg);
  WSeg w{};
  for (int l = 0; l < d.NL; ++l) {
    w.ptr[2 * l] = m->w.layer[l].wk;
    w.ptr[2 * l + 1] = m->w.layer[l].wv;
    w.row_end[2 * l] = (2 * l + 1) * d.KVD;
    w.row_end[2 * l + 1] = (2 * l + 2) * d.KVD;
  }
  w.n = 2 * d.NL;
  return w;
}

// Element offsets of each product's packed weights.
struct PackLayout {
  size_t fc, kv, lm, qkv[DFLASH_MAX_LAYERS], o[DFLASH_MAX_LAYERS], gu[DFLASH_MAX_LAYERS],
      down[DFLASH_MAX_LAYERS], total;
};
PackLayout pack_layout(const dflash_model* m) {
  const Dims d = dims_of(m->cfg);
  PackLayout P{};
  size_t off = 0;
  auto take = [&](int N, int K) {
    const size_t o = off;
    off += (packed_elems(N, K) + 127) / 128 * 128;   // 256-byte aligned
    return o;
  };
  P.fc = take(d.D, d.F);
  P.kv = take(2 * d.NL * d.KVD, d.D);
  P.lm = take(d.V, d.D);
  for (int l = 0; l < d.NL; ++l) {
    P.qkv[l] = take(d.QD + 2 * d.KVD, d.D);
    P.o[l] = take(d.D, d.QD);
    P.gu[l] = take(2 * d.I, d.D);
    P.down[l] = take(d.D, d.I);
  }
  P.total = off;
  return P;
}
const uint16_t* packed_at(const dflash_model* m, size_t off) {
  return m->packed ? m->packed + off : nullptr;
}

struct DraftLayout {
  size_t x, y, ss, rope, q, k, v, o, h, part, att_o, att_ml, best, total;
  AttnPlan ap;
  int parts;
  int groups;   // column groups of the LM-head argmax
  bool fused;
};

DraftLayout draft_layout(const dflash_model* m, int B, int gamma, int max_pages) {
  const Dims d = dims_of(m->cfg);
  const bool bf = m->bf16;
  const size_t M = (size_t)B * gamma;
  DraftLayout L{};
  L.fused = use_fused(m, (int)M);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  // Transient activations take 4 bytes per element: fp32, or two bf16 planes.
  L.x = take(M * d.D * 4);
  if (!L.fused) L.y = take(M * d.D * 4);
  L.ss = take(M * std::max(d.D / 64, 1) * 4);
  L.rope = take(M * d.dh * 4);   // (cos, sin) per row and dimension pair
  L.q = take(M * d.QD * 4);
  L.k = take(M * d.KVD * 4);
  L.v = take(M * d.KVD * 4);
  L.o = take(M * d.QD * 4);
  L.h = take(M * d.I * 4);
  const int Mi = (int)M;
  size_t pf;
  if (L.fused) {
    pf = skinny_part_floats(Mi, d.QD + 2 * d.KVD, d.D, SO_QKV, d.dh);
    pf = std::max(pf, skinny_part_floats(Mi, d.D, d.QD, SO_RESID, d.dh));
    pf = std::max(pf, skinny_part_floats(Mi, 2 * d.I, d.D, SO_SWIGLU, d.dh));
    pf = std::max(pf, skinny_part_floats(Mi, d.D, d.I, SO_RESID, d.dh));
  } else {
    pf = part_floats(bf, Mi, d.QD + 2 * d.KVD, d.D);
    pf = std::max(pf, part_floats(bf, Mi, d.D, d.QD));
    pf = std::max(pf, part_floats(bf, Mi, 2 * d.I, d.D));
    pf = std::max(pf, part_floats(bf, Mi, d.D, d.I));
  }
  L.part = take(pf * 4);
  L.ap = plan_attention(B, d.Hkv, max_pages, m->cfg.page_size);
  L.parts = bf ? L.ap.n_ctx_splits + 1 : 1;
  L.att_o = take((size_t)L.parts * M * d.Hq * d.dh * 4);
  L.att_ml = take((size_t)L.parts * M * d.Hq * 2 * 4);
  if (!L.fused) {   // the fused LM head merges its keys in the state buffer
    const GemmPlan lm = plan_gemm(bf, Mi, d.V, d.D, true);
    L.groups = gemm_argmax_groups(lm, d.V);
    L.best = take((size_t)L.groups * M * 8);
  }
  L.total = off;
  return L;
}

struct InjectLayout {
  size_t part, c, ss, rope, total;
  bool fused;
};

InjectLayout inject_layout(const dflash_model* m, int n_tok) {
  const Dims d = dims_of(m->cfg);
  const bool bf = m->bf16;
  InjectLayout L{};
  L.fused = use_fused(m, n_tok);
  size_t pf;
  if (L.fused) {
    pf = skinny_part_floats(n_tok, d.D, d.F, SO_STORE_SS, d.dh);
    pf = std::max(pf, skinny_part_floats(n_tok, 2 * d.NL * d.KVD, d.D, SO_KV, d.dh));
  } else {
    pf = part_floats(bf, n_tok, d.D, d.F);
    pf = std::max(pf, part_floats(bf, n_tok, 2 * d.NL * d.KVD, d.D));
  }
  size_t off = 0;
  L.part = off;
  off = align256(pf * 4);
  L.c = off;
  off = align256(off + (size_t)n_tok * d.D * 4);
  L.ss = off;
  off = align256(off + (size_t)n_tok * std::max(d.D / 64, 1) * 4);
  L.rope = off;
  off = align256(off + (size_t)n_tok * d.dh * 4);
  L.total = off;
  return L;
}

int check_config(const dflash_config* c) {
  if (c->hidden <= 0 || c->n_layers <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
      c->head_dim <= 0 || c->intermediate <= 0 || c->vocab <= 1 || c->n_target_feats <= 0)
    return fail(DFLASH_E_INVAL, "config: all dimensions must be positive (vocab >= 2)");
  if (c->n_layers > DFLASH_MAX_LAYERS)
    return fail(DFLASH_E_SHAPE, "config: n_layers %d > %d", c->n_layers, DFLASH_MAX_LAYERS);
  if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16)
    return fail(DFLASH_E_DTYPE, "config: unknown dtype %d", c->dtype);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(DFLASH_E_SHAPE, "config: head_dim must be 64 or 128 (got %d)", c->head_dim);
  if (c->n_q_heads % c->n_kv_heads != 0 || c->n_q_heads / c->n_kv_heads > 8)
    return fail(DFLASH_E_SHAPE, "config: n_q_heads must be a multiple of n_kv_heads, ratio <= 8");
  if (c->max_block < 1 || c->max_block > DFLASH_MAX_BLOCK)
    return fail(DFLASH_E_SHAPE, "config: max_block must be in [1, %d]", DFLASH_MAX_BLOCK);
  if (c->page_size != 16) return fail(DFLASH_E_SHAPE, "config: page_size must be 16");
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab)
    return fail(DFLASH_E_INVAL, "config: mask_token_id outside [0, vocab)");
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f))
    return fail(DFLASH_E_INVAL, "config: rope_theta must be > 0 and rms_eps >= 0");
  if (c->n_layers * 2 > WSEG_MAX) return fail(DFLASH_E_SHAPE, "config: too many layers");
  if (c->hidden % 4 || c->hidden > 8192)
    return fail(DFLASH_E_SHAPE, "config: hidden must be a multiple of 4 and at most 8192");
  if (c->dtype == DFLASH_BF16) {
    const int qd = c->n_q_heads * c->head_dim;
    if (c->hidden % 256 || c->intermediate % 256 || qd % 256)
      return fail(DFLASH_E_SHAPE,
                  "config: bf16 kernels need hidden, intermediate and n_q_heads*head_dim to be "
                  "multiples of 256");
  } else {
    if (c->head_dim > 256) return fail(DFLASH_E_SHAPE, "config: head_dim too large");
  }
  return DFLASH_OK;
}

}  // namespace

extern "C" {

const char* dflash_last_error(void) { return g_err.c_str(); }

int dflash_model_create(const dflash_config* cfg, const dflash_weights* w, void* state,
                        dflash_model** out) {
  if (!cfg || !w || !state || !out) return fail(DFLASH_E_INVAL, "model_create: null argument");
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!w->fc_w || !w->fc_norm || !w->embed || !w->lm_head || !w->final_norm)
    return fail(DFLASH_E_INVAL, "model_create: null global weight pointer");
  for (int l = 0; l < cfg->n_layers; ++l) {
    const dflash_layer_weights& L = w->layer[l];
    if (!L.attn_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.mlp_norm || !L.w_gate || !L.w_up ||
        !L.w_down)
      return fail(DFLASH_E_INVAL, "model_create: null weight pointer in layer %d", l);
  }
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  HIPCHK(hipMemset(state, 0, DFLASH_STATE_BYTES));
  resolve_scratch(dev);
  dflash_model* m = new dflash_model();
  m->cfg = *cfg;
  m->w = *w;
  m->err = (uint32_t*)state;
  m->ctr = (unsigned long long*)((char*)state + kCtrOffset);
  m->amax = (unsigned long long*)((char*)state + kAmaxOffset);
  m->actr = (unsigned long long*)((char*)state + kActrOffset);
  m->wctr = (unsigned int*)((char*)state + kActrOffset + 64);
  m->kvdone = (unsigned int*)((char*)state + kActrOffset + 128);
  m->qhint = (uint32_t*)((char*)state + kQhintOffset);
  m->hint_seq = 0;
  m->packed = nullptr;
  m->device = dev;
  m->bf16 = cfg->dtype == DFLASH_BF16;
  m->prof_on = false;
  m->prof_ms = 0.0;
  m->prof_count = 0;
  *out = m;
  return DFLASH_OK;
}

void dflash_model_destroy(dflash_model* m) {
  if (!m) return;
  for (auto& p : m->pending) {
    (void)hipEventDestroy(p.first);
    (void)hipEventDestroy(p.second);
  }
  for (auto& p : m->pool) {
    (void)hipEventDestroy(p.first);
    (void)hipEventDestroy(p.second);
  }
  delete m;
}

size_t dflash_workspace_bytes(const dflash_model* m, int32_t max_batch, int32_t max_block,
                              int32_t max_new_tokens, int32_t max_pages_per_seq) {
  if (!m || max_batch < 1 || max_block < 1 || max_block > m->cfg.max_block ||
      max_new_tokens < 0 || max_pages_per_seq < 1)
    return 0;
  size_t need = 0;
  for (int b = 1; b <= max_batch; ++b)
    for (int g = 1; g <= max_block; ++g)
      need = std::max(need, draft_layout(m, b, g, max_pages_per_seq).total);
  for (int n = 1; n <= max_new_tokens; ++n) need = std::max(need, inject_layout(m, n).total);
  // greedy verification of blocks over the model's vocabulary
  need = std::max(need, align256(verify_greedy_workspace(max_batch, max_block, m->cfg.vocab)));
  return need;
}

size_t dflash_packed_weight_bytes(const dflash_model* m) {
  if (!m || !m->bf16) return 0;
  return pack_layout(m).total * 2;
}

int dflash_pack_weights(dflash_model* m, void* packed, size_t bytes, void* stream) {
  if (!m || !packed) return fail(DFLASH_E_INVAL, "pack_weights: null argument");
  if (!m->bf16) return fail(DFLASH_E_DTYPE, "pack_weights: only bf16 models use packed weights");
  if (((uintptr_t)packed & 255) != 0)
    return fail(DFLASH_E_INVAL, "pack_weights: buffer must be 256-byte aligned");
  const PackLayout P = pack_layout(m);
  if (bytes < P.total * 2)
    return fail(DFLASH_E_CAPACITY, "pack_weights: buffer %zu bytes < %zu needed", bytes,
                P.total * 2);
  const Dims d = dims_of(m->cfg);
  hipStream_t st = (hipStream_t)stream;
  uint16_t* out = (uint16_t*)packed;
  HIPCHK(launch_pack(seg1(m->w.fc_w, d.D), d.D, d.F, 0, out + P.fc, st));
  HIPCHK(launch_pack(wseg_kv(m), 2 * d.NL * d.KVD, d.D, 0, out + P.kv, st));
  HIPCHK(launch_pack(seg1(m->w.lm_head, d.V), d.V, d.D, 0, out + P.lm, st));
  for (int l = 0; l < d.NL; ++l) {
    HIPCHK(launch_pack(wseg_qkv(m, l), d.QD + 2 * d.KVD, d.D, 0, out + P.qkv[l], st));
    HIPCHK(launch_pack(seg1(m->w.layer[l].wo, d.D), d.D, d.QD, 0, out + P.o[l], st));
    HIPCHK(launch_pack(wseg_gu(m, l), 2 * d.I, d.D, d.I, out + P.gu[l], st));
    HIPCHK(launch_pack(seg1(m->w.layer[l].w_down, d.D), d.D, d.I, 0, out + P.down[l], st));
  }
  m->packed = out;
  return DFLASH_OK;
}

int dflash_inject_ctx(const dflash_model* m, const dflash_kv* kv, const void* hidden,
                      const int32_t* cu_new, int32_t batch, int32_t n_tok, void* workspace,
                      size_t ws_bytes, void* stream) {
  if (!m || !kv || !cu_new) return fail(DFLASH_E_INVAL, "inject_ctx: null argument");
  if (!kv->pages || !kv->page_table || !kv->ctx_lens)
    return fail(DFLASH_E_INVAL, "inject_ctx: null pointer in the KV cache description");
  if (batch < 1) return fail(DFLASH_E_INVAL, "inject_ctx: batch must be >= 1");
  if (n_tok < 0) return fail(DFLASH_E_INVAL, "inject_ctx: n_tok must be >= 0");
  if (kv->n_pages < 1 || kv->max_pages_per_seq < 1)
    return fail(DFLASH_E_INVAL, "inject_ctx: empty page pool or page table");
  if (n_tok == 0) return DFLASH_OK;
  if (!hidden || !workspace) return fail(DFLASH_E_INVAL, "inject_ctx: null hidden or workspace");
  const InjectLayout L = inject_layout(m, n_tok);
  if (L.total > ws_bytes)
    return fail(DFLASH_E_CAPACITY, "inject_ctx: workspace %zu bytes < %zu needed", ws_bytes,
                L.total);
  const Dims d = dims_of(m->cfg);
  const bool bf = m->bf16;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* part = (float*)(ws + L.part);
  void* c = ws + L.c;

  const WSeg fc = seg1(m->w.fc_w, d.D);
  const WSeg kvw = wseg_kv(m);
  const int Nkv = 2 * d.NL * d.KVD;
  const PackLayout PL = pack_layout(m);

  if (L.fused) {
    // u = W_c f (fp32, with per-tile row sums of squares), then the K/V
    // product forms c = bf16(RMSNorm(u)) while staging it and writes the
    // pages itself.
    float* cx = (float*)c;
    float* ss = (float*)(ws + L.ss);
    SkinnyArgs a{};
    a.A = hidden;
    a.lda = d.F;
    a.M = n_tok;
    a.w = fc;
    a.packed = packed_at(m, PL.fc);
    a.N = d.D;
    a.K = d.F;
    a.part = part;
    a.ctr = m->ctr;
    a.err = m->err;
    a.dh = d.dh;
    a.I = d.I;
    a.x = cx;
    a.ss_out = ss;
    float* rope = (float*)(ws + L.rope);
    a.rope_out = rope;
    a.rope_rows = n_tok;
    a.cu_new = cu_new;
    a.batch = batch;
    a.ctx_lens = kv->ctx_lens;
    a.theta = m->cfg.rope_theta;
    GemmPlan p = plan_skinny(n_tok, d.D, d.F, SO_STORE_SS, d.dh);
    HIPCHK(run_skinny(m, p, SA_BF16, SO_STORE_SS, a, st));

    SkinnyArgs b{};
    b.A = cx;
    b.lda = d.D;
    b.M = n_tok;
    b.ss_in = ss;
    b.ss_tiles = d.D / 64;
    b.gain = m->w.fc_norm;
    b.eps = m->cfg.rms_eps;
    b.w = kvw;
    b.packed = packed_at(m, PL.kv);
    b.N = Nkv;
    b.K = d.D;
    b.part = part;
    b.ctr = m->ctr;
    b.err = m->err;
    b.Hkv = d.Hkv;
    b.dh = d.dh;
    b.I = d.I;
    b.ctx_lens = kv->ctx_lens;
    b.theta = m->cfg.rope_theta;
    b.rope = rope;
    b.pages = kv->pages;
    b.cu_new = cu_new;
    b.batch = batch;
    b.page_table = kv->page_table;
    b.max_pages = kv->max_pages_per_seq;
    b.n_pages = kv->n_pages;
    b.page_size = m->cfg.page_size;
    // the launch's last tile advances ctx_lens (no separate launch)
    b.kvdone = m->kvdone;
    b.ctx_lens_rw = kv->ctx_lens;
    p = plan_skinny(n_tok, Nkv, d.D, SO_KV, d.dh);
    HIPCHK(run_skinny(m, p, SA_NORM1, SO_KV, b, st));
    return DFLASH_OK;
  }

  GemmPlan p = plan_gemm(bf, n_tok, d.D, d.F, false);
  HIPCHK(launch_gemm(p, bf, hidden, nullptr, d.F, n_tok, fc, d.D, d.F, part, nullptr, nullptr, st));
  HIPCHK(launch_inject_norm(bf, part, p.splits, n_tok, d.D, m->w.fc_norm, m->cfg.rms_eps, c,
                            st));
  p = plan_gemm(bf, n_tok, Nkv, d.D, false);
  HIPCHK(launch_gemm(p, bf, c, nullptr, d.D, n_tok, kvw, Nkv, d.D, part, nullptr, nullptr, st));
  HIPCHK(launch_inject_scatter(bf, part, p.splits, n_tok, cu_new, batch, kv->ctx_lens,
                               kv->page_table, kv->max_pages_per_seq, kv->n_pages,
                               m->cfg.page_size, kv->pages, d.NL, d.Hkv, d.dh,
                               m->cfg.rope_theta, m->err, st));
  HIPCHK(launch_advance_ctx(kv->ctx_lens, cu_new, batch, st));
  return DFLASH_OK;
}

// A pass of the autoregressive variant: the rows' tokens come from
// tokens[b*stride + j], the block keys are causal, and row 0's output is an
// argmax like the others (no anchor substitution).
struct ArPass {
  const int32_t* tokens;
  int stride;
};

// One draft pass; dr.on turns the LM head's argmax into a Gumbel-max draw.
static int draft_impl(const dflash_model* mc, const dflash_kv* kv, const int32_t* anchor,
                      int32_t batch, int32_t gamma, int32_t* block_tokens, float* logits,
                      void* workspace, size_t ws_bytes, void* stream, const DrawArgs& dr,
                      const ArPass* ar = nullptr, bool may_profile = true) {
  dflash_model* m = const_cast<dflash_model*>(mc);
  if (!m || !kv || !anchor || !block_tokens || !workspace)
    return fail(DFLASH_E_INVAL, "draft_block: null argument");
  if (!kv->pages || !kv->page_table || !kv->ctx_lens)
    return fail(DFLASH_E_INVAL, "draft_block: null pointer in the KV cache description");
  if (batch < 1) return fail(DFLASH_E_INVAL, "draft_block: batch must be >= 1");
  if (gamma < 1 || gamma > m->cfg.max_block)
    return fail(DFLASH_E_CAPACITY, "draft_block: block_size %d outside [1, %d]", gamma,
                m->cfg.max_block);
  if (kv->n_pages < 1 || kv->max_pages_per_seq < 1)
    return fail(DFLASH_E_INVAL, "draft_block: empty page pool or page table");
  const DraftLayout L = draft_layout(m, batch, gamma, kv->max_pages_per_seq);
  if (L.total > ws_bytes)
    return fail(DFLASH_E_CAPACITY, "draft_block: workspace %zu bytes < %zu needed", ws_bytes,
                L.total);
  const Dims d = dims_of(m->cfg);
  const bool bf = m->bf16;
  const float eps = m->cfg.rms_eps;
  const int M = batch * gamma;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* x = (float*)(ws + L.x);
  void *y = ws + L.y, *q = ws + L.q, *o = ws + L.o, *h = ws + L.h;
  float* k = (float*)(ws + L.k);
  float* v = (float*)(ws + L.v);
  // planes of the split activations (bf16 models) and their lo halves
  const size_t y_pl = (size_t)M * d.D, q_pl = (size_t)M * d.QD, h_pl = (size_t)M * d.I;
  auto lo = [&](void* base, size_t plane) -> const void* {
    return bf ? (const void*)((const uint16_t*)base + plane) : nullptr;
  };
  float* part = (float*)(ws + L.part);
  float* att_o = (float*)(ws + L.att_o);
  float* att_ml = (float*)(ws + L.att_ml);
  uint64_t* best = (uint64_t*)(ws + L.best);

  float* ss = (float*)(ws + L.ss);

  // LM-head timing events (dflash_profile_enable)
  std::pair<hipEvent_t, hipEvent_t> ev{nullptr, nullptr};
  const bool prof = m->prof_on && may_profile;   // (event creation allocates)
  auto prof_begin = [&]() -> int {
    if (!prof) return DFLASH_OK;
    if (!m->pool.empty()) {
      ev = m->pool.back();
      m->pool.pop_back();
    } else {
      HIPCHK(hipEventCreate(&ev.first));
      HIPCHK(hipEventCreate(&ev.second));
    }
    HIPCHK(hipEventRecord(ev.first, st));
    return DFLASH_OK;
  };
  auto prof_end = [&]() -> int {
    if (!prof) return DFLASH_OK;
    HIPCHK(hipEventRecord(ev.second, st));
    m->pending.push_back(ev);
    return DFLASH_OK;
  };

  AttnArgs at{};
  at.q = q;
  at.q_plane = q_pl;
  at.k = k;
  at.v = v;
  at.pages = kv->pages;
  at.n_pages = kv->n_pages;
  at.max_pages = kv->max_pages_per_seq;
  at.page_size = m->cfg.page_size;
  at.page_table = kv->page_table;
  at.ctx_lens = kv->ctx_lens;
  at.batch = batch;
  at.gamma = gamma;
  at.Hq = d.Hq;
  at.Hkv = d.Hkv;
  at.dh = d.dh;
  at.part_o = att_o;
  at.part_ml = att_ml;
  at.err = m->err;
  at.causal = ar ? 1 : 0;

  const int Nqkv = d.QD + 2 * d.KVD;
  const WSeg lm = seg1(m->w.lm_head, d.V);
  const PackLayout PL = pack_layout(m);
  int rc;

  if (L.fused) {
    // Every product normalises its input while staging it and finishes its
    // own epilogue; the residual x carries per-tile row sums of squares ss.
    float* rope = (float*)(ws + L.rope);
    HIPCHK(launch_embed(bf, anchor, batch, gamma, m->cfg.mask_token_id, d.V, m->w.embed, d.D, x,
                        nullptr, eps, nullptr, 0, ss, rope, kv->ctx_lens, d.dh,
                        m->cfg.rope_theta, m->err, st, ar ? ar->tokens : nullptr,
                        ar ? ar->stride : 0));
    int ss_tiles = 1;
    SkinnyArgs base{};
    base.M = M;
    base.eps = eps;
    base.part = part;
    base.ctr = m->ctr;
    base.err = m->err;
    base.gamma = gamma;
    base.Hq = d.Hq;
    base.Hkv = d.Hkv;
    base.dh = d.dh;
    base.ctx_lens = kv->ctx_lens;
    base.theta = m->cfg.rope_theta;
    base.rope = rope;
    base.I = d.I;
    for (int l = 0; l < d.NL; ++l) {
      const dflash_layer_weights& W = m->w.layer[l];
      SkinnyArgs a = base;
      a.A = x;
      a.lda = d.D;
      a.ss_in = ss;
      a.ss_tiles = ss_tiles;
      a.gain = W.attn_norm;
      a.w = wseg_qkv(m, l);
      a.packed = packed_at(m, PL.qkv[l]);
      a.N = Nqkv;
      a.K = d.D;
      a.q = q;
      a.q_plane = q_pl;
      a.kb = k;
      a.vb = v;
      HIPCHK(run_skinny(m, plan_skinny(M, Nqkv, d.D, SO_QKV, d.dh), SA_NORM, SO_QKV, a, st));

      at.layer = l;
      HIPCHK(launch_attention(bf, at, L.ap, st));
      HIPCHK(launch_attn_combine(bf, att_o, att_ml, L.parts, batch, gamma, d.Hq, d.dh, o, q_pl,
                                 st));

      a = base;
      a.A = o;
      a.a_plane = q_pl;
      a.lda = d.QD;
      a.w = seg1(W.wo, d.D);
      a.packed = packed_at(m, PL.o[l]);
      a.N = d.D;
      a.K = d.QD;
      a.x = x;
      a.ss_out = ss;
      HIPCHK(run_skinny(m, plan_skinny(M, d.D, d.QD, SO_RESID, d.dh), SA_SPLIT, SO_RESID, a, st));
      ss_tiles = d.D / 64;

      a = base;
      a.A = x;
      a.lda = d.D;
      a.ss_in = ss;
      a.ss_tiles = ss_tiles;
      a.gain = W.mlp_norm;
      a.w = wseg_gu(m, l);
      a.packed = packed_at(m, PL.gu[l]);
      a.N = 2 * d.I;
      a.K = d.D;
      a.h = h;
      a.h_plane = h_pl;
      HIPCHK(run_skinny(m, plan_skinny(M, 2 * d.I, d.D, SO_SWIGLU, d.dh), SA_NORM, SO_SWIGLU, a,
                           st));

      a = base;
      a.A = h;
      a.a_plane = h_pl;
      a.lda = d.I;
      a.w = seg1(W.w_down, d.D);
      a.packed = packed_at(m, PL.down[l]);
      a.N = d.D;
      a.K = d.I;
      a.x = x;
      a.ss_out = ss;
      HIPCHK(run_skinny(m, plan_skinny(M, d.D, d.I, SO_RESID, d.dh), SA_SPLIT, SO_RESID, a, st));
    }
    SkinnyArgs a = base;
    a.A = x;
    a.lda = d.D;
    a.ss_in = ss;
    a.ss_tiles = ss_tiles;
    a.gain = m->w.final_norm;
    a.w = lm;
    a.packed = packed_at(m, PL.lm);
    a.N = d.V;
    a.K = d.D;
    a.amax = m->amax;
    a.actr = m->actr;
    a.wctr = m->wctr;
    a.anchor = ar ? nullptr : anchor;
    a.block_tokens = block_tokens;
    a.logits = logits;
    a.draw = dr;
    if ((rc = prof_begin()) != DFLASH_OK) return rc;
    HIPCHK(run_skinny(m, plan_skinny(M, d.V, d.D, SO_ARGMAX, d.dh), SA_NORM, SO_ARGMAX, a, st));
    if ((rc = prof_end()) != DFLASH_OK) return rc;
    return DFLASH_OK;
  }

  float* rope_t = (float*)(ws + L.rope);
  HIPCHK(launch_embed(bf, anchor, batch, gamma, m->cfg.mask_token_id, d.V, m->w.embed, d.D, x,
                      m->w.layer[0].attn_norm, eps, y, y_pl, nullptr, rope_t, kv->ctx_lens, d.dh,
                      m->cfg.rope_theta, m->err, st, ar ? ar->tokens : nullptr,
                        ar ? ar->stride : 0));
  for (int l = 0; l < d.NL; ++l) {
    const dflash_layer_weights& W = m->w.layer[l];
    WSeg qkv{};
    qkv.ptr[0] = W.wq;
    qkv.ptr[1] = W.wk;
    qkv.ptr[2] = W.wv;
    qkv.row_end[0] = d.QD;
    qkv.row_end[1] = d.QD + d.KVD;
    qkv.row_end[2] = Nqkv;
    qkv.n = 3;
    GemmPlan p = plan_gemm(bf, M, Nqkv, d.D, false);
    HIPCHK(launch_gemm(p, bf, y, lo(y, y_pl), d.D, M, qkv, Nqkv, d.D, part, nullptr, nullptr, st));
    HIPCHK(launch_qkv_epilogue(bf, part, p.splits, M, d.Hq, d.Hkv, d.dh, rope_t, q, q_pl, k, v,
                               st));
    at.layer = l;
    HIPCHK(launch_attention(bf, at, L.ap, st));
    HIPCHK(launch_attn_combine(bf, att_o, att_ml, L.parts, batch, gamma, d.Hq, d.dh, o, q_pl, st));

    WSeg wo{};
    wo.ptr[0] = W.wo;
    wo.row_end[0] = d.D;
    wo.n = 1;
    p = plan_gemm(bf, M, d.D, d.QD, false);
    HIPCHK(launch_gemm(p, bf, o, lo(o, q_pl), d.QD, M, wo, d.D, d.QD, part, nullptr, nullptr, st));
    HIPCHK(launch_residual_norm(bf, x, part, p.splits, M, d.D, W.mlp_norm, eps, y, y_pl, st));

    WSeg gu{};
    gu.ptr[0] = W.w_gate;
    gu.ptr[1] = W.w_up;
    gu.row_end[0] = d.I;
    gu.row_end[1] = 2 * d.I;
    gu.n = 2;
    p = plan_gemm(bf, M, 2 * d.I, d.D, false);
    if (bf && gemm_swiglu_ok(p, d.I)) {
      HIPCHK(launch_gemm_swiglu(p, y, lo(y, y_pl), d.D, M, gu, d.I, d.D, h, h_pl, st));
    } else {
      HIPCHK(launch_gemm(p, bf, y, lo(y, y_pl), d.D, M, gu, 2 * d.I, d.D, part, nullptr, nullptr,
                         st));
      HIPCHK(launch_swiglu(bf, part, p.splits, M, d.I, h, h_pl, st));
    }

    WSeg dn{};
    dn.ptr[0] = W.w_down;
    dn.row_end[0] = d.D;
    dn.n = 1;
    p = plan_gemm(bf, M, d.D, d.I, false);
    HIPCHK(launch_gemm(p, bf, h, lo(h, h_pl), d.I, M, dn, d.D, d.I, part, nullptr, nullptr, st));
    const void* g_next = l + 1 < d.NL ? m->w.layer[l + 1].attn_norm : m->w.final_norm;
    HIPCHK(launch_residual_norm(bf, x, part, p.splits, M, d.D, g_next, eps, y, y_pl, st));
  }

  const GemmPlan p = plan_gemm(bf, M, d.V, d.D, true);
  // On the large-product kernel (>= 128 rows, MFMA-bound) the LM head takes
  // its input in bf16, the workload's activation precision, which halves its
  // matrix-core work: the hi plane alone is the bf16 rounding of the fp32
  // row.  The lo plane carries the layers' fp32 activations; the LM head is
  // the last product, so its rounding only adds a bounded logit error
  // (sum over D of |h| * |W| * 2^-9) and is not amplified by later layers.
  const void* lm_lo = p.kind == GEMM_BIG ? nullptr : lo(y, y_pl);
  if ((rc = prof_begin()) != DFLASH_OK) return rc;
  HIPCHK(launch_gemm(p, bf, y, lm_lo, d.D, M, lm, d.V, d.D, nullptr, best, logits, st, dr));
  if ((rc = prof_end()) != DFLASH_OK) return rc;
  HIPCHK(launch_argmax_finalize(best, L.groups, ar ? nullptr : anchor, batch, gamma, block_tokens,
                                st));
  return DFLASH_OK;
}

int dflash_draft_block(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor,
                       int32_t batch, int32_t gamma, int32_t* block_tokens, float* logits,
                       void* workspace, size_t ws_bytes, void* stream) {
  return draft_impl(m, kv, anchor, batch, gamma, block_tokens, logits, workspace, ws_bytes,
                    stream, DrawArgs{});
}

int dflash_draft_block_noalloc(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor,
                               int32_t batch, int32_t gamma, int32_t* block_tokens, float* logits,
                               void* stream) {
  if (!m || !kv) return fail(DFLASH_E_INVAL, "draft_block_noalloc: null argument");
  int dev = -1;
  HIPCHK(hipGetDevice(&dev));
  if (dev != m->device)
    return fail(DFLASH_E_INVAL, "draft_block_noalloc: current device %d is not the model's (%d)",
                dev, m->device);
  void* ws = dev < kMaxDevices ? g_scratch[dev].load() : nullptr;
  if (ws == nullptr)
    return fail(DFLASH_E_HIP, "draft_block_noalloc: the scratch array of device %d is not "
                              "available", dev);
  if (batch >= 1 && gamma >= 1 && gamma <= m->cfg.max_block && kv->max_pages_per_seq >= 1) {
    const size_t need = draft_layout(m, batch, gamma, kv->max_pages_per_seq).total;
    if (need > DFLASH_NOALLOC_SCRATCH_BYTES)
      return fail(DFLASH_E_CAPACITY,
                  "draft_block_noalloc: batch %d, block %d, %d pages per sequence need %zu bytes "
                  "of scratch; the library holds %zu per GPU",
                  batch, gamma, kv->max_pages_per_seq, need,
                  (size_t)DFLASH_NOALLOC_SCRATCH_BYTES);
  }
  return draft_impl(m, kv, anchor, batch, gamma, block_tokens, logits, ws,
                    DFLASH_NOALLOC_SCRATCH_BYTES, stream, DrawArgs{}, nullptr, false);
}

// Autoregressive drafting workspace: a draft pass of up to block_size - 1
// rows per sequence, then the pass's row tokens [batch][block_size].
static size_t ar_layout_total(const dflash_model* m, int batch, int gamma, int max_pages,
                              size_t* tok_off) {
  size_t need = 0;
  for (int g = 1; g < gamma; ++g) need = std::max(need, draft_layout(m, batch, g, max_pages).total);
  need = align256(need);
  if (tok_off) *tok_off = need;
  return align256(need + (size_t)batch * gamma * 4);
}

size_t dflash_ar_workspace_bytes(const dflash_model* m, int32_t max_batch, int32_t max_block,
                                 int32_t max_pages_per_seq) {
  if (!m || max_batch < 1 || max_block < 1 || max_block > m->cfg.max_block ||
      max_pages_per_seq < 1)
    return 0;
  size_t need = 0;
  for (int b = 1; b <= max_batch; ++b)
    for (int g = 1; g <= max_block; ++g)
      need = std::max(need, ar_layout_total(m, b, g, max_pages_per_seq, nullptr));
  return need;
}

int dflash_draft_block_ar(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor,
                          int32_t batch, int32_t gamma, int32_t* block_tokens, float* logits,
                          void* workspace, size_t ws_bytes, void* stream) {
  if (!m || !kv || !anchor || !block_tokens || !workspace)
    return fail(DFLASH_E_INVAL, "draft_block_ar: null argument");
  if (batch < 1) return fail(DFLASH_E_INVAL, "draft_block_ar: batch must be >= 1");
  if (gamma < 1 || gamma > m->cfg.max_block)
    return fail(DFLASH_E_CAPACITY, "draft_block_ar: block_size %d outside [1, %d]", gamma,
                m->cfg.max_block);
  if (kv->max_pages_per_seq < 1)
    return fail(DFLASH_E_INVAL, "draft_block_ar: empty page table");
  size_t tok_off = 0;
  const size_t need = ar_layout_total(m, batch, gamma, kv->max_pages_per_seq, &tok_off);
  if (need > ws_bytes)
    return fail(DFLASH_E_CAPACITY, "draft_block_ar: workspace %zu bytes < %zu needed", ws_bytes,
                need);
  hipStream_t st = (hipStream_t)stream;
  int32_t* pass_tokens = (int32_t*)((char*)workspace + tok_off);
  HIPCHK(launch_ar_seed(anchor, batch, gamma, block_tokens, st));
  const ArPass ar{block_tokens, gamma};
  for (int i = 1; i < gamma; ++i) {
    const int rc = draft_impl(m, kv, anchor, batch, i, pass_tokens,
                              i == gamma - 1 ? logits : nullptr, workspace, tok_off, stream,
                              DrawArgs{}, &ar);
    if (rc != DFLASH_OK) return rc;
    HIPCHK(launch_ar_pick(pass_tokens, batch, i, gamma, block_tokens, st));
  }
  return DFLASH_OK;
}

int dflash_draft_block_sampled(const dflash_model* m, const dflash_kv* kv,
                               const int32_t* anchor, int32_t batch, int32_t gamma,
                               uint64_t seed, int32_t* block_tokens, float* logits,
                               void* workspace, size_t ws_bytes, void* stream) {
  if (!logits)
    return fail(DFLASH_E_INVAL, "draft_block_sampled: the drafter logits are required");
  DrawArgs dr{};
  dr.on = 1;
  dr.gamma = gamma;
  dr.seed = seed;
  return draft_impl(m, kv, anchor, batch, gamma, block_tokens, logits, workspace, ws_bytes,
                    stream, dr);
}

int dflash_verify_greedy(const int32_t* block_tokens, const void* target_logits,
                         int32_t logits_dtype, int32_t batch, int32_t gamma, int32_t vocab,
                         int32_t* accept_len, int32_t* out_tokens, int32_t* target_argmax,
                         void* workspace, size_t ws_bytes, void* stream) {
  if (!block_tokens || !target_logits || !accept_len || !out_tokens || !workspace)
    return fail(DFLASH_E_INVAL, "verify_greedy: null argument");
  if (logits_dtype != DFLASH_F32 && logits_dtype != DFLASH_BF16)
    return fail(DFLASH_E_DTYPE, "verify_greedy: unknown logits dtype %d", logits_dtype);
  if (batch < 1 || gamma < 1 || vocab < 1)
    return fail(DFLASH_E_INVAL, "verify_greedy: batch, block_size and vocab must be >= 1");
  if (gamma > kVerifyMaxBlock)
    return fail(DFLASH_E_CAPACITY, "verify_greedy: block_size %d > %d", gamma, kVerifyMaxBlock);
  const size_t need = verify_greedy_workspace(batch, gamma, vocab);
  if (ws_bytes < need)
    return fail(DFLASH_E_CAPACITY, "verify_greedy: workspace %zu bytes < %zu needed", ws_bytes,
                need);
  HIPCHK(launch_verify(logits_dtype == DFLASH_BF16, block_tokens, target_logits, batch, gamma,
                       vocab, (uint64_t*)workspace, accept_len, out_tokens, target_argmax,
                       (hipStream_t)stream));
  return DFLASH_OK;
}

// Packed forward workspace: the draft's own layout for n_blocks sequences,
// then the broadcast page table, the per-block context lengths, the block
// tokens and the cross-entropy scratch.
struct PackedLayout {
  size_t draft, table, lens, tokens, ce, total;
};

static PackedLayout packed_layout(const dflash_model* m, int n, int gamma, int max_pages) {
  PackedLayout L{};
  size_t off = align256(draft_layout(m, n, gamma, max_pages).total);
  L.draft = off;
  L.table = off;
  off = align256(off + (size_t)n * max_pages * 4);
  L.lens = off;
  off = align256(off + (size_t)n * 4);
  L.tokens = off;
  off = align256(off + (size_t)n * gamma * 4);
  L.ce = off;
  off = align256(off + (size_t)n * (gamma > 1 ? gamma - 1 : 1) * 8);
  L.total = off;
  return L;
}

size_t dflash_packed_workspace_bytes(const dflash_model* m, int32_t max_blocks, int32_t max_block,
                                     int32_t max_pages_per_seq) {
  if (!m || max_blocks < 1 || max_block < 1 || max_block > m->cfg.max_block ||
      max_pages_per_seq < 1)
    return 0;
  size_t need = 0;
  for (int n = 1; n <= max_blocks; ++n)
    for (int g = 1; g <= max_block; ++g)
      need = std::max(need, packed_layout(m, n, g, max_pages_per_seq).total);
  return need;
}

int dflash_packed_forward(const dflash_model* mc, const dflash_kv* ctx, const int32_t* anchors,
                          const int32_t* anchor_pos, int32_t n_blocks, int32_t gamma,
                          const int32_t* targets, float decay, float* logits,
                          int32_t* block_tokens, float* block_loss, float* loss, void* workspace,
                          size_t ws_bytes, void* stream) {
  dflash_model* m = const_cast<dflash_model*>(mc);
  if (!m || !ctx || !anchors || !anchor_pos || !logits || !workspace)
    return fail(DFLASH_E_INVAL, "packed_forward: null argument");
  if (!ctx->pages || !ctx->page_table || !ctx->ctx_lens)
    return fail(DFLASH_E_INVAL, "packed_forward: null pointer in the context description");
  if (n_blocks < 1) return fail(DFLASH_E_INVAL, "packed_forward: n_blocks must be >= 1");
  if (gamma < 1 || gamma > m->cfg.max_block)
    return fail(DFLASH_E_CAPACITY, "packed_forward: block_size %d outside [1, %d]", gamma,
                m->cfg.max_block);
  if (targets && (gamma < 2 || !(decay > 0.f)))
    return fail(DFLASH_E_INVAL, "packed_forward: the loss needs block_size >= 2 and decay > 0");
  if (!targets && (block_loss || loss))
    return fail(DFLASH_E_INVAL, "packed_forward: loss outputs without targets");
  if (ctx->n_pages < 1 || ctx->max_pages_per_seq < 1)
    return fail(DFLASH_E_INVAL, "packed_forward: empty page pool or page table");
  const PackedLayout L = packed_layout(m, n_blocks, gamma, ctx->max_pages_per_seq);
  if (L.total > ws_bytes)
    return fail(DFLASH_E_CAPACITY, "packed_forward: workspace %zu bytes < %zu needed", ws_bytes,
                L.total);
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  int32_t* table = (int32_t*)(ws + L.table);
  int32_t* lens = (int32_t*)(ws + L.lens);
  int32_t* toks = block_tokens ? block_tokens : (int32_t*)(ws + L.tokens);
  HIPCHK(launch_packed_setup(ctx->page_table, ctx->max_pages_per_seq, ctx->ctx_lens, anchor_pos,
                             n_blocks, table, lens, m->err, st));
  dflash_kv kv{};
  kv.pages = ctx->pages;
  kv.n_pages = ctx->n_pages;
  kv.max_pages_per_seq = ctx->max_pages_per_seq;
  kv.page_table = table;
  kv.ctx_lens = lens;
  int rc = draft_impl(m, &kv, anchors, n_blocks, gamma, toks, logits, workspace, L.draft, stream,
                      DrawArgs{});
  if (rc != DFLASH_OK) return rc;
  if (targets)
    HIPCHK(launch_block_loss(logits, targets, n_blocks, gamma, m->cfg.vocab, (double)decay,
                             (double*)(ws + L.ce), block_loss, loss, m->err, st));
  return DFLASH_OK;
}

size_t dflash_verify_greedy_workspace_bytes(int32_t batch, int32_t gamma, int32_t vocab) {
  if (batch < 1 || gamma < 1 || gamma > kVerifyMaxBlock || vocab < 1) return 0;
  return verify_greedy_workspace(batch, gamma, vocab);
}

size_t dflash_verify_stochastic_workspace_bytes(int32_t batch, int32_t gamma, int32_t vocab) {
  if (batch < 1 || gamma < 1 || vocab < 1) return 0;
  return verify_sampled_ws_bytes(batch, gamma, vocab);
}

int dflash_verify_stochastic(const int32_t* block_tokens, const float* draft_logits,
                             const void* target_logits, int32_t logits_dtype,
                             const float* uniforms, int32_t batch, int32_t gamma, int32_t vocab,
                             int32_t* accept_len, int32_t* out_tokens, void* workspace,
                             size_t ws_bytes, void* stream) {
  if (!block_tokens || !draft_logits || !target_logits || !uniforms || !accept_len ||
      !out_tokens || !workspace)
    return fail(DFLASH_E_INVAL, "verify_stochastic: null argument");
  if (logits_dtype != DFLASH_F32 && logits_dtype != DFLASH_BF16)
    return fail(DFLASH_E_DTYPE, "verify_stochastic: unknown logits dtype %d", logits_dtype);
  if (batch < 1 || gamma < 1 || vocab < 1)
    return fail(DFLASH_E_INVAL, "verify_stochastic: batch, block_size and vocab must be >= 1");
  if (gamma > kMaxVerifyBlock || (int64_t)batch * gamma > 65535)
    return fail(DFLASH_E_CAPACITY,
                "verify_stochastic: block_size %d > %d or batch * block_size > 65535", gamma,
                kMaxVerifyBlock);
  if (((uintptr_t)workspace & 15) != 0)
    return fail(DFLASH_E_INVAL, "verify_stochastic: workspace must be 16-byte aligned");
  const size_t need = verify_sampled_ws_bytes(batch, gamma, vocab);
  if (ws_bytes < need)
    return fail(DFLASH_E_CAPACITY, "verify_stochastic: workspace %zu bytes < %zu needed",
                ws_bytes, need);
  HIPCHK(launch_verify_sampled(logits_dtype == DFLASH_BF16, block_tokens, target_logits,
                               draft_logits, uniforms, batch, gamma, vocab, workspace,
                               accept_len, out_tokens, (hipStream_t)stream));
  return DFLASH_OK;
}

int dflash_device_error(const dflash_model* m, void* stream, int32_t* code) {
  if (!m || !code) return fail(DFLASH_E_INVAL, "device_error: null argument");
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(hipStreamSynchronize(st));
  uint32_t v = 0;
  HIPCHK(hipMemcpy(&v, m->err, sizeof v, hipMemcpyDeviceToHost));
  *code = (int32_t)v;
  if (v) {
    HIPCHK(launch_clear_word(m->err, st));
    HIPCHK(hipStreamSynchronize(st));
    return fail(DFLASH_E_DEVICE, "device error word 0x%x", v);
  }
  return DFLASH_OK;
}

int dflash_read_calibration(const void* src, size_t bytes, void* out, int32_t workgroups,
                            void* stream) {
  if (!src || !out) return fail(DFLASH_E_INVAL, "read_calibration: null argument");
  if (bytes == 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > 65535)
    return fail(DFLASH_E_INVAL, "read_calibration: bytes must be a positive multiple of 16 and "
                                "workgroups in [1, 65535]");
  HIPCHK(launch_read_calibration(src, bytes, out, workgroups, (hipStream_t)stream));
  return DFLASH_OK;
}

int dflash_profile_enable(dflash_model* m, int32_t on) {
  if (!m) return fail(DFLASH_E_INVAL, "profile_enable: null model");
  // Create the event pairs up front, so timed draft calls only record them.
  while (on && m->pool.size() + m->pending.size() < kProfPool) {
    std::pair<hipEvent_t, hipEvent_t> ev{nullptr, nullptr};
    HIPCHK(hipEventCreate(&ev.first));
    if (hipEventCreate(&ev.second) != hipSuccess) {
      (void)hipEventDestroy(ev.first);
      return fail(DFLASH_E_HIP, "profile_enable: hipEventCreate failed");
    }
    m->pool.push_back(ev);
  }
  m->prof_on = on != 0;
  return DFLASH_OK;
}

int dflash_profile_read(dflash_model* m, double* total_ms, int64_t* count, int32_t reset) {
  if (!m || !total_ms || !count) return fail(DFLASH_E_INVAL, "profile_read: null argument");
  for (auto& p : m->pending) {
    HIPCHK(hipEventSynchronize(p.second));
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, p.first, p.second));
    m->prof_ms += ms;
    m->prof_count += 1;
    m->pool.push_back(p);
  }
  m->pending.clear();
  *total_ms = m->prof_ms;
  *count = m->prof_count;
  if (reset) {
    m->prof_ms = 0.0;
    m->prof_count = 0;
  }
  return DFLASH_OK;
}

}  // extern "C"
