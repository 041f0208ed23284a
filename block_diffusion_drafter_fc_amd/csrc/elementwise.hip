// elementwise.hip -- row and element kernels around the dense products:
// embedding gather, RMSNorm, residual update, rotary embedding of q/k,
// SwiGLU, the draft argmax finaliser, context-injection scatter into the
// paged cache, and greedy verification.
//
// Split-K partial slices are always summed in slice order, so every result
// is deterministic.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kRowThreads = 256;

// Row r = b*gamma + j of the block: token (j == 0 ? anchor[b] : mask), its
// embedding into the fp32 residual x, and either y = RMSNorm(x) * g (the
// first layer's attention norm) or, when ss is given, only the row's sum of
// squares ss[r] (the next product normalises while staging x).  1024
// threads, 4 columns per thread per pass.
template <bool BF16>
__global__ __launch_bounds__(1024) void k_embed(const int32_t* __restrict__ anchor,
                                                int gamma, int mask_id, int vocab,
                                                const typename Act<BF16>::T* __restrict__ E,
                                                int D, float* __restrict__ x,
                                                const typename Act<BF16>::T* __restrict__ g,
                                                float eps, void* __restrict__ y,
                                                size_t y_plane, float* __restrict__ ss_out,
                                                float* __restrict__ rope,
                                                const int32_t* __restrict__ ctx_lens, int dh,
                                                float theta, uint32_t* err,
                                                const int32_t* __restrict__ tokens,
                                                int tok_stride) {
  __shared__ float red[16];
  const int r = blockIdx.x, b = r / gamma, j = r % gamma;
  int tok = tokens != nullptr ? tokens[(size_t)b * tok_stride + j] : (j == 0 ? anchor[b] : mask_id);
  if (tok < 0 || tok >= vocab) {
    if (threadIdx.x == 0) set_dev_error(err, 4u);
    tok = 0;
  }
  // four elements per thread and pass, loaded unconditionally (a clamped
  // column, D % 4 == 0) and selected afterwards: a predicated load here
  // becomes a branch that waits for each load in turn
  float v[2][4];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int d = (p * 1024 + threadIdx.x) * 4;
    const size_t src = (size_t)tok * D + (d < D ? d : 0);
    float t[4];
    if (BF16) {
      const uint2 raw = *(const uint2*)((const uint16_t*)E + src);
      t[0] = __uint_as_float(raw.x << 16);
      t[1] = __uint_as_float(raw.x & 0xFFFF0000u);
      t[2] = __uint_as_float(raw.y << 16);
      t[3] = __uint_as_float(raw.y & 0xFFFF0000u);
    } else {
      const f32x4 raw = *(const f32x4*)((const float*)E + src);
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = raw[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[p][e] = d < D ? t[e] : 0.f;
  }
  // the RoPE angles (fp64) while the embedding row is in flight
  if (rope != nullptr && (int)threadIdx.x < dh / 2) {
    float cs, sn;
    rope_cs(ctx_lens[b] + j, threadIdx.x, dh, (double)theta, &cs, &sn);
    rope[((size_t)r * (dh / 2) + threadIdx.x) * 2] = cs;
    rope[((size_t)r * (dh / 2) + threadIdx.x) * 2 + 1] = sn;
  }
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int d = (p * 1024 + threadIdx.x) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += v[p][e] * v[p][e];
    if (d < D) *(f32x4*)&x[(size_t)r * D + d] = f32x4{v[p][0], v[p][1], v[p][2], v[p][3]};
  }
  ss = block_sum(ss, red);
  if (ss_out != nullptr) {
    if (threadIdx.x == 0) ss_out[r] = ss;
    return;
  }
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int d = (p * 1024 + threadIdx.x) * 4;
    if (d < D)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Split<BF16>::store(y, y_plane, (size_t)r * D + d + e, v[p][e] * inv * Act<BF16>::load(g, d + e));
  }
}

template <bool BF16>
__global__ __launch_bounds__(kRowThreads) void k_rmsnorm(const float* __restrict__ x, int D,
                                                         const typename Act<BF16>::T* __restrict__ g,
                                                         float eps, void* __restrict__ y,
                                                         size_t y_plane) {
  __shared__ float red[16];
  const float* xr = x + (size_t)blockIdx.x * D;
  float ss = 0.f;
  for (int d = threadIdx.x; d < D; d += blockDim.x) ss = fmaf(xr[d], xr[d], ss);
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
  for (int d = threadIdx.x; d < D; d += blockDim.x)
    Split<BF16>::store(y, y_plane, (size_t)blockIdx.x * D + d, xr[d] * inv * Act<BF16>::load(g, d));
}

// x[r] += sum_s part[s][r]; then y[r] = RMSNorm(x[r]) * g.  One workgroup of
// 1024 threads per row, 4 consecutive columns per thread per pass; the loads
// of all partial slices are independent, so they are in flight together.
constexpr int kResThreads = 1024;
constexpr int kResMaxPass = 2;   // D <= 8192

// Four consecutive values (element i, a multiple of 4) to split planes
// (bf16 models: hi and lo, one 8-byte store each) or fp32 (one 16-byte store).
template <bool BF16>
DF_DEV void store4(void* base, size_t plane, size_t i, const f32x4& v) {
  if (BF16) {
    uint32_t h[2], l[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      h[e] = pack_bf2(v[2 * e], v[2 * e + 1]);
      l[e] = pack_bf2(v[2 * e] - __uint_as_float(h[e] << 16),
                      v[2 * e + 1] - __uint_as_float(h[e] & 0xFFFF0000u));
    }
    uint16_t* hi = (uint16_t*)base;
    *(uint2*)&hi[i] = make_uint2(h[0], h[1]);
    *(uint2*)&hi[plane + i] = make_uint2(l[0], l[1]);
  } else {
    *(f32x4*)&((float*)base)[i] = v;
  }
}

// Four consecutive gains as fp32 (one 8-byte load for bf16 gains).
template <bool BF16>
DF_DEV f32x4 load_gain4(const typename Act<BF16>::T* g, int d) {
  if (BF16) {
    const uint2 w = *(const uint2*)((const uint16_t*)g + d);
    return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
  }
  return *(const f32x4*)((const float*)g + d);
}

template <bool BF16>
__global__ __launch_bounds__(kResThreads) void k_residual_norm(float* __restrict__ x,
                                                               const float* __restrict__ part,
                                                               int splits, int M, int D,
                                                               const typename Act<BF16>::T* __restrict__ g,
                                                               float eps, void* __restrict__ y,
                                                               size_t y_plane) {
  __shared__ float red[16];
  const int r = blockIdx.x;
  float* xr = x + (size_t)r * D;
  // the residual and the gains (needed only after the row sum) load first,
  // at clamped in-bounds columns, so the wait for the partial slices that
  // follow covers them too
  f32x4 xv[kResMaxPass], gv[kResMaxPass];
#pragma unroll
  for (int p = 0; p < kResMaxPass; ++p) {
    const int d = (p * kResThreads + threadIdx.x) * 4, dc = d < D ? d : 0;
    xv[p] = *(const f32x4*)&xr[dc];
    gv[p] = load_gain4<BF16>(g, dc);
  }
  f32x4 v[kResMaxPass];
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < kResMaxPass; ++p) {
    const int d = (p * kResThreads + threadIdx.x) * 4;
    v[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (d < D) {
      f32x4 add = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int s = 0; s < splits; ++s) add += *(const f32x4*)&part[((size_t)s * M + r) * D + d];
      v[p] = xv[p] + add;
      *(f32x4*)&xr[d] = v[p];
      ss += v[p][0] * v[p][0] + v[p][1] * v[p][1] + v[p][2] * v[p][2] + v[p][3] * v[p][3];
    }
  }
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int p = 0; p < kResMaxPass; ++p) {
    const int d = (p * kResThreads + threadIdx.x) * 4;
    if (d < D) {
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = v[p][e] * inv * gv[p][e];
      store4<BF16>(y, y_plane, (size_t)r * D + d, o);
    }
  }
}

// Sum the QKV partials, rotate q and k (rotate-half form) with row r's
// (cos, sin) pairs from the call's RoPE table (positions ctx_lens[b] + j,
// angles evaluated once per call by the embedding kernel), store q
// [M][Hq][dh] (split planes for bf16 models) and the block's k and v
// [M][Hkv][dh] in fp32.
template <bool BF16>
__global__ void k_qkv_epilogue(const float* __restrict__ part, int splits, int M, int Hq,
                               int Hkv, int dh, const float* __restrict__ rope,
                               void* __restrict__ q, size_t q_plane, float* __restrict__ k,
                               float* __restrict__ v) {
  const int r = blockIdx.x, hh = blockIdx.y, i = threadIdx.x, half = dh / 2;
  const int N = (Hq + 2 * Hkv) * dh;
  (void)M;
  const int col = hh * dh + i;
  float a = 0.f, c2 = 0.f;
#pragma unroll 8
  for (int s = 0; s < splits; ++s) {
    a += part[((size_t)s * M + r) * N + col];
    c2 += part[((size_t)s * M + r) * N + col + half];
  }
  if (hh < Hq + Hkv) {
    const float2 t = ((const float2*)rope)[(size_t)r * half + i];
    const float cs = t.x, sn = t.y;
    const float a2 = a * cs - c2 * sn, b2 = c2 * cs + a * sn;
    a = a2;
    c2 = b2;
  }
  if (hh < Hq) {
    const size_t base = ((size_t)r * Hq + hh) * dh;
    Split<BF16>::store(q, q_plane, base + i, a);
    Split<BF16>::store(q, q_plane, base + i + half, c2);
  } else {
    float* dst = hh < Hq + Hkv ? k : v;
    const size_t base = ((size_t)r * Hkv + (hh < Hq + Hkv ? hh - Hq : hh - Hq - Hkv)) * dh;
    dst[base + i] = a;
    dst[base + i + half] = c2;
  }
}

// h = silu(gate) * up, gate = columns [0, I), up = columns [I, 2I).  VEC
// (I % 4 == 0): four columns per thread, 16-byte loads, one store per plane.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void k_swiglu(const float* __restrict__ part, int splits, int M,
                                                int I, void* __restrict__ h, size_t h_plane) {
  constexpr int C = VEC ? 4 : 1;
  const int r = blockIdx.y, c = (blockIdx.x * blockDim.x + threadIdx.x) * C;
  if (c >= I) return;
  f32x4 gt = {0.f, 0.f, 0.f, 0.f}, up = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int s = 0; s < splits; ++s) {
    const float* p = part + ((size_t)s * M + r) * (2 * (size_t)I);
    if (VEC) {
      gt += *(const f32x4*)&p[c];
      up += *(const f32x4*)&p[I + c];
    } else {
      gt[0] += p[c];
      up[0] += p[I + c];
    }
  }
  f32x4 o;
#pragma unroll
  for (int e = 0; e < C; ++e) o[e] = gt[e] / (1.0f + expf(-gt[e])) * up[e];
  if (VEC) store4<BF16>(h, h_plane, (size_t)r * I + c, o);
  else Split<BF16>::store(h, h_plane, (size_t)r * I + c, o[0]);
}

// Row r of the block: the anchor for j == 0, else the column of the largest
// argmax key of row r over the GEMM's column groups (keys[g][r]).
__global__ __launch_bounds__(256) void k_argmax_finalize(const uint64_t* __restrict__ keys,
                                                         int groups, int M,
                                                         const int32_t* __restrict__ anchor,
                                                         int gamma,
                                                         int32_t* __restrict__ block_tokens) {
  __shared__ uint64_t redk[4];
  const int r = blockIdx.x;
  uint64_t key = 0;
  for (int g = threadIdx.x; g < groups; g += blockDim.x) {
    const uint64_t k2 = keys[(size_t)g * M + r];
    key = k2 > key ? k2 : key;
  }
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = shfl_xor_u64(key, m);
    key = o > key ? o : key;
  }
  if ((threadIdx.x & 63) == 0) redk[threadIdx.x >> 6] = key;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) key = redk[w] > key ? redk[w] : key;
    const int j = r % gamma;
    block_tokens[r] = j == 0 && anchor ? anchor[r / gamma] : (int32_t)argmax_key_index(key);
  }
}

// c = RMSNorm(sum_s part[s]) * g   (the fused context H_t of each new token).
// Same shape of work as k_residual_norm: 1024 threads per token, 4 columns
// per thread per pass, all partial loads in flight together.
template <bool BF16>
__global__ __launch_bounds__(kResThreads) void k_inject_norm(const float* __restrict__ part,
                                                             int splits, int n, int D,
                                                             const typename Act<BF16>::T* __restrict__ g,
                                                             float eps, void* __restrict__ c) {
  __shared__ float red[16];
  const int t = blockIdx.x;
  f32x4 gv[kResMaxPass];   // loaded first: the slices' wait covers them
#pragma unroll
  for (int p = 0; p < kResMaxPass; ++p) {
    const int d = (p * kResThreads + threadIdx.x) * 4;
    gv[p] = load_gain4<BF16>(g, d < D ? d : 0);
  }
  f32x4 v[kResMaxPass];
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < kResMaxPass; ++p) {
    const int d = (p * kResThreads + threadIdx.x) * 4;
    v[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (d < D) {
#pragma unroll 8
      for (int s = 0; s < splits; ++s) v[p] += *(const f32x4*)&part[((size_t)s * n + t) * D + d];
      ss += v[p][0] * v[p][0] + v[p][1] * v[p][1] + v[p][2] * v[p][2] + v[p][3] * v[p][3];
    }
  }
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int p = 0; p < kResMaxPass; ++p) {
    const int d = (p * kResThreads + threadIdx.x) * 4;
    if (d < D) {
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = v[p][e] * inv * gv[p][e];
      if (BF16)   // c is held in the model dtype: one rounded bf16 plane
        *(uint2*)&((uint16_t*)c)[(size_t)t * D + d] = make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
      else
        *(f32x4*)&((float*)c)[(size_t)t * D + d] = o;
    }
  }
}

// Token t of the inject batch belongs to sequence b with cu_new[b] <= t <
// cu_new[b+1]; its position is ctx_lens[b] + (t - cu_new[b]).  Columns of
// the partial product are [K^0 | V^0 | K^1 | V^1 | ...], each Hkv*dh wide.
template <bool BF16>
__global__ void k_inject_scatter(const float* __restrict__ part, int splits, int n_tok,
                                 const int32_t* __restrict__ cu_new, int batch,
                                 const int32_t* __restrict__ ctx_lens,
                                 const int32_t* __restrict__ page_table, int max_pages,
                                 int n_pages, int page_size, typename Act<BF16>::T* __restrict__ pages,
                                 int n_layers, int Hkv, int dh, float theta, uint32_t* err) {
  const int t = blockIdx.x, y = blockIdx.y, i = threadIdx.x, half = dh / 2;
  const int kvh = y % Hkv, kv = (y / Hkv) % 2, layer = y / (2 * Hkv);
  int lo = 0, hi = batch;   // find b with cu_new[b] <= t < cu_new[b+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (cu_new[mid] <= t) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int pos = ctx_lens[b] + (t - cu_new[b]);
  const int pi = pos / page_size;
  if (pos < 0 || pi >= max_pages) {
    if (i == 0) set_dev_error(err, 2u);
    return;
  }
  const int pg = page_table[(size_t)b * max_pages + pi];
  if (pg < 0 || pg >= n_pages) {
    if (i == 0) set_dev_error(err, 1u);
    return;
  }
  const size_t N = (size_t)n_layers * 2 * Hkv * dh;
  const size_t col = (size_t)y * dh + i;
  float a = 0.f, c2 = 0.f;
#pragma unroll 8
  for (int s = 0; s < splits; ++s) {
    a += part[((size_t)s * n_tok + t) * N + col];
    c2 += part[((size_t)s * n_tok + t) * N + col + half];
  }
  if (kv == 0) {
    float cs, sn;
    rope_cs(pos, i, dh, (double)theta, &cs, &sn);
    const float a2 = a * cs - c2 * sn, b2 = c2 * cs + a * sn;
    a = a2;
    c2 = b2;
  }
  // K rows are [page_size][dh], values transposed [dh][page_size]
  const size_t page = ((((size_t)layer * n_pages + pg) * 2 + kv) * Hkv + kvh) * page_size * dh;
  const int slot = pos % page_size;
  if (kv == 0) {
    Act<BF16>::store(pages, page + (size_t)slot * dh + i, a);
    Act<BF16>::store(pages, page + (size_t)slot * dh + i + half, c2);
  } else {
    Act<BF16>::store(pages, page + (size_t)i * page_size + slot, a);
    Act<BF16>::store(pages, page + (size_t)(i + half) * page_size + slot, c2);
  }
}

__global__ void k_advance_ctx(int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ cu_new,
                              int batch) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) ctx_lens[b] += cu_new[b + 1] - cu_new[b];
}

__global__ void k_clear_word(uint32_t* w) { *w = 0u; }

// Row argmax of the target scores: workgroup (chunk, row) scans `chunk`
// columns with 16-byte loads and stores its key to best[row][chunk] (every
// slot is written on every call, so nothing needs clearing first).
template <bool BF16>
__global__ __launch_bounds__(256) void k_verify_argmax(const void* __restrict__ target, int vocab,
                                                       int chunk, uint64_t* __restrict__ best) {
  __shared__ uint64_t redk[4];
  const int row = blockIdx.y;
  const int c0 = blockIdx.x * chunk, c1 = min(vocab, c0 + chunk);
  uint64_t key = 0;
  // (vector paths: PU loads per thread are issued before any is used, at
  // clamped in-bounds columns whose keys are then skipped, so a thread waits
  // for memory once per PU loads rather than once per load)
  constexpr int PU = 4;
  if (BF16) {
    const uint16_t* p = (const uint16_t*)target + (size_t)row * vocab;
    if ((vocab & 7) == 0) {
      const int step = blockDim.x * 8;
      for (int c = c0 + threadIdx.x * 8; c < c1; c += step * PU) {
        u32x4 vs[PU];
#pragma unroll
        for (int u = 0; u < PU; ++u) vs[u] = ld16(p + min(c + u * step, c1 - 8));
#pragma unroll
        for (int u = 0; u < PU; ++u) {
          const int cu = c + u * step;
          if (cu >= c1) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint64_t k0 =
                argmax_key(bf2f((uint16_t)(vs[u][e] & 0xFFFFu)), (uint32_t)(cu + 2 * e));
            const uint64_t k1 =
                argmax_key(bf2f((uint16_t)(vs[u][e] >> 16)), (uint32_t)(cu + 2 * e + 1));
            key = k0 > key ? k0 : key;
            key = k1 > key ? k1 : key;
          }
        }
      }
    } else {
      for (int c = c0 + threadIdx.x; c < c1; c += blockDim.x) {
        const uint64_t k0 = argmax_key(bf2f(p[c]), (uint32_t)c);
        key = k0 > key ? k0 : key;
      }
    }
  } else {
    const float* p = (const float*)target + (size_t)row * vocab;
    if ((vocab & 3) == 0) {
      const int step = blockDim.x * 4;
      for (int c = c0 + threadIdx.x * 4; c < c1; c += step * PU) {
        u32x4 vs[PU];
#pragma unroll
        for (int u = 0; u < PU; ++u) vs[u] = ld16(p + min(c + u * step, c1 - 4));
#pragma unroll
        for (int u = 0; u < PU; ++u) {
          const int cu = c + u * step;
          if (cu >= c1) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint64_t k0 = argmax_key(__uint_as_float(vs[u][e]), (uint32_t)(cu + e));
            key = k0 > key ? k0 : key;
          }
        }
      }
    } else {
      for (int c = c0 + threadIdx.x; c < c1; c += blockDim.x) {
        const uint64_t k0 = argmax_key(p[c], (uint32_t)c);
        key = k0 > key ? k0 : key;
      }
    }
  }
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = shfl_xor_u64(key, m);
    key = o > key ? o : key;
  }
  if ((threadIdx.x & 63) == 0) redk[threadIdx.x >> 6] = key;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) key = redk[w] > key ? redk[w] : key;
    best[(size_t)row * gridDim.x + blockIdx.x] = key;
  }
}

// tau = n + 1 with n the longest prefix where block[j] == T_{j-1}.
// Workgroup b: thread j takes row j's maximum over its chunk keys, then the
// first mismatch is the minimum over the rows that break the prefix.
__global__ __launch_bounds__(256) void k_verify_finalize(
    const uint64_t* __restrict__ best, int nchunk, const int32_t* __restrict__ block_tokens,
    int gamma, int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ target_argmax) {
  __shared__ int n_s;
  __shared__ int32_t T_s[kVerifyMaxBlock];
  const int b = blockIdx.x;
  const int32_t* blk = block_tokens + (size_t)b * gamma;
  if (threadIdx.x == 0) n_s = gamma - 1;
  for (int j = threadIdx.x; j < gamma; j += blockDim.x) {
    const uint64_t* bk = best + ((size_t)b * gamma + j) * nchunk;
    uint64_t key = 0;
    for (int c = 0; c < nchunk; c += 8) {   // 8 loads in flight (clamped repeats are harmless)
      uint64_t k8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) k8[u] = bk[min(c + u, nchunk - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) key = k8[u] > key ? k8[u] : key;
    }
    T_s[j] = (int32_t)argmax_key_index(key);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < gamma - 1; j += blockDim.x)
    if (blk[j + 1] != T_s[j]) atomicMin(&n_s, j);
  __syncthreads();
  const int n = n_s;
  if (threadIdx.x == 0) accept_len[b] = n + 1;
  int32_t* out = out_tokens + (size_t)b * gamma;
  for (int j = threadIdx.x; j < gamma; j += blockDim.x) {
    out[j] = j < n ? blk[j + 1] : (j == n ? T_s[j] : -1);
    if (target_argmax) target_argmax[(size_t)b * gamma + j] = T_s[j];
  }
}

}  // namespace

hipError_t launch_embed(bool bf16, const int32_t* anchor, int batch, int gamma, int mask_id,
                        int vocab, const void* embed, int D, float* x, const void* g, float eps,
                        void* y, size_t y_plane, float* ss, float* rope, const int32_t* ctx_lens,
                        int dh, float theta, uint32_t* err, hipStream_t st,
                        const int32_t* tokens, int tok_stride) {
  dim3 grid(batch * gamma);
  if (D % 4 != 0 || D > 8192 || dh > 2048) return hipErrorInvalidValue;
  if (rope != nullptr && ctx_lens == nullptr) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(k_embed<true>, grid, dim3(1024), 0, st, anchor, gamma, mask_id,
                       vocab, (const uint16_t*)embed, D, x, (const uint16_t*)g, eps, y, y_plane,
                       ss, rope, ctx_lens, dh, theta, err, tokens, tok_stride);
  else
    hipLaunchKernelGGL(k_embed<false>, grid, dim3(1024), 0, st, anchor, gamma, mask_id,
                       vocab, (const float*)embed, D, x, (const float*)g, eps, y, y_plane, ss,
                       rope, ctx_lens, dh, theta, err, tokens, tok_stride);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(bool bf16, const float* x, int M, int D, const void* g, float eps,
                          void* y, size_t y_plane, hipStream_t st) {
  if (bf16)
    hipLaunchKernelGGL(k_rmsnorm<true>, dim3(M), dim3(kRowThreads), 0, st, x, D,
                       (const uint16_t*)g, eps, y, y_plane);
  else
    hipLaunchKernelGGL(k_rmsnorm<false>, dim3(M), dim3(kRowThreads), 0, st, x, D,
                       (const float*)g, eps, y, y_plane);
  return hipGetLastError();
}

hipError_t launch_residual_norm(bool bf16, float* x, const float* part, int splits, int M, int D,
                                const void* g, float eps, void* y, size_t y_plane,
                                hipStream_t st) {
  if (D % 4 != 0 || D > kResThreads * 4 * kResMaxPass) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(k_residual_norm<true>, dim3(M), dim3(kResThreads), 0, st, x, part, splits,
                       M, D, (const uint16_t*)g, eps, y, y_plane);
  else
    hipLaunchKernelGGL(k_residual_norm<false>, dim3(M), dim3(kResThreads), 0, st, x, part, splits,
                       M, D, (const float*)g, eps, y, y_plane);
  return hipGetLastError();
}

hipError_t launch_qkv_epilogue(bool bf16, const float* part, int splits, int M, int Hq,
                               int Hkv, int dh, const float* rope, void* q, size_t q_plane,
                               float* k, float* v, hipStream_t st) {
  dim3 grid(M, Hq + 2 * Hkv);
  dim3 block(dh / 2);
  if (bf16)
    hipLaunchKernelGGL(k_qkv_epilogue<true>, grid, block, 0, st, part, splits, M, Hq, Hkv, dh,
                       rope, q, q_plane, k, v);
  else
    hipLaunchKernelGGL(k_qkv_epilogue<false>, grid, block, 0, st, part, splits, M, Hq, Hkv, dh,
                       rope, q, q_plane, k, v);
  return hipGetLastError();
}

hipError_t launch_swiglu(bool bf16, const float* part, int splits, int M, int I, void* h,
                         size_t h_plane, hipStream_t st) {
  const bool vec = I % 4 == 0 && h_plane % 4 == 0;
  dim3 grid((I / (vec ? 4 : 1) + 255) / 256, M);
  if (bf16 && vec)
    hipLaunchKernelGGL((k_swiglu<true, true>), grid, dim3(256), 0, st, part, splits, M, I, h, h_plane);
  else if (bf16)
    hipLaunchKernelGGL((k_swiglu<true, false>), grid, dim3(256), 0, st, part, splits, M, I, h, h_plane);
  else if (vec)
    hipLaunchKernelGGL((k_swiglu<false, true>), grid, dim3(256), 0, st, part, splits, M, I, h, h_plane);
  else
    hipLaunchKernelGGL((k_swiglu<false, false>), grid, dim3(256), 0, st, part, splits, M, I, h, h_plane);
  return hipGetLastError();
}

hipError_t launch_argmax_finalize(const uint64_t* best, int groups, const int32_t* anchor,
                                  int batch, int gamma, int32_t* block_tokens, hipStream_t st) {
  const int M = batch * gamma;
  hipLaunchKernelGGL(k_argmax_finalize, dim3(M), dim3(256), 0, st, best, groups, M, anchor, gamma,
                     block_tokens);
  return hipGetLastError();
}

hipError_t launch_inject_norm(bool bf16, const float* part, int splits, int n, int D, const void* g,
                              float eps, void* c, hipStream_t st) {
  if (D % 4 != 0 || D > kResThreads * 4 * kResMaxPass) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(k_inject_norm<true>, dim3(n), dim3(kResThreads), 0, st, part, splits, n, D,
                       (const uint16_t*)g, eps, c);
  else
    hipLaunchKernelGGL(k_inject_norm<false>, dim3(n), dim3(kResThreads), 0, st, part, splits, n,
                       D, (const float*)g, eps, c);
  return hipGetLastError();
}

hipError_t launch_inject_scatter(bool bf16, const float* part, int splits, int n_tok,
                                 const int32_t* cu_new, int batch, const int32_t* ctx_lens,
                                 const int32_t* page_table, int max_pages, int n_pages,
                                 int page_size, void* pages, int n_layers, int Hkv, int dh,
                                 float theta, uint32_t* err, hipStream_t st) {
  dim3 grid(n_tok, n_layers * 2 * Hkv);
  dim3 block(dh / 2);
  if (bf16)
    hipLaunchKernelGGL(k_inject_scatter<true>, grid, block, 0, st, part, splits, n_tok, cu_new,
                       batch, ctx_lens, page_table, max_pages, n_pages, page_size,
                       (uint16_t*)pages, n_layers, Hkv, dh, theta, err);
  else
    hipLaunchKernelGGL(k_inject_scatter<false>, grid, block, 0, st, part, splits, n_tok, cu_new,
                       batch, ctx_lens, page_table, max_pages, n_pages, page_size,
                       (float*)pages, n_layers, Hkv, dh, theta, err);
  return hipGetLastError();
}

hipError_t launch_advance_ctx(int32_t* ctx_lens, const int32_t* cu_new, int batch,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_advance_ctx, dim3((batch + 255) / 256), dim3(256), 0, st, ctx_lens, cu_new,
                     batch);
  return hipGetLastError();
}

size_t verify_greedy_workspace(int batch, int gamma, int vocab) {
  return (size_t)batch * gamma * ((vocab + kVerifyChunk - 1) / kVerifyChunk) * 8;
}

hipError_t launch_verify(bool bf16, const int32_t* block_tokens, const void* target, int batch,
                         int gamma, int vocab, uint64_t* best, int32_t* accept_len,
                         int32_t* out_tokens, int32_t* target_argmax, hipStream_t st) {
  if (gamma > kVerifyMaxBlock) return hipErrorInvalidValue;
  const int rows = batch * gamma;
  const int chunk = kVerifyChunk;
  const int nchunk = (vocab + chunk - 1) / chunk;
  dim3 grid(nchunk, rows);
  if (bf16)
    hipLaunchKernelGGL(k_verify_argmax<true>, grid, dim3(256), 0, st, target, vocab, chunk, best);
  else
    hipLaunchKernelGGL(k_verify_argmax<false>, grid, dim3(256), 0, st, target, vocab, chunk, best);
  hipLaunchKernelGGL(k_verify_finalize, dim3(batch), dim3(gamma < 256 ? 64 : 256), 0, st, best,
                     nchunk, block_tokens, gamma, accept_len, out_tokens, target_argmax);
  return hipGetLastError();
}

hipError_t launch_clear_word(uint32_t* word, hipStream_t st) {
  hipLaunchKernelGGL(k_clear_word, dim3(1), dim3(1), 0, st, word);
  return hipGetLastError();
}
