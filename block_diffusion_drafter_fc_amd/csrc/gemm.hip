// gemm.hip -- out = A[M][K] * W[N][K]^T for the drafter's dense products.
//
// Three kernels:
//   k_gemm_skinny  bf16, M <= 64 (the block rows of a few sequences).  The
//                  product is a stream of the weight matrix: each lane loads
//                  16 contiguous bytes of a weight row straight into the
//                  B operand of a 16x16x32 bf16 MFMA (no LDS round trip),
//                  the A operand (activations, L2-resident) is reused across
//                  NT column tiles, and K is split over the waves of a group
//                  (LDS reduction in fixed order) and over groups (fp32
//                  partial slices) so that thousands of waves keep HBM busy.
//   k_gemm_tiled   bf16, larger M: 128x128 output tiles, both operands staged
//                  through double-buffered LDS, 4 waves of 64x64.
// With SPLIT the activations arrive as two bf16 planes (hi, lo) of an fp32
// value and every weight fragment meets both: acc += hi*W + lo*W.
//   k_gemm_f32     fp32 models: one thread per output, plain K loop.
// All three can end in a fused row argmax (the LM head): the row maximum of
// the tile is packed with its column into a 64-bit key (value order, then
// lowest column) and merged with an integer atomic max, which is exact and
// independent of the order in which groups finish.
#include "common.h"
#include "kernels.h"

namespace {

DF_DEV const uint16_t* seg_row_bf16(const WSeg& w, int row, int K) {
  int s = 0;
  while (s < w.n - 1 && row >= w.row_end[s]) ++s;
  const int start = s ? w.row_end[s - 1] : 0;
  return (const uint16_t*)w.ptr[s] + (size_t)(row - start) * K;
}

DF_DEV const float* seg_row_f32(const WSeg& w, int row, int K) {
  int s = 0;
  while (s < w.n - 1 && row >= w.row_end[s]) ++s;
  const int start = s ? w.row_end[s - 1] : 0;
  return (const float*)w.ptr[s] + (size_t)(row - start) * K;
}

// Merge the argmax keys of the 16 lanes that share lane / 16.
DF_DEV uint64_t max16(uint64_t k) {
  for (int m = 1; m < 16; m <<= 1) {
    uint64_t o = shfl_xor_u64(k, m);
    k = o > k ? o : k;
  }
  return k;
}

// ----------------------------------------------------------------------------
template <int MT, int NT, int U, bool SPLIT>
__global__ __launch_bounds__(256) void k_gemm_skinny(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Alo, int lda, int M, WSeg w,
    int N, int K, int kpw, float* __restrict__ part, uint64_t* __restrict__ best,
    float* __restrict__ logits) {
  extern __shared__ float red[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, W = blockDim.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * (16 * NT);
  const int split = blockIdx.y;
  const int kbeg = (split * W + wave) * kpw;

  const uint16_t* bp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int row = n0 + t * 16 + lr;
    row = row < N ? row : N - 1;
    bp[t] = seg_row_bf16(w, row, K) + kbeg + lg * 8;
  }
  const uint16_t* ap[MT];
  const uint16_t* apl[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    int row = m * 16 + lr;
    row = row < M ? row : M - 1;
    ap[m] = A + (size_t)row * lda + kbeg + lg * 8;
    apl[m] = SPLIT ? Alo + (size_t)row * lda + kbeg + lg * 8 : ap[m];
  }

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int iters = kpw / (32 * U);
  u32x4 bcur[U][NT];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) bcur[u][t] = ld16(bp[t] + u * 32);

  for (int it = 0; it < iters; ++it) {
    const int kk = it * 32 * U;
    u32x4 bnxt[U][NT];
    if (it + 1 < iters) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) bnxt[u][t] = ld16(bp[t] + kk + 32 * U + u * 32);
    }
    u32x4 a[U][MT], al[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        a[u][m] = ld16(ap[m] + kk + u * 32);
        if (SPLIT) al[u][m] = ld16(apl[m] + kk + u * 32);
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[m][t] = mfma_16x16x32(a[u][m], bcur[u][t], acc[m][t]);
          if (SPLIT) acc[m][t] = mfma_16x16x32(al[u][m], bcur[u][t], acc[m][t]);
        }
    if (it + 1 < iters) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) bcur[u][t] = bnxt[u][t];
    }
  }

  // K split inside the group: waves 1..W-1 hand their sums to wave 0, which
  // adds them in wave order.
  constexpr int E = MT * NT * 4;
  if (W > 1) {
    if (wave > 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            red[((size_t)(wave - 1) * E + (m * NT + t) * 4 + i) * 64 + lane] = acc[m][t][i];
    }
    __syncthreads();
    if (wave == 0) {
      for (int w2 = 1; w2 < W; ++w2)
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[m][t][i] += red[((size_t)(w2 - 1) * E + (m * NT + t) * 4 + i) * 64 + lane];
    }
  }
  if (wave != 0) return;

  if (best == nullptr) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + lg * 4 + i;
        if (row >= M) continue;
        float* dst = part + ((size_t)split * M + row) * N;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int col = n0 + t * 16 + lr;
          if (col < N) dst[col] = acc[m][t][i];
        }
      }
    return;
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m * 16 + lg * 4 + i;
      uint64_t key = 0;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int col = n0 + t * 16 + lr;
        if (col < N) {
          const float v = acc[m][t][i];
          const uint64_t k2 = argmax_key(v, (uint32_t)col);
          key = k2 > key ? k2 : key;
          if (logits != nullptr && row < M) logits[(size_t)row * N + col] = v;
        }
      }
      key = max16(key);
      if (lr == 0 && row < M) atomicMax((unsigned long long*)&best[row], (unsigned long long)key);
    }
}

// ----------------------------------------------------------------------------
constexpr int TBM = 128, TBN = 128, TPAD = 8;

// BK = 64 without split, 32 with split (two A planes must fit LDS).
template <bool SPLIT, int TBK>
__global__ __launch_bounds__(256) void k_gemm_tiled(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Alo, int lda, int M, WSeg w,
    int N, int K, int kps, float* __restrict__ part, uint64_t* __restrict__ best,
    float* __restrict__ logits) {
  constexpr int NP = SPLIT ? 2 : 1;               // A planes
  constexpr int CPR = TBK / 8;                    // 16-byte chunks per tile row
  constexpr int NCH = TBM * CPR / 256;            // chunks per thread per operand
  __shared__ __attribute__((aligned(16))) uint16_t As[2][NP][TBM][TBK + TPAD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][TBN][TBK + TPAD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * TBM, n0 = blockIdx.x * TBN, split = blockIdx.z;
  const int kbeg = split * kps;

  // Each thread moves NCH chunks of 16 bytes of every A plane and of B per
  // K step.
  const uint16_t* ag[NCH];
  const uint16_t* agl[NCH];
  const uint16_t* bg[NCH];
  int lrow[NCH], lcol[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + i * 256;
    lrow[i] = c / CPR;
    lcol[i] = (c % CPR) * 8;
    int ar = m0 + lrow[i];
    ar = ar < M ? ar : M - 1;
    ag[i] = A + (size_t)ar * lda + kbeg + lcol[i];
    agl[i] = SPLIT ? Alo + (size_t)ar * lda + kbeg + lcol[i] : ag[i];
    int br = n0 + lrow[i];
    br = br < N ? br : N - 1;
    bg[i] = seg_row_bf16(w, br, K) + kbeg + lcol[i];
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[NCH], ral[NCH], rb[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    ra[i] = ld16(ag[i]);
    if (SPLIT) ral[i] = ld16(agl[i]);
    rb[i] = ld16(bg[i]);
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    st16(&As[0][0][lrow[i]][lcol[i]], ra[i]);
    if (SPLIT) st16(&As[0][NP - 1][lrow[i]][lcol[i]], ral[i]);
    st16(&Bs[0][lrow[i]][lcol[i]], rb[i]);
  }
  __syncthreads();

  const int steps = kps / TBK;
  for (int s = 0; s < steps; ++s) {
    const int cur = s & 1;
    if (s + 1 < steps) {
      const int ko = (s + 1) * TBK;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        ra[i] = ld16(ag[i] + ko);
        if (SPLIT) ral[i] = ld16(agl[i] + ko);
        rb[i] = ld16(bg[i] + ko);
      }
    }
#pragma unroll
    for (int ks = 0; ks < TBK / 32; ++ks) {
      u32x4 fb[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) fb[b] = ld16(&Bs[cur][wn * 64 + b * 16 + lr][ks * 32 + lg * 8]);
#pragma unroll
      for (int pl = 0; pl < NP; ++pl) {
        u32x4 fa[4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
          fa[a] = ld16(&As[cur][pl][wm * 64 + a * 16 + lr][ks * 32 + lg * 8]);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = mfma_16x16x32(fa[a], fb[b], acc[a][b]);
      }
    }
    if (s + 1 < steps) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        st16(&As[cur ^ 1][0][lrow[i]][lcol[i]], ra[i]);
        if (SPLIT) st16(&As[cur ^ 1][NP - 1][lrow[i]][lcol[i]], ral[i]);
        st16(&Bs[cur ^ 1][lrow[i]][lcol[i]], rb[i]);
      }
    }
    __syncthreads();
  }

  if (best == nullptr) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + wm * 64 + a * 16 + lg * 4 + i;
        if (row >= M) continue;
        float* dst = part + ((size_t)split * M + row) * N;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int col = n0 + wn * 64 + b * 16 + lr;
          if (col < N) dst[col] = acc[a][b][i];
        }
      }
    return;
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + wm * 64 + a * 16 + lg * 4 + i;
      uint64_t key = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int col = n0 + wn * 64 + b * 16 + lr;
        if (col < N) {
          const float v = acc[a][b][i];
          const uint64_t k2 = argmax_key(v, (uint32_t)col);
          key = k2 > key ? k2 : key;
          if (logits != nullptr && row < M) logits[(size_t)row * N + col] = v;
        }
      }
      key = max16(key);
      if (lr == 0 && row < M) atomicMax((unsigned long long*)&best[row], (unsigned long long)key);
    }
}

// ----------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_gemm_f32(const float* __restrict__ A, int lda, int M,
                                                 WSeg w, int N, int K, float* __restrict__ part,
                                                 uint64_t* __restrict__ best,
                                                 float* __restrict__ logits) {
  const int n = blockIdx.x * 64 + threadIdx.x, m = blockIdx.y;
  float acc = 0.f;
  if (n < N) {
    const float* wr = seg_row_f32(w, n, K);
    const float* ar = A + (size_t)m * lda;
    for (int k = 0; k < K; ++k) acc = fmaf(ar[k], wr[k], acc);
  }
  if (best == nullptr) {
    if (n < N) part[(size_t)m * N + n] = acc;
    return;
  }
  uint64_t key = n < N ? argmax_key(acc, (uint32_t)n) : 0;
  if (n < N && logits != nullptr) logits[(size_t)m * N + n] = acc;
  for (int s = 1; s < 64; s <<= 1) {
    uint64_t o = shfl_xor_u64(key, s);
    key = o > key ? o : key;
  }
  if (threadIdx.x == 0) atomicMax((unsigned long long*)&best[m], (unsigned long long)key);
}

template <int MT, int NT, int U>
hipError_t run_skinny(const GemmPlan& p, const void* A, const void* Alo, int lda, int M,
                      const WSeg& w, int N, int K, float* part, uint64_t* best, float* logits,
                      hipStream_t st) {
  dim3 grid((N + 16 * NT - 1) / (16 * NT), p.splits);
  dim3 block(64 * p.waves);
  size_t lds = p.waves > 1 ? (size_t)(p.waves - 1) * MT * NT * 4 * 64 * sizeof(float) : 0;
  if (Alo)
    hipLaunchKernelGGL((k_gemm_skinny<MT, NT, U, true>), grid, block, lds, st,
                       (const uint16_t*)A, (const uint16_t*)Alo, lda, M, w, N, K, p.kpw, part,
                       best, logits);
  else
    hipLaunchKernelGGL((k_gemm_skinny<MT, NT, U, false>), grid, block, lds, st,
                       (const uint16_t*)A, (const uint16_t*)nullptr, lda, M, w, N, K, p.kpw,
                       part, best, logits);
  return hipGetLastError();
}

int largest_divisor_at_most(int n, int cap) {
  for (int d = cap < n ? cap : n; d >= 1; --d)
    if (n % d == 0) return d;
  return 1;
}

}  // namespace

GemmPlan plan_gemm(bool bf16, int M, int N, int K, bool argmax) {
  GemmPlan p{};
  if (!bf16) {
    p.kind = GEMM_F32;
    p.splits = 1;
    p.waves = 1;
    p.kpw = K;
    return p;
  }
  if (M <= 64) {
    p.kind = GEMM_SKINNY;
    p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    p.nt = ((N / 16) % 2 == 0) ? 2 : 1;
    p.unroll = p.mt == 1 ? 8 : (p.mt == 2 ? 4 : 2);
    const int groups = (N + 16 * p.nt - 1) / (16 * p.nt);
    const int nk = K / (32 * p.unroll);   // loop iterations without any split
    // Split K until about 2048 waves are in flight, keeping >= 2 iterations
    // per wave.
    int T = 1;
    for (int t = 1; t <= nk; ++t) {
      if (nk % t) continue;
      if (nk / t < 2 && t > 1) break;
      if (argmax && t != 1 && t != 2 && t != 4) continue;   // argmax: one group per tile
      T = t;
      if ((long)groups * t >= 2048) break;
    }
    p.waves = T % 4 == 0 ? 4 : (T % 2 == 0 ? 2 : 1);
    p.splits = T / p.waves;
    p.kpw = K / T;
    return p;
  }
  p.kind = GEMM_TILED;
  p.waves = 4;
  const long tiles = (long)((M + TBM - 1) / TBM) * ((N + TBN - 1) / TBN);
  int splits = 1;
  if (!argmax && tiles < 512) {
    const int want = (int)((512 + tiles - 1) / tiles);
    splits = largest_divisor_at_most(K / 64, want < 8 ? want : 8);
  }
  p.splits = splits;
  p.kpw = K / splits;
  return p;
}

hipError_t launch_gemm(const GemmPlan& p, bool bf16, const void* A, const void* Alo, int lda,
                       int M, const WSeg& w, int N, int K, float* part, uint64_t* best,
                       float* logits, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (p.kind == GEMM_F32) {
    dim3 grid((N + 63) / 64, M);
    hipLaunchKernelGGL(k_gemm_f32, grid, dim3(64), 0, st, (const float*)A, lda, M, w, N, K, part,
                       best, logits);
    return hipGetLastError();
  }
  (void)bf16;
  if (p.kind == GEMM_TILED) {
    dim3 grid((N + TBN - 1) / TBN, (M + TBM - 1) / TBM, p.splits);
    if (Alo)
      hipLaunchKernelGGL((k_gemm_tiled<true, 32>), grid, dim3(256), 0, st, (const uint16_t*)A,
                         (const uint16_t*)Alo, lda, M, w, N, K, p.kpw, part, best, logits);
    else
      hipLaunchKernelGGL((k_gemm_tiled<false, 64>), grid, dim3(256), 0, st, (const uint16_t*)A,
                         (const uint16_t*)nullptr, lda, M, w, N, K, p.kpw, part, best, logits);
    return hipGetLastError();
  }
#define DF_SKINNY(MT, NT, U) \
  if (p.mt == MT && p.nt == NT) return run_skinny<MT, NT, U>(p, A, Alo, lda, M, w, N, K, part, best, logits, st)
  DF_SKINNY(1, 2, 8);
  DF_SKINNY(1, 1, 8);
  DF_SKINNY(2, 2, 4);
  DF_SKINNY(2, 1, 4);
  DF_SKINNY(4, 2, 2);
  DF_SKINNY(4, 1, 2);
#undef DF_SKINNY
  return hipErrorInvalidValue;
}
