// gemm.hip -- out = A[M][K] * W[N][K]^T for the drafter's dense products.
//
// Three kernels:
//   k_gemm_skinny  bf16, M <= 64 (the block rows of a few sequences).  The
//                  product is a stream of the weight matrix: each lane loads
//                  16 contiguous bytes of a weight row straight into the
//                  B operand of a 16x16x32 bf16 MFMA (no LDS round trip); the
//                  activations are staged once per workgroup in LDS and
//                  shared by its 4 waves; K is split over workgroups (fp32
//                  partial slices) so that about a thousand groups keep HBM
//                  busy.
//   k_gemm_tiled   bf16, larger M: 128x128 output tiles, both operands staged
//                  through double-buffered LDS, 4 waves of 64x64.
// With SPLIT the activations arrive as two bf16 planes (hi, lo) of an fp32
// value and every weight fragment meets both: acc += hi*W + lo*W.
//   k_gemm_f32     fp32 models: one thread per output, plain K loop.
// All three can end in a fused row argmax (the LM head): the row maximum of
// a group's columns is packed with its column into a 64-bit key (value
// order, then lowest column) and stored per (group, row); a small kernel
// takes the maximum key of each row over the groups, which is exact and
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
// Skinny product.  A workgroup of 4 waves owns 64*NT output columns and one
// K slice [kbeg, kbeg + kps).  The activations of the slice are staged in
// LDS in sub-chunks of KC = 32*U columns (both planes, double-buffered) and
// shared by the 4 waves; each wave streams its own 16*NT weight rows from HBM
// straight into MFMA B operands (lane (r, g) reads 16 contiguous bytes of
// row n0 + 16t + r at column k + 32u + 8g).  Keeping the activations out of
// the load queue matters: loads retire in order, so activation loads issued
// between weight loads would make every MFMA wait for the slowest stream.
template <int MT, int NT, int U, bool SPLIT, bool ARGMAX>
__global__ __launch_bounds__(256) void k_gemm_skinny(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Alo, int lda, int M, WSeg w,
    int N, int K, int kps, float* __restrict__ part, uint64_t* __restrict__ best,
    float* __restrict__ logits, DrawArgs dr) {
  constexpr int KC = 32 * U, NP = SPLIT ? 2 : 1, ROWS = 16 * MT;
  constexpr int CPR = KC / 8;              // 16-byte chunks per activation row
  constexpr int NCH = ROWS * CPR / 256;    // chunks per thread per plane
  static_assert(ROWS * CPR % 256 == 0, "sub-chunk must split evenly over 256 threads");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][NP][ROWS][KC + 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = (blockIdx.x * 4 + wave) * 16 * NT;
  const bool active = n0 < N;
  const int split = blockIdx.y;
  const int kbeg = split * kps;

  const uint16_t* bp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int row = n0 + t * 16 + lr;
    row = row < N ? row : N - 1;
    bp[t] = seg_row_bf16(w, row, K) + kbeg + lg * 8;
  }
  // activation chunks this thread stages: row r_i, column c_i of a sub-chunk
  const uint16_t* ag[NCH];
  int srow[NCH], scol[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + i * 256;
    srow[i] = c / CPR;
    scol[i] = (c % CPR) * 8;
    const int r = srow[i] < M ? srow[i] : M - 1;
    ag[i] = A + (size_t)r * lda + kbeg + scol[i];
  }
  const size_t lo_off = SPLIT ? (size_t)(Alo - A) : 0;

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Issue order per sub-chunk: the next activation chunk, then the next
  // weight batch.  Loads retire in order, so the LDS store of the
  // activations never waits for weights, and two weight batches per wave
  // (the one being multiplied and the next) are in flight.
  u32x4 ra0[NCH], ra1[NCH];
  u32x4 bc[U][NT], bn[U][NT];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    ra0[i] = ld16(ag[i]);
    if (SPLIT) ra1[i] = ld16(ag[i] + lo_off);
  }
  if (active) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < NT; ++t) bc[u][t] = ld16_stream(bp[t] + u * 32);
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    st16(&As[0][0][srow[i]][scol[i]], ra0[i]);
    if (SPLIT) st16(&As[0][NP - 1][srow[i]][scol[i]], ra1[i]);
  }
  __syncthreads();

  int buf = 0;
  for (int k = 0; k < kps; k += KC) {
    const bool more = k + KC < kps;
    if (more) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        ra0[i] = ld16(ag[i] + k + KC);
        if (SPLIT) ra1[i] = ld16(ag[i] + lo_off + k + KC);
      }
      if (active) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int t = 0; t < NT; ++t) bn[u][t] = ld16_stream(bp[t] + k + KC + u * 32);
      }
    }
    if (active) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4 a = ld16(&As[buf][0][m * 16 + lr][u * 32 + lg * 8]);
          u32x4 al;
          if (SPLIT) al = ld16(&As[buf][NP - 1][m * 16 + lr][u * 32 + lg * 8]);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            acc[m][t] = mfma_16x16x32(a, bc[u][t], acc[m][t]);
            if (SPLIT) acc[m][t] = mfma_16x16x32(al, bc[u][t], acc[m][t]);
          }
        }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        st16(&As[buf ^ 1][0][srow[i]][scol[i]], ra0[i]);
        if (SPLIT) st16(&As[buf ^ 1][NP - 1][srow[i]][scol[i]], ra1[i]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) bc[u][t] = bn[u][t];
    }
    __syncthreads();
    buf ^= 1;
  }

  if (!ARGMAX) {
    if (!active) return;
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
  // Row argmax of the group's 64*NT columns: per wave over its columns
  // (lanes, then tiles), then over the 4 waves in LDS; one key per
  // (group, row) goes to keys[blockIdx.x][row] -- no atomics.
  __shared__ uint64_t wkeys[4][ROWS];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m * 16 + lg * 4 + i;
      uint64_t key = 0;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int col = n0 + t * 16 + lr;
        if (active && col < N) {
          const float v = acc[m][t][i];
          const float kv = dr.on && row < M ? v + gumbel_noise(dr.seed, (uint32_t)(row / dr.gamma),
                                                               (uint32_t)(row % dr.gamma), (uint32_t)col)
                                            : v;
          const uint64_t k2 = argmax_key(kv, (uint32_t)col);
          key = k2 > key ? k2 : key;
          if (logits != nullptr && row < M) logits[(size_t)row * N + col] = v;
        }
      }
      key = max16(key);
      if (lr == 0) wkeys[wave][row] = key;
    }
  __syncthreads();
  if (tid < ROWS && tid < M) {
    uint64_t key = wkeys[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) key = wkeys[w][tid] > key ? wkeys[w][tid] : key;
    best[(size_t)blockIdx.x * M + tid] = key;
  }
}

// ----------------------------------------------------------------------------
constexpr int TBM = 128, TBN = 128, TPAD = 8;

// BK = 64 without split, 32 with split (two A planes must fit LDS).
template <bool SPLIT, int TBK, bool ARGMAX>
__global__ __launch_bounds__(256) void k_gemm_tiled(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Alo, int lda, int M, WSeg w,
    int N, int K, int kps, float* __restrict__ part, uint64_t* __restrict__ best,
    float* __restrict__ logits, DrawArgs dr) {
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

  if (!ARGMAX) {
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
  // Row argmax of the tile's 128 columns: per wave (lanes, then tiles), then
  // over the two column halves in LDS; keys[blockIdx.x][row], no atomics.
  __shared__ uint64_t hkeys[2][TBM];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rloc = wm * 64 + a * 16 + lg * 4 + i;
      const int row = m0 + rloc;
      uint64_t key = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int col = n0 + wn * 64 + b * 16 + lr;
        if (col < N) {
          const float v = acc[a][b][i];
          const float kv = dr.on && row < M ? v + gumbel_noise(dr.seed, (uint32_t)(row / dr.gamma),
                                                               (uint32_t)(row % dr.gamma), (uint32_t)col)
                                            : v;
          const uint64_t k2 = argmax_key(kv, (uint32_t)col);
          key = k2 > key ? k2 : key;
          if (logits != nullptr && row < M) logits[(size_t)row * N + col] = v;
        }
      }
      key = max16(key);
      if (lr == 0) hkeys[wn][rloc] = key;
    }
  __syncthreads();
  if (tid < TBM && m0 + tid < M) {
    const uint64_t k0 = hkeys[0][tid], k1 = hkeys[1][tid];
    best[(size_t)blockIdx.x * M + m0 + tid] = k0 > k1 ? k0 : k1;
  }
}

// ----------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_gemm_f32(const float* __restrict__ A, int lda, int M,
                                                 WSeg w, int N, int K, float* __restrict__ part,
                                                 uint64_t* __restrict__ best,
                                                 float* __restrict__ logits, DrawArgs dr) {
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
  const float kv = dr.on ? acc + gumbel_noise(dr.seed, (uint32_t)(m / dr.gamma), (uint32_t)(m % dr.gamma),
                                              (uint32_t)n)
                        : acc;
  uint64_t key = n < N ? argmax_key(kv, (uint32_t)n) : 0;
  if (n < N && logits != nullptr) logits[(size_t)m * N + n] = acc;
  for (int s = 1; s < 64; s <<= 1) {
    uint64_t o = shfl_xor_u64(key, s);
    key = o > key ? o : key;
  }
  if (threadIdx.x == 0) best[(size_t)blockIdx.x * M + m] = key;
}

template <int MT, int NT, int U>
hipError_t run_skinny(const GemmPlan& p, const void* A, const void* Alo, int lda, int M,
                      const WSeg& w, int N, int K, float* part, uint64_t* best, float* logits,
                      hipStream_t st, const DrawArgs& dr) {
  dim3 grid((N + 64 * NT - 1) / (64 * NT), p.splits);
  dim3 block(256);
  const uint16_t* a = (const uint16_t*)A;
  const uint16_t* al = (const uint16_t*)Alo;
  if (al && best)
    hipLaunchKernelGGL((k_gemm_skinny<MT, NT, U, true, true>), grid, block, 0, st, a, al, lda, M,
                       w, N, K, p.kpw, part, best, logits, dr);
  else if (al)
    hipLaunchKernelGGL((k_gemm_skinny<MT, NT, U, true, false>), grid, block, 0, st, a, al, lda, M,
                       w, N, K, p.kpw, part, best, logits, dr);
  else if (best)
    hipLaunchKernelGGL((k_gemm_skinny<MT, NT, U, false, true>), grid, block, 0, st, a, al, lda,
                       M, w, N, K, p.kpw, part, best, logits, dr);
  else
    hipLaunchKernelGGL((k_gemm_skinny<MT, NT, U, false, false>), grid, block, 0, st, a, al, lda,
                       M, w, N, K, p.kpw, part, best, logits, dr);
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
    p.nt = 1;
    p.unroll = 8 / p.mt;
    p.waves = 4;
    const int groups = (N + 64 * p.nt - 1) / (64 * p.nt);
    const int nk = K / (32 * p.unroll);   // activation sub-chunks along K
    // Split K across workgroups until about 1024 groups are in flight.
    int S = 1;
    if (!argmax) {
      for (int t = 1; t <= nk; ++t) {
        if (nk % t) continue;
        S = t;
        if ((long)groups * t >= 1024) break;
      }
    }
    p.splits = S;
    p.kpw = K / S;
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

int gemm_argmax_groups(const GemmPlan& p, int N) {
  if (p.kind == GEMM_F32) return (N + 63) / 64;
  if (p.kind == GEMM_TILED) return (N + TBN - 1) / TBN;
  return (N + 64 * p.nt - 1) / (64 * p.nt);
}

hipError_t launch_gemm(const GemmPlan& p, bool bf16, const void* A, const void* Alo, int lda,
                       int M, const WSeg& w, int N, int K, float* part, uint64_t* best,
                       float* logits, hipStream_t st, const DrawArgs& dr) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (dr.on && (best == nullptr || dr.gamma < 1)) return hipErrorInvalidValue;
  if (p.kind == GEMM_F32) {
    dim3 grid((N + 63) / 64, M);
    hipLaunchKernelGGL(k_gemm_f32, grid, dim3(64), 0, st, (const float*)A, lda, M, w, N, K, part,
                       best, logits, dr);
    return hipGetLastError();
  }
  (void)bf16;
  if (p.kind == GEMM_TILED) {
    dim3 grid((N + TBN - 1) / TBN, (M + TBM - 1) / TBM, p.splits);
    const uint16_t* a = (const uint16_t*)A;
    const uint16_t* al = (const uint16_t*)Alo;
    if (al && best)
      hipLaunchKernelGGL((k_gemm_tiled<true, 32, true>), grid, dim3(256), 0, st, a, al, lda, M, w,
                         N, K, p.kpw, part, best, logits, dr);
    else if (al)
      hipLaunchKernelGGL((k_gemm_tiled<true, 32, false>), grid, dim3(256), 0, st, a, al, lda, M,
                         w, N, K, p.kpw, part, best, logits, dr);
    else if (best)
      hipLaunchKernelGGL((k_gemm_tiled<false, 64, true>), grid, dim3(256), 0, st, a, al, lda, M,
                         w, N, K, p.kpw, part, best, logits, dr);
    else
      hipLaunchKernelGGL((k_gemm_tiled<false, 64, false>), grid, dim3(256), 0, st, a, al, lda, M,
                         w, N, K, p.kpw, part, best, logits, dr);
    return hipGetLastError();
  }
#define DF_SKINNY(MT, NT, U) \
  if (p.mt == MT && p.nt == NT) return run_skinny<MT, NT, U>(p, A, Alo, lda, M, w, N, K, part, best, logits, st, dr)
  DF_SKINNY(1, 1, 8);
  DF_SKINNY(2, 1, 4);
  DF_SKINNY(4, 1, 2);
#undef DF_SKINNY
  return hipErrorInvalidValue;
}
