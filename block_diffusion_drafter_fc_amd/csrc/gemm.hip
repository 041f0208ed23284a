// gemm.hip -- out = A[M][K] * W[N][K]^T for the drafter's dense products.
//
// Four kernels (plan_gemm picks one; the fused products of the draft at
// M <= 64 live in skinny.hip):
//   k_gemm_big     bf16, M >= 128: the MFMA-bound products (batch-32 draft,
//                  large injections, packed passes of 8+ blocks).  Output
//                  tiles of 64*WM x BN; K moves in steps of 32 through a ring
//                  of LDS stages filled by global_load_lds (no register
//                  staging); waves work in two groups half a K step apart so
//                  one group's fragment reads overlap the other's MFMAs; tile
//                  order keeps the M tiles of a weight tile on one XCD.
//   k_gemm_skinny  bf16, M <= 64 (the block rows of a few sequences).  The
//                  product is a stream of the weight matrix: each lane loads
//                  16 contiguous bytes of a weight row straight into the
//                  B operand of a 16x16x32 bf16 MFMA (no LDS round trip); the
//                  activations are staged once per workgroup in LDS and
//                  shared by its 4 waves; K is split over workgroups (fp32
//                  partial slices) so that about a thousand groups keep HBM
//                  busy.
//   k_gemm_tiled   bf16, 64 < M < 128: 128x128 output tiles, both operands
//                  staged through double-buffered LDS, 4 waves of 64x64.
// With SPLIT the activations arrive as two bf16 planes (hi, lo) of an fp32
// value and every weight fragment meets both: acc += hi*W + lo*W.
//   k_gemm_f32     fp32 models: one thread per output, plain K loop.
// All four can end in a fused row argmax (the LM head): the row maximum of
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
  if (!dr.on && logits == nullptr) {
    // greedy: the short branch-free scan of the large product's epilogue
    // (columns past N become -inf; a strict > over ascending fragments keeps
    // the lowest column among equal values)
    if (n0 + TBN > N) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (n0 + wn * 64 + b * 16 + lr >= N)
#pragma unroll
          for (int a = 0; a < 4; ++a) acc[a][b] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float bv = acc[a][0][i];
        int bb = 0;
#pragma unroll
        for (int b = 1; b < 4; ++b) {
          const bool gt = acc[a][b][i] > bv;
          bv = gt ? acc[a][b][i] : bv;
          bb = gt ? b : bb;
        }
        const uint64_t key = max16(argmax_key(bv, (uint32_t)(n0 + wn * 64 + bb * 16 + lr)));
        if (lr == 0) hkeys[wn][wm * 64 + a * 16 + lg * 4 + i] = key;
      }
  } else {
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
  }
  __syncthreads();
  if (tid < TBM && m0 + tid < M) {
    const uint64_t k0 = hkeys[0][tid], k1 = hkeys[1][tid];
    best[(size_t)blockIdx.x * M + m0 + tid] = k0 > k1 ? k0 : k1;
  }
}

// ----------------------------------------------------------------------------
// Large product (M >= 128): 64*WM x BN output tiles (BN = 256, or 192 where
// 256-column tiles leave CUs idle), WM*NWN waves of 64 x BN/NWN (wide in N,
// so that the two activation planes share every weight fragment read from
// LDS), K in steps of 32 through a ring of LDS stages.  WM = 2 on 4 waves
// (one per SIMD, 4 stages): each wave reads the next step's MFMA fragments
// while the current step's MFMAs run.  8 waves (WM = 4, 3 stages; or WM = 2
// with NWN = 4 waves of 64 x BN/4 along N, 4 stages): two per SIMD in two
// groups half a step apart, one group reading fragments while the other runs
// MFMAs.
//
// Loads go straight from global memory to LDS (global_load_lds_dwordx4: lane
// l of a wave writes its 16 bytes at the instruction's LDS base + 16 l), so
// no registers stage the tiles and G - 1 steps of loads stay in flight.  A
// stage holds the tile rows back to back, 64 bytes each: the A planes'
// 64*WM rows each, then the BN weight rows; every wave issues the same number
// of 16-row load blocks, and blocks past the tile land in a spare area.  The four 16-byte
// chunks of row R sit XOR-swizzled (chunk c at slot c ^ ((R >> 1) & 3)), so
// the 16 rows a fragment read touches land in distinct banks; a load block
// of 16 rows (1 KB, one wave instruction) fetches the chunks in swizzled
// order.
constexpr int GBN = 256, GBK = 32;   // widest weight tile, K step
constexpr int big_stages(int wm) { return wm == 4 ? 3 : 4; }

typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __attribute__((address_space(1))) void* glb_void_t;

// SWIGLU (one K split, W = [W_gate; W_up] with I rows each): tile t takes
// the gate rows [t BN/2, t BN/2 + BN/2) as its first BN/2 columns and the
// same up rows as the rest; the up waves hand their accumulators to the
// gate waves through LDS, which write h = silu(gate) * up as split planes
// (N is then BN * ceil(I / (BN/2))).
template <bool SPLIT, bool ARGMAX, int WM, int BN, int NWN = 2, bool SWIGLU = false>
__global__ __launch_bounds__(64 * WM * NWN, 1) void k_gemm_big(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Alo, int lda, int M, WSeg w,
    int N, int K, int kps, float* __restrict__ part, uint64_t* __restrict__ best,
    float* __restrict__ logits, DrawArgs dr, void* __restrict__ hout, size_t h_plane, int I) {
  constexpr int BM = 64 * WM, NWAVE = WM * NWN, G = big_stages(WM);
  constexpr bool DBUF = NWAVE == 4;            // one wave per SIMD; else two groups
  constexpr int WCOL = BN / NWN;               // weight columns per wave
  constexpr int NP = SPLIT ? 2 : 1;
  constexpr int RA = NP * BM;                  // A rows per stage
  constexpr int NR = RA + BN;                  // rows per stage
  constexpr int NL = (NR / 16 + NWAVE - 1) / NWAVE;   // load instructions per wave per stage
  constexpr int SB = NL * NWAVE * 1024;        // bytes per stage (blocks past NR: spare)
  constexpr int NBF = WCOL / 16;               // 16-column weight fragments per wave
  static_assert(NR % 16 == 0 && BN % 64 == 0, "tile rows come in blocks of 16");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[G * SB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = wave / NWN, wn = wave % NWN;
  // Tile order: the dispatcher deals workgroup ids to the 8 XCDs round
  // robin, so ids equal mod 8 share an XCD (whatever XCD the rotation starts
  // at).  Within such a slot consecutive ids take the M tiles of one weight
  // tile, which then streams from HBM once and from that XCD's L2 for the
  // other M tiles.  Ids past the last weight tile (the N tiles are padded to
  // a multiple of 8) exit at once.
  const int mtiles = (M + BM - 1) / BM;
  const int slot = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int ntile = (q / mtiles) * 8 + slot;
  if (ntile * BN >= N) return;
  const int m0 = (q % mtiles) * BM, n0 = ntile * BN, split = blockIdx.z;
  const int kbeg = split * kps;

  // global source of each of this lane's loads (block wave + NWAVE j)
  const uint16_t* gp[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int R = (wave + NWAVE * j) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((R >> 1) & 3);
    const uint16_t* row;
    if (R < RA) {
      const int pl = R / BM;
      const int r = min(m0 + (R % BM), M - 1);
      row = (pl ? Alo : A) + (size_t)r * lda;
    } else {
      // (spare blocks past the tile re-read its first weight row)
      const int c = R < NR ? R - RA : 0;
      int vrow = min(n0 + c, N - 1);
      if (SWIGLU) {
        const int gi = min(ntile * (BN / 2) + c % (BN / 2), I - 1);
        vrow = c < BN / 2 ? gi : I + gi;
      }
      row = seg_row_bf16(w, vrow, K);
    }
    gp[j] = row + kbeg + c * 8;
  }
  auto issue = [&](int s) {
    unsigned char* base = lds + (s % G) * SB;
#pragma unroll
    for (int j = 0; j < NL; ++j)
      __builtin_amdgcn_global_load_lds((glb_void_t)(gp[j] + s * GBK),
                                       (lds_void_t)(base + (wave + NWAVE * j) * 1024), 16, 0, 0);
  };
  auto frag = [&](const unsigned char* base, int R) -> u32x4 {
    return *(const u32x4*)(base + R * 64 + ((lg ^ ((R >> 1) & 3)) << 4));
  };

  f32x4 acc[4][NBF];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NBF; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragments of one step: B (NBF x 16 weight rows) and A (4 x 16 rows per
  // plane).
  struct Frags {
    u32x4 b[NBF], a[NP][4];
  };
  auto read_frags = [&](Frags& f, int s) {
    const unsigned char* base = lds + (s % G) * SB;
#pragma unroll
    for (int b = 0; b < NBF; ++b) f.b[b] = frag(base, RA + wn * WCOL + b * 16 + lr);
#pragma unroll
    for (int pl = 0; pl < NP; ++pl)
#pragma unroll
      for (int a = 0; a < 4; ++a) f.a[pl][a] = frag(base, pl * BM + wm * 64 + a * 16 + lr);
  };
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int pl = 0; pl < NP; ++pl)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NBF; ++b) acc[a][b] = mfma_16x16x32(f.a[pl][a], f.b[b], acc[a][b]);
  };
  // Stage t is complete for the whole workgroup once every lane has waited
  // for its own loads of step t (at most the later steps' loads, `later`
  // steps of NL each, still outstanding) and the waves have met at a bare
  // s_barrier (__syncthreads' fence would also wait for the later steps'
  // loads).  Every wave's fragment reads of the stage that is refilled next
  // have completed: their MFMAs consumed them.
  auto stage_ready = [&](int later) {
    if (later >= 3)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * NL) : "memory");
    else if (later == 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NL) : "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NL) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int steps = kps / GBK;
  for (int s = 0; s < G - 1 && s < steps; ++s) issue(s);
  if (DBUF) {
    // Iteration s: stage s + 1 becomes ready, the stage that held step s - 1
    // receives step s + G - 1, the fragments of step s + 1 are read, then
    // step s's MFMAs run.  steps is even (launch_gemm checks), so each pass
    // of the loop does two steps.
    Frags f0, f1;
    stage_ready(min(steps - 1, G - 2));
    read_frags(f0, 0);
    for (int s = 0; s < steps; s += 2) {
      stage_ready(min(steps - 2 - s, G - 2));
      if (s + G - 1 < steps) issue(s + G - 1);
      read_frags(f1, s + 1);
      mfmas(f0);
      if (s + 2 < steps) {
        stage_ready(min(steps - 3 - s, G - 2));
        if (s + G < steps) issue(s + G);
        read_frags(f0, s + 2);
      }
      mfmas(f1);
    }
  } else {
    // Two wave groups (waves 0-3 and 4-7, one of each per SIMD) run half a
    // step apart: every wave runs read(s) | barrier | MFMAs(s) | barrier,
    // and group 1 starts one barrier late, so one group's fragment reads
    // overlap the other group's MFMAs on every SIMD (in lockstep, both
    // waves of a SIMD would wait for their reads together).  A wave issues
    // step s + G - 1 at the start of its read phase of step s; that stage
    // last held step s - 1, which both groups read before the previous
    // barrier.  Stage s + 1 must be complete at the barrier that ends group
    // 0's MFMA phase of step s: group 0 waits for it there, group 1 at the
    // end of its read phase of step s, which is the same barrier.
    Frags f;
    const int grp = wave >> 2;
    stage_ready(min(steps - 1, G - 2));
    if (grp == 1) __builtin_amdgcn_s_barrier();
    for (int s = 0; s < steps; ++s) {
      if (s + G - 1 < steps) issue(s + G - 1);
      read_frags(f, s);
      const int later = max(min(steps - 2 - s, G - 2), 0);   // steps' loads left in flight
      stage_ready(grp == 1 ? later : min(later + 1, steps - 1 - s));
      mfmas(f);
      stage_ready(later);
    }
    if (grp == 0) __builtin_amdgcn_s_barrier();
  }

  if constexpr (SWIGLU) {
    static_assert(!ARGMAX && NWN % 2 == 0 && (BN / 2) % 8 == 0, "SwiGLU pairs gate and up waves");
    constexpr int HN = NWN / 2;    // waves per half of the tile
    constexpr int HC = BN / 2;     // h columns of the tile
    constexpr int NT = 64 * WM * NWN;
    float* sm = (float*)lds;       // [BM rows][HC]: exchanged values, then h
    auto sidx = [&](int a, int i, int col) { return (wm * 64 + a * 16 + lg * 4 + i) * HC + col; };
    __syncthreads();               // every wave is past its last fragment reads
    if constexpr (NBF % 2 == 0) {
      // Gate wave wn and up wave wn + HN hold the gate and up values of the
      // same h columns.  Each keeps half of its fragments: the gate wave
      // passes the gate values of fragments NBF/2.. through LDS, the up wave
      // the up values of fragments 0..NBF/2-1, and each then forms
      // h = silu(g) u for the half it kept.  Both waves of a SIMD share the
      // exponentials and reciprocals (the gate waves alone took 6 us per
      // 256 x 96 tile, against 4 us here).
      constexpr int HB = NBF / 2;
      const int cw = (wn % HN) * WCOL;
      const bool up = wn >= HN;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int bb = 0; bb < HB; ++bb) {
            const int b = up ? bb : bb + HB;   // the half this wave passes on
            sm[sidx(a, i, cw + b * 16 + lr)] = acc[a][b][i];
          }
      __syncthreads();
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float other[4][HB];   // a row block's partner values, read before any write
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int bb = 0; bb < HB; ++bb)
            other[i][bb] = sm[sidx(a, i, cw + (up ? bb + HB : bb) * 16 + lr)];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int bb = 0; bb < HB; ++bb) {
            const int b = up ? bb + HB : bb;   // the half this wave kept
            const float g = up ? other[i][bb] : acc[a][b][i];
            const float u = up ? acc[a][b][i] : other[i][bb];
            sm[sidx(a, i, cw + b * 16 + lr)] = __fdividef(g, 1.0f + __expf(-g)) * u;   // silu(g) u
          }
      }
    } else {
      if (wn >= HN) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < NBF; ++b) sm[sidx(a, i, (wn - HN) * WCOL + b * 16 + lr)] = acc[a][b][i];
      }
      __syncthreads();
      if (wn < HN) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < NBF; ++b) {
              float* e = &sm[sidx(a, i, wn * WCOL + b * 16 + lr)];
              const float g = acc[a][b][i];
              *e = __fdividef(g, 1.0f + __expf(-g)) * *e;   // silu(gate) * up
            }
      }
    }
    __syncthreads();
    // h rows m0.., columns ntile * HC..: 8 consecutive columns per thread,
    // one 16-byte store per plane (I is a multiple of 8)
    auto store8 = [&](int r, int c8) {
      const f32x4 v0 = *(const f32x4*)&sm[r * HC + c8], v1 = *(const f32x4*)&sm[r * HC + c8 + 4];
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float x0 = v0[2 * k], x1 = v0[2 * k + 1], y0 = v1[2 * k], y1 = v1[2 * k + 1];
        hw[k] = pack_bf2(x0, x1);
        lw[k] = pack_bf2(x0 - __uint_as_float(hw[k] << 16), x1 - __uint_as_float(hw[k] & 0xFFFF0000u));
        hw[2 + k] = pack_bf2(y0, y1);
        lw[2 + k] = pack_bf2(y0 - __uint_as_float(hw[2 + k] << 16),
                             y1 - __uint_as_float(hw[2 + k] & 0xFFFF0000u));
      }
      uint16_t* hp = (uint16_t*)hout + (size_t)(m0 + r) * I + ntile * HC + c8;
      st16(hp, u32x4{hw[0], hw[1], hw[2], hw[3]});
      st16(hp + h_plane, u32x4{lw[0], lw[1], lw[2], lw[3]});
    };
    constexpr int NCHK = BM * (HC / 8);   // 8-column pieces of the tile
    if (NCHK % NT == 0 && m0 + BM <= M && (ntile + 1) * HC <= I) {
      // interior tile: every piece stored, no test per piece
#pragma unroll
      for (int q = 0; q < NCHK / NT; ++q) {
        const int e = tid + q * NT;
        store8(e / (HC / 8), (e % (HC / 8)) * 8);
      }
    } else {
      for (int e = tid; e < NCHK; e += NT) {
        const int r = e / (HC / 8), c8 = (e % (HC / 8)) * 8;
        if (m0 + r < M && ntile * HC + c8 < I) store8(r, c8);
      }
    }
    return;
  }
  if (!ARGMAX) {
    if (m0 + BM <= M && n0 + BN <= N) {
      // interior tile: stores without a bounds test each (one branch per
      // store was the epilogue's code)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float* dst = part + ((size_t)split * M + m0 + wm * 64 + a * 16 + lg * 4 + i) * N + n0 +
                       wn * WCOL + lr;
#pragma unroll
          for (int b = 0; b < NBF; ++b) dst[b * 16] = acc[a][b][i];
        }
      return;
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + wm * 64 + a * 16 + lg * 4 + i;
        if (row >= M) continue;
        float* dst = part + ((size_t)split * M + row) * N;
#pragma unroll
        for (int b = 0; b < NBF; ++b) {
          const int col = n0 + wn * WCOL + b * 16 + lr;
          if (col < N) dst[col] = acc[a][b][i];
        }
      }
    return;
  }
  // Row argmax over the tile's BN columns: per wave (NBF fragments, then the
  // 16 lanes of a row), then over the NWN column slices in LDS.
  __syncthreads();
  uint64_t* hkeys = (uint64_t*)lds;   // [NWN][BM], the stages are no longer read
  if (!dr.on && logits == nullptr) {
    // Greedy draft: a short branch-free scan.  This code runs once per tile
    // from a cold instruction cache, and the fully unrolled general path
    // below (noise, logits, a column test per element) measured 23 us per
    // 256 x 256 tile against 6 us for this one.  Columns past N (the last
    // tile) become -inf, which any real value beats.  Per lane a strict >
    // over ascending fragments keeps the lowest column among equal values
    // (-0 and +0 compare equal), which is the order of the keys.
    if (n0 + BN > N) {
#pragma unroll
      for (int b = 0; b < NBF; ++b)
        if (n0 + wn * WCOL + b * 16 + lr >= N)
#pragma unroll
          for (int a = 0; a < 4; ++a) acc[a][b] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float bv = acc[a][0][i];
        int bb = 0;
#pragma unroll
        for (int b = 1; b < NBF; ++b) {
          const bool gt = acc[a][b][i] > bv;
          bv = gt ? acc[a][b][i] : bv;
          bb = gt ? b : bb;
        }
        const uint64_t key = max16(argmax_key(bv, (uint32_t)(n0 + wn * WCOL + bb * 16 + lr)));
        if (lr == 0) hkeys[wn * BM + wm * 64 + a * 16 + lg * 4 + i] = key;
      }
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rloc = wm * 64 + a * 16 + lg * 4 + i;
        const int row = m0 + rloc;
        uint64_t key = 0;
#pragma unroll
        for (int b = 0; b < NBF; ++b) {
          const int col = n0 + wn * WCOL + b * 16 + lr;
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
        if (lr == 0) hkeys[wn * BM + rloc] = key;
      }
  }
  __syncthreads();
  if (tid < BM && m0 + tid < M) {
    uint64_t k0 = hkeys[tid];
#pragma unroll
    for (int x = 1; x < NWN; ++x) k0 = hkeys[x * BM + tid] > k0 ? hkeys[x * BM + tid] : k0;
    best[(size_t)ntile * M + m0 + tid] = k0;
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

// Tile height, waves, width and K splits of the large product, from a cost
// model fitted to measurements: a round of up to 256 workgroups (one per CU)
// costs steps/S K steps plus a fixed cost (filling the stage ring, writing the
// tile, dispatch); each extra partial slice costs its write-back and the
// reducer's read (2 * M * N * 4 bytes at ~5 TB/s).  Splits keep an even
// number of >= 4 steps.
// Per round: steps/S * t_step * BN/256 + fixed (us), least-squares fits to a
// sweep of every configuration on the Qwen3-8B and wide-drafter product shapes
// at 128, 256 and 512 rows (random bf16 data): 128-row tile on 4 waves, on 8
// waves, 256-row tile on 8 waves.
constexpr double kBigStep[3] = {0.885, 0.719, 1.021};
constexpr double kBigFixed[3] = {10.8, 11.6, 16.8};

struct BigChoice {
  int wm, splits, bn, waves;
};

BigChoice big_plan(int M, int N, int K, bool argmax) {
  BigChoice best{2, 1, GBN, 4};
  double best_cost = 1e300;
  const int steps = K / GBK;
  for (int bn = GBN; bn >= 192; bn -= 64) {
    if (argmax && bn != GBN) continue;
    const long ntiles = (N + bn - 1) / bn;
    for (int v = 0; v < 3; ++v) {   // (tile height, waves): (128, 4), (128, 8), (256, 8)
      const int wm = v == 2 ? 4 : 2, waves = v == 0 ? 4 : 8;
      const long tiles = (long)((M + 64 * wm - 1) / (64 * wm)) * ntiles;
      const double t_step = kBigStep[v] * bn / GBN, fixed = kBigFixed[v];
      for (int S = 1; S <= (argmax ? 1 : 16); ++S) {
        if (steps % S || (steps / S) % 2 || steps / S < 4) continue;
        const double rounds = (double)((tiles * S + 255) / 256);
        const double cost = rounds * ((double)(steps / S) * t_step + fixed) +
                            (double)(S - 1) * M * (double)N * 8.0 / 5e6;
        if (cost < best_cost) {
          best_cost = cost;
          best = BigChoice{wm, S, bn, waves};
        }
      }
    }
  }
  return best;
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
  p.waves = 4;
  if (M >= 128 && K % (2 * GBK) == 0) {
    // 128 x 256 or 256 x 256 tiles (or 192 wide).  At 128 rows (batch-8
    // draft of the wide drafter) they beat the 128 x 128 kernel on gate/up
    // (1.16x), down (1.25x) and the LM head (1.03x) and lose 7% on QKV;
    // below 128 rows the 128 x 128 kernel stays
    p.kind = GEMM_BIG;
    const BigChoice c = big_plan(M, N, K, argmax);
    p.mt = c.wm;
    p.nt = c.bn;
    p.waves = c.waves;
    p.splits = c.splits;
    p.kpw = K / p.splits;
    return p;
  }
  p.kind = GEMM_TILED;
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
  if (p.kind == GEMM_BIG) return (N + p.nt - 1) / p.nt;
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
  if (p.kind == GEMM_BIG) {
    if ((p.mt != 2 && p.mt != 4) || (p.nt != GBN && (p.nt != 192 || best)) ||
        (p.waves != 2 * p.mt && !(p.mt == 2 && p.waves == 8)) || p.kpw % (2 * GBK) != 0 ||
        (long)p.kpw * p.splits != K || lda % 8 != 0)
      return hipErrorInvalidValue;
    const int bm = 64 * p.mt;
    dim3 grid(((N + p.nt - 1) / p.nt + 7) / 8 * 8 * ((M + bm - 1) / bm), 1, p.splits);
    const uint16_t* a = (const uint16_t*)A;
    const uint16_t* al = (const uint16_t*)Alo;
#define DF_BIG(SPL, AM, WM, BN, NWN)                                                          \
  hipLaunchKernelGGL((k_gemm_big<SPL, AM, WM, BN, NWN>), grid, dim3(64 * WM * NWN), 0, st, a, al, \
                     lda, M, w, N, K, p.kpw, part, best, logits, dr, nullptr, (size_t)0, 0)
#define DF_BIG2(WM, NWN)                                       \
  if (al && best) DF_BIG(true, true, WM, GBN, NWN);             \
  else if (best) DF_BIG(false, true, WM, GBN, NWN);             \
  else if (al && p.nt == GBN) DF_BIG(true, false, WM, GBN, NWN); \
  else if (al) DF_BIG(true, false, WM, 192, NWN);               \
  else if (p.nt == GBN) DF_BIG(false, false, WM, GBN, NWN);     \
  else DF_BIG(false, false, WM, 192, NWN)
    if (p.mt == 4) {
      DF_BIG2(4, 2);
    } else if (p.waves == 8) {
      DF_BIG2(2, 4);
    } else {
      DF_BIG2(2, 2);
    }
#undef DF_BIG2
#undef DF_BIG
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

bool gemm_swiglu_ok(const GemmPlan& p, int I) {
  return p.kind == GEMM_BIG && p.splits == 1 && p.nt == 192 && I > 0 && I % 8 == 0 &&
         (p.mt == 4 || p.mt == 2);
}

hipError_t launch_gemm_swiglu(const GemmPlan& p, const void* A, const void* Alo, int lda, int M,
                              const WSeg& w, int I, int K, void* h, size_t h_plane,
                              hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (!gemm_swiglu_ok(p, I) || Alo == nullptr || p.kpw != K || K % (2 * GBK) != 0 ||
      lda % 8 != 0 || (p.waves != 2 * p.mt && !(p.mt == 2 && p.waves == 8)))
    return hipErrorInvalidValue;
  constexpr int BN = 192;
  const int N = BN * ((I + BN / 2 - 1) / (BN / 2));   // paired tiles, the last one ragged
  const int bm = 64 * p.mt;
  dim3 grid((N / BN + 7) / 8 * 8 * ((M + bm - 1) / bm), 1, 1);
  const uint16_t* a = (const uint16_t*)A;
  const uint16_t* al = (const uint16_t*)Alo;
  const DrawArgs dr{};
#define DF_SW(WM, NWN)                                                                         \
  hipLaunchKernelGGL((k_gemm_big<true, false, WM, BN, NWN, true>), grid, dim3(64 * WM * NWN), 0, \
                     st, a, al, lda, M, w, N, K, K, nullptr, nullptr, nullptr, dr, h, h_plane, I)
  if (p.mt == 4) DF_SW(4, 2);
  else if (p.waves == 8) DF_SW(2, 4);
  else DF_SW(2, 2);
#undef DF_SW
  return hipGetLastError();
}
