// skinny.hip -- bf16 weight-streaming product for M <= 64 rows (the block rows
// of up to 4 sequences, or up to 64 new context tokens) with the epilogue of
// the surrounding step fused in.
//
// Work split.  Output columns come in groups of 64; a workgroup of 4 waves
// owns one group and one K slice.  The activations of the slice are staged
// in LDS in sub-chunks of KC columns (double-buffered) as hi/lo bf16 planes
// and shared by the 4 waves; each wave streams its own 16 weight rows from
// HBM straight into 16x16x32 MFMA B operands (16 contiguous bytes per lane).
// Activation loads are issued before the weight batch (loads retire in
// order, so the LDS store never waits for weights) and two weight batches
// per wave are in flight.
//
// Activation sources (SkinnyA): split fp32 planes, exact bf16 inputs, or the
// fp32 residual x normalised on the fly (RMSNorm with the row sums of squares
// left by the producer of x, times the gain) -- so no separate norm kernel.
//
// Fused epilogues (SkinnyOut).  K is split over S workgroups; the groups of
// one output tile (one head, one [gate|up] pair, or one 64-column group) and
// all their K splits get workgroup ids congruent mod 8.  The dispatcher
// places workgroup i on XCD i mod 8, so they meet in that XCD's L2: each
// finished workgroup waits for its partial stores, adds its arrival to the
// tile's counter, and the last to arrive drops its L1, sums the partials in
// split order and applies the epilogue (RoPE, SwiGLU, residual + row sums of
// squares, K/V page store).  The dispatcher's round robin starts at an XCD
// that is fixed per hardware queue (not always XCD 0 once a process has
// several streams), so each launch takes the rotation workgroup 0 saw in the
// previous launch as the expected placement.  It reads that from one of two
// words of the state buffer and records its own in the other, so every
// workgroup of one launch expects the same placement.
// The counter also counts arrivals per XCD (read from the XCC_ID register).
// A workgroup away from the tile's home XCD
// writes its partials back with a device-scope fence; a reducer that saw
// arrivals from another XCD acquires at device scope; a reducer away from
// home while home workgroups also wrote (their partials then sit in another
// L2) raises an error bit.  No workgroup ever waits on another.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace {

constexpr int kXcds = 8;
// Workgroups a split-K launch aims for: every workgroup pays a start and
// publish latency, so fewer workgroups with longer K slices beat many short
// ones.  Measured with packed weights and streaming loads on the
// Qwen3-8B-shaped draft and inject (M <= 16): O, down and the fc were
// fastest at 256 workgroups (S = 4), QKV at 192 (S = 2), SwiGLU and K/V at
// 640-768 (S = 2 and 4).
constexpr int kWgTarget = 256;
constexpr int kWgTargetQkv = 192;
constexpr int kWgTargetPaired = 640;   // SO_SWIGLU, SO_KV
constexpr int kMaxSplits = 16;
constexpr int kMaxPer = 63;       // arrivals per tile (6-bit per-XCD fields)
constexpr int kMaxSsTiles = 128;  // row sum-of-squares pieces (hidden <= 8192)
constexpr uint32_t kErrXcd = 8u;

DF_DEV unsigned xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xFu; }

__host__ __device__ inline int tile_groups(int out, int dh) {
  if (out == SO_QKV || out == SO_KV) return dh / 64;
  if (out == SO_SWIGLU) return 2;
  return 1;
}

DF_DEV uint64_t max16(uint64_t k) {
  for (int m = 1; m < 16; m <<= 1) {
    const uint64_t o = shfl_xor_u64(k, m);
    k = o > k ? o : k;
  }
  return k;
}

// Weight row of the first column of 64-column group g.  SwiGLU interleaves
// gate and up groups so that one tile holds both halves of 64 outputs.
template <int OUT>
DF_DEV int group_row0(int g, int I) {
  if (OUT == SO_SWIGLU) return (g & 1) ? I + 64 * (g >> 1) : 64 * (g >> 1);
  return 64 * g;
}

// Sums over the S partial slices part[s][M][N] of two 4-column pieces at
// element offsets o1 and o2 of a slice, in split order.  Loads go out in
// batches of 8 per piece, so up to 16 are in flight at once.
DF_DEV void sum_parts2(const float* part, int S, size_t slice, size_t o1, size_t o2, f32x4& s1,
                       f32x4& s2) {
  s1 = f32x4{0.f, 0.f, 0.f, 0.f};
  s2 = s1;
  for (int s0 = 0; s0 < S; s0 += 8) {
    f32x4 a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < S) {
        a[j] = *(const f32x4*)&part[(size_t)(s0 + j) * slice + o1];
        b[j] = *(const f32x4*)&part[(size_t)(s0 + j) * slice + o2];
      }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < S) {
        s1 += a[j];
        s2 += b[j];
      }
  }
}

// Same for one piece.
DF_DEV f32x4 sum_parts1(const float* part, int S, size_t slice, size_t o) {
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 8) {
    f32x4 a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < S) a[j] = *(const f32x4*)&part[(size_t)(s0 + j) * slice + o];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < S) v += a[j];
  }
  return v;
}

// sequence of token t of an inject batch: cu_new[b] <= t < cu_new[b+1]
DF_DEV int seq_of(const int32_t* cu_new, int batch, int t) {
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_new[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Rotate the pairs (x1[e], x2[e]) = dims (i + e, i + e + dh/2) with the
// (cos, sin) values (c01, c23) = cs[0..7] of one table row: cs[2e], cs[2e+1]
// for pair e.
DF_DEV void rope4(f32x4 c01, f32x4 c23, f32x4& x1, f32x4& x2) {
  const float c[4] = {c01[0], c01[2], c23[0], c23[2]};
  const float sn[4] = {c01[1], c01[3], c23[1], c23[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = x1[e] * c[e] - x2[e] * sn[e], b = x2[e] * c[e] + x1[e] * sn[e];
    x1[e] = a;
    x2[e] = b;
  }
}

// ------------------------------------------------------------ tile epilogues
// All run on the 256 threads of the tile's last workgroup.

// x (+)= product over the 64 columns of `tile`; ss_out[tile][row] = sum x^2.
template <bool ADD>
DF_DEV void epi_resid(const SkinnyArgs& a, int S, int tile) {
  const int t = threadIdx.x, r16 = t >> 4, c = (t & 15) * 4;
  const int col = tile * 64 + c;
  for (int r0 = 0; r0 < a.M; r0 += 16) {
    const int row = r0 + r16;
    float ssq = 0.f;
    if (row < a.M) {
      f32x4 v = sum_parts1(a.part, S, (size_t)a.M * a.N, (size_t)row * a.N + col);
      float* xp = a.x + (size_t)row * a.N + col;
      if (ADD) v += *(const f32x4*)xp;
      *(f32x4*)xp = v;
      ssq = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    for (int m = 1; m < 16; m <<= 1) ssq += __shfl_xor(ssq, m, 64);
    if ((t & 15) == 0 && row < a.M) a.ss_out[(size_t)tile * a.M + row] = ssq;
  }
}

// Head hh of [Q heads | K heads | V heads]: RoPE on q and k at the row's
// position, q to split planes, k and v to fp32.
DF_DEV void epi_qkv(const SkinnyArgs& a, int S, int hh) {
  const int half = a.dh / 2, quads = half / 4;
  const int c0 = hh * a.dh;
  for (int task = threadIdx.x; task < a.M * quads; task += blockDim.x) {
    const int row = task / quads, i = (task % quads) * 4;
    // the row's cos/sin pairs load with the partials (one wait for both;
    // value heads read them too and leave them unused)
    const float* cs = a.rope + ((size_t)row * half + i) * 2;
    const f32x4 c01 = *(const f32x4*)cs, c23 = *(const f32x4*)(cs + 4);
    f32x4 x1, x2;
    const size_t o = (size_t)row * a.N + c0 + i;
    sum_parts2(a.part, S, (size_t)a.M * a.N, o, o + half, x1, x2);
    if (hh < a.Hq + a.Hkv) rope4(c01, c23, x1, x2);
    if (hh < a.Hq) {
      const size_t base = ((size_t)row * a.Hq + hh) * a.dh;
      split_store4(a.q, a.q_plane, base + i, x1);
      split_store4(a.q, a.q_plane, base + i + half, x2);
    } else {
      const bool isk = hh < a.Hq + a.Hkv;
      float* dst = isk ? a.kb : a.vb;
      const size_t base = ((size_t)row * a.Hkv + (isk ? hh - a.Hq : hh - a.Hq - a.Hkv)) * a.dh;
      *(f32x4*)&dst[base + i] = x1;
      *(f32x4*)&dst[base + i + half] = x2;
    }
  }
}

// Tile t: gate columns [64t, 64t+64) (group 2t) and up (group 2t+1).
DF_DEV void epi_swiglu(const SkinnyArgs& a, int S, int tile) {
  const int t = threadIdx.x, r16 = t >> 4, c = (t & 15) * 4;
  for (int r0 = 0; r0 < a.M; r0 += 16) {
    const int row = r0 + r16;
    if (row >= a.M) continue;
    f32x4 g, u;
    const size_t o = (size_t)row * a.N + (2 * tile) * 64 + c;
    sum_parts2(a.part, S, (size_t)a.M * a.N, o, o + 64, g, u);
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = g[e] / (1.0f + expf(-g[e])) * u[e];
    split_store4(a.h, a.h_plane, (size_t)row * a.I + tile * 64 + c, y);
  }
}

// Head y of [K^0 | V^0 | K^1 | V^1 | ...] for the inject tokens: RoPE on K at
// the token's position, store bf16 into its page (K row-major, V transposed).
DF_DEV void epi_kv(const SkinnyArgs& a, int S, int y) {
  const int half = a.dh / 2, quads = half / 4;
  const int kvh = y % a.Hkv, kv = (y / a.Hkv) % 2, layer = y / (2 * a.Hkv);
  const int c0 = y * a.dh;
  for (int task = threadIdx.x; task < a.M * quads; task += blockDim.x) {
    const int t = task / quads, i = (task % quads) * 4;
    const int b = seq_of(a.cu_new, a.batch, t);
    const int pos = a.ctx_lens[b] + (t - a.cu_new[b]);
    const int pi = pos / a.page_size;
    if (pos < 0 || pi >= a.max_pages) {
      if (i == 0) set_dev_error(a.err, 2u);
      continue;
    }
    const int pg = a.page_table[(size_t)b * a.max_pages + pi];
    if (pg < 0 || pg >= a.n_pages) {
      if (i == 0) set_dev_error(a.err, 1u);
      continue;
    }
    const float* cs = a.rope + ((size_t)t * half + i) * 2;
    const f32x4 c01 = *(const f32x4*)cs, c23 = *(const f32x4*)(cs + 4);
    f32x4 x1, x2;
    const size_t o = (size_t)t * a.N + c0 + i;
    sum_parts2(a.part, S, (size_t)a.M * a.N, o, o + half, x1, x2);
    if (kv == 0) rope4(c01, c23, x1, x2);
    // K rows are [page_size][dh], values transposed [dh][page_size]
    uint16_t* dst = (uint16_t*)a.pages +
                    ((((size_t)layer * a.n_pages + pg) * 2 + kv) * a.Hkv + kvh) * a.page_size * a.dh;
    const int slot = pos % a.page_size;
    const size_t rs = kv == 0 ? 1 : (size_t)a.page_size;              // step between dimensions
    dst += kv == 0 ? (size_t)slot * a.dh : (size_t)slot;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dst[(i + e) * rs] = f2bf(x1[e]);
      dst[(i + e + half) * rs] = f2bf(x2[e]);
    }
  }
}

// --------------------------------------------------------------- the kernel
// grid: (n_tiles rounded up to a multiple of 8) * per workgroups of 256 * KS
// threads, per = tile_groups * S.  The LM head (SO_ARGMAX) over packed
// weights: workgroup t takes the gpw consecutive 64-column groups
// [t * gpw, t * gpw + gpw) as one run of sub-chunks -- their packed tiles are
// adjacent, so the weight stream continues from group to group as one
// contiguous chunk and the activations are re-staged from column 0 -- and
// folds each group's argmax keys into running per-row maxima; n_tiles is then
// the number of workgroups.  Otherwise gpw = 1.
//
// DYN (LM head over packed weights): workgroup t starts with group t and then
// takes further groups from the counter a.wctr (zero between launches), so
// CUs that stream faster take more groups.  Thread 0 claims the group after
// the current one in the group's first sub-chunk, after that sub-chunk's
// loads, and publishes it through LDS in the second, after that sub-chunk's
// loads (so the wait for the claim only covers loads the MFMAs need anyway);
// the group's last sub-chunk starts loading the claimed group.  Needs an even
// number (>= 4) of sub-chunks per group (per wave set, with KS > 1).
//
// KS > 1 (dynamic LM head): KS sets of 4 waves share the group, set s taking
// the s-th 1/KS of K with its own activation stream, and the other sets'
// sums join set 0's through LDS when the group ends.  A group then takes
// 1/KS of the time, so the last groups claimed end the launch sooner (one
// such workgroup per CU: no second workgroup to compete for the CU).
template <int MT, int ASRC, int OUT, bool PACKED, int UW = 8, bool DYN = false, int KS = 1>
__global__ __launch_bounds__(256 * KS, KS > 1 ? 1 : (OUT == SO_ARGMAX || UW == 16 ? 2 : 4)) void k_skinny(SkinnyArgs a, int S, int kps, int n_tiles,
                                                   int gpw) {
  static_assert(!DYN || (OUT == SO_ARGMAX && PACKED), "dynamic groups: packed LM head only");
  static_assert(KS == 1 || DYN, "wave sets: dynamic LM head only");
  constexpr int U = UW / MT, KC = 32 * U, ROWS = 16 * MT, CPR = KC / 8;
  constexpr int NCH = ROWS * CPR / 256;
  constexpr bool NORM = ASRC == SA_NORM || ASRC == SA_NORM1;   // RMSNorm while staging
  constexpr bool TWO = ASRC == SA_SPLIT || ASRC == SA_NORM;     // two planes in LDS
  constexpr int NP = TWO ? 2 : 1;
  constexpr int LPR = 256 / ROWS;         // threads per row in the norm prologue
  static_assert(ROWS * CPR % 256 == 0 && 256 % CPR == 0,
                "sub-chunk must split evenly over 256 threads, same columns per thread");
  __shared__ __attribute__((aligned(16))) uint16_t As[KS][2][NP][ROWS][KC + 8];
  __shared__ float inv_s[ROWS];
  __shared__ unsigned long long sh_old;
  __shared__ int sh_grp[2];   // DYN: the group after group q, in slot (q + 1) & 1
  __shared__ float red[KS > 1 ? KS - 1 : 1][KS > 1 ? ROWS : 1][KS > 1 ? 68 : 1];   // wave-set sums

  // tid: the thread within its wave set (256 threads); ks: the set
  const int ks = KS > 1 ? (int)(threadIdx.x >> 8) : 0;
  const int tid = KS > 1 ? (int)(threadIdx.x & 255) : (int)threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int tg = tile_groups(OUT, a.dh);
  const int per = tg * S;
  const int id = blockIdx.x, xcd = id % kXcds, local = id / kXcds;
  const int tile = (local / per) * kXcds + xcd, member = local % per;
  if (tile >= n_tiles) return;
  // queue rotation of the workgroup -> XCD placement (see the publish step)
  const unsigned rot = (OUT != SO_ARGMAX && a.qhint_rd != nullptr) ? (*a.qhint_rd & 7u) : 0u;
  const int grp = OUT == SO_ARGMAX ? tile * gpw : tile * tg + member / S, split = member % S;
  const int kset = ks * (kps / KS);   // the set's first column within the slice
  const int kbeg = split * kps + kset;
  const int M = a.M, N = a.N, K = a.K;
  int vcol0 = grp * 64 + wave * 16;                        // virtual column of the wave
  const bool active = vcol0 < N;
  // Weight rows of this wave: virtual rows vcol0 .. vcol0 + 15.
  //  Plain layout: rows of the segments, 16 contiguous bytes per lane at
  //  column k + 32u + 8 lg (inner segment boundaries are multiples of 16; the
  //  segment lookup is wave-uniform).  Packed layout: 16-row x 32-column
  //  tiles of 1 KB in lane order, the product's virtual rows in order, the
  //  four tiles of a 64-row group adjacent per 32-column block.
  // Rows past the end (a partial last group, or a wave past N) re-read the
  // last row (group) and their products are discarded.
  const uint16_t* bp;
  int bstride;   // elements from one 32-column block to the next
  if (PACKED) {
    // [64-row group][32-column block][wave][1 KB tile]: the four waves of a
    // workgroup read 4 adjacent KB per block (rows padded to 64 with zeros)
    bp = a.packed + (((size_t)grp * (K / 32) + kbeg / 32) * 4 + wave) * 512 + lane * 8;
    bstride = 4 * 512;
  } else {
    const int nrows = a.w.row_end[a.w.n - 1];
    const int base = __builtin_amdgcn_readfirstlane(group_row0<OUT>(grp, a.I) + wave * 16);
    const int rfirst = base < nrows ? base : nrows - 1;
    int sgi = 0;
    while (sgi < a.w.n - 1 && rfirst >= a.w.row_end[sgi]) ++sgi;
    const int st = sgi ? a.w.row_end[sgi - 1] : 0, en = a.w.row_end[sgi];
    const int wrow = base + lr < en ? base + lr : en - 1;
    bp = (const uint16_t*)a.w.ptr[sgi] + (size_t)(wrow - st) * K + kbeg + lg * 8;
    bstride = 32;
  }
  // weights of block u of the sub-chunk at column k of the slice (DYN: of
  // the current group, whose base bp is)
  auto wload = [&](int k, int u) { return ld16_stream(bp + (size_t)(k / 32 + u) * bstride); };

  // activation chunks this thread stages per sub-chunk: row srow, column scol
  int srow[NCH], scol[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + i * 256;
    srow[i] = c / CPR;
    scol[i] = (c % CPR) * 8;
  }

  f32x4 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 bc[U], bn[U];

  // Raw activation data of one sub-chunk: two 16-byte pieces per chunk (the
  // hi and lo planes, or 8 fp32 values of x) plus, for SA_NORM, the 8 gains
  // of the thread's columns (the same for all its chunks).
  u32x4 r0[NCH], r1[NCH], rg;
  auto fetch = [&](int k) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int row = srow[i] < M ? srow[i] : M - 1;
      const int col = kbeg + k + scol[i];
      if (NORM) {
        const float* xp = (const float*)a.A + (size_t)row * a.lda + col;
        r0[i] = ld16(xp);
        r1[i] = ld16(xp + 4);
        if (i == 0) rg = ld16((const uint16_t*)a.gain + col);
      } else {
        const uint16_t* ap = (const uint16_t*)a.A + (size_t)row * a.lda + col;
        r0[i] = ld16(ap);
        if (TWO) r1[i] = ld16(ap + a.a_plane);
      }
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (NORM) {
        // y = x * inv * g, split into hi = bf16(y) and lo = bf16(y - hi)
        // (SA_NORM1: hi only)
        const float inv = inv_s[srow[i]];
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xa = __uint_as_float(e < 2 ? r0[i][2 * e] : r1[i][2 * e - 4]);
          const float xb = __uint_as_float(e < 2 ? r0[i][2 * e + 1] : r1[i][2 * e - 3]);
          const uint32_t gw = rg[e];
          const float ya = xa * inv * __uint_as_float(gw << 16);
          const float yb = xb * inv * __uint_as_float(gw & 0xFFFF0000u);
          hw[e] = pack_bf2(ya, yb);
          lw[e] = pack_bf2(ya - __uint_as_float(hw[e] << 16), yb - __uint_as_float(hw[e] & 0xFFFF0000u));
        }
        st16(&As[ks][buf][0][srow[i]][scol[i]], u32x4{hw[0], hw[1], hw[2], hw[3]});
        if (TWO) st16(&As[ks][buf][NP - 1][srow[i]][scol[i]], u32x4{lw[0], lw[1], lw[2], lw[3]});
      } else {
        st16(&As[ks][buf][0][srow[i]][scol[i]], r0[i]);
        if (TWO) st16(&As[ks][buf][NP - 1][srow[i]][scol[i]], r1[i]);
      }
    }
  };

  // Prologue.  Loads retire in order, so they are issued oldest-needed
  // first: the row sums of squares (SA_NORM), the activations of sub-chunk
  // 0, then its weights, which stay in flight while the rest is staged.
  constexpr int Q = kMaxSsTiles / LPR;
  const int nrm_row = tid / LPR, nrm_j = tid % LPR;
  float ssv[NORM ? Q : 1];
  if (NORM) {
    // fully unrolled, unpredicated loads (clamped index, masked use): a loop
    // or a branch here would make the compiler drain the loads in flight
    const int rr = nrm_row < M ? nrm_row : M - 1;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int i = q * LPR + nrm_j;
      ssv[q] = a.ss_in[(size_t)(i < a.ss_tiles ? i : a.ss_tiles - 1) * M + rr];
    }
  }
  fetch(0);
#pragma unroll
  for (int u = 0; u < U; ++u) bc[u] = wload(0, u);
  __builtin_amdgcn_sched_barrier(0);
  if (NORM) {
    // 1 / rms of each row from the producer's per-tile sums of squares
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) s += ssv[q] * (q * LPR + nrm_j < a.ss_tiles ? 1.f : 0.f);
    for (int m = 1; m < LPR; m <<= 1) s += __shfl_xor(s, m, 64);
    if (nrm_j == 0 && ks == 0) inv_s[nrm_row] = nrm_row < M ? 1.0f / sqrtf(s / (float)K + a.eps) : 0.f;
    __syncthreads();
  }
  stage(0);
  __syncthreads();

  // One sub-chunk k: if LOAD, issue the next sub-chunk's activation and
  // weight loads, then run the MFMAs on LDS buffer `buf` with the weights in
  // `bw` and stage the next activations.  Two weight register sets
  // alternate, so the batch loading for the next sub-chunk stays in flight
  // across the barrier, and the MFMAs wait only for their own batch (loads
  // retire in order).  The loads are not predicated (waves past N read a
  // clamped row), so the wait counts stay exact.
  const int nsub = kps / KS / KC;   // >= 1 sub-chunks per group (per wave set)
  const int ngroups = (N + 63) / 64;
  auto step = [&](auto load_tag, int J, int buf, const u32x4* bw, u32x4* bnext,
                  unsigned& claim) {
    constexpr bool LOAD = decltype(load_tag)::value;
    const int jq = J % nsub, q = J / nsub;
    if (LOAD) {
      // sub-chunk J + 1: its activations at column ((J + 1) mod nsub) * KC,
      // its weights J + 1 sub-chunks into this workgroup's stream (DYN: at
      // the start of the next group once J + 1 opens it)
      fetch(((J + 1) % nsub) * KC);
      if (DYN && jq == nsub - 1)
        bp = a.packed + (((size_t)sh_grp[(q + 1) & 1] * (K / 32) + kset / 32) * 4 + wave) * 512 +
             lane * 8;
#pragma unroll
      for (int u = 0; u < U; ++u) bnext[u] = wload((DYN ? (J + 1) % nsub : J + 1) * KC, u);
      __builtin_amdgcn_sched_barrier(0);
      // the claim made one sub-chunk earlier, older than this step's loads:
      // waiting for it waits for nothing the MFMAs below do not need anyway.
      // (Published before a claim is made in program order, so the compiler
      // never counts a claim of this same step as pending here.)
      if (DYN && jq == 1 && tid == 0 && ks == 0) sh_grp[(q + 1) & 1] = n_tiles + (int)claim;
      if (DYN && jq == 0 && tid == 0 && ks == 0) claim = atomicAdd(a.wctr, 1u);
      __builtin_amdgcn_sched_barrier(0);   // all loads issue before the MFMAs
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const u32x4 av = ld16(&As[ks][buf][0][m * 16 + lr][u * 32 + lg * 8]);
        acc[m] = mfma_16x16x32(av, bw[u], acc[m]);
        if (TWO) {
          const u32x4 al = ld16(&As[ks][buf][NP - 1][m * 16 + lr][u * 32 + lg * 8]);
          acc[m] = mfma_16x16x32(al, bw[u], acc[m]);
        }
      }
    if (LOAD) {
      __builtin_amdgcn_sched_barrier(0);   // staging (waits for the activations) after the MFMAs
      stage(buf ^ 1);
    }
    __syncthreads();
  };
  using Load = std::integral_constant<bool, true>;
  using Last = std::integral_constant<bool, false>;
  // LM head: argmax keys of the groups done so far, per (row tile, row)
  uint64_t best[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) best[m][i] = 0;
  // fold the finished group's columns into best (and store its logits), then
  // start the next group
  auto group_end = [&](int J) {
    if (OUT != SO_ARGMAX || (J + 1) % nsub != 0) return;
    if (KS > 1) {
      // the other wave sets' sums join set 0's, in set order (the last
      // step's barrier ordered every earlier read of red before this write)
      if (ks > 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[ks - 1][m * 16 + lg * 4 + i][wave * 16 + lr] = acc[m][i];
      }
      __syncthreads();
      if (ks == 0) {
#pragma unroll
        for (int s2 = 0; s2 < KS - 1; ++s2)
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][i] += red[s2][m * 16 + lg * 4 + i][wave * 16 + lr];
      }
    }
    if (!a.draw.on && a.logits == nullptr) {
      // greedy, no logits: a select per value, no branch (a branch per
      // value over the noise and store code costs an instruction fetch)
      const int col = vcol0 + lr;
      const bool ok = col < N && ks == 0;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint64_t key = argmax_key(acc[m][i], (uint32_t)col);
          best[m][i] = ok && key > best[m][i] ? key : best[m][i];
          acc[m][i] = 0.f;
        }
    } else {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m * 16 + lg * 4 + i;
          const int col = vcol0 + lr;
          if (col < N && ks == 0) {
            const float v = acc[m][i];
            const float kv = a.draw.on ? v + gumbel_noise(a.draw.seed, (uint32_t)(row / a.gamma),
                                                          (uint32_t)(row % a.gamma), (uint32_t)col)
                                       : v;
            const uint64_t key = argmax_key(kv, (uint32_t)col);
            best[m][i] = key > best[m][i] ? key : best[m][i];
            if (a.logits != nullptr && row < M) a.logits[(size_t)row * N + col] = v;
          }
          acc[m][i] = 0.f;
        }
    }
    vcol0 = DYN ? sh_grp[(J / nsub + 1) & 1] * 64 + wave * 16 : vcol0 + 64;
  };
  // DYN: sub-chunk J ends the stream when it closes a group and the group
  // claimed after it is past the end
  auto last_dyn = [&](int J) {
    return (J + 1) % nsub == 0 && sh_grp[(J / nsub + 1) & 1] >= ngroups;
  };
  const int ngrp = OUT == SO_ARGMAX ? min(gpw, ngroups - grp) : 1;
  const int nj = ngrp * nsub;   // sub-chunks of this workgroup (static runs)
  int j = 0;
  if (DYN) {
    // nsub is even (>= 4): a group starts at an even sub-chunk, so its claim
    // (sub-chunk 0) and its publication (sub-chunk 1) share an iteration, and
    // the stream can only end at an odd sub-chunk
    for (;; j += 2) {
      unsigned claim = 0;   // made and used within this iteration
      step(Load{}, j, 0, bc, bn, claim);
      group_end(j);
      if (last_dyn(j + 1)) {
        step(Last{}, j + 1, 1, bn, bc, claim);
        group_end(j + 1);
        break;
      }
      step(Load{}, j + 1, 1, bn, bc, claim);
      group_end(j + 1);
    }
  } else {
  unsigned claim = 0;   // unused by static runs
  for (; j + 2 < nj; j += 2) {
    step(Load{}, j, 0, bc, bn, claim);
    group_end(j);
    step(Load{}, j + 1, 1, bn, bc, claim);
    group_end(j + 1);
  }
  if (nj - j == 2) {
    step(Load{}, j, 0, bc, bn, claim);
    group_end(j);
    step(Last{}, j + 1, 1, bn, bc, claim);
    group_end(j + 1);
  } else {
    step(Last{}, j, 0, bc, bn, claim);
    group_end(j);
  }
  }

  if (OUT == SO_ARGMAX) {
    // Row argmax keys (ordered value bits | inverted column): per wave over
    // its 16 columns, then over the 4 waves, then a 64-bit atomic max into
    // this XCD's slot of the row.  The last workgroup to arrive reads the 8
    // slots of every row (device-scope atomic loads), writes the block
    // tokens, and re-zeroes the slots and the counter for the next launch.
    __shared__ uint64_t wkeys[4][ROWS];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + lg * 4 + i;
        const uint64_t key = max16(best[m][i]);
        if (lr == 0 && ks == 0) wkeys[wave][row] = key;
      }
    __syncthreads();
    const bool lead = ks == 0;   // wave sets > 0 hold no keys (they still meet the barriers)
    const unsigned slot = xcc_id() & 7u;
    if (lead && tid < ROWS && tid < M) {
      uint64_t key = wkeys[0][tid];
#pragma unroll
      for (int w = 1; w < 4; ++w) key = wkeys[w][tid] > key ? wkeys[w][tid] : key;
      atomicMax(&a.amax[slot * 64 + tid], (unsigned long long)key);
    }
    __builtin_amdgcn_s_waitcnt(0);   // the atomics are performed
    __syncthreads();
    if (lead && tid == 0) sh_old = atomicAdd(a.actr, 1ull);
    __syncthreads();
    if (sh_old != (unsigned long long)(n_tiles - 1)) return;
    if (lead && tid < M) {
      uint64_t ks8[kXcds];
#pragma unroll
      for (int x = 0; x < kXcds; ++x)
        ks8[x] = __hip_atomic_load(&a.amax[x * 64 + tid], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
      // the anchor loads behind the slots (one wait for all)
      const int32_t anc = a.anchor ? a.anchor[tid / a.gamma] : 0;
      uint64_t key = 0;
#pragma unroll
      for (int x = 0; x < kXcds; ++x) key = ks8[x] > key ? ks8[x] : key;
      const int j = tid % a.gamma;
      a.block_tokens[tid] = j == 0 && a.anchor ? anc : (int32_t)argmax_key_index(key);
    }
    __syncthreads();
    if (!lead) return;
    for (int i = tid; i < kXcds * 64; i += 256) atomicExch(&a.amax[i], 0ull);
    if (tid == 0) atomicExch(a.actr, 0ull);
    if (DYN && tid == 0) atomicExch(a.wctr, 0u);
    return;
  }

  if (OUT == SO_STORE_SS && a.rope_out != nullptr) {
    // Side job for the K/V product that follows: the rotary (cos, sin)
    // table of the new tokens, entry e = t * dh/2 + i, spread over the
    // workgroups (numbered densely by tile and member).
    const int half = a.dh / 2, e = (tile * per + member) * 256 + tid;
    if (e < a.rope_rows * half) {
      const int t = e / half, i = e % half;
      const int b = seq_of(a.cu_new, a.batch, t);
      float cs, sn;
      rope_cs(a.ctx_lens[b] + (t - a.cu_new[b]), i, a.dh, (double)a.theta, &cs, &sn);
      a.rope_out[2 * (size_t)e] = cs;
      a.rope_out[2 * (size_t)e + 1] = sn;
    }
  }

  // partial slice of this group
  if (active) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + lg * 4 + i;
        const int col = vcol0 + lr;
        if (row < M && col < N) a.part[((size_t)split * M + row) * N + col] = acc[m][i];
      }
  }
  if (OUT == SO_PART) return;

  // Publish the slice and count the arrival: bits 0..15 count all arrivals,
  // the 6-bit field at 16 + 6x counts those from XCD x.  Workgroup i is
  // expected on XCD (i + rot) mod 8, rot being the rotation that workgroup 0
  // of the previous launch observed (it is fixed per hardware queue).
  const unsigned xcc = xcc_id();
  const unsigned homex = (unsigned)(xcd + rot) & 7u;
  const bool home = xcc == homex;
  if (blockIdx.x == 0 && tid == 0 && a.qhint_wr != nullptr) *a.qhint_wr = (xcc - (unsigned)xcd) & 7u;
  if (home) __builtin_amdgcn_s_waitcnt(0);   // this wave's stores are in the XCD's L2
  else __threadfence();                       // write back for readers on other XCDs
  __syncthreads();
  const unsigned long long mine = 1ull + (1ull << (16 + 6 * (xcc & 7u)));
  if (tid == 0) sh_old = atomicAdd(&a.ctr[tile], mine);
  __syncthreads();
  const unsigned long long tot = sh_old + mine;
  if ((int)(tot & 0xFFFFu) != per) return;

  bool foreign = false;   // partials written on another XCD
#pragma unroll
  for (int x = 0; x < kXcds; ++x)
    if ((unsigned)x != (xcc & 7u) && ((tot >> (16 + 6 * x)) & 63u) != 0) foreign = true;
  if (foreign) {
    __threadfence();
    if (!home && ((tot >> (16 + 6 * homex)) & 63u) != 0 && tid == 0) set_dev_error(a.err, kErrXcd);
  } else {
    asm volatile("buffer_inv sc0" ::: "memory");   // drop this CU's L1 copies
  }
  if (tid == 0) atomicExch(&a.ctr[tile], 0ull);

  if (OUT == SO_RESID) epi_resid<true>(a, S, tile);
  if (OUT == SO_STORE_SS) epi_resid<false>(a, S, tile);
  if (OUT == SO_QKV) epi_qkv(a, S, tile);
  if (OUT == SO_SWIGLU) epi_swiglu(a, S, tile);
  if (OUT == SO_KV) {
    epi_kv(a, S, tile);
    if (a.kvdone != nullptr) {
      // Every tile's epilogue has read ctx_lens before its finisher counts
      // itself here, so the last one may advance the lengths (the next
      // launch on the stream reads them).
      __syncthreads();   // this workgroup's epilogue reads are done
      __shared__ int sh_last;
      if (tid == 0) sh_last = atomicAdd(a.kvdone, 1u) == (unsigned)n_tiles - 1u;
      __syncthreads();
      if (sh_last) {
        for (int b = tid; b < a.batch; b += 256) a.ctx_lens_rw[b] += a.cu_new[b + 1] - a.cu_new[b];
        if (tid == 0) atomicExch(a.kvdone, 0u);
      }
    }
  }
}

// Gate/up product with the SwiGLU at one row tile (M <= 16), without split
// K: workgroup b owns the 16-column output tiles [T b, T b + T) of h; its
// waves 0 .. T-1 stream the gate rows of those tiles and waves T .. 2T-1 the
// up rows, each over all of K, straight from the packed gate/up layout (tile
// w of 64-row group 2 (r / 64) for gate row r, of group 2 (r / 64) + 1 for
// the up row).  The normalised activations are staged as in k_skinny by the
// first 256 threads (the other waves issue the same loads, so every wave
// keeps the same count of loads in flight).  At the end the gate sums pass
// through LDS to the up waves, which form silu(gate) * up; the workgroup then
// stores its 16 x 16T block of h as split planes.  No partial slices,
// arrival counters or last-arrival epilogue: with T = 3 and I = 12288, one
// workgroup per CU over 256 CUs.  Waves past the last tile re-read the last
// tile and store nothing.
constexpr int kGluTiles = 3;
constexpr int kGluMaxWgs = 256;   // one round on the chip, else the split-K path

template <int U, int T>
__global__ __launch_bounds__(128 * T, 1) void k_glu1(SkinnyArgs a) {
  constexpr int KC = 32 * U, CPR = KC / 8, NCH = 16 * CPR / 256;
  constexpr int LPR = 16;   // threads per row in the norm prologue
  static_assert(16 * CPR % 256 == 0 && 256 % CPR == 0, "sub-chunk must split evenly over 256 threads");
  static_assert(2 * T >= 4, "the first four waves stage the activations");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][2][16][KC + 8];
  __shared__ float inv_s[16];
  __shared__ float gx[T][16][17];
  __shared__ __attribute__((aligned(16))) float hy[16][16 * T];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int stid = tid & 255;   // staging slot (waves 4.. mirror waves 0..)
  const bool stager = tid < 256;
  const int M = a.M, K = a.K, I = a.I, ntl = I / 16;
  const int t = wave % T, ht0 = (int)blockIdx.x * T;
  const bool up = wave >= T;
  const int ht = ht0 + t < ntl ? ht0 + t : ntl - 1;
  const int r = 16 * ht, g = 2 * (r / 64) + (up ? 1 : 0), wt = (r % 64) / 16;
  const uint16_t* bp = a.packed + ((size_t)g * (K / 32) * 4 + wt) * 512 + lane * 8;
  auto wload = [&](int k, int u) { return ld16_stream(bp + (size_t)(k / 32 + u) * (4 * 512)); };

  int srow[NCH], scol[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = stid + i * 256;
    srow[i] = c / CPR;
    scol[i] = (c % CPR) * 8;
  }
  u32x4 r0[NCH], r1[NCH], rg;
  auto fetch = [&](int k) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int row = srow[i] < M ? srow[i] : M - 1;
      const float* xp = (const float*)a.A + (size_t)row * a.lda + k + scol[i];
      r0[i] = ld16(xp);
      r1[i] = ld16(xp + 4);
      if (i == 0) rg = ld16((const uint16_t*)a.gain + k + scol[i]);
    }
  };
  // y = x * inv * g, split into hi = bf16(y) and lo = bf16(y - hi)
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const float inv = inv_s[srow[i]];
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xa = __uint_as_float(e < 2 ? r0[i][2 * e] : r1[i][2 * e - 4]);
        const float xb = __uint_as_float(e < 2 ? r0[i][2 * e + 1] : r1[i][2 * e - 3]);
        const uint32_t gw = rg[e];
        const float ya = xa * inv * __uint_as_float(gw << 16);
        const float yb = xb * inv * __uint_as_float(gw & 0xFFFF0000u);
        hw[e] = pack_bf2(ya, yb);
        lw[e] = pack_bf2(ya - __uint_as_float(hw[e] << 16), yb - __uint_as_float(hw[e] & 0xFFFF0000u));
      }
      st16(&As[buf][0][srow[i]][scol[i]], u32x4{hw[0], hw[1], hw[2], hw[3]});
      st16(&As[buf][1][srow[i]][scol[i]], u32x4{lw[0], lw[1], lw[2], lw[3]});
    }
  };

  // Prologue: row sums of squares, the activations of sub-chunk 0, then its
  // weights (loads retire in order; the weights stay in flight meanwhile).
  constexpr int Q = kMaxSsTiles / LPR;
  const int nrm_row = stid / LPR, nrm_j = stid % LPR;
  float ssv[Q];
  {
    const int rr = nrm_row < M ? nrm_row : M - 1;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int i = q * LPR + nrm_j;
      ssv[q] = a.ss_in[(size_t)(i < a.ss_tiles ? i : a.ss_tiles - 1) * M + rr];
    }
  }
  fetch(0);
  u32x4 bc[U], bn[U];
#pragma unroll
  for (int u = 0; u < U; ++u) bc[u] = wload(0, u);
  __builtin_amdgcn_sched_barrier(0);
  {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) s += ssv[q] * (q * LPR + nrm_j < a.ss_tiles ? 1.f : 0.f);
    for (int m = 1; m < LPR; m <<= 1) s += __shfl_xor(s, m, 64);
    if (nrm_j == 0 && tid < 256) inv_s[nrm_row] = nrm_row < M ? 1.0f / sqrtf(s / (float)K + a.eps) : 0.f;
  }
  __syncthreads();
  if (stager) stage(0);
  __syncthreads();

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto step = [&](auto load_tag, int J, int buf, const u32x4* bw, u32x4* bnext) {
    constexpr bool LOAD = decltype(load_tag)::value;
    if (LOAD) {
      fetch((J + 1) * KC);
#pragma unroll
      for (int u = 0; u < U; ++u) bnext[u] = wload((J + 1) * KC, u);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4 ah = ld16(&As[buf][0][lr][u * 32 + lg * 8]);
      acc = mfma_16x16x32(ah, bw[u], acc);
      const u32x4 al = ld16(&As[buf][1][lr][u * 32 + lg * 8]);
      acc = mfma_16x16x32(al, bw[u], acc);
    }
    if (LOAD) {
      __builtin_amdgcn_sched_barrier(0);
      if (stager) stage(buf ^ 1);
    }
    __syncthreads();
  };
  using Load = std::integral_constant<bool, true>;
  using Last = std::integral_constant<bool, false>;
  const int nsub = K / KC;
  int j = 0;
  for (; j + 2 < nsub; j += 2) {
    step(Load{}, j, 0, bc, bn);
    step(Load{}, j + 1, 1, bn, bc);
  }
  if (nsub - j == 2) {
    step(Load{}, j, 0, bc, bn);
    step(Last{}, j + 1, 1, bn, bc);
  } else {
    step(Last{}, j, 0, bc, bn);
  }

  // silu(gate) * up, as the split-K epilogue computes it
  if (!up) {
#pragma unroll
    for (int i = 0; i < 4; ++i) gx[t][lg * 4 + i][lr] = acc[i];
  }
  __syncthreads();
  if (up) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gv = gx[t][lg * 4 + i][lr];
      hy[lg * 4 + i][t * 16 + lr] = gv / (1.0f + expf(-gv)) * acc[i];
    }
  }
  __syncthreads();
  for (int p = tid; p < 16 * 4 * T; p += 128 * T) {
    const int row = p / (4 * T), c4 = (p % (4 * T)) * 4, col = ht0 * 16 + c4;
    if (row < M && col < I) split_store4(a.h, a.h_plane, (size_t)row * I + col, *(const f32x4*)&hy[row][c4]);
  }
  // keep the split-K launches' XCD rotation hint current (see the publish step)
  if (blockIdx.x == 0 && tid == 0 && a.qhint_wr != nullptr) *a.qhint_wr = xcc_id() & 7u;
}

// Whether the gate/up product at one row tile takes k_glu1.
bool glu1_fits(const GemmPlan& p, const SkinnyArgs& a) {
  const int wgs = (a.I / 16 + kGluTiles - 1) / kGluTiles;
  return p.mt == 1 && a.M <= 16 && a.packed != nullptr && a.K % 512 == 0 && a.I % 64 == 0 &&
         a.N == 2 * a.I && wgs <= kGluMaxWgs;
}

// LM head over packed weights: about this many workgroups, each streaming a
// contiguous run of groups (one long chunk per workgroup keeps HBM pages open
// and pays the start and publish latency once).
constexpr int kArgmaxWgTarget = 512;
// Dynamic LM head with two wave sets per group: one 8-wave workgroup per CU.
constexpr int kArgmaxWgTargetKs = 256;

template <int MT, int ASRC, int OUT>
hipError_t run(const GemmPlan& p, const SkinnyArgs& a, int n_tiles, hipStream_t st) {
  const int per = tile_groups(OUT, a.dh) * p.splits;
  int gpw = 1;
  const bool w16 = (OUT == SO_ARGMAX || (MT > 1 && OUT != SO_SWIGLU && OUT != SO_KV)) &&
                   a.packed != nullptr && p.kpw % (32 * 16 / MT) == 0;
  bool dyn = false;
  if (OUT == SO_ARGMAX && a.packed != nullptr) {
    // dynamic groups need an even number (>= 4) of sub-chunks per group: the
    // claim is made at sub-chunk 0, published at 1 and used from the last
    const int nsub = p.kpw / (32 * 16 / MT);
    dyn = a.wctr != nullptr && w16 && nsub >= 4 && nsub % 2 == 0;
    if constexpr (OUT == SO_ARGMAX && MT == 1) {
      // two wave sets (each needs an even number >= 4 of sub-chunks); one
      // row tile only: at four (64 rows) the kernel spills and the 4 x 32K
      // draft measured 1775 -> 1873 us
      if (dyn && nsub >= 8 && nsub % 4 == 0) {
        n_tiles = n_tiles < kArgmaxWgTargetKs ? n_tiles : kArgmaxWgTargetKs;   // workgroups
        const int padded = (n_tiles + kXcds - 1) / kXcds * kXcds;
        hipLaunchKernelGGL((k_skinny<MT, ASRC, OUT, true, 16, true, 2>), dim3(padded * per),
                           dim3(512), 0, st, a, p.splits, p.kpw, n_tiles, gpw);
        return hipGetLastError();
      }
    }
    if (dyn) {
      n_tiles = n_tiles < kArgmaxWgTarget ? n_tiles : kArgmaxWgTarget;   // workgroups
    } else {
      gpw = (n_tiles + kArgmaxWgTarget - 1) / kArgmaxWgTarget;
      n_tiles = (n_tiles + gpw - 1) / gpw;   // workgroups
    }
  }
  const int padded = (n_tiles + kXcds - 1) / kXcds * kXcds;
  if (OUT == SO_ARGMAX && dyn) {
    hipLaunchKernelGGL((k_skinny<MT, ASRC, OUT, true, 16, OUT == SO_ARGMAX>), dim3(padded * per),
                       dim3(256), 0, st, a, p.splits, p.kpw, n_tiles, gpw);
    return hipGetLastError();
  }
  // 16 weight blocks per batch (512 columns at one row tile): half the
  // staging rounds and barriers per byte, at two workgroups per CU.  The LM
  // head always; with 2 or 4 row tiles also the unpaired products (at one row
  // tile they measured slower, and the paired ones at 640+ workgroups would
  // no longer fit one round).
  if (w16)
    hipLaunchKernelGGL((k_skinny<MT, ASRC, OUT, true, 16>), dim3(padded * per), dim3(256), 0, st,
                       a, p.splits, p.kpw, n_tiles, gpw);
  else if (a.packed != nullptr)
    hipLaunchKernelGGL((k_skinny<MT, ASRC, OUT, true>), dim3(padded * per), dim3(256), 0, st, a,
                       p.splits, p.kpw, n_tiles, gpw);
  else
    hipLaunchKernelGGL((k_skinny<MT, ASRC, OUT, false>), dim3(padded * per), dim3(256), 0, st, a,
                       p.splits, p.kpw, n_tiles, gpw);
  return hipGetLastError();
}

template <int ASRC, int OUT>
hipError_t run_mt(const GemmPlan& p, const SkinnyArgs& a, int n_tiles, hipStream_t st) {
  if (p.mt == 1) return run<1, ASRC, OUT>(p, a, n_tiles, st);
  if (p.mt == 2) return run<2, ASRC, OUT>(p, a, n_tiles, st);
  if (p.mt == 4) return run<4, ASRC, OUT>(p, a, n_tiles, st);
  return hipErrorInvalidValue;
}

// Pack the virtual rows [0, N) of a product's weight matrix (segments w;
// with swiglu_I > 0 the gate/up interleave of 64-row groups) into 16-row x
// 32-column tiles of 1 KB in MFMA lane order, ordered [64-row group g]
// [32-column block kb][16-row group w of the 64][tile]: 16-byte unit u =
// 64 t + l of tile t = (g * K/32 + kb) * 4 + w holds row 64 g + 16 w + l % 16,
// columns 32 kb + 8 (l / 16) .. + 7.  Rows N .. 64 ceil(N/64) - 1 are zero.
__global__ __launch_bounds__(256) void k_pack(WSeg w, int N, int K, int swiglu_I,
                                             uint16_t* __restrict__ out, size_t units) {
  const int kbs = K / 32;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
       u += (size_t)gridDim.x * blockDim.x) {
    const size_t t = u / 64;
    const int l = (int)(u % 64), wv = (int)(t % 4), kb = (int)((t / 4) % kbs);
    const int g = (int)(t / 4 / kbs);
    const int vrow = g * 64 + wv * 16 + l % 16, col = kb * 32 + (l / 16) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (vrow < N) {
      int row = vrow;
      if (swiglu_I > 0) {
        const int gg = vrow / 64;
        row = ((gg & 1) ? swiglu_I + 64 * (gg >> 1) : 64 * (gg >> 1)) + vrow % 64;
      }
      int sg = 0;
      while (sg < w.n - 1 && row >= w.row_end[sg]) ++sg;
      const int st = sg ? w.row_end[sg - 1] : 0;
      v = ld16((const uint16_t*)w.ptr[sg] + (size_t)(row - st) * K + col);
    }
    st16(out + u * 8, v);
  }
}

}  // namespace

size_t packed_elems(int N, int K) { return (size_t)((N + 63) / 64 * 64) * (size_t)K; }

hipError_t launch_pack(const WSeg& w, int N, int K, int swiglu_I, uint16_t* out, hipStream_t st) {
  if (N <= 0 || K % 32 || w.n < 1 || w.row_end[w.n - 1] < (swiglu_I > 0 ? 2 * swiglu_I : N))
    return hipErrorInvalidValue;
  if (swiglu_I > 0 && (N != 2 * swiglu_I || swiglu_I % 64)) return hipErrorInvalidValue;
  const size_t units = packed_elems(N, K) / 8;
  const size_t blocks = (units + 255) / 256;
  hipLaunchKernelGGL(k_pack, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, st,
                     w, N, K, swiglu_I, out, units);
  return hipGetLastError();
}

GemmPlan plan_skinny(int M, int N, int K, int out, int dh) {
  GemmPlan p{};
  p.kind = GEMM_SKINNY;
  p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.nt = 1;
  p.unroll = 8 / p.mt;
  p.waves = 4;
  const int kc = 32 * p.unroll, nk = K / kc;
  const int groups = (N + 63) / 64, tg = tile_groups(out, dh);
  int S = 1;
  if (out != SO_ARGMAX) {
    for (int s = 1; s <= nk; ++s) {
      if (nk % s) continue;
      if (s > kMaxSplits || tg * s > kMaxPer) break;
      S = s;
      const int target = (out == SO_SWIGLU || out == SO_KV) ? kWgTargetPaired
                         : out == SO_QKV                      ? kWgTargetQkv
                                                              : kWgTarget;
      if (groups * s >= target) break;
    }
  }
  p.splits = S;
  p.kpw = K / S;
  return p;
}

int skinny_tiles(int out, int N, int dh, int I) {
  if (out == SO_QKV || out == SO_KV) return (dh % 64 || N % dh) ? -1 : N / dh;
  if (out == SO_SWIGLU) return (N != 2 * I || I % 64) ? -1 : I / 64;
  if (out == SO_RESID || out == SO_STORE_SS) return N % 64 ? -1 : N / 64;
  return (N + 63) / 64;
}

hipError_t launch_skinny(const GemmPlan& p, int asrc, int out, const SkinnyArgs& a,
                         hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.M > 64 || p.kind != GEMM_SKINNY || p.splits < 1 || p.kpw * p.splits != a.K ||
      p.kpw % (32 * p.unroll) != 0 || p.unroll * p.mt != 8)
    return hipErrorInvalidValue;
  if ((p.mt == 1 && a.M > 16) || (p.mt == 2 && a.M > 32)) return hipErrorInvalidValue;
  const int n_tiles = skinny_tiles(out, a.N, a.dh, a.I);
  if (n_tiles < 0) return hipErrorInvalidValue;
  if (out == SO_ARGMAX && (p.splits != 1 || a.amax == nullptr || a.actr == nullptr ||
                           a.block_tokens == nullptr || a.gamma < 1))
    return hipErrorInvalidValue;
  if (tile_groups(out, a.dh) * p.splits > kMaxPer) return hipErrorInvalidValue;
  if ((asrc == SA_NORM || asrc == SA_NORM1) && (a.ss_in == nullptr || a.ss_tiles < 1 || a.ss_tiles > kMaxSsTiles ||
                          a.gain == nullptr))
    return hipErrorInvalidValue;
  if ((out == SO_QKV || out == SO_KV) && a.rope == nullptr) return hipErrorInvalidValue;
  if (out == SO_STORE_SS && a.rope_out != nullptr) {
    const long long wgs = (long long)n_tiles * tile_groups(out, a.dh) * p.splits;
    if (a.cu_new == nullptr || a.ctx_lens == nullptr || a.dh % 2 ||
        (long long)a.rope_rows * (a.dh / 2) > wgs * 256)
      return hipErrorInvalidValue;
  }
  if (asrc == SA_NORM && out == SO_SWIGLU && glu1_fits(p, a)) {
    const int wgs = (a.I / 16 + kGluTiles - 1) / kGluTiles;
    hipLaunchKernelGGL((k_glu1<16, kGluTiles>), dim3(wgs), dim3(128 * kGluTiles), 0, st, a);
    return hipGetLastError();
  }
#define DF_RUN(A_, O_) \
  if (asrc == A_ && out == O_) return run_mt<A_, O_>(p, a, n_tiles, st)
  DF_RUN(SA_NORM, SO_QKV);
  DF_RUN(SA_SPLIT, SO_RESID);
  DF_RUN(SA_NORM, SO_SWIGLU);
  DF_RUN(SA_NORM, SO_ARGMAX);
  DF_RUN(SA_BF16, SO_STORE_SS);
  DF_RUN(SA_NORM1, SO_KV);
#undef DF_RUN
  return hipErrorInvalidValue;
}
