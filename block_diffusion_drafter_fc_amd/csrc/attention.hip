// attention.hip -- block attention of the draft step.
//
// Every block query of sequence b sees the sequence's ctx_lens[b] cached
// context keys and all gamma block keys, with no mask inside the block
// (summary page, "Block Diffusion Makes Draft Cost Nearly Independent of Block
// Length" and Figure 2; paper §4.1).  Query head h reads KV head
// h / (Hq / Hkv).
//
// Split-context (flash-decode) layout: workgroup (s, kvh, b) owns one KV head
// of one sequence and one slice of keys -- context slice s < n_ctx_splits, or
// the block's own keys for query head kvh * G + (s - n_ctx_splits) -- and writes an
// unnormalised partial (running max in log2 units, sum of weights, weighted
// values) that k_attn_combine merges in split order.  Both kinds of slice run
// in one launch (the block's slice takes a uniform branch).
//
// bf16 context kernel: one wave per query head of the KV group, the gamma
// (<= 16) queries of that head form the N side of 16x16x32 MFMAs.  32 cached
// keys at a time are staged in LDS (K row-major, V transposed).  Scores are
// computed as S^T = K Q^T with the key rows of the two 16-row MFMA tiles
// interleaved so that each lane ends up holding 8 consecutive keys of one
// query -- exactly the B operand the P V product needs -- and the softmax
// max/sum runs over the 4 lanes of a query with two cross-lane shuffles.
// The cached K/V are exact bf16; the queries and the softmax weights are fp32
// values carried as hi+lo bf16 pairs, so each product is two MFMAs.
#include "common.h"
#include "kernels.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxCtxSplits = 256;            // bounded by plan_attention
constexpr int kMaxChunk = 1024;               // context keys per workgroup (64 pages)

// The block's own gamma keys: one workgroup per query head h of the KV
// group (workgroups s = n_ctx_splits + (h mod G) of the same grid), in fp32
// on the vector ALUs, since the block keys and values are transient fp32
// values.  The head's gamma queries (hi + lo planes summed), the KV head's
// block keys and values are staged in LDS; thread (j, k) of the first 256
// forms the score of query j and key k over the whole head dimension, the
// softmax runs over the 16 lanes of a query with shuffles, and thread
// (j, d8) then sums 8 output dimensions over the keys.  One head per
// workgroup keeps each thread's work to ~2 x DH multiply-adds.
template <int DH>
__device__ __forceinline__ void attn_block_keys(
    const uint16_t* __restrict__ q, size_t q_plane, const float* __restrict__ kb,
    const float* __restrict__ vb, int gamma, int Hq, int Hkv, int h, int kvh, int b, int B,
    int split, float* __restrict__ part_o, float* __restrict__ part_ml, float* __restrict__ lds,
    int causal) {
  constexpr int RS = DH + 4;   // padded row stride (floats)
  float* ks = lds;             // [16][RS] block keys
  float* vs = ks + 16 * RS;    // [16][RS] block values
  float* qs = vs + 16 * RS;    // [16][RS] the head's queries (fp32)
  float* ps = qs + 16 * RS;    // [16][16] weights of query j, key k
  const int tid = threadIdx.x, nthr = blockDim.x;
  for (int c = tid; c < gamma * (DH / 4); c += nthr) {
    const int r = c / (DH / 4), d = (c % (DH / 4)) * 4;
    const size_t off = ((size_t)(b * gamma + r) * Hkv + kvh) * DH + d;
    *(f32x4*)&ks[r * RS + d] = *(const f32x4*)&kb[off];
    *(f32x4*)&vs[r * RS + d] = *(const f32x4*)&vb[off];
    const size_t qo = ((size_t)(b * gamma + r) * Hq + h) * DH + d;
    const uint2 hi = *(const uint2*)(q + qo), lo = *(const uint2*)(q + q_plane + qo);
    qs[r * RS + d + 0] = bf2f((uint16_t)(hi.x & 0xFFFFu)) + bf2f((uint16_t)(lo.x & 0xFFFFu));
    qs[r * RS + d + 1] = bf2f((uint16_t)(hi.x >> 16)) + bf2f((uint16_t)(lo.x >> 16));
    qs[r * RS + d + 2] = bf2f((uint16_t)(hi.y & 0xFFFFu)) + bf2f((uint16_t)(lo.y & 0xFFFFu));
    qs[r * RS + d + 3] = bf2f((uint16_t)(hi.y >> 16)) + bf2f((uint16_t)(lo.y >> 16));
  }
  __syncthreads();
  const float sl2 = kLog2e / sqrtf((float)DH);
  const size_t prow = ((size_t)(split * B + b) * Hq + h) * gamma;   // partial row of query 0
  if (tid < 256) {
    // score of query j = tid / 16 and key k = tid % 16 (log2 units)
    const int j = tid >> 4, k = tid & 15;
    float dot = 0.f;
    if (j < gamma && k < gamma) {
#pragma unroll 8
      for (int d = 0; d < DH; d += 4) {
        const f32x4 qv = *(const f32x4*)&qs[j * RS + d];
        const f32x4 kv = *(const f32x4*)&ks[k * RS + d];
        dot = fmaf(qv[0], kv[0], dot);
        dot = fmaf(qv[1], kv[1], dot);
        dot = fmaf(qv[2], kv[2], dot);
        dot = fmaf(qv[3], kv[3], dot);
      }
    }
    const float sc = k < gamma && (!causal || k <= j) ? dot * sl2 : -INFINITY;
    float mx = sc;
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
    // key 0 is visible to every query, so mx is finite for j < gamma
    const float pw = j < gamma ? exp2f(sc - mx) : 0.f;
    float l = pw;
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) l += __shfl_xor(l, m, 64);
    ps[j * 16 + k] = pw;
    if (k == 0 && j < gamma) {
      part_ml[(prow + j) * 2 + 0] = mx;
      part_ml[(prow + j) * 2 + 1] = l;
    }
  }
  __syncthreads();
  // output dimensions 8 d8 .. 8 d8 + 7 of query j
  for (int c = tid; c < gamma * (DH / 8); c += nthr) {
    const int j = c / (DH / 8), d = (c % (DH / 8)) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < gamma; ++k) {
      const float pw = ps[j * 16 + k];
      const f32x4 v0 = *(const f32x4*)&vs[k * RS + d], v1 = *(const f32x4*)&vs[k * RS + d + 4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(pw, v0[e], acc[e]);
        acc[4 + e] = fmaf(pw, v1[e], acc[4 + e]);
      }
    }
    float* po = part_o + (prow + j) * DH + d;
    *(f32x4*)po = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4*)(po + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

// Context path.  A tile is 32 keys; a stage of the LDS ring holds its K rows
// (32 x DH bf16, row-major) and its values transposed (DH x 32), so both MFMA
// operands read 16 contiguous bytes per lane.  The cache stores each page's
// values already transposed ([head_dim][16]), so both halves of a stage are
// 1 KB blocks of contiguous memory that global_load_lds_dwordx4 moves straight
// into LDS (lane l's 16 bytes land at the block base + 16 l): no registers
// stage the tiles, the loads are fully coalesced, and NST - 1 tiles stay in
// flight.  The W waves of a workgroup issue the stage's blocks evenly; waves
// past the G query heads of the KV group only load.  Chunks sit
// XOR-swizzled within their rows (K: by kswz, V: by (row >> 1) & 3) so that
// the 16 rows a fragment read touches land in distinct banks; the swizzle is
// applied to the global source of each lane, the LDS placement being fixed.
template <int DH>
DF_DEV int kswz(int R) {
  return DH == 128 ? ((((R >> 3) << 2) | (R & 3)) & 15) : ((((R >> 3) << 1) | ((R >> 1) & 1)) & 7);
}
DF_DEV int vswz(int R) { return (R >> 1) & 3; }

typedef __attribute__((address_space(3))) void* attn_lds_t;

// Maximum over lanes l, l ^ 16, l ^ 32 and l ^ 48 of the wave, with the
// VALU row swaps (16-lane rows, then 32-lane halves) instead of two LDS
// permutes: each swap hands every lane the value of its partner row, so the
// max of the two returned halves is max(x[l], x[partner]).
DF_DEV float wave_max_xor16_32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// One direct-to-LDS load: the wave's 64 lanes each move 16 bytes from `src`
// to LDS address lds_base + 16 lane (lds_base wave-uniform, in M0).  Issued
// as inline assembly so that the compiler does not track the LDS write:
// given a load it cannot tell apart from the stage being read, it would wait
// for every load in flight before each LDS read and serialise the ring.  The
// caller orders reads after these loads itself (vmcnt wait, then s_barrier).
DF_DEV void lds_dma16(const void* src, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory", "m0");
}

// Workgroup -> (split, sequence) when the grid is larger than the GPU holds
// at once.  In launch order, Hkv consecutive workgroups (one per KV head)
// take one (split, sequence) pair, and the pairs run longest first: every
// sequence's full context splits, then the partly filled ones, then the
// block keys, then the empty splits.  Dealt in grid order, the pairs of a
// mixed batch would leave full splits waiting behind short ones for a
// second round of workgroups.  Every wave computes the same uniform result
// from the B <= 64 context lengths (one per lane): per sequence the counts
// of full, partial and empty splits, their running sums over sequences, and
// the first sequence whose running sum passes the pair's rank.
struct AttnItem {
  int s, b, L;
};
DF_DEV AttnItem attn_item_longest_first(int pair, const int32_t* __restrict__ ctx_lens, int B,
                                        int P, int G, int chunk, int cap, int report,
                                        uint32_t* err) {
  const int lane = threadIdx.x & 63;
  const int Lb = lane < B ? ctx_lens[lane] : 0;
  if (report && __ballot(lane < B && (Lb < 0 || Lb > cap)) != 0 && threadIdx.x == 0)
    set_dev_error(err, 2u);
  const int Lc = Lb < 0 ? 0 : Lb;
  const int fb = lane < B ? min(Lc / chunk, P) : 0;
  const int pb = lane < B && fb < P && Lc % chunk != 0 ? 1 : 0;
  const int eb = lane < B ? P - fb - pb : 0;
  int incf = fb, incp = pb, ince = eb;   // inclusive running sums over sequences
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int tf = __shfl_up(incf, o, 64), tp = __shfl_up(incp, o, 64),
              te = __shfl_up(ince, o, 64);
    if (lane >= o) {
      incf += tf;
      incp += tp;
      ince += te;
    }
  }
  const int F = __shfl(incf, 63, 64), Pp = __shfl(incp, 63, 64);
  int b, s;
  if (pair < F) {
    b = __ffsll((long long)__ballot(incf > pair)) - 1;
    s = pair - (__shfl(incf, b, 64) - __shfl(fb, b, 64));
  } else if (pair < F + Pp) {
    b = __ffsll((long long)__ballot(incp > pair - F)) - 1;
    s = __shfl(fb, b, 64);
  } else if (pair < F + Pp + B * G) {
    b = (pair - F - Pp) / G;           // the block keys: G heads per sequence
    s = P + (pair - F - Pp) % G;
  } else {
    const int idx = pair - F - Pp - B * G;
    b = __ffsll((long long)__ballot(ince > idx)) - 1;
    s = __shfl(fb, b, 64) + __shfl(pb, b, 64) + idx - (__shfl(ince, b, 64) - __shfl(eb, b, 64));
  }
  AttnItem it;
  it.b = __builtin_amdgcn_readfirstlane(b);
  it.s = __builtin_amdgcn_readfirstlane(s);
  it.L = __builtin_amdgcn_readfirstlane(__shfl(Lb, it.b, 64));
  return it;
}

template <int DH, int W, int NST>
// (4 waves: three workgroups per CU by registers; 8 waves: two)
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W == 4 ? 3 : 4))) void k_attn_ctx(
    const uint16_t* __restrict__ q, size_t q_plane, const float* __restrict__ kb,
    const float* __restrict__ vb, const uint16_t* __restrict__ pages, int n_pages,
    const int32_t* __restrict__ page_table, int max_pages, const int32_t* __restrict__ ctx_lens,
    int gamma, int Hq, int Hkv, int layer, int chunk, int n_ctx_splits,
    float* __restrict__ part_o, float* __restrict__ part_ml, uint32_t* err, int causal,
    int longest_first) {
  constexpr int KT = 32 * DH * 2;              // bytes of the K tile (= the V tile)
  constexpr int SB = 2 * KT;                   // bytes per stage
  constexpr int NB = SB / 1024;                // 1 KB load blocks per stage
  constexpr int NLW = NB / W;                  // blocks per wave
  static_assert(NB % W == 0, "stage blocks must split evenly over the waves");
  constexpr int CPR = DH / 8;                  // 16-byte chunks per K row
  constexpr int KPB = 1024 / (DH * 2);         // K rows per block
  constexpr int CTX_LDS = NST * SB;
  constexpr int BLK_LDS = (3 * 16 * (DH + 4) + 256) * 4;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[CTX_LDS > BLK_LDS ? CTX_LDS : BLK_LDS];
  __shared__ int pg_s[64];
  const int B = gridDim.z;
  const int G = Hq / Hkv;
  int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z, L = 0;
  if (longest_first) {
    const int lin = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    kvh = lin % Hkv;
    const AttnItem it = attn_item_longest_first(lin / Hkv, ctx_lens, B, n_ctx_splits, G, chunk,
                                                max_pages * 16, lin == 0, err);
    s = it.s;
    b = it.b;
    L = it.L;
  }
  if (s >= n_ctx_splits) {   // the block keys, one query head per workgroup
    attn_block_keys<DH>(q, q_plane, kb, vb, gamma, Hq, Hkv, kvh * G + (s - n_ctx_splits), kvh, b,
                        B, n_ctx_splits, part_o, part_ml, (float*)lds, causal);
    return;
  }
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const bool comp = wave < G;
  const int h = kvh * G + (comp ? wave : 0);
  const int kbeg = s * chunk;
  const int pg0 = kbeg >> 4;   // page-table slot of the split's first key
  constexpr int NI = DH / 32;   // MFMA K steps over the head dimension
  constexpr int ND = DH / 16;   // 16-row tiles of the head dimension
  // The context length, the Q fragments and the page-table entries of the
  // split's whole chunk (at most 64 pages; splits start at multiples of 16
  // keys) are loaded together, so the split waits for memory once before
  // its first tile.  Entries past the context are read (clamped to the
  // table) but not used.
  if (!longest_first) L = ctx_lens[b];
  int pg_raw = 0;
  if (wave == 0) {
    const int pi = pg0 + lane;
    pg_raw = page_table[(size_t)b * max_pages + (pi < max_pages ? pi : max_pages - 1)];
  }
  u32x4 qop[NI], qlo[NI];
  {
    const int row = b * gamma + (lr < gamma ? lr : 0);
    const uint16_t* qp = q + ((size_t)row * Hq + h) * DH + lg * 8;
#pragma unroll
    for (int i = 0; i < NI; ++i) {   // unpredicated loads, then a select (no branch)
      const u32x4 hi = ld16(qp + i * 32), lo = ld16(qp + q_plane + i * 32);
      qop[i] = lr < gamma ? hi : u32x4{0u, 0u, 0u, 0u};
      qlo[i] = lr < gamma ? lo : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // The splits cover the page table's capacity; a longer context (or a
  // negative one) cannot be read whole: report it (longest-first grids
  // report it while mapping their workgroups).
  if (!longest_first && s == 0 && kvh == 0 && tid == 0 && (L < 0 || L > max_pages * 16))
    set_dev_error(err, 2u);
  const int kend = min(kbeg + chunk, L);
  const size_t prow = ((size_t)(s * B + b) * Hq + h) * gamma;   // partial row of query 0
  if (kend <= kbeg) {
    if (comp && lg == 0 && lr < gamma) {
      part_ml[(prow + lr) * 2 + 0] = -INFINITY;
      part_ml[(prow + lr) * 2 + 1] = 0.f;
    }
    return;
  }
  // pages kbeg/16 .. (kend-1)/16 of the split; slots past the last repeat it
  const int npg = ((kend - 1) >> 4) - pg0 + 1;
  if (wave == 0) {
    const int sl = lane < npg ? lane : npg - 1;
    const int pg = __shfl(pg_raw, sl, 64);
    const int pi = pg0 + sl;
    const bool bad = pi >= max_pages || pg < 0 || pg >= n_pages;
    if (bad && lane < npg) set_dev_error(err, pi < max_pages ? 1u : 2u);
    pg_s[lane] = bad ? -1 : pg;
  }
  __syncthreads();   // pg_s; the Q loads are complete too

  const size_t kv_stride = (size_t)Hkv * 16 * DH;   // K part of a page -> its V part
  const uint16_t* lpages = pages + ((size_t)layer * n_pages * 2 * Hkv + kvh) * 16 * DH;
  const int ntile = (kend - kbeg + 31) >> 5;
  // Sources of this lane's blocks, relative to the page: K blocks hold KPB
  // key rows, V blocks 16 dimension rows of 4 chunks (8 keys each; chunks
  // 0-1 from the tile's first page, 2-3 from its second).
  int src_off[NLW];
  bool src_second[NLW];
#pragma unroll
  for (int jj = 0; jj < NLW; ++jj) {
    const int blk = wave + W * jj;
    if (blk < NB / 2) {
      const int R = blk * KPB + lane / CPR;
      const int c = (lane % CPR) ^ kswz<DH>(R);
      src_off[jj] = (R & 15) * DH + c * 8;
      src_second[jj] = R >= 16;
    } else {
      const int d = (blk - NB / 2) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ vswz(d);
      src_off[jj] = (int)kv_stride + d * 16 + (c & 1) * 8;
      src_second[jj] = c >= 2;
    }
  }
  auto page_of = [&](int slot) {   // page-table slot relative to pg0, clamped; bad -> page 0
    const int pg = pg_s[slot < npg ? slot : npg - 1];
    return pg < 0 ? 0 : pg;
  };
  auto issue = [&](int t) {
    unsigned char* base = lds + (t % NST) * SB;
    const int slot = 2 * t;   // kbeg is a multiple of 32 keys
    const size_t p0 = (size_t)page_of(slot) * 2 * kv_stride;
    const size_t p1 = (size_t)page_of(slot + 1) * 2 * kv_stride;
#pragma unroll
    for (int jj = 0; jj < NLW; ++jj)
      lds_dma16(lpages + (src_second[jj] ? p1 : p0) + src_off[jj],
                (uint32_t)(size_t)(attn_lds_t)(base + (wave + W * jj) * 1024));
  };
  // Stage t is complete for the workgroup once every lane has waited for
  // its own loads of tile t (at most `later` younger tiles' loads still
  // outstanding) and the waves have met at a bare s_barrier (the fence of
  // __syncthreads would also wait for the younger tiles' loads).
  auto stage_ready = [&](int later) {
    if (later >= 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NLW) : "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLW) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x4 o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = kLog2e / sqrtf((float)DH);
  const int ra = 8 * (lr >> 2) + (lr & 3), rb = ra + 4;

  // The running maximum m_run is kept in raw score units (the scale sl2 > 0
  // keeps the order) and folded into each exponent with one FMA.
  auto score = [&](int t, int valid, bool bad0, bool bad1) {
    const unsigned char* st = lds + (t % NST) * SB;
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = 4 * i + lg;   // dimensions i*32 + lg*8 .. +7
      const u32x4 ka = *(const u32x4*)(st + ra * (DH * 2) + ((c ^ kswz<DH>(ra)) << 4));
      const u32x4 kb2 = *(const u32x4*)(st + rb * (DH * 2) + ((c ^ kswz<DH>(rb)) << 4));
      sa = mfma_16x16x32(ka, qop[i], sa);
      sa = mfma_16x16x32(ka, qlo[i], sa);
      sb = mfma_16x16x32(kb2, qop[i], sb);
      sb = mfma_16x16x32(kb2, qlo[i], sb);
    }
    // lane (query lr, group lg) now holds keys 8*lg + 0..7 of the tile
    float sv[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = sa[r];
      sv[4 + r] = sb[r];
    }
    if (valid < 32 || bad0 || bad1) {   // uniform: only a split's last tile or a bad page
      const bool bad = lg < 2 ? bad0 : bad1;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (bad || 8 * lg + e >= valid) sv[e] = -INFINITY;
    }
    float mt = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    mt = wave_max_xor16_32(mt);
    const float m_new = fmaxf(m_run, mt);
    // while every key so far is masked the maximum stays -inf: using 0 in
    // the exponents then gives weights exp2(-inf) = 0
    const float mu = m_new == -INFINITY ? 0.f : m_new * sl2;
    const float alpha = __builtin_amdgcn_exp2f(m_run * sl2 - mu);   // 1 unless the max grew
    uint32_t pw[4], lw[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pa = __builtin_amdgcn_exp2f(fmaf(sv[2 * e], sl2, -mu));
      const float pb = __builtin_amdgcn_exp2f(fmaf(sv[2 * e + 1], sl2, -mu));
      pw[e] = pack_bf2(pa, pb);
      lw[e] = pack_bf2(pa - __uint_as_float(pw[e] << 16), pb - __uint_as_float(pw[e] & 0xFFFF0000u));
      psum += pa + pb;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
      for (int d = 0; d < ND; ++d) o[d] *= alpha;
    }
    const u32x4 pop = {pw[0], pw[1], pw[2], pw[3]}, plo = {lw[0], lw[1], lw[2], lw[3]};
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const int R = d * 16 + lr;
      const u32x4 vt = *(const u32x4*)(st + KT + R * 64 + ((lg ^ vswz(R)) << 4));
      o[d] = mfma_16x16x32(vt, pop, o[d]);
      o[d] = mfma_16x16x32(vt, plo, o[d]);
    }
  };

  // The Q fragments must be in registers before the ring starts: the
  // compiler does not count the ring's loads, and a wait of its own for Q
  // placed inside the loop would also wait for every tile in flight.
#pragma unroll
  for (int i = 0; i < NI; ++i) asm volatile("" ::"v"(qop[i]), "v"(qlo[i]));
  for (int t = 0; t < NST - 1 && t < ntile; ++t) issue(t);
  for (int t = 0; t < ntile; ++t) {
    stage_ready(min(ntile - 1 - t, NST - 2));
    if (t + NST - 1 < ntile) issue(t + NST - 1);
    const int valid = min(32, kend - (kbeg + 32 * t));
    const bool bad0 = pg_s[2 * t] < 0, bad1 = valid > 16 && pg_s[2 * t + 1] < 0;
    if (valid < 32 || bad0 || bad1) {
      // masked keys (past the split, or in a page outside the pool) get
      // zero values, so their zero weights never meet stale non-finite bits
      unsigned char* vt = lds + (t % NST) * SB + KT;
      for (int e = tid; e < DH * 32; e += 64 * W) {
        const int d = e >> 5, k = e & 31;
        if (k >= valid || (k < 16 ? bad0 : bad1))
          *(uint16_t*)(vt + d * 64 + ((((k >> 3) ^ vswz(d))) << 4) + (k & 7) * 2) = 0;
      }
      __syncthreads();
    }
    if (comp) score(t, valid, bad0, bad1);
  }
  if (!comp) return;
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (lr < gamma) {
    float* po = part_o + (prow + lr) * DH;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) po[d * 16 + 4 * lg + r] = o[d][r];
    if (lg == 0) {
      part_ml[(prow + lr) * 2 + 0] = m_run * sl2;   // log2 units (-inf stays -inf)
      part_ml[(prow + lr) * 2 + 1] = l_run;
    }
  }
}

// fp32 models: one workgroup per (query, head, sequence) over all keys, in
// chunks of 256 with an online softmax; writes the same partial layout as a
// single split.
__global__ __launch_bounds__(256) void k_attn_f32(
    const float* __restrict__ q, const float* __restrict__ kb, const float* __restrict__ vb,
    const float* __restrict__ pages, int n_pages, const int32_t* __restrict__ page_table,
    int max_pages, int page_size, const int32_t* __restrict__ ctx_lens, int gamma, int Hq,
    int Hkv, int dh, int layer, float* __restrict__ part_o, float* __restrict__ part_ml,
    uint32_t* err, int causal) {
  __shared__ float qs[256];
  __shared__ float ps[256];
  __shared__ const float* vrow[256];
  __shared__ int vstep[256];   // element stride of a value row (transposed pages: page_size)
  __shared__ float red[16];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, B = gridDim.z;
  const int kvh = h / (Hq / Hkv), tid = threadIdx.x;
  const int L = ctx_lens[b], total = L + gamma;
  const size_t qrow = (size_t)(b * gamma + j);
  if (tid < dh) qs[tid] = q[(qrow * Hq + h) * dh + tid];
  __syncthreads();
  const float sl2 = kLog2e / sqrtf((float)dh);
  float m_run = -INFINITY, l_run = 0.f, o_acc = 0.f;
  const size_t head_stride = (size_t)page_size * dh, kv_stride = (size_t)Hkv * head_stride;
  for (int c0 = 0; c0 < total; c0 += 256) {
    const int key = c0 + tid;
    float sc = -INFINITY;
    const float* kp = nullptr;
    const float* vp = nullptr;
    int vs = 1;
    if (key < total) {
      if (key < L) {
        const int pi = key / page_size;
        const int pg = pi < max_pages ? page_table[(size_t)b * max_pages + pi] : -1;
        if (pg >= 0 && pg < n_pages) {
          const float* page = pages + (((size_t)layer * n_pages + pg) * 2 * Hkv + kvh) * head_stride;
          kp = page + (size_t)(key % page_size) * dh;
          vp = page + kv_stride + key % page_size;   // values stored [dh][page_size]
          vs = page_size;
        } else {
          set_dev_error(err, pi < max_pages ? 1u : 2u);
        }
      } else if (!causal || key - L <= j) {
        kp = kb + ((size_t)(b * gamma + key - L) * Hkv + kvh) * dh;
        vp = vb + ((size_t)(b * gamma + key - L) * Hkv + kvh) * dh;
      }
      if (kp) {
        float acc = 0.f;
        for (int d = 0; d < dh; ++d) acc = fmaf(qs[d], kp[d], acc);
        sc = acc * sl2;
      }
    }
    vrow[tid] = vp;
    vstep[tid] = vs;
    // chunk maximum
    float mx = sc;
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) mx = fmaxf(mx, red[i]);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    const float p = (sc == -INFINITY) ? 0.f : exp2f(sc - m_new);
    ps[tid] = p;
    const float psum = block_sum(p, red);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    __syncthreads();
    if (tid < dh) {
      float acc = o_acc * alpha;
      const int n = min(256, total - c0);
      for (int t = 0; t < n; ++t)
        if (ps[t] != 0.f) acc = fmaf(ps[t], vrow[t][(size_t)tid * vstep[t]], acc);
      o_acc = acc;
    }
    __syncthreads();
  }
  const size_t prow = ((size_t)b * Hq + h) * gamma + j;   // split 0
  (void)B;
  if (tid < dh) part_o[prow * dh + tid] = o_acc;
  if (tid == 0) {
    part_ml[prow * 2 + 0] = m_run;
    part_ml[prow * 2 + 1] = l_run;
  }
}

// Workgroup (h, b, z) merges rows z*R .. z*R+R-1 of query head h of
// sequence b; thread t takes row z*R + t / (dh/4) and columns 4 (t % (dh/4))
// .. +3.  Each thread forms its row's weights 2^(m_s - max) in registers (the
// threads of a row read the same (max, sum) pairs, which the caches serve)
// and sums its columns over the parts in part order.  Up to PG parts
// (SINGLE) every load is issued before any arithmetic, so a thread waits for
// memory once; longer part lists run a max pass, then groups of PG parts.
template <bool BF16, int PG, bool SINGLE>
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      int n_parts, int gamma, int Hq, int dh,
                                                      int rows, void* __restrict__ o,
                                                      size_t o_plane) {
  const int h = blockIdx.x, b = blockIdx.y, B = gridDim.y;
  const int per = dh / 4;
  const int j = blockIdx.z * rows + threadIdx.x / per, d0 = (threadIdx.x % per) * 4;
  if (j >= gamma) return;
  const size_t stride = (size_t)B * Hq * gamma;            // partial rows per part
  const size_t pr0 = ((size_t)b * Hq + h) * gamma + j;
  const float2* ml_row = (const float2*)part_ml + pr0;
  // parts s0 .. s0+PG-1 of this thread's row and columns (past the end: empty)
  auto load = [&](int s0, float2* ml, f32x4* v) {
#pragma unroll
    for (int u = 0; u < PG; ++u) {
      if (s0 + u < n_parts) {
        ml[u] = ml_row[(s0 + u) * stride];
        v[u] = *(const f32x4*)(part_o + (pr0 + (s0 + u) * stride) * dh + d0);
      } else {
        ml[u] = make_float2(-INFINITY, 0.f);
        v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  float mx = -INFINITY;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  // an empty part (sum 0) may hold stale values: it is selected away, not
  // multiplied by a zero weight
  auto accumulate = [&](const float2* ml, const f32x4* v) {
#pragma unroll
    for (int u = 0; u < PG; ++u) {
      const bool live = ml[u].y > 0.f;
      const float w = live ? exp2f(ml[u].x - mx) : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = live ? acc[e] + w * v[u][e] : acc[e];
      den = live ? den + w * ml[u].y : den;
    }
  };
  if (SINGLE) {
    float2 ml[PG];
    f32x4 v[PG];
    load(0, ml, v);
#pragma unroll
    for (int u = 0; u < PG; ++u)
      if (ml[u].y > 0.f) mx = fmaxf(mx, ml[u].x);
    accumulate(ml, v);
  } else {
    for (int s0 = 0; s0 < n_parts; s0 += PG) {
      float2 ml[PG];
#pragma unroll
      for (int u = 0; u < PG; ++u)
        ml[u] = s0 + u < n_parts ? ml_row[(s0 + u) * stride] : make_float2(-INFINITY, 0.f);
#pragma unroll
      for (int u = 0; u < PG; ++u)
        if (ml[u].y > 0.f) mx = fmaxf(mx, ml[u].x);
    }
    for (int s0 = 0; s0 < n_parts; s0 += PG) {
      float2 ml[PG];
      f32x4 v[PG];
      load(s0, ml, v);
      accumulate(ml, v);
    }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  const size_t dst = ((size_t)(b * gamma + j) * Hq + h) * dh + d0;
#pragma unroll
  for (int e = 0; e < 4; ++e) Split<BF16>::store(o, o_plane, dst + e, acc[e] * inv);
}

// Longest-first order when the grid exceeds what the GPU holds at once
// (768 workgroups: three per CU), for batches of 2..64 sequences.
int longest_first(const AttnArgs& a, const AttnPlan& p) {
  const long wgs = (long)(p.n_ctx_splits + a.Hq / a.Hkv) * a.Hkv * a.batch;
  return a.batch > 1 && a.batch <= 64 && wgs > 768 ? 1 : 0;
}

template <int DH, int W, int NST>
hipError_t run_ctx1(const AttnArgs& a, const AttnPlan& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((k_attn_ctx<DH, W, NST>), grid, dim3(64 * W), 0, st, (const uint16_t*)a.q,
                     a.q_plane, (const float*)a.k, (const float*)a.v, (const uint16_t*)a.pages,
                     a.n_pages, a.page_table, a.max_pages, a.ctx_lens, a.gamma, a.Hq, a.Hkv,
                     a.layer, p.chunk, p.n_ctx_splits, a.part_o, a.part_ml, a.err, a.causal,
                     longest_first(a, p));
  return hipGetLastError();
}

// W = 4 waves for up to 4 query heads per KV head, else 8; NST stages of
// 2 * 32 * DH * 2 bytes (head dim 128: 3 stages, 48 KB, three workgroups per
// CU; head dim 64: 4 stages, 32 KB).
template <int DH>
hipError_t run_ctx(const AttnArgs& a, const AttnPlan& p, dim3 grid, hipStream_t st) {
  constexpr int NST = DH == 128 ? 3 : 4;
  if (a.Hq / a.Hkv <= 4) return run_ctx1<DH, 4, NST>(a, p, grid, st);
  return run_ctx1<DH, 8, NST>(a, p, grid, st);
}

}  // namespace

AttnPlan plan_attention(int batch, int n_kv_heads, int max_pages, int page_size) {
  AttnPlan p;
  const long cap = (long)max_pages * page_size;
  long chunk = (cap * batch * n_kv_heads + 1023) / 1024;
  const long min_chunk = (cap + kMaxCtxSplits - 1) / kMaxCtxSplits;
  if (chunk < min_chunk) chunk = min_chunk;
  const long merge_chunk = (cap + 22) / 23;
  if (chunk <= 128 && merge_chunk <= 128) {
    // small grids (batch 1): the shortest whole-tile chunk that keeps at
    // most 23 context splits, so the merge takes every part in one batch of
    // loads (96 keys for a 2048-token context, measured 2 us less per draft
    // than 128-key chunks)
    if (chunk < merge_chunk) chunk = merge_chunk;
    chunk = ((chunk + 31) / 32) * 32;
  } else {
    chunk = ((chunk + 127) / 128) * 128;   // whole groups of 4 tiles
  }
  if (chunk > kMaxChunk) chunk = kMaxChunk;
  p.chunk = (int)chunk;
  p.n_ctx_splits = (int)((cap + chunk - 1) / chunk);
  if (p.n_ctx_splits < 1) p.n_ctx_splits = 1;
  return p;
}

hipError_t launch_attention(bool bf16, const AttnArgs& a, const AttnPlan& p, hipStream_t st) {
  if (!bf16) {
    dim3 grid(a.gamma, a.Hq, a.batch);
    hipLaunchKernelGGL(k_attn_f32, grid, dim3(256), 0, st, (const float*)a.q, (const float*)a.k,
                       (const float*)a.v, (const float*)a.pages, a.n_pages, a.page_table,
                       a.max_pages, a.page_size, a.ctx_lens, a.gamma, a.Hq, a.Hkv, a.dh, a.layer,
                       a.part_o, a.part_ml, a.err, a.causal);
    return hipGetLastError();
  }
  // splits 0 .. n_ctx_splits-1: cached context; split n_ctx_splits: block keys
  dim3 grid(p.n_ctx_splits + a.Hq / a.Hkv, a.Hkv, a.batch);
  if (a.gamma > 16 || p.chunk > kMaxChunk || p.chunk % 32 || p.n_ctx_splits > kMaxCtxSplits ||
      a.page_size != 16 || a.Hq % a.Hkv != 0 || a.Hq / a.Hkv > 8 || a.n_pages < 1)
    return hipErrorInvalidValue;
  if (a.dh == 128) return run_ctx<128>(a, p, grid, st);
  if (a.dh == 64) return run_ctx<64>(a, p, grid, st);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_combine(bool bf16, const float* part_o, const float* part_ml, int n_parts,
                               int batch, int gamma, int Hq, int dh, void* o, size_t o_plane,
                               hipStream_t st) {
  if (dh % 4 != 0 || dh > 1024 || gamma < 1 || n_parts < 1) return hipErrorInvalidValue;
  // rows per workgroup: at least one full wave, then more rows while the
  // grid keeps >= 1024 workgroups, at most 256 threads
  const int per = dh / 4;
  int rows = 1;
  while (rows < gamma && rows * per < 64) rows *= 2;
  while (rows < gamma && 2 * rows * per <= 256 &&
         (long long)Hq * batch * ((gamma + 2 * rows - 1) / (2 * rows)) >= 1024)
    rows *= 2;
  if (rows > gamma) rows = gamma;
  dim3 grid(Hq, batch, (gamma + rows - 1) / rows);
  dim3 block(rows * per);
#define DF_COMB(BF, PG, SINGLE)                                                               \
  hipLaunchKernelGGL((k_attn_combine<BF, PG, SINGLE>), grid, block, 0, st, part_o, part_ml, n_parts, \
                     gamma, Hq, dh, rows, o, o_plane)
  if (bf16) {
    if (n_parts <= 8) DF_COMB(true, 8, true);
    else if (n_parts <= 24) DF_COMB(true, 24, true);
    else DF_COMB(true, 8, false);
  } else {
    if (n_parts <= 8) DF_COMB(false, 8, true);
    else if (n_parts <= 24) DF_COMB(false, 24, true);
    else DF_COMB(false, 8, false);
  }
#undef DF_COMB
  return hipGetLastError();
}
