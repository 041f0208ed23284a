// Lossless verification of sampled blocks (DFlash summary page, section on
// the target verifier as the correctness anchor).  Proposal k >= 1 was drawn
// from the drafter's row k; it is kept while u_k * p_d(x_k) < p_t(x_k), with
// p_t the target's row k - 1.  The first rejection is replaced by a draw
// from the positive part of p_t - p_d (from p_t itself when that part has no
// mass) and the rest of the block is dropped; a block kept whole earns a
// bonus token drawn from the target's last row.  A draw from r with uniform
// u is the smallest token v whose running sum of r exceeds u * sum(r).
//
// Every decision is the one fp64 softmax values give.  Five launches:
//   k_stats_fast   (chunk, row, target|drafter): max and sum of exp(x - max)
//                  of a 4096-column chunk, fp32 exponentials (HBM-bound);
//   k_decide_fast  (sequence): all proposals at once, one lane each, with
//                  the fp32 normalisers; a decision whose relative margin is
//                  below 1e-4 sends the sequence down the exact path;
//   k_stats_exact  (chunk, sequence, target|drafter): fp64 chunk statistics
//                  of the two rows the final draw reads, or of every row of
//                  a sequence on the exact path;
//   k_draw_units   (chunk, sequence): the final draw's weights summed over
//                  16-column units (fp64);
//   k_draw_finish  (sequence): scans the unit sums, walks the unit that holds
//                  the threshold and writes accept_len and out_tokens.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace {

constexpr int kChunk = 4096;                 // vocabulary columns per chunk
constexpr int kThreads = 256;                // threads of the chunk kernels
constexpr int kPer = kChunk / kThreads;      // columns per thread / per unit
constexpr int kFinishThreads = 1024;
// A decision taken with the fp32 normalisers is final when its relative
// margin exceeds this; their error is a few 1e-6 (fp32 exponentials of
// arguments that matter, |x - max| < 30, and 16-term fp32 partial sums).
constexpr double kCertify = 1e-4;

template <bool BF16>
DF_DEV float logit_at(const void* p, size_t i) {
  if (BF16) return bf2f(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

DF_DEV double wave_sum(double v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

DF_DEV double wave_max(double v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmax(v, __shfl_xor(v, m, 64));
  return v;
}

// The 16 columns of one chunk a thread reads, in registers.  Coalesced:
// piece j of lane l covers columns c0 + (j * 256 + tid) * W .. +W (W = 8 for
// bf16, 4 for fp32); columns at or past c1 read as -inf.  vec: the row base
// is 16-byte aligned and the chunk is whole, so 16-byte loads are used.
template <bool BF16>
DF_DEV void load_chunk(const void* row, int c0, int c1, bool vec, float (&x)[kPer]) {
  const int tid = threadIdx.x;
  if (BF16) {
    const uint16_t* p = (const uint16_t*)row;
    if (vec) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 v = ld16(p + c0 + (j * kThreads + tid) * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[j * 8 + 2 * e] = bf2f((uint16_t)(v[e] & 0xFFFFu));
          x[j * 8 + 2 * e + 1] = bf2f((uint16_t)(v[e] >> 16));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = c0 + (j * kThreads + tid) * 8 + e;
          x[j * 8 + e] = c < c1 ? bf2f(p[c]) : -INFINITY;
        }
    }
  } else {
    const float* p = (const float*)row;
    if (vec) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 v = ld16(p + c0 + (j * kThreads + tid) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[j * 4 + e] = __uint_as_float(v[e]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = c0 + (j * kThreads + tid) * 4 + e;
          x[j * 4 + e] = c < c1 ? p[c] : -INFINITY;
        }
    }
  }
}

// (max, sum of exp(x - max)) of the chunk over the workgroup; EXACT: terms
// in fp64, else fp32 exponentials summed per thread in fp32.  Every thread
// returns the result.
template <bool EXACT>
DF_DEV double2 chunk_stats(const float (&x)[kPer], double* red) {
  const int tid = threadIdx.x, w = tid >> 6;
  float m = x[0];
#pragma unroll
  for (int i = 1; i < kPer; ++i) m = fmaxf(m, x[i]);
  double md = wave_max((double)m);
  if ((tid & 63) == 0) red[w] = md;
  __syncthreads();
  md = red[0];
  for (int i = 1; i < kThreads / 64; ++i) md = fmax(md, red[i]);
  __syncthreads();
  double s = 0.0;
  if (md > -INFINITY) {
    if (EXACT) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) s += exp((double)x[i] - md);
    } else {
      const float mf = (float)md;
      float sf = 0.f;
#pragma unroll
      for (int i = 0; i < kPer; ++i) sf += __expf(x[i] - mf);
      s = sf;
    }
  }
  s = wave_sum(s);
  if ((tid & 63) == 0) red[w] = s;
  __syncthreads();
  double t = red[0];
  for (int i = 1; i < kThreads / 64; ++i) t += red[i];
  __syncthreads();
  return make_double2(md, t);
}

DF_DEV bool vec_ok(const void* base, int vocab, int c0, int c1, bool bf16) {
  return (((uintptr_t)base & 15) == 0) && (vocab % (bf16 ? 8 : 4)) == 0 && c1 - c0 == kChunk;
}

// Fast row statistics of every row: fast[(z * rows + r) * chunks + c] for
// z = 0 (target row r) and z = 1 (drafter row r; rows r % gamma == 0 hold
// the anchor and are skipped).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_stats_fast(const void* __restrict__ target,
                                                         const float* __restrict__ draft,
                                                         int rows, int gamma, int vocab,
                                                         int chunks, double2* __restrict__ fast) {
  __shared__ double red[kThreads / 64];
  const int z = blockIdx.z, r = blockIdx.y, c = blockIdx.x;
  if (z == 1 && r % gamma == 0) return;
  const int c0 = c * kChunk, c1 = min(vocab, c0 + kChunk);
  float x[kPer];
  if (z == 0) {
    const void* row = (const uint16_t*)target + (size_t)r * vocab * (BF16 ? 1 : 2);
    load_chunk<BF16>(row, c0, c1, vec_ok(target, vocab, c0, c1, BF16), x);
  } else {
    const float* row = draft + (size_t)r * vocab;
    load_chunk<false>(row, c0, c1, vec_ok(draft, vocab, c0, c1, false), x);
  }
  const double2 st = chunk_stats<false>(x, red);
  if (threadIdx.x == 0) fast[((size_t)z * rows + r) * chunks + c] = st;
}

// (max, sum of exp(x - max)) of a whole row from its chunk statistics, by
// one wave (lanes over chunks, fixed reduction order).
DF_DEV double2 combine_row(const double2* __restrict__ st, int chunks) {
  const int lane = threadIdx.x & 63;
  double m = -INFINITY;
  for (int c = lane; c < chunks; c += 64) m = fmax(m, st[c].x);
  m = wave_max(m);
  double s = 0.0;
  if (m > -INFINITY)
    for (int c = lane; c < chunks; c += 64)
      if (st[c].x > -INFINITY) s += st[c].y * exp(st[c].x - m);
  return make_double2(m, wave_sum(s));
}

// Combines rows of sequence b into rs[] (LDS, 2 * gamma entries: target rows
// 0..gamma-1, then drafter rows): all of them, or only the target row trow
// and the drafter row drow (drow < 0: none).  Rows are spread over waves.
DF_DEV void combine_rows(const double2* __restrict__ stats, int b, int rows, int gamma,
                         int chunks, bool all, int trow, int drow, double2* rs) {
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const size_t r0 = (size_t)b * gamma;
  if (all) {
    for (int ri = w; ri < 2 * gamma; ri += nw) {
      if (ri == gamma) continue;   // drafter row 0
      const int z = ri / gamma, j = ri % gamma;
      const double2 v = combine_row(stats + ((size_t)z * rows + r0 + j) * chunks, chunks);
      if ((threadIdx.x & 63) == 0) rs[ri] = v;
    }
  } else {
    if (w == 0) {
      const double2 v = combine_row(stats + (r0 + trow) * chunks, chunks);
      if ((threadIdx.x & 63) == 0) rs[trow] = v;
    }
    if (w == nw - 1 && drow >= 0) {
      const double2 v = combine_row(stats + ((size_t)rows + r0 + drow) * chunks, chunks);
      if ((threadIdx.x & 63) == 0) rs[gamma + drow] = v;
    }
  }
  __syncthreads();
}

// The accept/reject pass from the normalisers in rs[], by wave 0 (lane l
// takes proposal k = l + 1).  Writes tau, rej and (certify) whether a
// decision up to the first rejection lies within the certification margin.
template <bool BF16>
DF_DEV void proposals(const int32_t* __restrict__ blk, const void* __restrict__ target,
                      const float* __restrict__ draft, const float* __restrict__ uniforms,
                      const double2* rs, int b, int gamma, int vocab, bool certify, int* out3) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x, k = lane + 1;
    const size_t r0 = (size_t)b * gamma;
    bool rej = false, unc = false;
    if (k < gamma) {
      const int32_t x = blk[r0 + k];
      double p = 0.0, q = 0.0;   // a token outside the vocabulary is never kept
      if (x >= 0 && x < vocab) {
        p = exp((double)logit_at<BF16>(target, (r0 + k - 1) * vocab + x) - rs[k - 1].x) /
            rs[k - 1].y;
        q = exp((double)draft[(r0 + k) * vocab + x] - rs[gamma + k].x) / rs[gamma + k].y;
      }
      const double lhs = (double)uniforms[r0 + k] * q;
      rej = !(lhs < p);
      unc = certify && x >= 0 && x < vocab && !(fabs(lhs - p) > kCertify * fmax(lhs, p));
    }
    const uint64_t rm = __ballot(rej), um = __ballot(unc);
    if (lane == 0) {
      const int first = rm ? __builtin_ctzll(rm) : 64;       // lane of the first rejection
      const uint64_t upto = first >= 63 ? ~0ull : ((2ull << first) - 1);
      out3[0] = rm ? first + 1 : gamma;
      out3[1] = rm ? 1 : 0;
      out3[2] = (um & upto) ? 1 : 0;
    }
  }
  __syncthreads();
}

// Fast decision per sequence: dec[b] = (tau, rej, needs the exact path).
// 16 waves, so that the 2 * gamma row combines run two per wave.
template <bool BF16>
__global__ __launch_bounds__(kFinishThreads) void k_decide_fast(
    const int32_t* __restrict__ blk, const void* __restrict__ target,
    const float* __restrict__ draft, const float* __restrict__ uniforms,
    const double2* __restrict__ fast, int rows, int gamma, int vocab, int chunks,
    int4* __restrict__ dec) {
  __shared__ double2 rs[2 * kMaxVerifyBlock];
  __shared__ int d3[3];
  const int b = blockIdx.x;
  combine_rows(fast, b, rows, gamma, chunks, true, 0, -1, rs);
  proposals<BF16>(blk, target, draft, uniforms, rs, b, gamma, vocab, true, d3);
  if (threadIdx.x == 0) dec[b] = make_int4(d3[0], d3[1], d3[2], 0);
}

// Exact (fp64) chunk statistics of the rows the final draw reads (target
// row tau - 1 or gamma - 1, drafter row tau after a rejection), or of every
// row of a sequence whose fast decision was not certified.  z = 0 target,
// z = 1 drafter.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_stats_exact(
    const void* __restrict__ target, const float* __restrict__ draft,
    const int4* __restrict__ dec, int rows, int gamma, int vocab, int chunks,
    double2* __restrict__ exact) {
  __shared__ double red[kThreads / 64];
  const int z = blockIdx.z, b = blockIdx.y, c = blockIdx.x;
  const int4 d = dec[b];
  const int c0 = c * kChunk, c1 = min(vocab, c0 + kChunk);
  int j0, j1;
  if (d.z) {                       // every row of this kind
    j0 = z == 0 ? 0 : 1;
    j1 = gamma;
  } else if (z == 0) {
    j0 = d.y ? d.x - 1 : gamma - 1;
    j1 = j0 + 1;
  } else {
    if (!d.y) return;
    j0 = d.x;
    j1 = j0 + 1;
  }
  for (int j = j0; j < j1; ++j) {
    const size_t r = (size_t)b * gamma + j;
    float x[kPer];
    if (z == 0)
      load_chunk<BF16>((const uint16_t*)target + r * vocab * (BF16 ? 1 : 2), c0, c1,
                       vec_ok(target, vocab, c0, c1, BF16), x);
    else
      load_chunk<false>(draft + r * vocab, c0, c1, vec_ok(draft, vocab, c0, c1, false), x);
    const double2 st = chunk_stats<true>(x, red);
    if (threadIdx.x == 0) exact[((size_t)z * rows + r) * chunks + c] = st;
  }
}

struct Decision {
  int tau;        // accepted proposals + 1
  int rej;        // 1: proposal tau was rejected (draw from the residual)
  size_t trow;    // target row of the final draw
  size_t drow;    // drafter row of the residual (rej only)
  double2 t;      // exact (max, 1 / sum of exp) of the target row
  double2 d;      // exact (max, 1 / sum of exp) of the drafter row (rej only)
};

// The final decision of sequence b with exact normalisers of the draw rows:
// the fast one when it was certified, else the accept/reject pass redone
// from exact statistics of every row.  Whole workgroup; result in *dec.
template <bool BF16>
DF_DEV void final_decision(const int32_t* __restrict__ blk, const void* __restrict__ target,
                           const float* __restrict__ draft, const float* __restrict__ uniforms,
                           const int4* __restrict__ fdec, const double2* __restrict__ exact,
                           int b, int rows, int gamma, int vocab, int chunks, double2* rs,
                           int* d3, Decision* dec) {
  const int4 f = fdec[b];
  int tau = f.x, rej = f.y;
  if (f.z) {
    combine_rows(exact, b, rows, gamma, chunks, true, 0, -1, rs);
    proposals<BF16>(blk, target, draft, uniforms, rs, b, gamma, vocab, false, d3);
    tau = d3[0];
    rej = d3[1];
  } else {
    combine_rows(exact, b, rows, gamma, chunks, false, rej ? tau - 1 : gamma - 1,
                 rej ? tau : -1, rs);
  }
  if (threadIdx.x == 0) {
    const size_t r0 = (size_t)b * gamma;
    dec->tau = tau;
    dec->rej = rej;
    dec->trow = r0 + (rej ? tau - 1 : gamma - 1);
    dec->drow = r0 + (rej ? tau : 0);
    const double2 t = rs[rej ? tau - 1 : gamma - 1];
    const double2 dr = rej ? rs[gamma + tau] : make_double2(0.0, 1.0);
    dec->t = make_double2(t.x, 1.0 / t.y);
    dec->d = make_double2(dr.x, 1.0 / dr.y);
  }
  __syncthreads();
}

// Target probability and final-draw weight of a token from its target and
// drafter logits: the residual max(0, p_t - p_d) after a rejection, p_t
// itself for the bonus token.
DF_DEV void weights_from(float xt, float xd, const Decision& d, double& pt, double& res) {
  // p_t and p_d are each rounded before the difference: a fused multiply-add
  // would leave rounding noise where the two rows agree and the residual
  // must be empty.
#pragma clang fp contract(off)
  pt = exp((double)xt - d.t.x) * d.t.y;
  res = pt;
  if (d.rej) {
    const double pd = exp((double)xd - d.d.x) * d.d.y;
    res = fmax(pt - pd, 0.0);
  }
}

// Sums of the final draw's weights over 16-column units:
// units[(b * chunks + c) * 256 + t] = (sum of residual, sum of p_t) over
// columns [c * kChunk + t * kPer, +kPer).  Both sums are kept so that an
// empty residual can fall back to p_t without another pass.  Four lanes
// share a unit (4 columns each) and add their parts in a fixed order.
template <bool BF16>
__global__ __launch_bounds__(kFinishThreads) void k_draw_units(
    const int32_t* __restrict__ blk, const void* __restrict__ target,
    const float* __restrict__ draft, const float* __restrict__ uniforms,
    const int4* __restrict__ fdec, const double2* __restrict__ exact, int rows, int gamma,
    int vocab, int chunks, double2* __restrict__ units) {
  __shared__ double2 rs[2 * kMaxVerifyBlock];
  __shared__ int d3[3];
  __shared__ Decision dec;
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  final_decision<BF16>(blk, target, draft, uniforms, fdec, exact, b, rows, gamma, vocab, chunks,
                       rs, d3, &dec);
  const Decision d = dec;
  const int unit = t >> 2, part = t & 3;
  const int v0 = c * kChunk + unit * kPer + part * 4, v1 = min(vocab, v0 + 4);
  float xt[4], xd[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {           // every load in flight before any arithmetic
    const bool in = v0 + e < v1;
    xt[e] = in ? logit_at<BF16>(target, d.trow * vocab + v0 + e) : -INFINITY;
    xd[e] = in && d.rej ? draft[d.drow * vocab + v0 + e] : -INFINITY;
  }
  double sr = 0.0, stt = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (v0 + e < v1) {
      double pt, res;
      weights_from(xt[e], xd[e], d, pt, res);
      sr += res;
      stt += pt;
    }
  }
  sr += __shfl_xor(sr, 1, 64);
  stt += __shfl_xor(stt, 1, 64);
  sr += __shfl_xor(sr, 2, 64);
  stt += __shfl_xor(stt, 2, 64);
  if (part == 0) units[((size_t)b * chunks + c) * (kChunk / kPer) + unit] = make_double2(sr, stt);
}

DF_DEV double wave_incl_scan(double v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double n = __shfl_up(v, d, 64);
    if (lane >= d) v += n;
  }
  return v;
}

// Exclusive prefix of one double per thread over the workgroup (wave scans,
// then the wave totals in wave order); the total lands in *total.
DF_DEV double block_excl_scan(double v, double* wsum, double* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const double inc = wave_incl_scan(v);
  double ex = __shfl_up(inc, 1, 64);
  if (lane == 0) ex = 0.0;
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  double base = 0.0, tot = 0.0;
  for (int k = 0; k < nw; ++k) {
    if (k == w) base = tot;
    tot += wsum[k];
  }
  __syncthreads();
  *total = tot;
  return base + ex;
}

// Final draw and outputs of sequence b.  Thread i owns units [i * per,
// (i + 1) * per); the owner of the threshold T = u_0 * total is the first
// thread whose prefix plus its own sum exceeds T.  The owner's wave then
// scans the owner's units, and the chosen unit's 16 columns, lane-parallel,
// taking the first position whose running sum exceeds T.  Should rounding
// leave no sum above T, the last position of positive weight is taken.
template <bool BF16>
__global__ __launch_bounds__(kFinishThreads) void k_draw_finish(
    const int32_t* __restrict__ blk, const void* __restrict__ target,
    const float* __restrict__ draft, const float* __restrict__ uniforms,
    const int4* __restrict__ fdec, const double2* __restrict__ exact,
    const double2* __restrict__ units, int rows, int gamma, int vocab, int chunks,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tokens) {
  __shared__ double2 rs[2 * kMaxVerifyBlock];
  __shared__ int d3[3];
  __shared__ Decision dec;
  __shared__ double wsum[kFinishThreads / 64];
  __shared__ int owner, last_pos, token;
  const int b = blockIdx.x, i = threadIdx.x, lane = i & 63;
  final_decision<BF16>(blk, target, draft, uniforms, fdec, exact, b, rows, gamma, vocab, chunks,
                       rs, d3, &dec);
  const Decision d = dec;
  const int n_units = chunks * kThreads;
  const int per = (n_units + kFinishThreads - 1) / kFinishThreads;
  const int u0 = min(n_units, i * per), u1 = min(n_units, u0 + per);
  const double2* un = units + (size_t)b * n_units;

  double g = 0.0, total;
  for (int u = u0; u < u1; ++u) g += un[u].x;
  double pre = block_excl_scan(g, wsum, &total);
  const bool use_t = !(total > 0.0);   // empty residual: draw from p_t
  if (use_t) {
    g = 0.0;
    for (int u = u0; u < u1; ++u) g += un[u].y;
    pre = block_excl_scan(g, wsum, &total);
  }
  const double T = (double)uniforms[(size_t)b * gamma] * total;
  if (i == 0) {
    owner = 0x7FFFFFFF;
    last_pos = -1;
    token = 0;
  }
  __syncthreads();
  {  // one LDS atomic per wave: its lowest lane above T, its highest positive lane
    const uint64_t above = __ballot(pre + g > T), pos = __ballot(g > 0.0);
    if (lane == 0 && above) atomicMin(&owner, (i & ~63) + __builtin_ctzll(above));
    if (lane == 0 && pos) atomicMax(&last_pos, (i & ~63) + 63 - __builtin_clzll(pos));
  }
  __syncthreads();
  const bool found = owner != 0x7FFFFFFF;
  const int own = found ? owner : last_pos;
  if (own >= 0 && (i >> 6) == (own >> 6)) {
    // the unit: first whose running sum exceeds T, else the last positive one
    const int ou0 = min(n_units, own * per), ou1 = min(n_units, ou0 + per);
    double acc = __shfl(pre, own & 63, 64);
    int unit = -1, last_u = -1;
    double unit_acc = acc, last_acc = acc;
    for (int base = ou0; base < ou1 && unit < 0; base += 64) {
      const int u = base + lane;
      const bool in = u < ou1;
      const double sv = in ? (use_t ? un[u].y : un[u].x) : 0.0;
      const double inc = wave_incl_scan(sv);
      double ex = __shfl_up(inc, 1, 64);
      if (lane == 0) ex = 0.0;
      const uint64_t hm = __ballot(found && in && acc + inc > T);
      const uint64_t pm = __ballot(in && sv > 0.0);
      if (hm) {
        const int l = __builtin_ctzll(hm);
        unit = base + l;
        unit_acc = acc + __shfl(ex, l, 64);
      } else {
        if (pm) {
          const int l = 63 - __builtin_clzll(pm);
          last_u = base + l;
          last_acc = acc + __shfl(ex, l, 64);
        }
        acc += __shfl(inc, 63, 64);
      }
    }
    if (unit < 0) {
      unit = last_u;
      unit_acc = last_acc;
    }
    int tok = 0;
    if (unit >= 0) {
      const int c = unit / kThreads, t = unit % kThreads;
      const int v0 = c * kChunk + t * kPer, v1 = min(vocab, v0 + kPer);
      const int v = v0 + lane;
      const bool in = lane < kPer && v < v1;
      double wv = 0.0;
      if (in) {
        const float xt = logit_at<BF16>(target, d.trow * vocab + v);
        const float xd = d.rej ? draft[d.drow * vocab + v] : -INFINITY;
        double pt, res;
        weights_from(xt, xd, d, pt, res);
        wv = use_t ? pt : res;
      }
      const double inc = wave_incl_scan(wv);
      const uint64_t hm = __ballot(in && unit_acc + inc > T);
      const uint64_t pm = __ballot(in && wv > 0.0);
      tok = hm ? v0 + __builtin_ctzll(hm) : (pm ? v0 + 63 - __builtin_clzll(pm) : v0);
    }
    if (i == own) token = tok;
  }
  __syncthreads();
  if (i < gamma) {
    const size_t r0 = (size_t)b * gamma;
    out_tokens[r0 + i] = i < d.tau - 1 ? blk[r0 + i + 1] : (i == d.tau - 1 ? token : -1);
    if (i == 0) accept_len[b] = d.tau;
  }
}

}  // namespace

size_t verify_sampled_ws_bytes(int batch, int gamma, int vocab) {
  const size_t chunks = ((size_t)vocab + kChunk - 1) / kChunk;
  return 16 * (chunks * ((size_t)4 * batch * gamma + (size_t)batch * kThreads) + (size_t)batch);
}

hipError_t launch_verify_sampled(bool bf16, const int32_t* block_tokens, const void* target,
                                 const float* draft, const float* uniforms, int batch, int gamma,
                                 int vocab, void* workspace, int32_t* accept_len,
                                 int32_t* out_tokens, hipStream_t st) {
  if (batch < 1 || gamma < 1 || gamma > kMaxVerifyBlock || vocab < 1 ||
      (long long)batch * gamma > 65535)
    return hipErrorInvalidValue;
  const int rows = batch * gamma;
  const int chunks = (vocab + kChunk - 1) / kChunk;
  double2* fast = (double2*)workspace;
  double2* exact = fast + (size_t)2 * rows * chunks;
  double2* units = exact + (size_t)2 * rows * chunks;
  int4* dec = (int4*)(units + (size_t)batch * chunks * kThreads);
  const dim3 g_rows(chunks, rows, 2), g_seq2(chunks, batch, 2), g_seq(chunks, batch);
#define DF_VS(B)                                                                               \
  hipLaunchKernelGGL(k_stats_fast<B>, g_rows, dim3(kThreads), 0, st, target, draft, rows,     \
                     gamma, vocab, chunks, fast);                                              \
  hipLaunchKernelGGL(k_decide_fast<B>, dim3(batch), dim3(kFinishThreads), 0, st, block_tokens, \
                     target, draft, uniforms, fast, rows, gamma, vocab, chunks, dec);          \
  hipLaunchKernelGGL(k_stats_exact<B>, g_seq2, dim3(kThreads), 0, st, target, draft, dec,     \
                     rows, gamma, vocab, chunks, exact);                                       \
  hipLaunchKernelGGL(k_draw_units<B>, g_seq, dim3(kFinishThreads), 0, st, block_tokens, target,\
                     draft, uniforms, dec, exact, rows, gamma, vocab, chunks, units);          \
  hipLaunchKernelGGL(k_draw_finish<B>, dim3(batch), dim3(kFinishThreads), 0, st,              \
                     block_tokens, target, draft, uniforms, dec, exact, units, rows, gamma,    \
                     vocab, chunks, accept_len, out_tokens)
  if (bf16) {
    DF_VS(true);
  } else {
    DF_VS(false);
  }
#undef DF_VS
  return hipGetLastError();
}
