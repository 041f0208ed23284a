// Lossless verification of sampled blocks (DFlash summary page, section on
// the target verifier as the correctness anchor).  Proposal k >= 1 was drawn
// from the drafter's row k; it is kept while u_k * p_d(x_k) < p_t(x_k), with
// p_t the target's row k - 1.  The first rejection is replaced by a draw
// from the positive part of p_t - p_d (from p_t itself when that part has no
// mass) and the rest of the block is dropped; a block kept whole earns a
// bonus token drawn from the target's last row.  A draw from r with uniform
// u is the smallest token v whose running sum of r exceeds u * sum(r).
//
// Probabilities are softmax values evaluated in fp64 from the fp32 or bf16
// logits, so every accept/reject decision and every draw is taken in fp64.
//
// Three launches:
//   k_row_stats    (chunk, row, target|draft): max and sum of exp(x - max)
//                  of one 4096-column chunk of one row;
//   k_draw_units   (chunk, sequence): repeats the accept/reject decision
//                  (cheap: 2 * gamma row combines and gamma - 1 lookups) and
//                  sums the final draw's distribution over 16-column units;
//   k_draw_finish  (sequence): scans the unit sums, walks the unit that holds
//                  the threshold and writes accept_len and out_tokens.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace {

constexpr int kChunk = 4096;                 // vocabulary columns per chunk
constexpr int kThreads = 256;                // threads of the chunk kernels
constexpr int kPer = kChunk / kThreads;      // columns per unit (one thread)
constexpr int kFinishThreads = 1024;

struct Decision {
  int tau;        // accepted proposals + 1
  int rej;        // 1: proposal tau was rejected (draw from the residual)
  size_t trow;    // target row of the final draw
  size_t drow;    // drafter row of the residual (rej only)
  double2 t;      // (max, sum of exp) of the target row
  double2 d;      // (max, sum of exp) of the drafter row (rej only)
};

template <bool BF16>
DF_DEV float logit_at(const void* p, size_t i) {
  if (BF16) return bf2f(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

DF_DEV double wave_sum(double v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

DF_DEV float wave_max(float v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Row statistics of one chunk: stats[(z * rows + r) * chunks + c] =
// (max, sum of exp(x - max)) over the chunk's columns; a chunk whose
// columns are all -inf stores (-inf, 0).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_row_stats(const void* __restrict__ target,
                                                         const float* __restrict__ draft,
                                                         int rows, int gamma, int vocab,
                                                         int chunks,
                                                         double2* __restrict__ stats) {
  __shared__ float redm[kThreads / 64];
  __shared__ double reds[kThreads / 64];
  const int z = blockIdx.z, r = blockIdx.y, c = blockIdx.x;
  if (z == 1 && r % gamma == 0) return;   // drafter row 0 holds the anchor: unused
  const int tid = threadIdx.x, w = tid >> 6;
  const int c0 = c * kChunk, c1 = min(vocab, c0 + kChunk);
  const size_t off = (size_t)r * vocab;
  auto x_at = [&](int v) -> float {
    return z == 0 ? logit_at<BF16>(target, off + v) : draft[off + v];
  };
  float m = -INFINITY;
  for (int v = c0 + tid; v < c1; v += kThreads) m = fmaxf(m, x_at(v));
  m = wave_max(m);
  if ((tid & 63) == 0) redm[w] = m;
  __syncthreads();
  m = redm[0];
  for (int i = 1; i < kThreads / 64; ++i) m = fmaxf(m, redm[i]);
  double s = 0.0;
  if (m > -INFINITY)
    for (int v = c0 + tid; v < c1; v += kThreads) s += exp((double)x_at(v) - (double)m);
  s = wave_sum(s);
  if ((tid & 63) == 0) reds[w] = s;
  __syncthreads();
  if (tid == 0) {
    double t = reds[0];
    for (int i = 1; i < kThreads / 64; ++i) t += reds[i];
    stats[((size_t)z * rows + r) * chunks + c] = make_double2((double)m, t);
  }
}

// (max, sum of exp(x - max)) of a whole row from its chunk statistics.
DF_DEV double2 combine_row(const double2* __restrict__ st, int chunks) {
  double m = -INFINITY;
  for (int c = 0; c < chunks; ++c) m = fmax(m, st[c].x);
  double s = 0.0;
  if (m > -INFINITY)
    for (int c = 0; c < chunks; ++c)
      if (st[c].x > -INFINITY) s += st[c].y * exp(st[c].x - m);
  return make_double2(m, s);
}

// The accept/reject pass of sequence b, run by a whole workgroup (at least
// 2 * gamma threads).  rs is LDS of 2 * gamma entries; the result lands in
// *dec for every thread.
template <bool BF16>
DF_DEV void decide(const int32_t* __restrict__ blk, const void* __restrict__ target,
                   const float* __restrict__ draft, const float* __restrict__ uniforms,
                   const double2* __restrict__ stats, int b, int rows, int gamma, int vocab,
                   int chunks, double2* rs, Decision* dec) {
  const int t = threadIdx.x;
  const size_t r0 = (size_t)b * gamma;
  if (t < 2 * gamma) {
    const int z = t / gamma, j = t % gamma;
    if (!(z == 1 && j == 0))
      rs[t] = combine_row(stats + ((size_t)z * rows + r0 + j) * chunks, chunks);
  }
  __syncthreads();
  if (t == 0) {
    int tau = gamma, rej = 0;
    for (int k = 1; k < gamma; ++k) {
      const int32_t x = blk[r0 + k];
      double p = 0.0, q = 0.0;   // a token outside the vocabulary is never kept
      if (x >= 0 && x < vocab) {
        p = exp((double)logit_at<BF16>(target, (r0 + k - 1) * vocab + x) - rs[k - 1].x) /
            rs[k - 1].y;
        q = exp((double)draft[(r0 + k) * vocab + x] - rs[gamma + k].x) / rs[gamma + k].y;
      }
      if (!((double)uniforms[r0 + k] * q < p)) {
        tau = k;
        rej = 1;
        break;
      }
    }
    dec->tau = tau;
    dec->rej = rej;
    dec->trow = r0 + (rej ? tau - 1 : gamma - 1);
    dec->drow = r0 + (rej ? tau : 0);
    dec->t = rs[rej ? tau - 1 : gamma - 1];
    dec->d = rej ? rs[gamma + tau] : make_double2(0.0, 1.0);
  }
  __syncthreads();
}

// Target probability and final-draw weight of token v: the residual
// max(0, p_t - p_d) after a rejection, p_t itself for the bonus token.
template <bool BF16>
DF_DEV void weights_at(const void* __restrict__ target, const float* __restrict__ draft,
                       const Decision& d, int vocab, int v, double& pt, double& res) {
  pt = exp((double)logit_at<BF16>(target, d.trow * vocab + v) - d.t.x) / d.t.y;
  res = pt;
  if (d.rej) {
    const double pd = exp((double)draft[d.drow * vocab + v] - d.d.x) / d.d.y;
    res = fmax(pt - pd, 0.0);
  }
}

// Sums of the final draw's weights over 16-column units:
// units[(b * chunks + c) * kThreads + t] = (sum of residual, sum of p_t) over
// columns [c * kChunk + t * kPer, +kPer).  Both sums are kept so that an
// empty residual can fall back to p_t without another pass.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_draw_units(
    const int32_t* __restrict__ blk, const void* __restrict__ target,
    const float* __restrict__ draft, const float* __restrict__ uniforms,
    const double2* __restrict__ stats, int rows, int gamma, int vocab, int chunks,
    double2* __restrict__ units) {
  __shared__ double2 rs[2 * kMaxVerifyBlock];
  __shared__ Decision dec;
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  decide<BF16>(blk, target, draft, uniforms, stats, b, rows, gamma, vocab, chunks, rs, &dec);
  const Decision d = dec;
  const int v0 = c * kChunk + t * kPer, v1 = min(vocab, v0 + kPer);
  double sr = 0.0, stt = 0.0;
  for (int v = v0; v < v1; ++v) {
    double pt, res;
    weights_at<BF16>(target, draft, d, vocab, v, pt, res);
    sr += res;
    stt += pt;
  }
  units[((size_t)b * chunks + c) * kThreads + t] = make_double2(sr, stt);
}

// Scan of one double per thread over the workgroup (Hillis-Steele in LDS,
// fixed order): the thread's exclusive prefix, and the total in *total.
DF_DEV double block_scan(double v, double* buf, double* total) {
  const int t = threadIdx.x, n = blockDim.x;
  buf[t] = v;
  __syncthreads();
  int src = 0;
  for (int d = 1; d < n; d <<= 1) {
    const double* in = buf + src * n;
    double* out = buf + (src ^ 1) * n;
    out[t] = t >= d ? in[t] + in[t - d] : in[t];
    __syncthreads();
    src ^= 1;
  }
  *total = buf[src * n + n - 1];
  return t > 0 ? buf[src * n + t - 1] : 0.0;
}

// Final draw and outputs of sequence b.  Thread i owns units [i * per,
// (i + 1) * per); the owner of the threshold T = u_0 * total is the first
// thread whose prefix plus its own sum exceeds T; it walks its units, then
// the unit's columns, with the same running sums.  Should rounding leave
// no sum above T, the last column of positive weight is taken.
template <bool BF16>
__global__ __launch_bounds__(kFinishThreads) void k_draw_finish(
    const int32_t* __restrict__ blk, const void* __restrict__ target,
    const float* __restrict__ draft, const float* __restrict__ uniforms,
    const double2* __restrict__ stats, const double2* __restrict__ units, int rows, int gamma,
    int vocab, int chunks, int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tokens) {
  __shared__ double2 rs[2 * kMaxVerifyBlock];
  __shared__ Decision dec;
  __shared__ double scan[2 * kFinishThreads];
  __shared__ int owner, last_pos, token;
  const int b = blockIdx.x, i = threadIdx.x;
  decide<BF16>(blk, target, draft, uniforms, stats, b, rows, gamma, vocab, chunks, rs, &dec);
  const Decision d = dec;
  const int n_units = chunks * kThreads;
  const int per = (n_units + kFinishThreads - 1) / kFinishThreads;
  const int u0 = min(n_units, i * per), u1 = min(n_units, u0 + per);
  const double2* un = units + (size_t)b * n_units;

  double g = 0.0, total;
  for (int u = u0; u < u1; ++u) g += un[u].x;
  double pre = block_scan(g, scan, &total);
  const bool use_t = !(total > 0.0);   // empty residual: draw from p_t
  if (use_t) {
    __syncthreads();
    g = 0.0;
    for (int u = u0; u < u1; ++u) g += un[u].y;
    pre = block_scan(g, scan, &total);
  }
  const double T = (double)uniforms[(size_t)b * gamma] * total;
  if (i == 0) {
    owner = 0x7FFFFFFF;
    last_pos = -1;
    token = 0;
  }
  __syncthreads();
  if (pre + g > T) atomicMin(&owner, i);
  if (g > 0.0) atomicMax(&last_pos, i);
  __syncthreads();
  const bool found = owner != 0x7FFFFFFF;
  if (i == (found ? owner : last_pos)) {
    // the unit: first whose running sum exceeds T, else the last positive one
    double acc = pre, acc_last = pre;
    int unit = -1, unit_last = -1;
    for (int u = u0; u < u1; ++u) {
      const double s = use_t ? un[u].y : un[u].x;
      if (found && acc + s > T) {
        unit = u;
        break;
      }
      if (s > 0.0) {
        unit_last = u;
        acc_last = acc;
      }
      acc += s;
    }
    if (unit < 0) {
      unit = unit_last;
      acc = acc_last;
    }
    int tok = -1, tok_last = -1;
    if (unit >= 0) {
      const int c = unit / kThreads, t = unit % kThreads;
      const int v0 = c * kChunk + t * kPer, v1 = min(vocab, v0 + kPer);
      for (int v = v0; v < v1; ++v) {
        double pt, res;
        weights_at<BF16>(target, draft, d, vocab, v, pt, res);
        const double wv = use_t ? pt : res;
        if (acc + wv > T) {
          tok = v;
          break;
        }
        if (wv > 0.0) tok_last = v;
        acc += wv;
      }
      if (tok < 0) tok = tok_last >= 0 ? tok_last : v0;
    }
    token = tok < 0 ? 0 : tok;
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
  return 16 * chunks * ((size_t)2 * batch * gamma + (size_t)batch * kThreads);
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
  double2* stats = (double2*)workspace;
  double2* units = stats + (size_t)2 * rows * chunks;
  const dim3 g1(chunks, rows, 2), g2(chunks, batch);
  if (bf16) {
    hipLaunchKernelGGL(k_row_stats<true>, g1, dim3(kThreads), 0, st, target, draft, rows, gamma,
                       vocab, chunks, stats);
    hipLaunchKernelGGL(k_draw_units<true>, g2, dim3(kThreads), 0, st, block_tokens, target, draft,
                       uniforms, stats, rows, gamma, vocab, chunks, units);
    hipLaunchKernelGGL(k_draw_finish<true>, dim3(batch), dim3(kFinishThreads), 0, st,
                       block_tokens, target, draft, uniforms, stats, units, rows, gamma, vocab,
                       chunks, accept_len, out_tokens);
  } else {
    hipLaunchKernelGGL(k_row_stats<false>, g1, dim3(kThreads), 0, st, target, draft, rows, gamma,
                       vocab, chunks, stats);
    hipLaunchKernelGGL(k_draw_units<false>, g2, dim3(kThreads), 0, st, block_tokens, target,
                       draft, uniforms, stats, rows, gamma, vocab, chunks, units);
    hipLaunchKernelGGL(k_draw_finish<false>, dim3(batch), dim3(kFinishThreads), 0, st,
                       block_tokens, target, draft, uniforms, stats, units, rows, gamma, vocab,
                       chunks, accept_len, out_tokens);
  }
  return hipGetLastError();
}
