// Packed multi-block forward (DFlash summary page, section "Training
// Rehearses the Same Masked Blocks Used at Runtime", Figure 4; paper §4.2):
// several blocks of one sequence in one pass, block b anchored at position
// anchor_pos[b], its rows seeing the context keys [0, anchor_pos[b]) and the
// keys of their own block.  That mask is the draft's own attention for a
// batch whose sequences share one page table and whose context lengths are
// the anchor positions, so the pass is a draft over such a batch; this file
// holds the set-up of that batch and the loss.
//
// Loss (summary page, section "Early Positions Receive More Learning
// Budget"; paper §4.2 eq. 1): block b's loss is sum_k w_k CE_k / sum_k w_k
// over its predicted positions k = 1 .. gamma-1, w_k = exp(-(k-1)/decay),
// CE_k = logsumexp(logits_k) - logits_k[target_k]; the pass's loss is the
// mean of the block losses.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace {

constexpr int kCeThreads = 1024;

// table[b][p] = row[p]; lens[b] = anchor_pos[b], which must lie in
// [0, ctx_len] (else DFLASH_DEVERR_POS and the nearest bound).
__global__ void k_packed_setup(const int32_t* __restrict__ row, int max_pages,
                               const int32_t* __restrict__ ctx_len,
                               const int32_t* __restrict__ anchor_pos, int n_blocks,
                               int32_t* __restrict__ table, int32_t* __restrict__ lens,
                               uint32_t* __restrict__ err) {
  const int b = blockIdx.x;
  for (int p = threadIdx.x; p < max_pages; p += blockDim.x)
    table[(size_t)b * max_pages + p] = row[p];
  if (threadIdx.x == 0) {
    const int L = ctx_len[0];
    int a = anchor_pos[b];
    if (a < 0 || a > L) {
      set_dev_error(err, 2u);
      a = a < 0 ? 0 : L;
    }
    lens[b] = a;
  }
}

// Cross-entropy of row (b, k), k = 1 .. gamma-1: max and sum of exp in one
// workgroup (fp32 exponentials summed per thread, then in fp64), then
// ce[b][k-1] = max + log(sum) - logit[target].  A target outside the
// vocabulary gives NaN and sets DFLASH_DEVERR_TOKEN.
__global__ __launch_bounds__(kCeThreads) void k_block_ce(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ targets,
                                                         int gamma, int vocab,
                                                         double* __restrict__ ce,
                                                         uint32_t* __restrict__ err) {
  __shared__ float redm[kCeThreads / 64];
  __shared__ double reds[kCeThreads / 64];
  const int r = blockIdx.x, b = r / (gamma - 1), k = 1 + r % (gamma - 1);
  const float* x = logits + ((size_t)b * gamma + k) * vocab;
  const int tid = threadIdx.x, w = tid >> 6;
  float m = -INFINITY;
  for (int v = tid; v < vocab; v += kCeThreads) m = fmaxf(m, x[v]);
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  if ((tid & 63) == 0) redm[w] = m;
  __syncthreads();
  m = redm[0];
  for (int i = 1; i < kCeThreads / 64; ++i) m = fmaxf(m, redm[i]);
  float sf = 0.f;
  for (int v = tid; v < vocab; v += kCeThreads) sf += __expf(x[v] - m);
  double s = sf;
  for (int sh = 32; sh >= 1; sh >>= 1) s += __shfl_xor(s, sh, 64);
  if ((tid & 63) == 0) reds[w] = s;
  __syncthreads();
  if (tid == 0) {
    double t = reds[0];
    for (int i = 1; i < kCeThreads / 64; ++i) t += reds[i];
    const int tg = targets[(size_t)b * gamma + k];
    double c;
    if (tg < 0 || tg >= vocab) {
      set_dev_error(err, 4u);
      c = __builtin_nan("");
    } else {
      c = (double)m + log(t) - (double)x[tg];
    }
    ce[r] = c;
  }
}

// block_loss[b] = sum_k w_k ce / sum_k w_k; loss = mean over the blocks,
// summed in block order by one thread.
__global__ void k_block_loss(const double* __restrict__ ce, int n_blocks, int gamma,
                             double decay, float* __restrict__ block_loss,
                             float* __restrict__ loss) {
  double den = 0.0;
  for (int k = 1; k < gamma; ++k) den += exp(-(double)(k - 1) / decay);
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < n_blocks; b += gridDim.x * blockDim.x) {
    double num = 0.0;
    for (int k = 1; k < gamma; ++k)
      num += exp(-(double)(k - 1) / decay) * ce[(size_t)b * (gamma - 1) + k - 1];
    if (block_loss) block_loss[b] = (float)(num / den);
  }
  if (loss && blockIdx.x == 0 && threadIdx.x == 0) {
    double t = 0.0;
    for (int b = 0; b < n_blocks; ++b) {
      double num = 0.0;
      for (int k = 1; k < gamma; ++k)
        num += exp(-(double)(k - 1) / decay) * ce[(size_t)b * (gamma - 1) + k - 1];
      t += num / den;
    }
    *loss = (float)(t / n_blocks);
  }
}

// Autoregressive drafting: block[b][0] = anchor[b].
__global__ void k_ar_seed(const int32_t* __restrict__ anchor, int batch, int gamma,
                          int32_t* __restrict__ block) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) block[(size_t)b * gamma] = anchor[b];
}

// After pass i (rows 0..i-1 of each sequence): block[b][i] = the argmax of
// the pass's last row, pass_tokens[b*i + i-1].
__global__ void k_ar_pick(const int32_t* __restrict__ pass_tokens, int batch, int i, int gamma,
                          int32_t* __restrict__ block) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) block[(size_t)b * gamma + i] = pass_tokens[(size_t)b * i + i - 1];
}

}  // namespace

hipError_t launch_ar_seed(const int32_t* anchor, int batch, int gamma, int32_t* block,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_ar_seed, dim3((batch + 255) / 256), dim3(256), 0, st, anchor, batch, gamma,
                     block);
  return hipGetLastError();
}

hipError_t launch_ar_pick(const int32_t* pass_tokens, int batch, int i, int gamma, int32_t* block,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_ar_pick, dim3((batch + 255) / 256), dim3(256), 0, st, pass_tokens, batch, i,
                     gamma, block);
  return hipGetLastError();
}

hipError_t launch_packed_setup(const int32_t* page_row, int max_pages, const int32_t* ctx_len,
                               const int32_t* anchor_pos, int n_blocks, int32_t* table,
                               int32_t* lens, uint32_t* err, hipStream_t st) {
  if (n_blocks < 1 || max_pages < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_packed_setup, dim3(n_blocks), dim3(256), 0, st, page_row, max_pages,
                     ctx_len, anchor_pos, n_blocks, table, lens, err);
  return hipGetLastError();
}

hipError_t launch_block_loss(const float* logits, const int32_t* targets, int n_blocks, int gamma,
                             int vocab, double decay, double* ce, float* block_loss, float* loss,
                             uint32_t* err, hipStream_t st) {
  if (n_blocks < 1 || gamma < 2 || vocab < 1 || !(decay > 0.0)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_block_ce, dim3(n_blocks * (gamma - 1)), dim3(kCeThreads), 0, st, logits,
                     targets, gamma, vocab, ce, err);
  hipLaunchKernelGGL(k_block_loss, dim3((n_blocks + 255) / 256), dim3(256), 0, st, ce, n_blocks,
                     gamma, decay, block_loss, loss);
  return hipGetLastError();
}
