/* synth.c -- seeded, counter-based synthetic inputs shared by the tests, the
 * benchmark and the CPU baseline.
 *
 * It holds none of the drafter's arithmetic: only random numbers and the
 * planting of target scores for the verification inputs.  Every value is a
 * pure function of (seed, stream, element index), so the result does not
 * depend on the thread count or on which slice is generated.
 *
 *   key(seed, stream) = splitmix64(splitmix64(seed) ^ stream)
 *   bits(i)           = splitmix64(key + i)
 *   normal(i)         = Box-Muller on the uniform pair drawn from
 *                       bits(2*(i/2)) and bits(2*(i/2)+1): the cosine branch
 *                       for even i, the sine branch for odd i
 *
 * SplitMix64 follows its published definition (Steele, Lea, Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return splitmix64(splitmix64(seed) ^ stream);
}

static double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  uint64_t b1 = splitmix64(key + 2 * p), b2 = splitmix64(key + 2 * p + 1);
  double u1 = (double)((b1 >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
  double u2 = (double)(b2 >> 11) * 0x1.0p-53;       /* [0, 1) */
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

/* fp32 -> bf16 bits, round to nearest even (the generator's storage rule). */
static uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* out[i] = mean + std * normal(offset + i), i < n, stored as fp32. */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                      double mean, double std, float* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = (float)(mean + std * normal_at(key, offset + (uint64_t)i));
}

/* Same values rounded to bf16 (through fp32), stored as raw bits. */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                       double mean, double std, uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16((float)(mean + std * normal_at(key, offset + (uint64_t)i)));
}

/* Uniform integers in [lo, hi] (inclusive). */
void synth_uniform_int(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                       int64_t lo, int64_t hi, int64_t* out) {
  uint64_t key = stream_key(seed, stream);
  uint64_t range = (uint64_t)(hi - lo) + 1u;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t b = splitmix64(key + offset + (uint64_t)i);
    /* 128-bit multiply-shift maps 64 random bits onto [0, range) */
    unsigned __int128 m = (unsigned __int128)b * range;
    out[i] = lo + (int64_t)(uint64_t)(m >> 64);
  }
}

/* Uniform doubles in [0, 1). */
void synth_uniform_f64(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                       double* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = (double)(splitmix64(key + offset + (uint64_t)i) >> 11) * 0x1.0p-53;
}

/* Target scores for verification with a planted accepted length.
 *
 * For each of the n_seq sequences: gamma rows of V scores drawn N(0, 1)
 * (stream `stream`, sequence s at element offset s*gamma*V).  Then, with
 * tau = tau_star[s] and block = blocks[s]:
 *   rows j <= tau-2: score[block[j+1]] = rowmax + margin, so the target's
 *                    argmax of row j is the block's next proposal (accepted);
 *   row tau-1 (only if tau < gamma): score[c] = rowmax + margin for
 *                    c = (block[tau] + 1) mod V, so the target's choice
 *                    differs from the proposal block[tau] (rejected).
 * The planted value is formed in fp32 and then stored in the output type
 * (out_bf16 != 0: bf16 bits in out (uint16), else fp32).
 */
void synth_plant_target(uint64_t seed, uint64_t stream, int32_t n_seq, int32_t gamma,
                        int32_t V, const int32_t* blocks, const int32_t* tau_star,
                        double margin, int32_t out_bf16, void* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)n_seq * gamma; ++r) {
    int s = (int)(r / gamma), j = (int)(r % gamma);
    const int32_t* blk = blocks + (int64_t)s * gamma;
    int tau = tau_star[s];
    float rowmax = -INFINITY;
    int64_t base = r * (int64_t)V;
    float* of = (float*)out;
    uint16_t* ob = (uint16_t*)out;
    /* pass 1: draw, remember the fp32 row maximum */
    for (int64_t i = 0; i < V; ++i) {
      float v = (float)normal_at(key, (uint64_t)(base + i));
      if (v > rowmax) rowmax = v;
      if (out_bf16) ob[base + i] = f32_to_bf16(v); else of[base + i] = v;
    }
    int target = -1;
    if (j <= tau - 2) target = blk[j + 1];
    else if (j == tau - 1 && tau < gamma) target = (blk[tau] + 1) % V;
    if (target >= 0) {
      float v = (float)((double)rowmax + margin);
      if (out_bf16) ob[base + target] = f32_to_bf16(v); else of[base + target] = v;
    }
  }
}
