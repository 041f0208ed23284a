// common.h -- device helpers shared by the gfx950 kernels of the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define DF_DEV __device__ __forceinline__

DF_DEV float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even (inputs are finite).
DF_DEV uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 values -> two bf16 in one word (a in the low half), round to
// nearest, ties to even: one v_cvt_pk_bf16_f32, equal to f2bf for finite
// inputs.
DF_DEV uint32_t pack_bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Round an fp32 value to the nearest bf16 value, kept in fp32.
DF_DEV float round_bf(float f) { return bf2f(f2bf(f)); }

// Storage of the model dtype (weights, gains, hidden-state inputs, the K/V
// cache): bf16 bits (BF16 = true) or fp32.
template <bool BF16> struct Act;
template <> struct Act<true> {
  typedef uint16_t T;
  static DF_DEV float load(const T* p, size_t i) { return bf2f(p[i]); }
  static DF_DEV void store(T* p, size_t i, float v) { p[i] = f2bf(v); }
};
template <> struct Act<false> {
  typedef float T;
  static DF_DEV float load(const T* p, size_t i) { return p[i]; }
  static DF_DEV void store(T* p, size_t i, float v) { p[i] = v; }
};

// Transient activations that feed a matrix product.  fp32 models keep one
// fp32 plane.  bf16 models keep the fp32 value as two bf16 planes, hi and lo
// (hi = bf16(v), lo = bf16(v - hi), |v - hi - lo| <= 2^-17 |v|), laid out
// back to back: lo starts `plane` elements after hi.  The products then run
// as two bf16 MFMAs (hi and lo against the same weights).
template <bool BF16> struct Split;
template <> struct Split<true> {
  static DF_DEV void store(void* base, size_t plane, size_t i, float v) {
    uint16_t* hi = (uint16_t*)base;
    const uint16_t h = f2bf(v);
    hi[i] = h;
    hi[plane + i] = f2bf(v - bf2f(h));
  }
  static DF_DEV float load(const void* base, size_t plane, size_t i) {
    const uint16_t* hi = (const uint16_t*)base;
    return bf2f(hi[i]) + bf2f(hi[plane + i]);
  }
};
// Four consecutive values (element i, i a multiple of 4) as hi and lo bf16
// planes, 8 bytes per plane, rounded as Split<true>::store rounds.
DF_DEV void split_store4(void* base, size_t plane, size_t i, f32x4 v) {
  uint16_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = f2bf(v[e]);
    l[e] = f2bf(v[e] - bf2f(h[e]));
  }
  uint16_t* hp = (uint16_t*)base + i;
  *(uint2*)hp = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
  *(uint2*)(hp + plane) = make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
}

template <> struct Split<false> {
  static DF_DEV void store(void* base, size_t, size_t i, float v) { ((float*)base)[i] = v; }
  static DF_DEV float load(const void* base, size_t, size_t i) { return ((const float*)base)[i]; }
};

// D = A * B + C for one 16x16x32 bf16 MFMA tile.  Lane l (r = l % 16,
// g = l / 16) supplies A[r][8g..8g+7] and B[8g..8g+7][r]; it receives
// D[4g + i][r], i = 0..3.
DF_DEV f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

DF_DEV u32x4 ld16(const void* p) { return *(const u32x4*)p; }
// Streaming load of data read once per launch (weights): the non-temporal
// hint keeps it from displacing reused lines in the caches.
DF_DEV u32x4 ld16_stream(const void* p) { return __builtin_nontemporal_load((const u32x4*)p); }
DF_DEV void st16(void* p, u32x4 v) { *(u32x4*)p = v; }

// Order-preserving map of an fp32 value onto uint32 (finite inputs).  -0.0
// maps to the key of +0.0: the two compare equal, so a tie between them goes
// to the lower index like any other tie.
DF_DEV uint32_t f32_order(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u << 1) ? u : 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Argmax key: larger value wins; among equal values the lower index wins.
DF_DEV uint64_t argmax_key(float v, uint32_t idx) {
  return ((uint64_t)f32_order(v) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
DF_DEV uint32_t argmax_key_index(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu); }

// n-th output (n >= 1) of the SplitMix64 generator started at seed (Steele,
// Lea and Flood, "Fast splittable pseudorandom number generators", 2014):
// the state advances by the golden-ratio constant and goes through the
// generator's finaliser.
DF_DEV uint64_t splitmix64_at(uint64_t seed, uint64_t n) {
  uint64_t z = seed + n * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Gumbel noise -log(-log(w)) of the drafter's draw at (sequence, block
// position, token): w = (top 23 bits of output n + 1/2) / 2^23 with counter
// n = (seq << 40 | pos << 32 | token) + 1.  2 * bits + 1 < 2^24, so w is
// exact in fp32 and never reaches 1.
DF_DEV float gumbel_noise(uint64_t seed, uint32_t seq, uint32_t pos, uint32_t tok) {
  const uint64_t n = (((uint64_t)seq << 40) | ((uint64_t)pos << 32) | tok) + 1ull;
  const uint32_t bits = (uint32_t)(splitmix64_at(seed, n) >> 41);
  const float w = (float)(2u * bits + 1u) * (1.0f / 16777216.0f);
  return -logf(-logf(w));
}

DF_DEV uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m, 64);
  hi = __shfl_xor(hi, m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Block-wide sum over blockDim.x threads (blockDim.x a multiple of 64,
// at most 1024).  `red` is shared scratch of >= 16 floats.  All threads get
// the result.  The summation order is fixed.
DF_DEV float block_sum(float v, float* red) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

// Rotary angle pair for dimension pair i of a head of size dh at position
// pos: (cos, sin) of pos * theta^(-2i/dh), evaluated in double.
DF_DEV void rope_cs(int pos, int i, int dh, double theta, float* c, float* s) {
  double inv = pow(theta, -2.0 * (double)i / (double)dh);
  double phi = (double)pos * inv;
  double sd, cd;
  sincos(phi, &sd, &cd);
  *c = (float)cd;
  *s = (float)sd;
}

// Sticky device error word.
DF_DEV void set_dev_error(uint32_t* word, uint32_t bit) { atomicOr(word, bit); }
