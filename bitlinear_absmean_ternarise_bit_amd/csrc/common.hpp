// Shared device helpers for the BitLinear kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitlinear {

constexpr int kWave = 64;
constexpr float kEps = 1e-5f;  // eps of both quantisers, a float32 constant

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ unsigned wave_or(unsigned v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= __shfl_xor(v, o, kWave);
  return v;
}

// bfloat16 bit pattern -> float32 (exact widening)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Byte offset of 16-byte unit u of row n in a packed matrix of N rows of U
// units.  Rows are stored in blocks of 16 (the last block holds N % 16 rows
// if that is not 0) and a block's units in chunks of 4 (the last chunk holds
// U % 4 units if that is not 0); within a chunk each row of the block stores
// its units of the chunk contiguously.  A full chunk is 16 rows x 64 bytes in
// one contiguous KiB, and a block takes as many bytes as its rows stored one
// after another.  Requires n < N and u < U.
__device__ __forceinline__ uint32_t unit_offset(uint32_t n, uint32_t u, uint32_t N, uint32_t U) {
  const uint32_t b = n >> 4, j = n & 15u, c = u >> 2, g = u & 3u;
  const uint32_t R = min(16u, N - 16u * b);
  const uint32_t W = min(4u, U - 4u * c);
  return (16u * b * U + c * R * 4u + j * W + g) * 16u;
}

// Four 2-bit codes per byte lane: (word >> 2i) & 0x03030303 gives the int8
// codes of k = 16j + 4i .. 16j + 4i + 3, so the four results are the sixteen
// codes of a packed word in k order.
__device__ __forceinline__ v4i unpack_word(uint32_t w) {
  v4i r;
  r[0] = static_cast<int>(w & 0x03030303u);
  r[1] = static_cast<int>((w >> 2) & 0x03030303u);
  r[2] = static_cast<int>((w >> 4) & 0x03030303u);
  r[3] = static_cast<int>((w >> 6) & 0x03030303u);
  return r;
}

// Ternary codes without a division.  [PMV] section 1: W_q = RoundClip(W / d)
// with d = gamma + eps, here fp32(gamma + eps), an IEEE float32 quotient and
// round half to even.  The code is nonzero exactly when fp32(|w| / d) > 1/2
// (a quotient of exactly 1/2 rounds to 0), that is when the real |w| / d
// exceeds 1/2 + 2^-25 (the tie above 1/2 rounds down to the even 1/2), that is
// when |w| > d/2 + d 2^-25.  No float32 lies in (d/2, d/2 + d 2^-25]: d/2 is
// exact and the float32 spacing there is larger than d 2^-25.  So for float32
// weights the test is |w| > d/2.  Likewise fp32(|w| / d) <= 1 exactly when
// |w| <= d (the STE range mask).
struct TernaryThresholds {
  float nonzero;   // |w| > nonzero  <=>  Round(Clip(fp32(w / d), -1, 1)) != 0
  float in_range;  // |w| <= in_range  <=>  |fp32(w / d)| <= 1
};

__device__ __forceinline__ TernaryThresholds ternary_thresholds(float gamma) {
  const float d = __fadd_rn(gamma, kEps);  // >= eps: d/2 is exact
  return {__fmul_rn(d, 0.5f), d};
}

// Offset code c = q + 1 in {0, 1, 2} of one weight; padding (valid false) is
// a zero weight, c = 1.
__device__ __forceinline__ uint32_t ternary_code(float w, float nonzero, bool valid) {
  const uint32_t q = fabsf(w) > nonzero ? (w > 0.0f ? 2u : 0u) : 1u;
  return valid ? q : 1u;
}

// Activation code of one value: rint(x * s) (half to even) clipped to [-128, 127].
__device__ __forceinline__ int act_code(float x, float s) {
  float v = __fmul_rn(x, s);
  float r = __builtin_rintf(v);
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return static_cast<int>(r);
}

}  // namespace bitlinear
