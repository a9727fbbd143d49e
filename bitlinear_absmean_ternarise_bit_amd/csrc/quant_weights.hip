// Offline weight quantisation: AbsMean scale, RoundClip ternary codes, and
// either the 2-bit pack or the radix-3 pack (five weights per byte).
//
// [PMV] = produtoramaxvision.com.br article on BitNet b1.58 (ternary
// quantisation, BitLinear, Zero-GEMM).  gamma = (1/(n m)) sum |W_ij| and
// W_q = Round(Clip(W / (gamma + eps), -1, 1)) are its section-1 AbsMean
// equations; 2 bits per weight is its section-3 packing; five weights per
// byte (3^5 = 243 <= 256) is the Radix-3 packing of its section on bitnet.cpp.
//
// gamma is computed exactly and order-independently: each |w| is an integer
// significand times a power of two, so the sum is an integer in units of
// 2^-149.  Lanes accumulate it as base-2^32 "digits" held carry-save in
// uint64 registers (a value lands in two adjacent digits); one block-wide
// table of ten digits per workgroup goes to the workspace, and a single
// workgroup adds the tables, propagates carries, rounds the exact sum once to
// float64 and divides by N*K.  Any grid shape gives bit-identical results.
#include "kernels.hpp"

namespace bitlinear {

namespace {

constexpr int kDigits = kAbsmeanDigits;

struct DigitAcc {
  unsigned long long a0 = 0, a1 = 0, a2 = 0;  // digits T0, T0+1, T0+2
};

// Split |w| (float32 bit pattern) into (digit index t, low 32 bits, high bits)
// of sig << r, where |w| = sig * 2^(32 t + r) * 2^-149.
__device__ __forceinline__ void split_abs(uint32_t bits, uint32_t& t, uint32_t& lo, uint32_t& hi) {
  const uint32_t b = bits & 0x7fffffffu;
  const uint32_t e = b >> 23;
  const uint32_t m = b & 0x7fffffu;
  const uint32_t sig = e ? (m | 0x800000u) : m;
  const uint32_t s = e ? e - 1u : 0u;
  t = s >> 5;
  const uint64_t v = static_cast<uint64_t>(sig) << (s & 31u);
  lo = static_cast<uint32_t>(v);
  hi = static_cast<uint32_t>(v >> 32);
}

__device__ __forceinline__ void add_abs(uint32_t bits, uint32_t T0, DigitAcc& acc,
                                        unsigned long long* sdig) {
  uint32_t t, lo, hi;
  split_abs(bits, t, lo, hi);
  if (t == T0) {
    acc.a0 += lo;
    acc.a1 += hi;
  } else if (t == T0 + 1u) {
    acc.a1 += lo;
    acc.a2 += hi;
  } else if (lo | hi) {  // outside the wave's window (rare): block table
    atomicAdd(&sdig[t], static_cast<unsigned long long>(lo));
    atomicAdd(&sdig[t + 1], static_cast<unsigned long long>(hi));
  }
}

__global__ __launch_bounds__(256) void absmean_digits_kernel(const float* __restrict__ W,
                                                             uint64_t n,
                                                             unsigned long long* __restrict__ partial) {
  __shared__ unsigned long long sdig[kDigits];
  if (threadIdx.x < kDigits) sdig[threadIdx.x] = 0;
  __syncthreads();

  const uint64_t n4 = n >> 2;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  const uint64_t tid = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const uint4* W4 = reinterpret_cast<const uint4*>(W);

  // Window base: one digit below the largest digit among the wave's first
  // loads (any choice is exact; this one keeps nearly every value in-window).
  uint4 first = make_uint4(0, 0, 0, 0);
  if (tid < n4) first = W4[tid];
  uint32_t tmax = 0;
  {
    uint32_t t, lo, hi;
    split_abs(first.x, t, lo, hi); tmax = max(tmax, (lo | hi) ? t : 0u);
    split_abs(first.y, t, lo, hi); tmax = max(tmax, (lo | hi) ? t : 0u);
    split_abs(first.z, t, lo, hi); tmax = max(tmax, (lo | hi) ? t : 0u);
    split_abs(first.w, t, lo, hi); tmax = max(tmax, (lo | hi) ? t : 0u);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tmax = max(tmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(tmax), o, kWave)));
  // (a wave whose first loads are all zero -- e.g. zeroed rows -- takes the
  // window of magnitudes below 4, where trained and synthetic weights live)
  uint32_t any = 0;
  {
    uint32_t t, lo, hi;
    split_abs(first.x | first.y | first.z | first.w, t, lo, hi);
    any = lo | hi;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) any |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(any), o, kWave));
  const uint32_t T0 = any ? (tmax ? tmax - 1u : 0u) : 2u;

  DigitAcc acc;
  if (tid < n4) {
    add_abs(first.x, T0, acc, sdig);
    add_abs(first.y, T0, acc, sdig);
    add_abs(first.z, T0, acc, sdig);
    add_abs(first.w, T0, acc, sdig);
  }
  // four independent 16-byte loads in flight per lane; indices past the end
  // re-read the last vector and are then zeroed (no branches around loads)
  const uint64_t last = n4 ? n4 - 1 : 0;
  for (uint64_t i0 = tid + stride; i0 < n4; i0 += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t idx = i0 + u * stride;
      const uint4 x = W4[idx < n4 ? idx : last];
      v[u] = idx < n4 ? x : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      add_abs(v[u].x, T0, acc, sdig);
      add_abs(v[u].y, T0, acc, sdig);
      add_abs(v[u].z, T0, acc, sdig);
      add_abs(v[u].w, T0, acc, sdig);
    }
  }
  // scalar tail (n not a multiple of 4)
  const uint64_t tail = n4 << 2;
  if (tid < n - tail) add_abs(__float_as_uint(W[tail + tid]), T0, acc, sdig);

  const unsigned long long s0 = wave_sum_u64(acc.a0);
  const unsigned long long s1 = wave_sum_u64(acc.a1);
  const unsigned long long s2 = wave_sum_u64(acc.a2);
  if ((threadIdx.x & (kWave - 1)) == 0) {
    if (s0) atomicAdd(&sdig[T0], s0);
    if (s1) atomicAdd(&sdig[T0 + 1], s1);
    if (s2) atomicAdd(&sdig[T0 + 2], s2);
  }
  __syncthreads();
  if (threadIdx.x < kDigits) partial[static_cast<uint64_t>(blockIdx.x) * kDigits + threadIdx.x] = sdig[threadIdx.x];
}

// Sum the per-workgroup digit tables, round the exact sum to float64 once,
// gamma = float32(sum / count).
__global__ __launch_bounds__(256) void absmean_finalize_kernel(const unsigned long long* __restrict__ partial,
                                                               int nparts, double count,
                                                               float* __restrict__ gamma) {
  __shared__ unsigned long long red[kDigits][256 / kWave];
  unsigned long long d[kDigits];
#pragma unroll
  for (int i = 0; i < kDigits; ++i) d[i] = 0;
  for (int p = threadIdx.x; p < nparts; p += blockDim.x) {
#pragma unroll
    for (int i = 0; i < kDigits; ++i) d[i] += partial[static_cast<uint64_t>(p) * kDigits + i];
  }
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int i = 0; i < kDigits; ++i) {
    const unsigned long long s = wave_sum_u64(d[i]);
    if ((threadIdx.x & (kWave - 1)) == 0) red[i][wave] = s;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;

  // carry-propagate into 32-bit limbs: S = sum_i limb[i] * 2^(32 i)
  uint32_t limb[kDigits + 2];
  unsigned long long carry = 0;
#pragma unroll
  for (int i = 0; i < kDigits; ++i) {
    unsigned long long v = carry;
    for (int w = 0; w < 256 / kWave; ++w) v += red[i][w];  // < 2^64 for N*K < 2^32
    limb[i] = static_cast<uint32_t>(v);
    carry = v >> 32;
  }
  limb[kDigits] = static_cast<uint32_t>(carry);
  limb[kDigits + 1] = static_cast<uint32_t>(carry >> 32);

  int top = kDigits + 1;
  while (top >= 0 && limb[top] == 0) --top;
  double sum = 0.0;
  if (top >= 0) {
    // top 64 significant bits T, exponent so that S ~= T * 2^(32 top - 32 - lz)
    const int lz = __clz(limb[top]);
    const uint64_t h = (static_cast<uint64_t>(limb[top]) << 32) | (top >= 1 ? limb[top - 1] : 0u);
    const uint64_t l = static_cast<uint64_t>(top >= 2 ? limb[top - 2] : 0u) << 32;
    uint64_t T = lz ? ((h << lz) | (l >> (64 - lz))) : h;
    bool sticky = lz ? ((l << lz) != 0) : (l != 0);
    for (int i = top - 3; i >= 0; --i) sticky |= (limb[i] != 0);
    if (sticky) T |= 1u;  // below the float64 round bit: decides ties correctly
    // hi * 2^32 is exact and the one addition rounds once: correctly rounded
    const double t = static_cast<double>(static_cast<uint32_t>(T >> 32)) * 4294967296.0 +
                     static_cast<double>(static_cast<uint32_t>(T));
    sum = ldexp(t, 32 * top - 32 - lz - 149);
  }
  gamma[0] = static_cast<float>(sum / count);
}

typedef float v4f __attribute__((ext_vector_type(4)));

// Ternarise and pack.  Each lane turns four consecutive weights (k = 4f..4f+3)
// into the four bytes' bit pair 2i of word f/4 (i = f%4); four adjacent lanes
// OR their parts into one word, stored at its place in the interleaved row
// order (unit_offset).  The codes come from one comparison per weight with
// the threshold of ternary_thresholds (no division).  A lane handles four
// grid-stride items per round, their 16-byte loads (streaming: every weight
// is read once) issued together; its (row, quad) position advances by the
// stride without a division.
template <bool VEC>
__global__ __launch_bounds__(256) void ternarise_pack_kernel(const float* __restrict__ W, int64_t N,
                                                             int64_t K, int64_t Kp,
                                                             const float* __restrict__ gamma,
                                                             uint32_t* __restrict__ packed) {
  constexpr int U = 4;
  const float thr = ternary_thresholds(gamma[0]).nonzero;
  const int64_t qpr = Kp >> 2;       // quads (four weights) per row
  const int64_t total = N * qpr;     // a multiple of 16: groups of 4 lanes stay together
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;  // a multiple of 4
  const int64_t row_step = stride / qpr, quad_step = stride - row_step * qpr;
  int64_t f = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t n = f / qpr, q = f - n * qpr;
  const int i = static_cast<int>(threadIdx.x & 3);
  for (; f < total; f += U * stride) {
    int64_t nu[U], qu[U];
    float w[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      nu[u] = n;
      qu[u] = q;
      const int64_t kq = q << 2;
      const float* row = W + n * K;
      if (f + u * stride < total) {
        if (VEC && kq + 3 < K) {
          const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(row + kq));
          w[u][0] = v[0]; w[u][1] = v[1]; w[u][2] = v[2]; w[u][3] = v[3];
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b) w[u][b] = (kq + b < K) ? row[kq + b] : 0.0f;
        }
      }
      n += row_step;
      q += quad_step;
      if (q >= qpr) {
        q -= qpr;
        ++n;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (f + u * stride >= total) break;  // the same for all four lanes of a word
      const int64_t kq = qu[u] << 2;
      uint32_t part = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) part |= ternary_code(w[u][b], thr, kq + b < K) << (8 * b);
      part <<= 2 * i;
      part |= __shfl_xor(part, 1, 4);
      part |= __shfl_xor(part, 2, 4);
      if (i == 0) {
        const uint32_t wi = static_cast<uint32_t>(kq >> 4);  // word of the row
        const uint32_t off = unit_offset(static_cast<uint32_t>(nu[u]), wi >> 2, static_cast<uint32_t>(N),
                                         static_cast<uint32_t>(Kp >> 6));
        packed[(off >> 2) + (wi & 3u)] = part;
      }
    }
  }
}

// Ternarise and pack five weights per byte.  One lane writes one 32-bit word
// of a row: 20 weights k = 20j + 4t + b (byte b, digit t).  Byte b holds
// v = sum_t c_t 3^(4-t) as ceil(256 v / 243), so a decoder reads the digits
// most significant first by repeated multiplication by three.
template <bool VEC>
__global__ __launch_bounds__(256) void ternarise_pack_r3_kernel(const float* __restrict__ W, int64_t N,
                                                                int64_t K, int64_t words_per_row,
                                                                const float* __restrict__ gamma,
                                                                uint32_t* __restrict__ packed) {
  const float thr = ternary_thresholds(gamma[0]).nonzero;
  const int64_t total = N * words_per_row;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t f = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; f < total; f += stride) {
    const int64_t n = f / words_per_row;
    const int64_t k0 = (f - n * words_per_row) * 20;
    const float* row = W + n * K;
    uint32_t v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 5; ++t) {
      const int64_t k = k0 + 4 * t;
      float w[4];
      if (VEC && k + 3 < K) {
        const float4 x = *reinterpret_cast<const float4*>(row + k);
        w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) w[b] = (k + b < K) ? row[k + b] : 0.0f;
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) v[b] = 3u * v[b] + ternary_code(w[b], thr, k + b < K);
    }
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) word |= ((256u * v[b] + 242u) / 243u) << (8 * b);
    const uint32_t wi = static_cast<uint32_t>(f - n * words_per_row);  // word of the row
    const uint32_t off = unit_offset(static_cast<uint32_t>(n), wi >> 2, static_cast<uint32_t>(N),
                                     static_cast<uint32_t>(words_per_row >> 2));
    packed[(off >> 2) + (wi & 3u)] = word;
  }
}

void launch_gamma(const float* W, int64_t N, int64_t K, float* gamma, void* workspace,
                  hipStream_t stream) {
  const uint64_t n = static_cast<uint64_t>(N) * static_cast<uint64_t>(K);
  auto* partial = static_cast<unsigned long long*>(workspace);
  const uint64_t want = (n / 4 + 255) / 256;
  const int blocks = static_cast<int>(want < 1 ? 1 : (want > kAbsmeanBlocks ? kAbsmeanBlocks : want));
  absmean_digits_kernel<<<blocks, 256, 0, stream>>>(W, n, partial);
  absmean_finalize_kernel<<<1, 256, 0, stream>>>(partial, blocks, static_cast<double>(n), gamma);
}

}  // namespace

hipError_t launch_quantize_weights_r3(const float* W, int64_t N, int64_t K, uint8_t* packed,
                                      float* gamma, void* workspace, hipStream_t stream) {
  launch_gamma(W, N, K, gamma, workspace, stream);
  const int64_t wpr = r3_padded_k(K) / 20;
  const int64_t total = N * wpr;
  int64_t pblocks = (total + 255) / 256;
  if (pblocks > 65536) pblocks = 65536;
  uint32_t* out = reinterpret_cast<uint32_t*>(packed);
  if ((K & 3) == 0)
    ternarise_pack_r3_kernel<true><<<static_cast<int>(pblocks), 256, 0, stream>>>(W, N, K, wpr, gamma, out);
  else
    ternarise_pack_r3_kernel<false><<<static_cast<int>(pblocks), 256, 0, stream>>>(W, N, K, wpr, gamma, out);
  return hipGetLastError();
}

hipError_t launch_quantize_weights(const float* W, int64_t N, int64_t K, uint32_t* packed,
                                   float* gamma, void* workspace, hipStream_t stream) {
  launch_gamma(W, N, K, gamma, workspace, stream);
  const int64_t Kp = padded_k(K);
  const int64_t total = N * (Kp / 4);
  // four items per lane (the kernel's batch), at most 65536 workgroups
  int64_t pblocks = (total + 1023) / 1024;
  if (pblocks > 65536) pblocks = 65536;
  if ((K & 3) == 0)
    ternarise_pack_kernel<true><<<static_cast<int>(pblocks), 256, 0, stream>>>(W, N, K, Kp, gamma, packed);
  else
    ternarise_pack_kernel<false><<<static_cast<int>(pblocks), 256, 0, stream>>>(W, N, K, Kp, gamma, packed);
  return hipGetLastError();
}


}  // namespace bitlinear
