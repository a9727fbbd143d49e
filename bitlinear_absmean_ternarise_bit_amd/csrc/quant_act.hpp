// Per-token AbsMax INT8 quantisation of one activation row by one wavefront.
//
// [PMV] = produtoramaxvision.com.br article on BitNet b1.58; its section-1
// AbsMax equations: gamma_A = max_k |A_k| per token and
// A_q = Clip(Round(A * (127 / (gamma_A + eps))), -128, 127).
//
// Float32 arithmetic: one IEEE division per token for the scale, then
// rint(x * s) (half to even).  The max and the code sum are exact, so the
// wave reductions' order does not matter.
#pragma once

#include "common.hpp"

namespace bitlinear {

// Wave reductions on the quantiser's critical path: within each row of 16
// lanes by DPP moves (swap neighbours, swap pairs, mirror the half-rows,
// mirror the row), then the four row results read as scalars.  Every lane
// gets the result.  A maximum and an integer sum do not depend on the order.
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float quant_wave_max(float v) {
  v = fmaxf(v, __int_as_float(dpp<0xb1>(__float_as_int(v))));   // quad_perm 1,0,3,2
  v = fmaxf(v, __int_as_float(dpp<0x4e>(__float_as_int(v))));   // quad_perm 2,3,0,1
  v = fmaxf(v, __int_as_float(dpp<0x141>(__float_as_int(v))));  // row_half_mirror
  v = fmaxf(v, __int_as_float(dpp<0x140>(__float_as_int(v))));  // row_mirror
  const int b = __float_as_int(v);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}
__device__ __forceinline__ int quant_wave_sum(int v) {
  v += dpp<0xb1>(v);
  v += dpp<0x4e>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// DT: 0 = float32, 1 = bfloat16.  VEC: rows are 16-byte aligned and hold a
// whole number of 16-byte chunks.
template <int DT>
struct ActTraits;
template <>
struct ActTraits<0> {
  static constexpr int kPerChunk = 4;  // float32 values per 16 bytes
};
template <>
struct ActTraits<1> {
  static constexpr int kPerChunk = 8;  // bfloat16 values per 16 bytes
};

template <int DT>
__device__ __forceinline__ void chunk_to_f32(const uint4 v, float* f) {
  if constexpr (DT == 0) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  } else {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(u[i] << 16);
      f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
}

template <int DT>
__device__ __forceinline__ float load_one(const void* row, int64_t k) {
  if constexpr (DT == 0) return static_cast<const float*>(row)[k];
  else return bf16_to_f32(static_cast<const uint16_t*>(row)[k]);
}

// Codes of one 16-byte chunk (P values) with scale s, stored at dst; returns
// their sum.
template <int DT>
__device__ __forceinline__ int quantize_chunk(const uint4 v, float s, int8_t* __restrict__ dst) {
  constexpr int P = ActTraits<DT>::kPerChunk;
  float f[P];
  chunk_to_f32<DT>(v, f);
  int sum = 0;
  uint32_t w[P / 4];
#pragma unroll
  for (int q = 0; q < P / 4; ++q) {
    uint32_t packedq = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int code = act_code(f[4 * q + b], s);
      sum += code;
      packedq |= (static_cast<uint32_t>(code) & 0xffu) << (8 * b);
    }
    w[q] = packedq;
  }
  if constexpr (P == 8) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  } else {
    *reinterpret_cast<uint32_t*>(dst) = w[0];
  }
  return sum;
}

// Codes of row `row` (K values) with scale s into dst[0..Kp) (zeros in
// [K, Kp)), one pass; returns this lane's part of the code sum.
template <int DT, bool VEC>
__device__ __forceinline__ int codes_pass(const void* __restrict__ row, int64_t K, int64_t Kp, int lane,
                                          int8_t* __restrict__ dst, float s) {
  constexpr int P = ActTraits<DT>::kPerChunk;
  int sum = 0;
  if constexpr (VEC) {
    const uint4* r4 = static_cast<const uint4*>(row);
    const int64_t nc = K / P;
    for (int64_t c = lane; c < nc; c += kWave) sum += quantize_chunk<DT>(r4[c], s, dst + c * P);
  } else {
    for (int64_t k = lane; k < K; k += kWave) {
      const int code = act_code(load_one<DT>(row, k), s);
      sum += code;
      dst[k] = static_cast<int8_t>(code);
    }
  }
  for (int64_t k = K + lane; k < Kp; k += kWave) dst[k] = 0;
  return sum;
}

// Quantise row `row` (K values) into dst[0..Kp) (zeros in [K, Kp)); every lane
// of the wave must call it.  Returns gamma_A and the code sum in all lanes.
// RC: a row of at most RC 16-byte chunks per lane stays in registers between
// the two passes (one read of X instead of two).
template <int DT, bool VEC, int RC = 4>
__device__ __forceinline__ void quantize_row_wave(const void* __restrict__ row, int64_t K, int64_t Kp,
                                                  int lane, int8_t* __restrict__ dst,
                                                  float& gamma_a, int& codesum) {
  constexpr int P = ActTraits<DT>::kPerChunk;
  if constexpr (VEC) {
    const uint4* r4 = static_cast<const uint4*>(row);
    const int64_t nc = K / P;
    if (nc <= RC * kWave) {
      uint4 v[RC];
      float mx = 0.0f;
#pragma unroll
      for (int u = 0; u < RC; ++u) {
        const int64_t c = lane + u * kWave;
        v[u] = r4[c < nc ? c : nc - 1];
      }
#pragma unroll
      for (int u = 0; u < RC; ++u) {
        float f[P];
        chunk_to_f32<DT>(v[u], f);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < P; ++i) m = fmaxf(m, fabsf(f[i]));
        mx = (lane + u * kWave < nc) ? fmaxf(mx, m) : mx;
      }
      mx = quant_wave_max(mx);
      const float s = __fdiv_rn(127.0f, __fadd_rn(mx, kEps));
      int sum = 0;
#pragma unroll
      for (int u = 0; u < RC; ++u) {
        const int64_t c = lane + u * kWave;
        if (c < nc) sum += quantize_chunk<DT>(v[u], s, dst + c * P);
      }
      for (int64_t k = K + lane; k < Kp; k += kWave) dst[k] = 0;
      gamma_a = mx;
      codesum = quant_wave_sum(sum);
      return;
    }
  }
  float mx = 0.0f;
  if constexpr (VEC) {
    // four 16-byte loads in flight per lane; chunks past the row re-read the
    // last chunk (in bounds) and are dropped by the select
    const uint4* r4 = static_cast<const uint4*>(row);
    const int64_t nc = K / P;
    for (int64_t c0 = lane; c0 < nc; c0 += 4 * kWave) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t c = c0 + u * kWave;
        v[u] = r4[c < nc ? c : nc - 1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float f[P];
        chunk_to_f32<DT>(v[u], f);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < P; ++i) m = fmaxf(m, fabsf(f[i]));
        mx = (c0 + u * kWave < nc) ? fmaxf(mx, m) : mx;
      }
    }
  } else {
    for (int64_t k = lane; k < K; k += kWave) mx = fmaxf(mx, fabsf(load_one<DT>(row, k)));
  }
  mx = quant_wave_max(mx);
  const float s = __fdiv_rn(127.0f, __fadd_rn(mx, kEps));

  gamma_a = mx;
  codesum = quant_wave_sum(codes_pass<DT, VEC>(row, K, Kp, lane, dst, s));
}

// A row of at most RC 16-byte chunks per lane, loaded into registers (its
// loads can go out before other work), then quantised as quantize_row_wave
// does.  Chunks past the row re-read its last chunk and are not used.
template <int DT, int RC = 4>
__device__ __forceinline__ void load_row_chunks(const void* __restrict__ row, int64_t nc, int lane, uint4 (&v)[RC]) {
  const uint4* r4 = static_cast<const uint4*>(row);
#pragma unroll
  for (int u = 0; u < RC; ++u) {
    const int64_t c = lane + u * kWave;
    v[u] = r4[c < nc ? c : nc - 1];
  }
}
template <int DT, int RC = 4>
__device__ __forceinline__ void quantize_loaded_row(const uint4 (&v)[RC], int64_t nc, int64_t K, int64_t Kp,
                                                    int lane, int8_t* __restrict__ dst, float& gamma_a,
                                                    int& codesum) {
  constexpr int P = ActTraits<DT>::kPerChunk;
  float mx = 0.0f;
#pragma unroll
  for (int u = 0; u < RC; ++u) {
    float f[P];
    chunk_to_f32<DT>(v[u], f);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < P; ++i) m = fmaxf(m, fabsf(f[i]));
    mx = (lane + u * kWave < nc) ? fmaxf(mx, m) : mx;
  }
  mx = quant_wave_max(mx);
  const float s = __fdiv_rn(127.0f, __fadd_rn(mx, kEps));
  int sum = 0;
#pragma unroll
  for (int u = 0; u < RC; ++u) {
    const int64_t c = lane + u * kWave;
    if (c < nc) sum += quantize_chunk<DT>(v[u], s, dst + c * P);
  }
  for (int64_t k = K + lane; k < Kp; k += kWave) dst[k] = 0;
  gamma_a = mx;
  codesum = quant_wave_sum(sum);
}

// Two rows by one wave, both held in registers: their loads go out together,
// so the wave waits for one memory round trip instead of two.  Rows of more
// than RC 16-byte chunks per lane are quantised one after the other.  The
// codes, gamma_A and code sums are those of quantize_row_wave.
template <int DT, bool VEC, int RC = 4>
__device__ __forceinline__ void quantize_two_rows_wave(const void* __restrict__ row0, const void* __restrict__ row1,
                                                       int64_t K, int64_t Kp, int lane, int8_t* __restrict__ dst0,
                                                       int8_t* __restrict__ dst1, float (&gamma_a)[2], int (&codesum)[2]) {
  constexpr int P = ActTraits<DT>::kPerChunk;
  const int64_t nc = K / P;
  if (!VEC || nc > RC * kWave) {
    quantize_row_wave<DT, VEC, RC>(row0, K, Kp, lane, dst0, gamma_a[0], codesum[0]);
    quantize_row_wave<DT, VEC, RC>(row1, K, Kp, lane, dst1, gamma_a[1], codesum[1]);
    return;
  }
  const uint4* r4[2] = {static_cast<const uint4*>(row0), static_cast<const uint4*>(row1)};
  int8_t* dst[2] = {dst0, dst1};
  uint4 v[2][RC];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < RC; ++u) {
      const int64_t c = lane + u * kWave;
      v[t][u] = r4[t][c < nc ? c : nc - 1];
    }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float mx = 0.0f;
#pragma unroll
    for (int u = 0; u < RC; ++u) {
      float f[P];
      chunk_to_f32<DT>(v[t][u], f);
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < P; ++i) m = fmaxf(m, fabsf(f[i]));
      mx = (lane + u * kWave < nc) ? fmaxf(mx, m) : mx;
    }
    mx = quant_wave_max(mx);
    const float s = __fdiv_rn(127.0f, __fadd_rn(mx, kEps));
    int sum = 0;
#pragma unroll
    for (int u = 0; u < RC; ++u) {
      const int64_t c = lane + u * kWave;
      if (c < nc) sum += quantize_chunk<DT>(v[t][u], s, dst[t] + c * P);
    }
    for (int64_t k = K + lane; k < Kp; k += kWave) dst[t][k] = 0;
    gamma_a[t] = mx;
    codesum[t] = quant_wave_sum(sum);
  }
}

}  // namespace bitlinear
