// Decode path (M <= 16 tokens): one fused kernel per call.
//
//   phase A  each workgroup quantises the (few) tokens into LDS with the
//            per-token AbsMax quantiser (one wave per token);
//   phase B  each wave streams the packed codes of 16 weight rows once from
//            HBM (16 bytes per lane per load, 64 contiguous bytes per row per
//            load instruction), unpacks them in registers and contracts them
//            against the LDS codes with v_mfma_i32_16x16x64_i8;
//   epilogue INT32 accumulator -> float32 times gamma * gamma_A / 127.
//
// [PMV] = produtoramaxvision.com.br article on BitNet b1.58: section 2's
// Zero-GEMM adds the activation for a +1 weight, subtracts it for -1 and skips
// 0, accumulating in INT32, then rescales once by gamma_A * gamma / 127.
// gfx950 has no ternary ALU (the article's trade-off section notes GPUs lack
// one), so the same integer sum is formed branch-free: the stored codes are
// c = q + 1 in {0,1,2}, the matrix cores form sum_k c * x, and the exact
// token code sum is subtracted: sum_k q x = sum_k c x - sum_k x.
//
// MFMA operands: for a 16x16x64 int8 MFMA lane l supplies 16 bytes of row
// (l % 16) of A and of column (l % 16) of B, both for the same 16 k positions
// (chosen by l / 16).  Here lane l feeds weight row n0 + l%16 from its own
// packed word (16 weights = one B operand) and token l%16 from the same 16 k
// of the LDS codes, so every k is paired consistently.
#include "kernels.hpp"
#include "quant_act.hpp"

namespace bitlinear {

namespace {

constexpr int kRowsPerWave = 16;   // one MFMA column block of weight rows
constexpr int kDecodeThreads = 256;
constexpr int kWaves = kDecodeThreads / kWave;
constexpr int kUnroll = 8;         // 16-byte loads per lane per batch (8 KiB per wave)

// A wave owns `groups` blocks of 16 weight rows and walks them in batches of
// kUnroll 16-word chunks; the loads of batch b+1 are issued before batch b is
// contracted, and the first batch is in flight while phase A quantises X.
template <int DT, bool VEC, bool WRITE_ACC>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const void* __restrict__ X, int M, int64_t K, int64_t Kp, const uint32_t* __restrict__ packed,
    int64_t N, const float* __restrict__ gamma, float* __restrict__ Y, int32_t* __restrict__ acc,
    int blocks_per_layer, int groups) {
  extern __shared__ __align__(16) int8_t sxq[];
  __shared__ float s_ga[kDecodeMaxM];
  __shared__ int s_rs[kDecodeMaxM];

  constexpr int esize = DT == 0 ? 4 : 2;
  const int64_t layer = blockIdx.x / blocks_per_layer;
  const int rb = static_cast<int>(blockIdx.x - layer * blocks_per_layer);
  const int64_t words = Kp >> 4;
  const int64_t lds_stride = Kp + 16;  // +16 bytes: token rows start on different banks
  X = static_cast<const char*>(X) + layer * M * K * esize;
  packed += layer * N * words;
  Y += layer * M * N;
  if constexpr (WRITE_ACC) acc += layer * M * N;
  gamma += layer;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & (kWave - 1);
  const int j = lane & 15;
  const int g = lane >> 4;
  const int64_t n_base = (static_cast<int64_t>(rb) * kWaves + wave) * groups * kRowsPerWave;
  const int chunks = static_cast<int>((words + 15) >> 4);           // 16-word chunks per row
  const int bpg = (chunks + kUnroll - 1) / kUnroll;                   // batches per row group
  const int nbatch = groups * bpg;

  auto load_batch = [&](int b, uint4 (&r)[kUnroll]) {
    const int gi = b / bpg;
    const int cb = b - gi * bpg;
    const int64_t n = n_base + gi * kRowsPerWave + j;
    const uint32_t* prow = packed + (n < N ? n : 0) * words;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t w0 = static_cast<int64_t>(cb * kUnroll + u) * 16 + 4 * g;
      r[u] = (n < N && w0 < words) ? *reinterpret_cast<const uint4*>(prow + w0) : make_uint4(0, 0, 0, 0);
    }
  };

  uint4 buf0[kUnroll], buf1[kUnroll];
  load_batch(0, buf0);

  // phase A: AbsMax INT8 codes of every token into LDS (one wave per token)
  for (int m = wave; m < M; m += kWaves) {
    float ga;
    int rs;
    quantize_row_wave<DT, VEC>(static_cast<const char*>(X) + m * K * esize, K, Kp, lane,
                               sxq + m * lds_stride, ga, rs);
    if (lane == 0) {
      s_ga[m] = ga;
      s_rs[m] = rs;
    }
  }
  __syncthreads();

  const bool avalid = j < M;
  const int8_t* arow = sxq + j * lds_stride;
  const v4i zero = {0, 0, 0, 0};
  const float gm = gamma[0];
  v4i c = zero;

  auto contract = [&](int b, const uint4 (&r)[kUnroll]) {
    const int gi = b / bpg;
    const int cb = b - gi * bpg;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c0 = static_cast<int64_t>(cb * kUnroll + u) * 16;
      if (c0 >= words) break;  // wave-uniform
      const int64_t w0 = c0 + 4 * g;
      const bool kvalid = w0 < words;
      const uint32_t wd[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const v4i bop = unpack_word(wd[t]);
        const v4i a = (avalid && kvalid) ? *reinterpret_cast<const v4i*>(arow + 16 * (w0 + t)) : zero;
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bop, c, 0, 0, 0);
      }
    }
    if (cb == bpg - 1) {
      // epilogue: lane holds tokens 4g + r of weight row n
      const int64_t n = n_base + gi * kRowsPerWave + j;
      if (n < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * g + r;
          if (i < M) {
            const int v = c[r] - s_rs[i];
            if constexpr (WRITE_ACC) acc[static_cast<int64_t>(i) * N + n] = v;
            const float scale = __fdiv_rn(__fmul_rn(gm, s_ga[i]), 127.0f);
            Y[static_cast<int64_t>(i) * N + n] = __fmul_rn(static_cast<float>(v), scale);
          }
        }
      }
      c = zero;
    }
  };

  for (int b = 0; b < nbatch; b += 2) {
    if (b + 1 < nbatch) load_batch(b + 1, buf1);
    contract(b, buf0);
    if (b + 1 >= nbatch) break;
    if (b + 2 < nbatch) load_batch(b + 2, buf0);
    contract(b + 1, buf1);
  }
}

// Rows per workgroup = 64 * groups.  Larger blocks quantise X less often and
// stream longer runs; the choice keeps >= 2048 workgroups in flight (8 per
// CU) when the work allows and wastes at most 1/16 of a layer in its last block.
int pick_groups(int64_t L, int64_t N) {
  for (int gsz = 16; gsz > 1; gsz >>= 1) {
    const int64_t rows = int64_t(kWaves) * kRowsPerWave * gsz;
    const int64_t bpl = (N + rows - 1) / rows;
    if (L * bpl >= 2048 && (bpl * rows - N) * 16 <= N) return gsz;
  }
  return 1;
}

template <int DT, bool VEC>
hipError_t launch_v(const void* X, int64_t M, int64_t K, const uint32_t* packed, int64_t N,
                    const float* gamma, float* Y, int32_t* acc, int64_t L, hipStream_t stream) {
  const int64_t Kp = padded_k(K);
  const int groups = pick_groups(L, N);
  const int64_t rows = int64_t(kWaves) * kRowsPerWave * groups;
  const int bpl = static_cast<int>((N + rows - 1) / rows);
  const int64_t blocks = L * bpl;
  const size_t lds = static_cast<size_t>(M) * static_cast<size_t>(Kp + 16);
  if (acc)
    decode_kernel<DT, VEC, true><<<static_cast<unsigned>(blocks), kDecodeThreads, lds, stream>>>(
        X, static_cast<int>(M), K, Kp, packed, N, gamma, Y, acc, bpl, groups);
  else
    decode_kernel<DT, VEC, false><<<static_cast<unsigned>(blocks), kDecodeThreads, lds, stream>>>(
        X, static_cast<int>(M), K, Kp, packed, N, gamma, Y, acc, bpl, groups);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const void* X, int x_dtype, int64_t M, int64_t K, const uint32_t* packed,
                         int64_t N, const float* gamma, float* Y, int32_t* acc, int64_t L,
                         hipStream_t stream) {
  const int esize = x_dtype == 0 ? 4 : 2;
  const bool vec = (reinterpret_cast<uintptr_t>(X) % 16 == 0) && ((K * esize) % 16 == 0);
  if (x_dtype == 0)
    return vec ? launch_v<0, true>(X, M, K, packed, N, gamma, Y, acc, L, stream)
               : launch_v<0, false>(X, M, K, packed, N, gamma, Y, acc, L, stream);
  return vec ? launch_v<1, true>(X, M, K, packed, N, gamma, Y, acc, L, stream)
             : launch_v<1, false>(X, M, K, packed, N, gamma, Y, acc, L, stream);
}

}  // namespace bitlinear
