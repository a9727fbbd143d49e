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

  // Packed rows are read, and outputs written, through buffer resources over
  // this layer's arrays.  Every load and store is unconditional: offsets that
  // must not touch memory (rows past N, words past a row's end, batches past
  // the last, outputs that are not due yet) are set past the resource and the
  // hardware bounds check turns them into zeros / dropped stores.  Without
  // branches the compiler keeps the next batch of loads in flight while the
  // current one is contracted.
  constexpr uint32_t kOff = 0xfffffff0u;  // past every resource
  const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(packed), 0, static_cast<int>(N * words * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t ysrc = __builtin_amdgcn_make_buffer_rsrc(
      Y, 0, static_cast<int>(static_cast<int64_t>(M) * N * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t asrc = __builtin_amdgcn_make_buffer_rsrc(
      WRITE_ACC ? static_cast<void*>(acc) : static_cast<void*>(Y), 0,
      WRITE_ACC ? static_cast<int>(static_cast<int64_t>(M) * N * 4) : 0, 0x00020000);
  const uint32_t words32 = static_cast<uint32_t>(words);
  const uint32_t N32 = static_cast<uint32_t>(N);
  auto load_batch = [&](int b, bool valid, uint4 (&r)[kUnroll]) {
    const int gi = b / bpg;
    const int cb = b - gi * bpg;
    const uint32_t row_off = static_cast<uint32_t>(n_base + gi * kRowsPerWave + j) * words32 * 4u;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t w0 = static_cast<uint32_t>(cb * kUnroll + u) * 16u + 4u * g;
      const uint32_t off = (valid && w0 < words32) ? row_off + 4u * w0 : kOff;
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(wsrc, off, 0, 0);
      r[u] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };

  uint4 buf0[kUnroll], buf1[kUnroll];
  load_batch(0, true, buf0);
  __builtin_amdgcn_sched_barrier(0);

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
  const int8_t* arow = sxq + (avalid ? j : 0) * lds_stride;
  const v4i zero = {0, 0, 0, 0};
  const float gm = gamma[0];
  v4i c = zero;

  auto contract = [&](int b, const uint4 (&r)[kUnroll]) {
    const int gi = b / bpg;
    const int cb = b - gi * bpg;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t w0 = static_cast<uint32_t>(cb * kUnroll + u) * 16u + 4u * g;
      const bool use = avalid && w0 < words32;
      const uint32_t wd[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const v4i bop = unpack_word(wd[t]);
        const v4i araw = *reinterpret_cast<const v4i*>(arow + (use ? 16u * (w0 + t) : 0u));
        const v4i a = use ? araw : zero;
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bop, c, 0, 0, 0);
      }
    }
    // epilogue of the row group after its last batch: lane holds tokens
    // 4g + r of weight row n
    const bool last = cb == bpg - 1;
    const uint32_t n = static_cast<uint32_t>(n_base + gi * kRowsPerWave + j);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * g + r;
      const int ic = i < M ? i : M - 1;
      const int v = c[r] - s_rs[ic];
      const float scale = __fdiv_rn(__fmul_rn(gm, s_ga[ic]), 127.0f);
      const float y = __fmul_rn(static_cast<float>(v), scale);
      const uint32_t off = (last && i < M && n < N32) ? (static_cast<uint32_t>(i) * N32 + n) * 4u : kOff;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), ysrc, off, 0, 0);
      if constexpr (WRITE_ACC) __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(v), asrc, off, 0, 0);
    }
    c = last ? zero : c;
  };

  // sched_barrier keeps the scheduler from sinking a batch's loads into the
  // contraction that follows them.
  int b = 0;
  for (; b + 1 < nbatch; b += 2) {
    load_batch(b + 1, true, buf1);
    __builtin_amdgcn_sched_barrier(0);
    contract(b, buf0);
    load_batch(b + 2, b + 2 < nbatch, buf0);
    __builtin_amdgcn_sched_barrier(0);
    contract(b + 1, buf1);
  }
  if (b < nbatch) contract(b, buf0);
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
