// LUT contraction (comparison variant of the decode GEMV).
//
// [PMV] = produtoramaxvision.com.br article on BitNet b1.58, section 4 (how
// bitnet.cpp speeds up CPU inference), LUT-GEMM figure: for a block of four
// INT8 activations every one of the 3^4 = 81 ternary weight patterns has a
// pre-computed sum, so the packed weights index a table instead of being
// unpacked; the looked-up entries are summed in INT32.  CPUs keep the table in
// L1 and index it with byte shuffles; here each workgroup builds the tables of
// the tokens in LDS and every thread looks up entries for one weight row.
//
// Blocks of four activations follow the 2-bit format: byte b of packed word j
// holds the codes of k = 16j + b + 4t (t = 0..3, bits 2t..2t+1), so that byte
// is one block and its table is built from x[16j + b + 4t].  The table index
// is the base-3 number of the byte's codes c_0 c_1 c_2 c_3 (first weight most
// significant), so index 0 is all -1, 40 all 0 and 80 all +1 as in the figure;
// entry e holds sum_t (c_t(e) - 1) a_t, at most 4 * 127 in magnitude (int16).
//
// A workgroup owns 256 weight rows of one layer (a thread per row) and walks
// K in slices of 256 weights (128 for 5 to 8 tokens, 64 beyond, so a slice
// has at most 256 tables): it builds each token's tables for the slice, a
// thread per table, then every thread turns its row's packed bytes of the
// slice into table indices with SWAR arithmetic and adds one table entry per
// token.  Rows are read 64 contiguous bytes (four units) at a time, so no
// line is fetched twice.  The accumulators stay in registers and the epilogue
// applies the same rescale as the other paths.  The tables cost 81 entries
// per block per token per workgroup, paid back only because a workgroup's
// 256 rows share them; the lookups are LDS reads, one per block per token,
// which bounds the scheme well below the matrix-core GEMV as M grows.
#include "kernels.hpp"

namespace bitlinear {

namespace {

constexpr int kLutRows = 256;    // weight rows per workgroup, one per thread
constexpr int kLutStride = 41;   // 32-bit words per table: 81 int16 entries + 1 pad

// Index bytes of four packed-code bytes: per byte, the base-3 number of its
// four 2-bit codes with the code in bits 0-1 most significant.  Every partial
// value stays below 81, so the four bytes never carry into each other.
__device__ __forceinline__ uint32_t lut_index4(uint32_t w) {
  const uint32_t c0 = w & 0x03030303u, c1 = (w >> 2) & 0x03030303u;
  const uint32_t c2 = (w >> 4) & 0x03030303u, c3 = (w >> 6) & 0x03030303u;
  uint32_t v = c0 * 3u + c1;
  v = v * 3u + c2;
  return v * 3u + c3;
}

// The 81 pre-sums of (a0, a1, a2, a3), entry e = 27 c0 + 9 c1 + 3 c2 + c3
// holding sum_t (c_t - 1) a_t, stored as int16 pairs in table[0 .. 40].
__device__ __forceinline__ void build_table(uint32_t* table, int a0, int a1, int a2, int a3) {
  int t3[27];
#pragma unroll
  for (int c1 = 0; c1 < 3; ++c1)
#pragma unroll
    for (int c2 = 0; c2 < 3; ++c2)
#pragma unroll
      for (int c3 = 0; c3 < 3; ++c3) t3[9 * c1 + 3 * c2 + c3] = (c1 - 1) * a1 + (c2 - 1) * a2 + (c3 - 1) * a3;
  int e[82];
#pragma unroll
  for (int c0 = 0; c0 < 3; ++c0)
#pragma unroll
    for (int r = 0; r < 27; ++r) e[27 * c0 + r] = (c0 - 1) * a0 + t3[r];
  e[81] = 0;
#pragma unroll
  for (int p = 0; p < kLutStride; ++p)
    table[p] = (static_cast<uint32_t>(e[2 * p]) & 0xffffu) | (static_cast<uint32_t>(e[2 * p + 1]) << 16);
}

// M tokens (<= 16).  A slice is SU 16-byte units of every row (16 SU blocks);
// the tables of token m, block g of the slice start at word (m * 16 SU + g) * 41
// of LDS.  Rows are read a chunk of four units (64 contiguous bytes) at a time.
template <int M>
__global__ __launch_bounds__(kLutRows) void lut_gemv_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ gamma_a, int64_t Kp,
    const uint32_t* __restrict__ packed, int64_t N, const float* __restrict__ gamma, float* __restrict__ Y,
    int32_t* __restrict__ acc_out, int blocks_per_layer) {
  constexpr int SU = M <= 4 ? 4 : M <= 8 ? 2 : 1;  // units per slice: at most 256 tables, 42 KB of LDS
  constexpr int G = 16 * SU;          // blocks per slice
  __shared__ uint32_t tables[M * G * kLutStride];
  const int tid = threadIdx.x;
  // workgroups are dealt round-robin to the 8 XCDs: give each XCD a
  // contiguous run of (layer, row block) pairs, so a layer's workgroups share
  // one L2 for its token codes
  const uint32_t per_xcd = gridDim.x >> 3;
  const uint32_t v = blockIdx.x < 8u * per_xcd ? (blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3) : blockIdx.x;
  const int64_t layer = v / blocks_per_layer;
  const uint32_t n = static_cast<uint32_t>(v % blocks_per_layer) * kLutRows + tid;
  const uint32_t U = static_cast<uint32_t>(Kp >> 6);  // 16-byte units per row
  const uint32_t N32 = static_cast<uint32_t>(N);
  Xq += layer * M * Kp;
  gamma_a += layer * M;
  packed += layer * N * (Kp >> 4);
  const char* wbase = reinterpret_cast<const char*>(packed);
  const bool row_ok = n < N32;
  const int16_t* t16 = reinterpret_cast<const int16_t*>(tables);

  int acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0;

  const uint32_t chunks = (U + 3) >> 2;
  for (uint32_t c = 0; c < chunks; ++c) {
    // the row's units of the chunk, requested before the first tables are built
    v4u w[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t u = 4u * c + h;
      w[h] = row_ok && u < U ? *reinterpret_cast<const v4u*>(wbase + unit_offset(n, u, N32, U)) : v4u{0, 0, 0, 0};
    }
#pragma unroll
    for (int sl = 0; sl < 4 / SU; ++sl) {
      const uint32_t u0 = 4u * c + SU * sl;  // first unit of the slice
      if (u0 >= U) break;
      // tables of the slice: thread tt builds token tt / G, block tt % G
      for (int tt = tid; tt < M * G; tt += kLutRows) {
        const int m = tt / G, g = tt % G;
        const uint32_t u = u0 + g / 16;
        if (u < U) {
          const uint32_t j = 4u * u + ((g >> 2) & 3);  // packed word of the block
          const int b = g & 3;                          // byte of the block in that word
          const v4u x = *reinterpret_cast<const v4u*>(Xq + m * Kp + 16 * j);
          // bytes b, b + 4, b + 8, b + 12 of the word's 16 activations, sign-extended
          const int sh = 8 * b;
          const int a0 = static_cast<int>(x[0] << (24 - sh)) >> 24;
          const int a1 = static_cast<int>(x[1] << (24 - sh)) >> 24;
          const int a2 = static_cast<int>(x[2] << (24 - sh)) >> 24;
          const int a3 = static_cast<int>(x[3] << (24 - sh)) >> 24;
          build_table(tables + tt * kLutStride, a0, a1, a2, a3);
        }
      }
      __syncthreads();
      if (row_ok) {
#pragma unroll
        for (int h = 0; h < SU; ++h) {
          if (u0 + h < U) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t idx4 = lut_index4(w[SU * sl + h][q]);
#pragma unroll
              for (int b = 0; b < 4; ++b) {
                const int g = 16 * h + 4 * q + b;
                const uint32_t e = (idx4 >> (8 * b)) & 0xffu;
#pragma unroll
                for (int m = 0; m < M; ++m) acc[m] += t16[(m * G + g) * (2 * kLutStride) + e];
              }
            }
          }
        }
      }
      __syncthreads();
    }
  }

  if (!row_ok) return;
  const float gm = gamma[layer];
  float* Yl = Y + layer * M * N;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float scale = __fdiv_rn(__fmul_rn(gm, gamma_a[m]), 127.0f);
    if (acc_out) acc_out[layer * M * N + m * N + n] = acc[m];
    Yl[m * N + n] = __fmul_rn(static_cast<float>(acc[m]), scale);
  }
}

template <int M>
hipError_t launch_m(int64_t m, const int8_t* Xq, const float* gamma_a, int64_t Kp, const uint32_t* packed, int64_t N,
                    const float* gamma, float* Y, int32_t* acc, int64_t L, hipStream_t stream) {
  if constexpr (M < kDecodeMaxM) {
    if (m != M) return launch_m<M + 1>(m, Xq, gamma_a, Kp, packed, N, gamma, Y, acc, L, stream);
  }
  const int blocks_per_layer = static_cast<int>((N + kLutRows - 1) / kLutRows);
  const unsigned grid = static_cast<unsigned>(L * blocks_per_layer);
  lut_gemv_kernel<M><<<grid, kLutRows, 0, stream>>>(Xq, gamma_a, Kp, packed, N, gamma, Y, acc, blocks_per_layer);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lut_gemv(const int8_t* Xq, const float* gamma_a, int64_t M, int64_t K, const uint32_t* packed,
                           int64_t N, const float* gamma, float* Y, int32_t* acc, int64_t L, hipStream_t stream) {
  return launch_m<1>(M, Xq, gamma_a, padded_k(K), packed, N, gamma, Y, acc, L, stream);
}

}  // namespace bitlinear
