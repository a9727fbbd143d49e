// Prefill path (large M): INT8-MFMA GEMM of the activation codes against the
// packed ternary codes, with the dequantisation fused into the epilogue.
//
// [PMV] = produtoramaxvision.com.br article on BitNet b1.58: section 2's
// Zero-GEMM (add / subtract / skip, INT32 accumulation, one rescale by
// gamma_A * gamma / 127).  At large M the contraction is a dense GEMM, so it
// runs on the matrix cores: codes c = q + 1 in {0,1,2} are unpacked from the
// 2-bit words in registers and fed to v_mfma_i32_32x32x32_i8 as the B operand;
// the exact token code sum is subtracted in the epilogue
// (sum_k q x = sum_k c x - sum_k x).
//
// Tiling: a 256-thread workgroup owns a 256 (tokens) x 256 (weight rows)
// output tile; its four waves each own 128 x 128 (4 x 4 MFMA tiles of
// 32 x 32).  K advances 128 per step through two LDS stages: activation codes
// [256][128] (rows padded to 144 bytes) and packed words [256][8] (rows
// padded to 48 bytes), so 8 consecutive lanes reading 16 bytes each touch
// distinct banks.
//
// MFMA operands: for 32x32x32 int8, lane l supplies 16 bytes of A row l % 32
// and of B column l % 32, for the same 16 k positions (chosen by l / 32).  In
// K step s (32 k) of a 128-k stage, lane group h = l / 32 uses packed word
// 4h + s of its weight row (16 weights) and the 16 activation codes at
// k = 64h + 16s of its token row: the same k on both sides.
#include "kernels.hpp"

namespace bitlinear {

namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int A_STRIDE = BK + 16;       // bytes per activation row in LDS
constexpr int B_STRIDE = 48;            // bytes per packed weight row in LDS (32 used)
constexpr int A_BYTES = BM * A_STRIDE;  // 36864
constexpr int B_BYTES = BN * B_STRIDE;  // 12288
constexpr int STAGE = A_BYTES + B_BYTES;

template <bool WRITE_ACC>
__global__ __launch_bounds__(256, 1) void prefill_gemm_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ gamma_a,
    const int32_t* __restrict__ rowsum, int64_t M, int64_t Kp, const uint32_t* __restrict__ packed,
    int64_t N, const float* __restrict__ gamma, float* __restrict__ Y, int32_t* __restrict__ acc,
    int tiles_n) {
  __shared__ __align__(16) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tm = blockIdx.x / tiles_n;
  const int tn = blockIdx.x - tm * tiles_n;
  const int64_t m0 = static_cast<int64_t>(tm) * BM;
  const int64_t n0 = static_cast<int64_t>(tn) * BN;
  const int64_t words = Kp >> 4;
  const int niter = static_cast<int>((Kp + BK - 1) / BK);

  // global -> register staging: A 8 x 16 B per thread, B 2 x 16 B per thread
  uint4 ra[8], rb[2];
  const int a_row = tid >> 3, a_col = tid & 7;  // + 32 p rows
  const int b_row = tid >> 1, b_half = tid & 1; // + 128 p rows

  auto gload = [&](int it) {
    const int64_t k0 = static_cast<int64_t>(it) * BK;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int64_t m = m0 + a_row + 32 * p;
      const int64_t kk = k0 + 16 * a_col;
      ra[p] = (m < M && kk < Kp) ? *reinterpret_cast<const uint4*>(Xq + m * Kp + kk)
                                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int64_t n = n0 + b_row + 128 * p;
      const int64_t w = (k0 >> 4) + 4 * b_half;
      rb[p] = (n < N && w < words) ? *reinterpret_cast<const uint4*>(packed + n * words + w)
                                   : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
    char* sa = smem + buf * STAGE;
    char* sb = sa + A_BYTES;
#pragma unroll
    for (int p = 0; p < 8; ++p)
      *reinterpret_cast<uint4*>(sa + (a_row + 32 * p) * A_STRIDE + 16 * a_col) = ra[p];
#pragma unroll
    for (int p = 0; p < 2; ++p)
      *reinterpret_cast<uint4*>(sb + (b_row + 128 * p) * B_STRIDE + 16 * b_half) = rb[p];
  };

  v16i c[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) c[mi][ni][r] = 0;

  const int lr = lane & 31;
  const int lh = lane >> 5;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int it = 0; it < niter; ++it) {
    const int buf = it & 1;
    if (it + 1 < niter) gload(it + 1);
    const char* sa = smem + buf * STAGE;
    const char* sb = sa + A_BYTES;
    uint4 bw[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      bw[ni] = *reinterpret_cast<const uint4*>(sb + (wn * 128 + ni * 32 + lr) * B_STRIDE + 16 * lh);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4i a[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        a[mi] = *reinterpret_cast<const v4i*>(sa + (wm * 128 + mi * 32 + lr) * A_STRIDE + 64 * lh + 16 * s);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const uint32_t wd = s == 0 ? bw[ni].x : s == 1 ? bw[ni].y : s == 2 ? bw[ni].z : bw[ni].w;
        const v4i b = unpack_word(wd);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          c[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[mi], b, c[mi][ni], 0, 0, 0);
      }
    }
    if (it + 1 < niter) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 8*(r/4) + 4*(l/32) + r%4, column l%32 of each 32x32 tile
  const float gm = gamma[0];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = m0 + wm * 128 + mi * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (m >= M) continue;
      const int rs = rowsum[m];
      const float scale = __fdiv_rn(__fmul_rn(gm, gamma_a[m]), 127.0f);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int64_t n = n0 + wn * 128 + ni * 32 + lr;
        if (n < N) {
          const int v = c[mi][ni][r] - rs;
          if constexpr (WRITE_ACC) acc[m * N + n] = v;
          Y[m * N + n] = __fmul_rn(static_cast<float>(v), scale);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill_gemm(const int8_t* Xq, const float* gamma_a, const int32_t* rowsum,
                               int64_t M, int64_t K, const uint32_t* packed, int64_t N,
                               const float* gamma, float* Y, int32_t* acc, hipStream_t stream) {
  const int64_t Kp = padded_k(K);
  const int tiles_m = static_cast<int>((M + BM - 1) / BM);
  const int tiles_n = static_cast<int>((N + BN - 1) / BN);
  const unsigned blocks = static_cast<unsigned>(tiles_m) * static_cast<unsigned>(tiles_n);
  if (acc)
    prefill_gemm_kernel<true><<<blocks, 256, 0, stream>>>(Xq, gamma_a, rowsum, M, Kp, packed, N,
                                                          gamma, Y, acc, tiles_n);
  else
    prefill_gemm_kernel<false><<<blocks, 256, 0, stream>>>(Xq, gamma_a, rowsum, M, Kp, packed, N,
                                                           gamma, Y, acc, tiles_n);
  return hipGetLastError();
}

}  // namespace bitlinear
