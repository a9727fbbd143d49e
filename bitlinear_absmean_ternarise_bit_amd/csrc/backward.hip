// Backward of BitLinear with the straight-through estimator (STE).
//
// [PMV] = produtoramaxvision.com.br article on BitNet b1.58: its STE passage
// takes the quantiser's gradient as the identity, dW_q/dW = 1, for values
// inside the valid range.  The forward is Y = A_hat W_hat^T with
// A_hat = (gamma_A / 127) A_q and W_hat = gamma W_q, so
//     dX = dY W_hat = gamma (dY W_q)
//     dW = (dY^T A_hat) * 1[|fp32(W / fp32(gamma + eps))| <= 1]
// (the activation clip never binds; gamma and gamma_A are constants).
// Training precision: dY and A_hat in bfloat16, float32 accumulation.
//
// Both contractions run on one bf16 MFMA GEMM, C[p, q] = sum_r A[p, r] B[q, r],
// whose operands both have the contraction index contiguous:
//   dX: A = dY (in place when its rows start on 16-byte boundaries, else a
//       zero-padded copy), B = the ternary codes of W^T, packed in
//       the 2-bit format (pack_transposed_kernel) and expanded to bf16 {-1,0,1}
//       while they are staged into LDS;
//   dW: A = dY^T, B = A_hat^T (transposed copies, zero-padded along M).
#include "kernels.hpp"

namespace bitlinear {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 64;  // transpose / pack tiles

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t offset_code(float w, float d, bool valid) {
  const float t = __fdiv_rn(w, d);
  const float q = __builtin_rintf(fminf(fmaxf(t, -1.0f), 1.0f));
  return valid ? static_cast<uint32_t>(static_cast<int>(q) + 1) : 1u;
}

// Codes of W^T ([K rows of Np = padded_k(N) codes]) in the 2-bit format and
// its interleaved row order.  One workgroup per 64 (n) x 64 (k) tile of W:
// codes go through LDS transposed, then each thread writes one word (16
// consecutive n of one k).
__global__ __launch_bounds__(256) void pack_transposed_kernel(const float* __restrict__ W, int64_t N,
                                                              int64_t K, const float* __restrict__ gamma,
                                                              uint32_t* __restrict__ packedT, int64_t Np) {
  __shared__ uint8_t codes[kTile][kTile + 4];  // [k][n]
  const float d = __fadd_rn(gamma[0], kEps);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kTile;
  const int64_t k0 = static_cast<int64_t>(blockIdx.y) * kTile;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < kTile * kTile; idx += 256) {
    const int nl = idx >> 6, kl = idx & 63;  // consecutive threads: consecutive k of one row n
    const int64_t n = n0 + nl, k = k0 + kl;
    const bool valid = n < N && k < K;
    const float w = valid ? W[n * K + k] : 0.0f;
    codes[kl][nl] = static_cast<uint8_t>(offset_code(w, d, n < N));
  }
  __syncthreads();
  const int kl = tid >> 2, jw = tid & 3;
  const int64_t k = k0 + kl;
  if (k >= K) return;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int b = 0; b < 4; ++b) word |= static_cast<uint32_t>(codes[kl][16 * jw + 4 * i + b]) << (8 * b + 2 * i);
  const uint32_t off = unit_offset(static_cast<uint32_t>(k), static_cast<uint32_t>(n0 >> 6),
                                   static_cast<uint32_t>(K), static_cast<uint32_t>(Np >> 6));
  packedT[(off >> 2) + jw] = word;
}

// dYp[m, n] = dY[m, n] for n < N, 0 for N <= n < Np (bf16 bit patterns).
__global__ __launch_bounds__(256) void pad_rows_bf16_kernel(const uint16_t* __restrict__ src, int64_t M, int64_t N,
                                                            uint16_t* __restrict__ dst, int64_t Np) {
  const int64_t total = M * Np;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t m = i / Np, n = i - m * Np;
    dst[i] = n < N ? src[m * N + n] : static_cast<uint16_t>(0);
  }
}

// Transposes of the M-major operands into rows of Mp (zero-padded) entries:
//   MODE 0: dst[n, m] = dY[m, n]                          (src bf16 [M, N])
//   MODE 1: dst[k, m] = bf16(fp32(fp32(gamma_A[m] / 127) * Xq[m, k]))  (Xq int8 [M, ld])
template <int MODE>
__global__ __launch_bounds__(256) void transpose_kernel(const void* __restrict__ src, int64_t M, int64_t R,
                                                        int64_t ld, const float* __restrict__ gamma_a,
                                                        uint16_t* __restrict__ dst, int64_t Mp) {
  __shared__ uint16_t tile[kTile][kTile + 2];  // [m][r]
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kTile;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kTile;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < kTile * kTile; idx += 256) {
    const int ml = idx >> 6, rl = idx & 63;
    const int64_t m = m0 + ml, r = r0 + rl;
    uint16_t v = 0;
    if (m < M && r < R) {
      if constexpr (MODE == 0) {
        v = static_cast<const uint16_t*>(src)[m * ld + r];
      } else {
        const float c = __fdiv_rn(gamma_a[m], 127.0f);
        const int8_t q = static_cast<const int8_t*>(src)[m * ld + r];
        v = f32_to_bf16_rne(__fmul_rn(c, static_cast<float>(q)));
      }
    }
    tile[ml][rl] = v;
  }
  __syncthreads();
  for (int idx = tid; idx < kTile * kTile; idx += 256) {
    const int rl = idx >> 6, ml = idx & 63;
    const int64_t m = m0 + ml, r = r0 + rl;
    if (r < R && m < Mp) dst[r * Mp + m] = tile[ml][rl];
  }
}

// bf16 MFMA GEMM, C[p, q] = sum_r A[p, r] B[q, r] over r < Rp (a multiple of 64).
// A: bf16 [P, Rp] with row stride lda >= Rp, or, when B is packed, lda >= the
// number of real columns (padding codes are zero weights, so whatever A holds
// past a row's end only meets zeros); rows 16-byte aligned.  B: bf16 [Q, Rp]
// (BMODE 0) or the 2-bit ternary codes of a [Q, Rp] matrix in the packed
// format (BMODE 1), expanded to bf16 c - 1.
// EPI 0: C * gamma;  EPI 1: C where |fp32(W[p, q] / fp32(gamma + eps))| <= 1, else 0.
// Tile 128 x 128, 4 waves of 64 x 64 (2 x 2 MFMA tiles of 32 x 32), 64 r per
// LDS stage, two stages; rows of an operand stage are 128 bytes with 16-byte
// slot c of row r stored at slot c ^ (r & 7).
template <int BMODE, int EPI>
__global__ __launch_bounds__(256) void bf16_gemm_nt_kernel(const uint16_t* __restrict__ A, int64_t P,
                                                           int64_t lda, const void* __restrict__ B, int64_t Q,
                                                           int64_t Rp,
                                                           float* __restrict__ C, int64_t ldc,
                                                           const float* __restrict__ gamma,
                                                           const float* __restrict__ W, int64_t ldw,
                                                           int bytes_a, int bytes_b) {
  constexpr int BM = 128, BN = 128, BK = 64;
  constexpr int ROWB = BK * 2;
  constexpr int A_BYTES = BM * ROWB;
  constexpr int STAGE = A_BYTES + BN * ROWB;
  __shared__ __align__(16) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t p0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t q0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int niter = static_cast<int>(Rp / BK);
  const uint32_t rowbytes = static_cast<uint32_t>(Rp) * 2u;
  const uint32_t rowbytes_a = static_cast<uint32_t>(lda) * 2u;

  const __amdgpu_buffer_rsrc_t rsrc_a =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A), 0, bytes_a, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_b =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(B), 0, bytes_b, 0x00020000);
  constexpr uint32_t kOff = 0x80000000u;  // past every resource: reads zeros

  // A (and dense B): 128 rows x 8 slots per stage, 4 slots per thread
  uint32_t a_off[4], a_dst[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = tid + 256 * i, r = s >> 3, c = s & 7;
    a_off[i] = (p0 + r < P) ? static_cast<uint32_t>(p0 + r) * rowbytes_a + 16u * c : kOff;
    b_off[i] = (q0 + r < Q) ? static_cast<uint32_t>(q0 + r) * rowbytes + 16u * c : kOff;
    a_dst[i] = r * ROWB + 16 * (c ^ (r & 7));
  }
  // packed B: thread tid < 128 stages row tid (one 16-byte unit of 64 codes)
  const uint32_t units = static_cast<uint32_t>(Rp >> 6);
  const bool pb_row = tid < BN && q0 + tid < Q;

  v4u ra[4], rb[4];
  auto gload = [&](int it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, a_off[i] == kOff ? kOff : a_off[i] + 128u * it, 0, 0);
    if constexpr (BMODE == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, b_off[i] == kOff ? kOff : b_off[i] + 128u * it, 0, 0);
    } else {
      const uint32_t off = pb_row ? unit_offset(static_cast<uint32_t>(q0 + tid), static_cast<uint32_t>(it),
                                                static_cast<uint32_t>(Q), units)
                                  : kOff;
      rb[0] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, off, 0, 0);
    }
  };
  auto swrite = [&](char* st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<v4u*>(st + a_dst[i]) = ra[i];
    char* sb = st + A_BYTES;
    if constexpr (BMODE == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<v4u*>(sb + a_dst[i]) = rb[i];
    } else if (tid < BN) {
      // 64 codes -> 64 bf16 values c - 1 through two byte tables (v_perm):
      // high bytes {0xBF, 0x00, 0x3F} and low bytes {0x80, 0x00, 0x80} for c = 0, 1, 2
      constexpr uint32_t kHi = 0x003F00BFu, kLo = 0x00800080u;
      const int r = tid;
#pragma unroll
      for (int c = 0; c < 8; ++c) {  // slot c: k = 8c .. 8c + 7 = word c/2, fields i = 2(c%2), 2(c%2)+1
        const uint32_t w = rb[0][c >> 1];
        v4u out;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t x = (w >> (2 * (2 * (c & 1) + h))) & 0x03030303u;
          const uint32_t hi = __builtin_amdgcn_perm(0u, kHi, x);
          const uint32_t lo = __builtin_amdgcn_perm(0u, kLo, x);
          out[2 * h] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
          out[2 * h + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
        }
        *reinterpret_cast<v4u*>(sb + r * ROWB + 16 * (c ^ (r & 7))) = out;
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int lr = lane & 31, lh = lane >> 5;
  gload(0);
  swrite(smem);
  __syncthreads();
  for (int it = 0; it < niter; ++it) {
    char* cur = smem + (it & 1) * STAGE;
    gload(it + 1 < niter ? it + 1 : it);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int slot = 2 * ks + lh;
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + lr;
        a[i] = *reinterpret_cast<const bf16x8*>(cur + r * ROWB + 16 * (slot ^ (r & 7)));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + lr;
        b[j] = *reinterpret_cast<const bf16x8*>(cur + A_BYTES + r * ROWB + 16 * (slot ^ (r & 7)));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    swrite(smem + ((it + 1) & 1) * STAGE);
    __syncthreads();
  }

  // epilogue: lane holds rows 8 (e / 4) + 4 lh + e % 4, column lr of each 32 x 32 tile
  const float g = gamma[0];
  const float d = __fadd_rn(g, kEps);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t p = p0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
      if (p >= P) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t q = q0 + wn * 64 + j * 32 + lr;
        if (q >= Q) continue;
        float v = acc[i][j][e];
        if constexpr (EPI == 0) {
          v = __fmul_rn(v, g);
        } else {
          const float t = __fdiv_rn(W[p * ldw + q], d);
          v = fabsf(t) <= 1.0f ? v : 0.0f;
        }
        C[p * ldc + q] = v;
      }
    }
}

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

size_t backward_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int64_t Mp = ((M + 63) / 64) * 64, Np = padded_k(N);
  return align256(static_cast<size_t>(M * Np * 2)) + align256(static_cast<size_t>(N * Mp * 2)) +
         align256(static_cast<size_t>(K * Mp * 2));
}

hipError_t launch_pack_transposed(const float* W, int64_t N, int64_t K, const float* gamma, uint32_t* packedT,
                                  hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((N + kTile - 1) / kTile), static_cast<unsigned>((K + kTile - 1) / kTile));
  pack_transposed_kernel<<<grid, 256, 0, stream>>>(W, N, K, gamma, packedT, padded_k(N));
  return hipGetLastError();
}

hipError_t launch_backward(const uint16_t* dY, int64_t M, int64_t N, int64_t K, const uint32_t* packedT,
                           const float* gamma, const int8_t* Xq, const float* gamma_a, const float* W, float* dX,
                           float* dW, void* workspace, hipStream_t stream) {
  const int64_t Mp = ((M + 63) / 64) * 64, Np = padded_k(N), Kp = padded_k(K);
  char* ws = static_cast<char*>(workspace);
  uint16_t* dYp = reinterpret_cast<uint16_t*>(ws);
  ws += align256(static_cast<size_t>(M * Np * 2));
  uint16_t* dYt = reinterpret_cast<uint16_t*>(ws);
  ws += align256(static_cast<size_t>(N * Mp * 2));
  uint16_t* At = reinterpret_cast<uint16_t*>(ws);
  if (dX) {
    // dY's rows serve as they are when they start on 16-byte boundaries
    const bool direct = N % 8 == 0 && reinterpret_cast<uintptr_t>(dY) % 16 == 0;
    if (!direct) {
      int64_t blocks = (M * Np + 255) / 256;
      if (blocks > 65536) blocks = 65536;
      pad_rows_bf16_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(dY, M, N, dYp, Np);
    }
    const dim3 grid(static_cast<unsigned>((K + 127) / 128), static_cast<unsigned>((M + 127) / 128));
    bf16_gemm_nt_kernel<1, 0><<<grid, 256, 0, stream>>>(direct ? dY : dYp, M, direct ? N : Np, packedT, K, Np,
                                                         dX, K, gamma, nullptr, 0,
                                                         static_cast<int>(M * (direct ? N : Np) * 2),
                                                         static_cast<int>(K * (Np / 4)));
  }
  if (dW) {
    const dim3 g0(static_cast<unsigned>((N + kTile - 1) / kTile), static_cast<unsigned>(Mp / kTile));
    transpose_kernel<0><<<g0, 256, 0, stream>>>(dY, M, N, N, nullptr, dYt, Mp);
    const dim3 g1(static_cast<unsigned>((K + kTile - 1) / kTile), static_cast<unsigned>(Mp / kTile));
    transpose_kernel<1><<<g1, 256, 0, stream>>>(Xq, M, K, Kp, gamma_a, At, Mp);
    const dim3 grid(static_cast<unsigned>((K + 127) / 128), static_cast<unsigned>((N + 127) / 128));
    bf16_gemm_nt_kernel<0, 1><<<grid, 256, 0, stream>>>(dYt, N, Mp, At, K, Mp, dW, K, gamma, W, K,
                                                         static_cast<int>(N * Mp * 2),
                                                         static_cast<int>(K * Mp * 2));
  }
  return hipGetLastError();
}

}  // namespace bitlinear
