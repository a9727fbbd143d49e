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
// dX runs on a bf16 MFMA GEMM, C[p, q] = sum_r A[p, r] B[q, r], whose operands
// both have the contraction index contiguous: A = dY (in place when its rows
// start on 16-byte boundaries, else a zero-padded copy), B = the ternary codes
// of W^T, packed in the 2-bit format (pack_transposed_kernel) and expanded to
// bf16 {-1,0,1} while they are staged into LDS.
// dW contracts over the tokens, the row index of both dY and A_hat.  When dY
// has N % 8 == 0 and 16-byte aligned rows (and so do the codes), it is read
// as it lies, A_hat is formed once in that layout, and the matrix-core
// operands come from gfx950's transposing LDS reads (bf16_gemm_tn_kernel);
// otherwise dY^T and A_hat^T are copied out (zero-padded along M) for the
// first GEMM.  Both give the same bits: the matrix cores see the same operands
// in the same order.
#include <type_traits>

#include "kernels.hpp"

namespace bitlinear {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 64;  // transpose / pack tiles

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Codes of W^T ([K rows of Np = padded_k(N) codes]) in the 2-bit format and
// its interleaved row order, and the range mask of W as bits (bit k % 32 of
// word k / 32 of row n: |fp32(W[n, k] / fp32(gamma + eps))| <= 1; bits past K
// are 0; words per row Kw).  One workgroup per 64 (n) x 64 (k) tile of W:
// codes go through LDS transposed, then each thread writes one word (16
// consecutive n of one k); a wave reads 64 consecutive k of one row, so one
// ballot is that row's two mask words.  Either output may be NULL.
__global__ __launch_bounds__(256) void pack_transposed_kernel(const float* __restrict__ W, int64_t N,
                                                              int64_t K, const float* __restrict__ gamma,
                                                              uint32_t* __restrict__ packedT, int64_t Np,
                                                              uint32_t* __restrict__ mask, int64_t Kw) {
  __shared__ uint8_t codes[kTile][kTile + 4];  // [k][n]
  const TernaryThresholds thr = ternary_thresholds(gamma[0]);  // codes and mask without a division
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kTile;
  const int64_t k0 = static_cast<int64_t>(blockIdx.y) * kTile;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < kTile * kTile; idx += 256) {
    const int nl = idx >> 6, kl = idx & 63;  // a wave: k0 .. k0 + 63 of one row n
    const int64_t n = n0 + nl, k = k0 + kl;
    const bool valid = n < N && k < K;
    const float w = valid ? W[n * K + k] : 0.0f;
    codes[kl][nl] = static_cast<uint8_t>(ternary_code(w, thr.nonzero, n < N));
    if (mask) {
      const uint64_t bits = __ballot(valid && fabsf(w) <= thr.in_range);
      if ((tid & 63) == 0 && n < N) {
        const int64_t wd = k0 >> 5;
        mask[n * Kw + wd] = static_cast<uint32_t>(bits);
        if (wd + 1 < Kw) mask[n * Kw + wd + 1] = static_cast<uint32_t>(bits >> 32);
      }
    }
  }
  if (!packedT) return;
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
// 64 x 64 tiles through LDS with 16-byte global accesses: a source chunk is
// 8 bf16 (MODE 0) or 16 int8 (MODE 1) of one row, read whole when it lies
// inside the row and is 16-byte aligned, else element by element; an output
// chunk is 8 consecutive m of one row of dst (Mp is a multiple of 64, so
// always whole).
template <int MODE>
__global__ __launch_bounds__(256) void transpose_kernel(const void* __restrict__ src, int64_t M, int64_t R,
                                                        int64_t ld, const float* __restrict__ gamma_a,
                                                        uint16_t* __restrict__ dst, int64_t Mp) {
  __shared__ uint16_t tile[kTile][kTile + 2];  // [m][r]
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kTile;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kTile;
  const int tid = threadIdx.x;
  constexpr int PER = MODE == 0 ? 8 : 16;          // source elements per 16-byte chunk
  constexpr int CPR = kTile / PER;                 // chunks per tile row
  constexpr int esize = MODE == 0 ? 2 : 1;
  for (int idx = tid; idx < kTile * CPR; idx += 256) {
    const int ml = idx / CPR, rl = (idx % CPR) * PER;
    const int64_t m = m0 + ml, r = r0 + rl;
    uint16_t v[PER];
    if (m < M && r + PER <= R && ((m * ld + r) * esize) % 16 == 0) {
      const uint4 c = *reinterpret_cast<const uint4*>(static_cast<const char*>(src) + (m * ld + r) * esize);
      const uint32_t u[4] = {c.x, c.y, c.z, c.w};
      if constexpr (MODE == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = static_cast<uint16_t>(u[i >> 1] >> (16 * (i & 1)));
      } else {
        const float sc = __fdiv_rn(gamma_a[m], 127.0f);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int8_t q = static_cast<int8_t>(u[i >> 2] >> (8 * (i & 3)));
          v[i] = f32_to_bf16_rne(__fmul_rn(sc, static_cast<float>(q)));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        uint16_t e = 0;
        if (m < M && r + i < R) {
          if constexpr (MODE == 0) {
            e = static_cast<const uint16_t*>(src)[m * ld + r + i];
          } else {
            const float sc = __fdiv_rn(gamma_a[m], 127.0f);
            e = f32_to_bf16_rne(__fmul_rn(sc, static_cast<float>(static_cast<const int8_t*>(src)[m * ld + r + i])));
          }
        }
        v[i] = e;
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) tile[ml][rl + i] = v[i];
  }
  __syncthreads();
  // output chunk (row r, m = 8 c .. 8 c + 7); eight consecutive threads
  // write one row's 128 contiguous bytes
  for (int idx = tid; idx < kTile * (kTile / 8); idx += 256) {
    const int rl = idx >> 3, c = idx & 7;
    const int64_t r = r0 + rl;
    if (r >= R) continue;
    uint4 out;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(tile[8 * c + 2 * i][rl]) | (static_cast<uint32_t>(tile[8 * c + 2 * i + 1][rl]) << 16);
    out.x = w[0]; out.y = w[1]; out.z = w[2]; out.w = w[3];
    if (m0 + 8 * c < Mp) *reinterpret_cast<uint4*>(dst + r * Mp + m0 + 8 * c) = out;
  }
}

// Masked store of a finished tile: C[p, q] = acc where bit q of row p of the
// range mask is set, else 0.  The lane holds rows lrow + 32 i + 8 (e / 4) +
// e % 4 and columns lcol + 32 j of the tile.  The tile's mask words go into
// LDS first (every wave is past the last stage's LDS reads): vector-memory
// operations complete in order, so mask loads interleaved with the output
// stores would each wait for the stores before them.  The outputs are written
// nontemporally: they are not read again here, and streaming them evicts less
// of the operand panels that other tiles on this XCD still read.
template <int BM, int BN, int THREADS, int MI, int NI>
__device__ __forceinline__ void store_masked(const f32x16 (&acc)[MI][NI], char* smem, int tid, int lrow, int lcol,
                                             int lr, int64_t p0, int64_t q0, int64_t P, int64_t Q,
                                             float* __restrict__ C, int64_t ldc, const uint32_t* __restrict__ mask,
                                             int64_t kw) {
  constexpr int WPR32 = BN / 32;  // mask words per tile row
  uint32_t* mb = reinterpret_cast<uint32_t*>(smem);
  const int64_t w0 = q0 >> 5;
  for (int idx = tid; idx < BM * WPR32; idx += THREADS) {
    const int row = idx / WPR32, wi = idx % WPR32;
    const int64_t p = p0 + row, w = w0 + wi;
    mb[idx] = (p < P && w < kw) ? mask[p * kw + w] : 0u;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = lrow + i * 32 + 8 * (e >> 2) + (e & 3);
      const int64_t p = p0 + row;
      if (p >= P) continue;
      // bit lr of words (row, lcol / 32 + j): columns lcol + 32 j
      const uint32_t* wrow = mb + row * WPR32 + (lcol >> 5);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int64_t q = q0 + lcol + j * 32;
        if (q >= Q) continue;
        __builtin_nontemporal_store((wrow[j] >> lr) & 1u ? acc[i][j][e] : 0.0f, C + p * ldc + q);
      }
    }
}

// bf16 MFMA GEMM, C[p, q] = sum_r A[p, r] B[q, r] over r < Rp (a multiple of 64).
// A: bf16 [P, Rp] with row stride lda >= Rp, or, when B is packed, lda >= the
// number of real columns (padding codes are zero weights, so whatever A holds
// past a row's end only meets zeros); rows 16-byte aligned.  B: bf16 [Q, Rp]
// (BMODE 0) or the 2-bit ternary codes of a [Q, Rp] matrix in the packed
// format (BMODE 1), expanded to bf16 c - 1.
// EPI 0: C * gamma;  EPI 1: C where bit q of row p of the range mask is set
// (mask: rows of kw 32-bit words, bit q % 32 of word q / 32), else 0.
//
// Tile BM x BN, WM x WN waves each owning (BM/WM) x (BN/WN) (64 or 128 rows)
// of 32 x 32 MFMA tiles; 64 r per LDS stage, two stages.  Global loads run two
// stages ahead into two register sets, and the next stage is written to LDS
// halfway through the contraction of the current one, so one barrier per
// stage suffices and the matrix cores keep working while loads are in flight.
// Operand rows of a stage are 128 bytes with 16-byte slot c of row r stored at
// slot c ^ ((r >> 1) & 7): the 16 lanes one LDS cycle serves (16 consecutive
// rows, same slot) hit distinct bank groups of the 64-bank LDS.
template <int BM, int BN, int WM, int WN, int BMODE, int EPI>
__global__ __launch_bounds__(64 * WM * WN, 1) void bf16_gemm_nt_kernel(
    const uint16_t* __restrict__ A, int64_t P, int64_t lda, const void* __restrict__ B, int64_t Q, int64_t Rp,
    float* __restrict__ C, int64_t ldc, const float* __restrict__ gamma, const uint32_t* __restrict__ mask,
    int64_t kw, int bytes_a, int bytes_b, int tiles_p, int tiles_q) {
  constexpr int BK = 64;
  constexpr int ROWB = BK * 2;
  constexpr int THREADS = 64 * WM * WN;
  constexpr int A_BYTES = BM * ROWB;
  constexpr int STAGE = A_BYTES + BN * ROWB;
  constexpr int WROWS = BM / WM;  // rows of a wave's tile
  constexpr int MI = WROWS / 32, NI = BN / WN / 32;
  constexpr int A_LOADS = BM * 8 / THREADS;
  constexpr int B_LOADS = BMODE == 0 ? BN * 8 / THREADS : BN * 4 / THREADS;  // 16-byte slots, or packed words
  static_assert((WROWS == 64 || WROWS == 128) && A_LOADS >= 1 && B_LOADS >= 1 && NI >= 1, "tile shape");
  static_assert(BMODE == 0 || (B_LOADS <= 4 && BN * 4 == B_LOADS * THREADS), "packed B: whole words per thread");
  __shared__ __align__(1024) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // Workgroup -> tile: each XCD (workgroups are dealt round-robin to the 8
  // XCDs) gets a contiguous run of tiles, walked in groups of 8 tile rows so
  // resident tiles share operand panels in the XCD's L2.
  const int num_tiles = tiles_p * tiles_q;
  int t = blockIdx.x;
  if (num_tiles % 8 == 0) t = (t & 7) * (num_tiles >> 3) + (t >> 3);
  constexpr int GROUP = 8;
  const int group = t / (GROUP * tiles_q);
  const int first_p = group * GROUP;
  const int gsize = min(tiles_p - first_p, GROUP);
  const int in_group = t - group * GROUP * tiles_q;
  const int64_t p0 = static_cast<int64_t>(first_p + in_group % gsize) * BM;
  const int64_t q0 = static_cast<int64_t>(in_group / gsize) * BN;

  const int niter = static_cast<int>(Rp / BK);
  const uint32_t rowbytes = static_cast<uint32_t>(Rp) * 2u;
  const uint32_t rowbytes_a = static_cast<uint32_t>(lda) * 2u;

  const __amdgpu_buffer_rsrc_t rsrc_a =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A), 0, bytes_a, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_b =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(B), 0, bytes_b, 0x00020000);
  constexpr uint32_t kOff = 0x80000000u;  // past every resource: reads zeros

  // operand slot s = tid + THREADS i: row s / 8, logical slot s % 8
  uint32_t a_off[A_LOADS], a_dst[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int s = tid + THREADS * i, r = s >> 3, c = s & 7;
    a_off[i] = (p0 + r < P) ? static_cast<uint32_t>(p0 + r) * rowbytes_a + 16u * c : kOff;
    a_dst[i] = r * ROWB + 16 * (c ^ ((r >> 1) & 7));
  }
  uint32_t b_off[B_LOADS], b_dst[B_LOADS];
  if constexpr (BMODE == 0) {
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int s = tid + THREADS * i, r = s >> 3, c = s & 7;
      b_off[i] = (q0 + r < Q) ? static_cast<uint32_t>(q0 + r) * rowbytes + 16u * c : kOff;
      b_dst[i] = A_BYTES + r * ROWB + 16 * (c ^ ((r >> 1) & 7));
    }
  }
  // packed B: word s % 4 of row s / 4's unit (16 codes, two 16-byte slots of
  // bf16) for s = tid + THREADS i, so the expansion is spread over every wave
  const uint32_t units = static_cast<uint32_t>(Rp >> 6);
  const int pb_w = tid & 3;

  v4u ra[2][A_LOADS], rb[2][BMODE == 0 ? B_LOADS : 1];  // packed B: word i in element i
  auto gload = [&](int it, auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      ra[S][i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, a_off[i] == kOff ? kOff : a_off[i] + 128u * it, 0, 0);
    if constexpr (BMODE == 0) {
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i)
        rb[S][i] =
            __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, b_off[i] == kOff ? kOff : b_off[i] + 128u * it, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i) {
        const int r = (tid + THREADS * i) >> 2;
        const uint32_t off = q0 + r < Q ? unit_offset(static_cast<uint32_t>(q0 + r), static_cast<uint32_t>(it),
                                                      static_cast<uint32_t>(Q), units) + 4u * pb_w
                                        : kOff;
        rb[S][0][i] = __builtin_amdgcn_raw_buffer_load_b32(rsrc_b, off, 0, 0);
      }
    }
  };
  auto swrite = [&](char* st, auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) *reinterpret_cast<v4u*>(st + a_dst[i]) = ra[S][i];
    if constexpr (BMODE == 0) {
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i) *reinterpret_cast<v4u*>(st + b_dst[i]) = rb[S][i];
    } else {
      // 16 codes -> 16 bf16 values c - 1 through two byte tables (v_perm):
      // high bytes {0xBF, 0x00, 0x3F} and low bytes {0x80, 0x00, 0x80} for c = 0, 1, 2
      constexpr uint32_t kHi = 0x003F00BFu, kLo = 0x00800080u;
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i) {
        const int r = (tid + THREADS * i) >> 2;
        char* sb = st + A_BYTES + r * ROWB;
        const uint32_t w = rb[S][0][i];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {  // slot c = 2 pb_w + cc: k = 8c .. 8c + 7, fields i = 2 cc, 2 cc + 1
          const int c = 2 * pb_w + cc;
          v4u out;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t x = (w >> (2 * (2 * cc + h))) & 0x03030303u;
            const uint32_t hi = __builtin_amdgcn_perm(0u, kHi, x);
            const uint32_t lo = __builtin_amdgcn_perm(0u, kLo, x);
            out[2 * h] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
            out[2 * h + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
          }
          *reinterpret_cast<v4u*>(sb + 16 * (c ^ ((r >> 1) & 7))) = out;
        }
      }
    }
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int lr = lane & 31, lh = lane >> 5;
  // LDS byte offsets of this lane's operands for k step ks of a stage (slot
  // 2 ks + lh of its row); tile mi / ni adds 32 rows = 4096 bytes
  int a_rd[4], b_rd[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int sw = 16 * ((2 * ks + lh) ^ ((lr >> 1) & 7));
    a_rd[ks] = (wm * WROWS + lr) * ROWB + sw;
    b_rd[ks] = A_BYTES + (wn * (BN / WN) + lr) * ROWB + sw;
  }
  auto contract_half = [&](const char* st, int hs) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ks = 2 * hs + kk;
      bf16x8 a[MI], b[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) a[i] = *reinterpret_cast<const bf16x8*>(st + a_rd[ks] + i * 32 * ROWB);
#pragma unroll
      for (int j = 0; j < NI; ++j) b[j] = *reinterpret_cast<const bf16x8*>(st + b_rd[ks] + j * 32 * ROWB);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // prologue: stage 0 -> LDS 0; stage 1 in register set 1; stage 2 loading into set 0
  gload(0, S0());
  gload(min(1, niter - 1), S1());
  swrite(smem, S0());
  gload(min(2, niter - 1), S0());
  __syncthreads();

  // Iteration it contracts LDS stage it % 2; halfway it writes stage it + 1
  // (register set (it + 1) % 2, loaded two iterations earlier) into the other
  // LDS stage and reloads that register set with stage it + 3 (past the last
  // stage: the last stage again, written to the idle LDS stage, harmless).
  auto iteration = [&](int it, auto set_tag) {
    const char* cur = smem + (it & 1) * STAGE;
    char* nxt = smem + ((it + 1) & 1) * STAGE;
    contract_half(cur, 0);
    swrite(nxt, set_tag);
    gload(min(it + 3, niter - 1), set_tag);
    contract_half(cur, 1);
    __syncthreads();
  };
  int it = 0;
  for (; it + 1 < niter; it += 2) {
    iteration(it, S1());
    iteration(it + 1, S0());
  }
  if (it < niter) iteration(it, S1());

  // epilogue: lane holds rows 8 (e / 4) + 4 lh + e % 4, column lr of each
  // 32 x 32 tile.  The lane's first row and column are opaque to the
  // compiler, so it does not compute the output addresses before the main
  // loop and keep them live (spilled) across it.  The outputs are written
  // nontemporally (see store_masked).
  int lrow = wm * WROWS + 4 * lh;
  int lcol = wn * (BN / WN) + lr;
  asm volatile("" : "+v"(lrow), "+v"(lcol));
  if constexpr (EPI == 0) {
    const float g = gamma[0];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t p = p0 + lrow + i * 32 + 8 * (e >> 2) + (e & 3);
        if (p >= P) continue;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int64_t q = q0 + lcol + j * 32;
          if (q < Q) __builtin_nontemporal_store(__fmul_rn(acc[i][j][e], g), C + p * ldc + q);
        }
      }
  } else {
    store_masked<BM, BN, THREADS, MI, NI>(acc, smem, tid, lrow, lcol, lr, p0, q0, P, Q, C, ldc, mask, kw);
  }
}

template <int BM, int BN, int WM, int WN, int BMODE, int EPI>
void launch_gemm(const uint16_t* A, int64_t P, int64_t lda, const void* B, int64_t Q, int64_t Rp, float* C,
                 int64_t ldc, const float* gamma, const uint32_t* mask, int64_t kw, int bytes_a, int bytes_b,
                 hipStream_t stream) {
  const int tiles_p = static_cast<int>((P + BM - 1) / BM), tiles_q = static_cast<int>((Q + BN - 1) / BN);
  bf16_gemm_nt_kernel<BM, BN, WM, WN, BMODE, EPI><<<static_cast<unsigned>(tiles_p * tiles_q), 64 * WM * WN, 0,
                                                    stream>>>(A, P, lda, B, Q, Rp, C, ldc, gamma, mask, kw, bytes_a,
                                                              bytes_b, tiles_p, tiles_q);
}


// A_hat = bf16(fp32(fp32(gamma_a[m] / 127) * Xq[m, k])) (round half to even),
// r-major [M, ld] with ld a multiple of 8; 16 codes per thread and step.
// Columns K .. ld - 1 hold whatever the codes' padding gives: they meet only
// outputs past K.
__global__ __launch_bounds__(256) void ahat_kernel(const int8_t* __restrict__ Xq, int64_t M, int64_t ldq,
                                                   int64_t ld, const float* __restrict__ gamma_a,
                                                   uint16_t* __restrict__ out) {
  const int64_t cpr = ld / 16 + (ld % 16 ? 1 : 0);  // 16-code chunks per row (the last may be half)
  const int64_t total = M * cpr;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t m = i / cpr, c = i - m * cpr;
    const uint4 w = *reinterpret_cast<const uint4*>(Xq + m * ldq + 16 * c);
    const float sc = __fdiv_rn(gamma_a[m], 127.0f);
    const float bias = -128.0f * sc;
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    uint32_t h[8];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint32_t u = wd[x] ^ 0x80808080u;
      const f32x2 lo = {__fmaf_rn(sc, static_cast<float>(u & 0xffu), bias),
                        __fmaf_rn(sc, static_cast<float>((u >> 8) & 0xffu), bias)};
      const f32x2 hi = {__fmaf_rn(sc, static_cast<float>((u >> 16) & 0xffu), bias),
                        __fmaf_rn(sc, static_cast<float>(u >> 24), bias)};
      h[2 * x] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
      h[2 * x + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
    }
    uint16_t* dst = out + m * ld + 16 * c;
    *reinterpret_cast<uint4*>(dst) = uint4{h[0], h[1], h[2], h[3]};
    if (16 * c + 8 < ld) *reinterpret_cast<uint4*>(dst + 8) = uint4{h[4], h[5], h[6], h[7]};
  }
}

// dW without transposed copies: C[p, q] = sum_r A[r, p] B[r, q] * mask, with
// both operands r-major: A = dY as it lies (bf16 [R, P]) and B = A_hat from
// ahat_kernel (bf16 [R, ldb]), rows 16-byte aligned.  Forming A_hat once
// costs less than forming it in every tile (the 43 row tiles of a 11008-row
// dW would each repeat it).  An LDS stage holds 64 r-rows of both tiles in
// that layout; the matrix cores' operand (8 consecutive r of one column per
// lane) comes from two transposing LDS reads
// (ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte rows that lanes 4 j + i / 4 address, j = 0..3).  For
// 32 x 32 x 16 operands, lane l = 16 g + i addresses r-row 8 (g / 2) + 4 s +
// i / 4 of the k step (read s = 0, 1) and columns 16 (g % 2) + 4 (i % 4) of
// its 32-column block.  One such read touches 8 r-rows x 64 bytes; 16-byte
// chunk c of row r is stored at chunk c ^ 4 (r % 4), so rows r .. r + 3 fall
// on distinct quarters of the LDS banks.  Tiles, waves, the two-stage
// pipeline and the epilogue are those of bf16_gemm_nt_kernel.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void bf16_gemm_tn_kernel(
    const uint16_t* __restrict__ A, int64_t R, int64_t P, const uint16_t* __restrict__ B, int64_t ldb, int64_t Q,
    float* __restrict__ C, int64_t ldc, const uint32_t* __restrict__ mask, int64_t kw, int bytes_a, int bytes_b,
    int tiles_p, int tiles_q) {
  constexpr int BK = 64;
  constexpr int THREADS = 64 * WM * WN;
  constexpr int ROWA = BM * 2, ROWB = BN * 2;  // LDS bytes of one r-row of each tile
  constexpr int A_BYTES = BK * ROWA;
  constexpr int STAGE = A_BYTES + BK * ROWB;
  constexpr int WROWS = BM / WM;
  constexpr int MI = WROWS / 32, NI = BN / WN / 32;
  constexpr int A_CPR = BM / 8, B_CPR = BN / 8;  // 16-byte chunks per row
  constexpr int A_LOADS = BK * A_CPR / THREADS;
  constexpr int B_LOADS = BK * B_CPR / THREADS;
  static_assert((WROWS == 64 || WROWS == 128) && NI >= 1 && A_LOADS >= 1 && B_LOADS >= 1 &&
                    BK * A_CPR == A_LOADS * THREADS && BK * B_CPR == B_LOADS * THREADS,
                "tile shape");
  __shared__ __align__(1024) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const int num_tiles = tiles_p * tiles_q;
  int t = blockIdx.x;
  if (num_tiles % 8 == 0) t = (t & 7) * (num_tiles >> 3) + (t >> 3);
  constexpr int GROUP = 8;
  const int group = t / (GROUP * tiles_q);
  const int first_p = group * GROUP;
  const int gsize = min(tiles_p - first_p, GROUP);
  const int in_group = t - group * GROUP * tiles_q;
  const int64_t p0 = static_cast<int64_t>(first_p + in_group % gsize) * BM;
  const int64_t q0 = static_cast<int64_t>(in_group / gsize) * BN;

  const int niter = static_cast<int>((R + BK - 1) / BK);
  const uint32_t rowbytes_a = static_cast<uint32_t>(P) * 2u;
  const uint32_t rowbytes_b = static_cast<uint32_t>(ldb) * 2u;

  const __amdgpu_buffer_rsrc_t rsrc_a =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A), 0, bytes_a, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_b =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(B), 0, bytes_b, 0x00020000);
  constexpr uint32_t kOff = 0x80000000u;  // past every resource: reads zeros

  // chunk s = tid + THREADS i of a stage: A row s / A_CPR, column chunk
  // s % A_CPR; B likewise.  The
  // rows of thread tid step by THREADS / CPR per i, the chunk stays, and so
  // does row % 4 (THREADS / CPR is a multiple of 4): one global offset and one
  // LDS offset per operand, plus multiples of the row pitch.  Rows past R read
  // zeros through the resources' range (R * row bytes); it goes in voffset,
  // which the range check covers.
  static_assert((THREADS / A_CPR) % 4 == 0 && (THREADS / B_CPR) % 4 == 0, "row step keeps row % 4");
  constexpr int A_RSTEP = THREADS / A_CPR, B_RSTEP = THREADS / B_CPR;
  const int ar = tid / A_CPR, ac = tid % A_CPR, br = tid / B_CPR, bc = tid % B_CPR;
  const bool a_ok = p0 + 8 * ac < P, b_ok = q0 + 8 * bc < ldb;
  const uint32_t a_off = static_cast<uint32_t>(ar) * rowbytes_a + static_cast<uint32_t>(p0 + 8 * ac) * 2u;
  const uint32_t b_off = static_cast<uint32_t>(br) * rowbytes_b + static_cast<uint32_t>(q0 + 8 * bc) * 2u;
  const int a_dst = ar * ROWA + 16 * (ac ^ (4 * (ar & 3)));
  const int b_dst = A_BYTES + br * ROWB + 16 * (bc ^ (4 * (br & 3)));

  v4u ra[2][A_LOADS], rb[2][B_LOADS];
  auto gload = [&](int it, auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
    const uint32_t ra0 = static_cast<uint32_t>(it) * BK * rowbytes_a;
    const uint32_t rb0 = static_cast<uint32_t>(it) * BK * rowbytes_b;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      ra[S][i] = __builtin_amdgcn_raw_buffer_load_b128(
          rsrc_a, a_ok ? a_off + ra0 + static_cast<uint32_t>(i * A_RSTEP) * rowbytes_a : kOff, 0, 0);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i)
      rb[S][i] = __builtin_amdgcn_raw_buffer_load_b128(
          rsrc_b, b_ok ? b_off + rb0 + static_cast<uint32_t>(i * B_RSTEP) * rowbytes_b : kOff, 0, 0);
  };
  auto swrite = [&](char* st, auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) *reinterpret_cast<v4u*>(st + a_dst + i * A_RSTEP * ROWA) = ra[S][i];
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) *reinterpret_cast<v4u*>(st + b_dst + i * B_RSTEP * ROWB) = rb[S][i];
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // this lane's transposing-read offsets (k step 0, read 0) for each block;
  // k step ks and read s add (16 ks + 4 s) rows, which keeps r % 4
  const int g = lane >> 4, li = lane & 15;
  const int rrow = 8 * (g >> 1) + (li >> 2);
  const int cin = 2 * (g & 1) + ((li & 3) >> 1);  // chunk within the 32-column block
  const int swz = 4 * (li >> 2);
  int a_rd[MI], b_rd[NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
    a_rd[i] = rrow * ROWA + 16 * ((((wm * WROWS + 32 * i) >> 3) ^ swz) + cin) + 8 * (li & 1);
#pragma unroll
  for (int j = 0; j < NI; ++j)
    b_rd[j] = A_BYTES + rrow * ROWB + 16 * ((((wn * (BN / WN) + 32 * j) >> 3) ^ swz) + cin) + 8 * (li & 1);

  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  auto tr_operand = [&](const char* base) -> bf16x8 {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + 4 * ROWA));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto tr_operand_b = [&](const char* base) -> bf16x8 {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + 4 * ROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto contract_half = [&](const char* st, int hs) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ks = 2 * hs + kk;
      bf16x8 a[MI], b[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) a[i] = tr_operand(st + a_rd[i] + 16 * ks * ROWA);
#pragma unroll
      for (int j = 0; j < NI; ++j) b[j] = tr_operand_b(st + b_rd[j] + 16 * ks * ROWB);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  gload(0, S0());
  gload(min(1, niter - 1), S1());
  swrite(smem, S0());
  gload(min(2, niter - 1), S0());
  __syncthreads();
  auto iteration = [&](int it, auto set_tag) {
    const char* cur = smem + (it & 1) * STAGE;
    char* nxt = smem + ((it + 1) & 1) * STAGE;
    contract_half(cur, 0);
    swrite(nxt, set_tag);
    gload(min(it + 3, niter - 1), set_tag);
    contract_half(cur, 1);
    __syncthreads();
  };
  int it = 0;
  for (; it + 1 < niter; it += 2) {
    iteration(it, S1());
    iteration(it + 1, S0());
  }
  if (it < niter) iteration(it, S1());

  const int lr = lane & 31, lh = lane >> 5;
  int lrow = wm * WROWS + 4 * lh;
  int lcol = wn * (BN / WN) + lr;
  asm volatile("" : "+v"(lrow), "+v"(lcol));
  store_masked<BM, BN, THREADS, MI, NI>(acc, smem, tid, lrow, lcol, lr, p0, q0, P, Q, C, ldc, mask, kw);
}

}  // namespace

hipError_t launch_pack_transposed(const float* W, int64_t N, int64_t K, const float* gamma, uint32_t* packedT,
                                  uint32_t* mask, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((N + kTile - 1) / kTile), static_cast<unsigned>((K + kTile - 1) / kTile));
  pack_transposed_kernel<<<grid, 256, 0, stream>>>(W, N, K, gamma, packedT, padded_k(N), mask, mask_words(K));
  return hipGetLastError();
}

hipError_t launch_backward(const uint16_t* dY, int64_t M, int64_t N, int64_t K, const uint32_t* packedT,
                           const float* gamma, const int8_t* Xq, const float* gamma_a, const uint32_t* mask,
                           float* dX, float* dW, void* workspace, hipStream_t stream) {
  const int64_t Mp = ((M + 63) / 64) * 64, Np = padded_k(N), Kp = padded_k(K);
  char* ws = static_cast<char*>(workspace);
  uint16_t* dYp = reinterpret_cast<uint16_t*>(ws);
  ws += backward_ws_part(M, Np);
  uint16_t* dYt = reinterpret_cast<uint16_t*>(ws);
  ws += backward_ws_part(N, Mp);
  uint16_t* At = reinterpret_cast<uint16_t*>(ws);
  if (dX) {
    // dY's rows serve as they are when they start on 16-byte boundaries
    const bool direct = N % 8 == 0 && reinterpret_cast<uintptr_t>(dY) % 16 == 0;
    if (!direct) {
      int64_t blocks = (M * Np + 255) / 256;
      if (blocks > 65536) blocks = 65536;
      pad_rows_bf16_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(dY, M, N, dYp, Np);
    }
    // 256 x 128 tiles: a 2048-token, 4096-column dX is 256 tiles, one per CU
    launch_gemm<256, 128, 4, 2, 1, 0>(direct ? dY : dYp, M, direct ? N : Np, packedT, K, Np, dX, K, gamma,
                                      nullptr, 0, static_cast<int>(M * (direct ? N : Np) * 2),
                                      static_cast<int>(K * (Np / 4)), stream);
  }
  if (dW && N % 8 == 0 && reinterpret_cast<uintptr_t>(dY) % 16 == 0 && reinterpret_cast<uintptr_t>(Xq) % 16 == 0) {
    // operands as they are: no transposed copies
    constexpr int BM = 256, BN = 256;
    const int tiles_p = static_cast<int>((N + BM - 1) / BM), tiles_q = static_cast<int>((K + BN - 1) / BN);
    const unsigned grid = static_cast<unsigned>(tiles_p * tiles_q);
    // A_hat once, r-major with rows of K rounded up to 8, in the space of the
    // transposed copies (dYt and At, contiguous: N Mp + K Mp >= M (K + 7) for N >= 8)
    const int64_t ld = (K + 7) / 8 * 8;
    int64_t blocks = (M * ((ld + 15) / 16) + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    ahat_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(Xq, M, Kp, ld, gamma_a, dYt);
    bf16_gemm_tn_kernel<BM, BN, 4, 2><<<grid, 512, 0, stream>>>(dY, M, N, dYt, ld, K, dW, K, mask, mask_words(K),
                                                               static_cast<int>(M * N * 2),
                                                               static_cast<int>(M * ld * 2), tiles_p, tiles_q);
  } else if (dW) {
    const dim3 g0(static_cast<unsigned>((N + kTile - 1) / kTile), static_cast<unsigned>(Mp / kTile));
    transpose_kernel<0><<<g0, 256, 0, stream>>>(dY, M, N, N, nullptr, dYt, Mp);
    const dim3 g1(static_cast<unsigned>((K + kTile - 1) / kTile), static_cast<unsigned>(Mp / kTile));
    transpose_kernel<1><<<g1, 256, 0, stream>>>(Xq, M, K, Kp, gamma_a, At, Mp);
    launch_gemm<256, 256, 4, 2, 0, 1>(dYt, N, Mp, At, K, Mp, dW, K, gamma, mask, mask_words(K),
                                      static_cast<int>(N * Mp * 2), static_cast<int>(K * Mp * 2), stream);
  }
  return hipGetLastError();
}

}  // namespace bitlinear
