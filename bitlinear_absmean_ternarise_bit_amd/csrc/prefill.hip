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
// Tiling: a workgroup of WM x WN waves owns a BM (tokens) x BN (weight rows)
// output tile; each wave owns a (BM/WM) x (BN/WN) sub-tile made of 32 x 32
// MFMA tiles (256 x 256 with 4 x 2 waves for large problems).  K advances 128 per stage through two LDS stages.
// Workgroups are persistent, one per CU: each walks every gridDim.x-th tile,
// and requests the next tile's first stage before it writes the finished
// tile's outputs.  The per-row dequantisation terms (gamma * gamma_A / 127 and
// the token code sum) of a tile are formed once, by one thread per row, into
// LDS, so the epilogue issues no global loads (a load there would wait for the
// stores before it: vector-memory completions are counted in order).
// Global loads run two stages ahead into two register sets (buffer loads with
// 32-bit offsets; rows past M or N read as zeros from the hardware bounds
// check), and the stage after the one being contracted is written to LDS
// halfway through the contraction, so one barrier per stage suffices and the
// matrix cores keep working while loads and LDS writes are in flight.
//
// LDS layout per stage: activation codes [BM][128 B], dense, with 16-byte
// slot c of row r stored at slot c ^ ((r >> 1) & 7), so the 16 lanes that one
// LDS cycle serves (16 consecutive rows, same logical slot) hit 16 distinct
// bank groups; packed words as [hs][h][BN] 8-byte pairs (words 4hs + 2h and
// 4hs + 2h + 1 of every row contiguous), so the 32 lanes of a 64-bit read
// cover 256 contiguous bytes.
//
// MFMA operands: for 32x32x32 int8, lane l supplies 16 bytes of A row l % 32
// and of B column l % 32 for the same 16 k positions (chosen by h = l / 32).
// In K step s (0..3) of a stage, lane half h uses packed word
// w(s, h) = 4 (s / 2) + 2 h + s % 2 of its weight row (16 weights) and the
// 16 activation codes at k = 16 w(s, h) of its token row: the same k on both
// sides.  Steps 0 and 1 use words 0..3 only, so a final half stage (Kp not a
// multiple of 128) just skips steps 2 and 3.
#include <algorithm>
#include <type_traits>

#include "kernels.hpp"

namespace bitlinear {

namespace {

constexpr int BK = 128;

// Buffer resource word 3 for raw (unformatted, stride 0) accesses on gfx9.
constexpr int kBufferFlags = 0x00020000;

// s_waitcnt immediate (gfx9 encoding): wait until at most n LDS operations
// are outstanding (vector-memory and export counters left free).
constexpr int lgkmcnt_imm(int n) { return 15 | (3 << 14) | (7 << 4) | ((n & 15) << 8); }

// EPI: 0 = Y, 1 = Y and the INT32 accumulators, 2 = ReLU^2 of Y (the hidden
// activation of a BitNet FFN block)
template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(64 * WM * WN, 1) void prefill_gemm_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ gamma_a,
    const int32_t* __restrict__ rowsum, int64_t M, int64_t Kp, const uint32_t* __restrict__ packed,
    int64_t N, int64_t ldy, const float* __restrict__ gamma, float* __restrict__ Y,
    int32_t* __restrict__ acc,
    int tiles_m, int tiles_n, int bytes_a, int bytes_b) {
  constexpr int A_BYTES = BM * 128;
  constexpr int B_BYTES = BN * 32;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int THREADS = 64 * WM * WN;
  constexpr int MI = BM / WM / 32;      // 32-row MFMA tiles per wave
  constexpr int NI = BN / WN / 32;      // 32-column MFMA tiles per wave
  constexpr int A_LOADS = BM * 8 / THREADS;  // 16-byte loads per thread per stage (activations)
  constexpr int B_SLOTS = BN * 2;            // 16-byte packed slots per stage
  constexpr int B_LOADS = B_SLOTS >= THREADS ? B_SLOTS / THREADS : 1;
  constexpr bool B_ALL = B_SLOTS >= THREADS;  // else only threads < B_SLOTS load packed words
  static_assert(A_LOADS >= 1 && MI >= 1 && NI >= 1, "tile too small for the workgroup");
  __shared__ __align__(1024) char smem[2 * STAGE];
  // dequantisation terms of the current tile's rows: gamma * gamma_A / 127 and
  // the token code sum
  __shared__ float row_scale[BM];
  __shared__ int row_sum[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // Tile index -> tile.  Workgroups are dealt round-robin to the 8 XCDs and
  // each walks the tiles t = blockIdx.x + gridDim.x i (gridDim.x is a multiple
  // of 8 or covers every tile), so a workgroup stays on one XCD; give each XCD
  // a contiguous run of tiles, walked in groups of 8 tile rows so the tiles
  // resident on one XCD share activation and weight panels in its L2.
  const int num_tiles = tiles_m * tiles_n;
  constexpr int GROUP = 8;
  int64_t m0 = 0, n0 = 0;
  auto place = [&](int t) {
    if (num_tiles % 8 == 0) t = (t & 7) * (num_tiles >> 3) + (t >> 3);
    const int group = t / (GROUP * tiles_n);
    const int first_m = group * GROUP;
    const int gsize = min(tiles_m - first_m, GROUP);
    const int in_group = t - group * GROUP * tiles_n;
    m0 = static_cast<int64_t>(first_m + in_group % gsize) * BM;
    n0 = static_cast<int64_t>(in_group / gsize) * BN;
  };

  // Global sources: buffer resources over the whole code arrays, 32-bit lane
  // offsets; rows past M or N fall outside the resource and read as zeros
  // (their outputs are discarded).  In a final half stage the slots past Kp
  // re-read the 64 weights before them; they only reach the skipped steps.
  const __amdgpu_buffer_rsrc_t rsrc_a =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(Xq), 0, bytes_a, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsrc_b =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(packed), 0, bytes_b, kBufferFlags);
  const uint32_t kp32 = static_cast<uint32_t>(Kp);
  // thread -> 16-byte slots: activation slot tid + THREADS q is row
  // (tid >> 3) + (THREADS / 8) q, logical column tid & 7; packed slot
  // tid + THREADS q is row (tid >> 1) + (THREADS / 2) q, half tid & 1
  const int a_r = tid >> 3, a_c = tid & 7;
  const int b_r = tid >> 1, b_c = tid & 1;
  const uint32_t a_row_step = (THREADS / 8) * kp32;          // rows of activation codes per q
  static_assert(B_LOADS == 1, "one packed slot per thread per stage");
  static_assert(BM <= THREADS, "one thread per tile row loads its dequantisation terms");
  const uint32_t units = kp32 >> 6;
  const uint32_t N32 = static_cast<uint32_t>(N);
  // per-tile source offsets: the activation slot, and packed row b_n in the
  // interleaved row order (see unit_offset): block base, row within the
  // block, rows of the block
  uint32_t voff_a = 0, b_blk = 0, b_j = 0, b_R = 0;
  bool b_ok = false;
  int row_rs = 0;
  float row_ga = 0.0f;
  auto set_tile = [&](int t) {
    place(t);
    voff_a = static_cast<uint32_t>(m0 + a_r) * kp32 + 16u * a_c;
    const uint32_t b_n = static_cast<uint32_t>(n0 + b_r);
    b_ok = b_n < N32;
    // rows past N: an offset past the resource (2^31 + at most 48), read as zeros
    b_blk = b_ok ? (b_n & ~15u) * units * 16u : 0x80000000u;
    b_j = b_ok ? b_n & 15u : 0u;
    b_R = b_ok ? min(16u, N32 - (b_n & ~15u)) : 0u;
    const int64_t m = m0 + tid;
    if (tid < BM && m < M) {
      row_rs = rowsum[m];
      row_ga = gamma_a[m];
    }
  };
  // LDS destinations (swizzled)
  int a_dst[A_LOADS], b_dst[B_LOADS];  // b_dst: LDS offset of the slot's first 8-byte half
#pragma unroll
  for (int q = 0; q < A_LOADS; ++q) {
    const int r = a_r + (THREADS / 8) * q;
    a_dst[q] = r * 128 + 16 * (a_c ^ ((r >> 1) & 7));
  }
#pragma unroll
  for (int q = 0; q < B_LOADS; ++q) {
    const int r = b_r + (THREADS / 2) * q;
    b_dst[q] = A_BYTES + ((2 * b_c) * BN + r) * 8;  // words 4c, 4c+1; words 4c+2, 4c+3 at +BN*8
  }

  v4u ra[2][A_LOADS], rb[2][B_LOADS];
  auto gload = [&](int it, auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
    const uint32_t k0 = static_cast<uint32_t>(it) * BK;
    const uint32_t a_adj = (k0 + 16u * a_c >= kp32) ? 64u : 0u;
    // unit 2 it + b_c of the row; past Kp (final half stage) the unit before it
    uint32_t u = 2u * static_cast<uint32_t>(it) + static_cast<uint32_t>(b_c);
    u = u >= units ? u - 1u : u;
    const uint32_t cu = u >> 2;
    const uint32_t W = min(4u, units - 4u * cu);
    const uint32_t voff_b = b_blk + (cu * b_R * 4u + b_j * W + (u & 3u)) * 16u;
    // The whole offset, row step included, goes in the lane offset: the
    // hardware range check covers the lane offset (plus the instruction's
    // immediate) but not the scalar offset, so only this way does a row past
    // M land past the resource and read as zeros.
    const uint32_t a_base = voff_a + k0 - a_adj;
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q)
      ra[S][q] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, a_base + q * a_row_step, 0, 0);
    if (B_ALL || tid < B_SLOTS)
      rb[S][0] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, voff_b, 0, 0);
  };
  auto swrite = [&](char* st, auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q) *reinterpret_cast<v4u*>(st + a_dst[q]) = ra[S][q];
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q)
      if (B_ALL || tid < B_SLOTS) {
        *reinterpret_cast<uint2*>(st + b_dst[q]) = make_uint2(rb[S][q][0], rb[S][q][1]);
        *reinterpret_cast<uint2*>(st + b_dst[q] + BN * 8) = make_uint2(rb[S][q][2], rb[S][q][3]);
      }
  };

  v16i c[MI][NI];

  const int lr = lane & 31;
  const int lh = lane >> 5;
  // LDS byte offsets of this lane's operands within a stage.  The swizzle
  // terms depend on lr only (tile row bases are multiples of 8), so tile mi /
  // ni adds a constant that the ds_read instruction carries as its offset.
  int a_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int cl = 4 * (s >> 1) + 2 * lh + (s & 1);
    a_off[s] = (wm * (BM / WM) + lr) * 128 + 16 * (cl ^ ((lr >> 1) & 7));
  }
  int b_off[2];
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) b_off[hs] = A_BYTES + ((2 * hs + lh) * BN + wn * (BN / WN) + lr) * 8;

  // Contract half hs (steps 2hs, 2hs+1: 64 k) of an LDS stage.  The packed
  // words of both steps are read first, and the activation operands of the
  // second step are requested before the first step's MFMAs are issued, so
  // LDS latency overlaps matrix-core work.
  auto contract_half = [&](const char* st, int hs) {
    uint2 bw[NI];
    v4i a0[MI], a1[MI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) bw[ni] = *reinterpret_cast<const uint2*>(st + b_off[hs] + ni * 256);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) a0[mi] = *reinterpret_cast<const v4i*>(st + a_off[2 * hs] + mi * 4096);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) a1[mi] = *reinterpret_cast<const v4i*>(st + a_off[2 * hs + 1] + mi * 4096);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const v4i b = unpack_word(bw[ni].x);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        c[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0[mi], b, c[mi][ni], 0, 0, 0);
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const v4i b = unpack_word(bw[ni].y);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        c[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1[mi], b, c[mi][ni], 0, 0, 0);
    }
  };

  const int nfull = static_cast<int>(Kp / BK);
  const int niter = static_cast<int>((Kp + BK - 1) / BK);
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  const float gm = gamma[0];
  int t = blockIdx.x;
  set_tile(t);
  gload(0, S0());
  gload(min(1, niter - 1), S1());
  for (;;) {
    // Prologue: stage 0 -> LDS 0; stage 1 in register set 1; stage 2 loading
    // into set 0.  Stages 0 and 1 were requested before the previous tile's
    // epilogue, and every wave is past that epilogue's LDS reads.
    swrite(smem, S0());
    if (tid < BM) {
      row_scale[tid] = __fdiv_rn(__fmul_rn(gm, row_ga), 127.0f);
      row_sum[tid] = row_rs;
    }
    gload(min(2, niter - 1), S0());
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[mi][ni][r] = 0;
    __builtin_amdgcn_s_waitcnt(lgkmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // Iteration it contracts LDS stage it % 2; halfway it writes stage it + 1
    // (register set (it + 1) % 2, loaded two iterations earlier) into the
    // other LDS stage and reloads that register set with stage it + 3.  Past
    // the last stage the write lands in the idle LDS stage and the reload
    // repeats the last stage: harmless, and the loop stays free of branches,
    // which keeps the compiler's count of outstanding loads exact (it then
    // waits only for the older register set).
    auto iteration = [&](int it, auto set_tag) {
      const char* cur = smem + (it & 1) * STAGE;
      char* nxt = smem + ((it + 1) & 1) * STAGE;
      contract_half(cur, 0);
      swrite(nxt, set_tag);
      gload(min(it + 3, niter - 1), set_tag);
      contract_half(cur, 1);
      __builtin_amdgcn_s_waitcnt(lgkmcnt_imm(0));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");  // LDS traffic stays on its side of the barrier
    };
    int it = 0;
    for (; it + 1 < nfull; it += 2) {
      iteration(it, S1());
      iteration(it + 1, S0());
    }
    if (it < nfull) iteration(it, S1());
    if (nfull < niter) contract_half(smem + (nfull & 1) * STAGE, 0);  // final half stage

    // Request the next tile's first stage and row terms, so they arrive while
    // this tile's outputs are written.
    const int64_t em0 = m0, en0 = n0;
    const int tn = t + static_cast<int>(gridDim.x);
    const bool more = tn < num_tiles;
    if (more) {
      set_tile(tn);
      gload(0, S0());
    }

    // epilogue: lane holds rows 8*(r/4) + 4*(l/32) + r%4, column l%32 of each
    // 32x32 tile.  The lane's first row and column are made opaque to the
    // compiler: otherwise it hoists the per-row index arithmetic out of the
    // tile loop, where the results stay live across the main loop and spill.
    int lrow = wm * (BM / WM) + 4 * lh;
    int lcol = wn * (BN / WN) + lr;
    asm volatile("" : "+v"(lrow), "+v"(lcol));
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = lrow + mi * 32 + 8 * (r >> 2) + (r & 3);
        const int64_t m = em0 + row;
        if (m >= M) continue;
        const int rs = row_sum[row];
        const float scale = row_scale[row];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int64_t n = en0 + lcol + ni * 32;
          if (n < N) {
            const int v = c[mi][ni][r] - rs;
            if constexpr (EPI == 1) acc[m * ldy + n] = v;
            float y = __fmul_rn(static_cast<float>(v), scale);
            if constexpr (EPI == 2) {
              const float r = fmaxf(y, 0.0f);
              y = __fmul_rn(r, r) + 0.0f;  // + 0: no negative zero
            }
            // Y streams past the caches (nontemporal), so it evicts less of
            // the operand panels the other tiles on this XCD still read; the
            // FFN hidden layer (EPI 2) is read again right away and is not
            if constexpr (EPI == 2) Y[m * ldy + n] = y;
            else __builtin_nontemporal_store(y, Y + m * ldy + n);
          }
        }
      }
    }
    if (!more) break;
    t = tn;
    gload(min(1, niter - 1), S1());
    __builtin_amdgcn_s_barrier();  // every wave is done with this tile's LDS
    asm volatile("" ::: "memory");
  }
}

constexpr int64_t kCUs = 256;  // compute units of an MI355X: one workgroup each

// Rows [0, N) of the packed matrix against the tokens; Y and acc have row
// stride ldy (N when the launch covers all output columns).
template <int BM, int BN, int WM, int WN>
hipError_t launch_tile(const int8_t* Xq, const float* gamma_a, const int32_t* rowsum, int64_t M,
                       int64_t Kp, const uint32_t* packed, int64_t N, int64_t ldy, const float* gamma,
                       float* Y, int32_t* acc, bool relu2, hipStream_t stream) {
  // Buffer offsets are 32-bit: run the tokens in chunks of < 2^31 code bytes.
  const int64_t chunk = ((int64_t(1) << 31) - 1) / Kp / BM * BM;
  const int bytes_b = static_cast<int>(N * (Kp / 4));
  for (int64_t r0 = 0; r0 < M; r0 += chunk) {
    const int64_t Mc = min(M - r0, chunk);
    const int tiles_m = static_cast<int>((Mc + BM - 1) / BM);
    const int tiles_n = static_cast<int>((N + BN - 1) / BN);
    // persistent workgroups, one per CU, each walking every gridDim.x-th tile
    const unsigned blocks = static_cast<unsigned>(std::min<int64_t>(int64_t(tiles_m) * tiles_n, kCUs));
    const int bytes_a = static_cast<int>(Mc * Kp);
    if (relu2)
      prefill_gemm_kernel<BM, BN, WM, WN, 2><<<blocks, 64 * WM * WN, 0, stream>>>(
          Xq + r0 * Kp, gamma_a + r0, rowsum + r0, Mc, Kp, packed, N, ldy, gamma, Y + r0 * ldy,
          nullptr, tiles_m, tiles_n, bytes_a, bytes_b);
    else if (acc)
      prefill_gemm_kernel<BM, BN, WM, WN, 1><<<blocks, 64 * WM * WN, 0, stream>>>(
          Xq + r0 * Kp, gamma_a + r0, rowsum + r0, Mc, Kp, packed, N, ldy, gamma, Y + r0 * ldy,
          acc + r0 * ldy, tiles_m, tiles_n, bytes_a, bytes_b);
    else
      prefill_gemm_kernel<BM, BN, WM, WN, 0><<<blocks, 64 * WM * WN, 0, stream>>>(
          Xq + r0 * Kp, gamma_a + r0, rowsum + r0, Mc, Kp, packed, N, ldy, gamma, Y + r0 * ldy,
          nullptr, tiles_m, tiles_n, bytes_a, bytes_b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_prefill_gemm(const int8_t* Xq, const float* gamma_a, const int32_t* rowsum,
                               int64_t M, int64_t K, const uint32_t* packed, int64_t N,
                               const float* gamma, float* Y, int32_t* acc, hipStream_t stream,
                               bool relu2) {
  const int64_t Kp = padded_k(K);
  if (relu2) acc = nullptr;
  // One workgroup per CU.  The 256 x 256 tile (8 waves of 64 x 128) has the
  // best ratio of matrix-core work to LDS traffic; smaller tiles are used only
  // when the big one would leave more than a quarter of the CUs idle.
  auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  const int64_t big = tiles(256, 256);
  const int64_t rounds = big / kCUs;
  const int64_t rest = big - rounds * kCUs;
  // A few rounds of big tiles with a short last round: the first output
  // columns take whole rounds of big tiles and the rest one round of
  // 128 x 256 tiles (two launches; the packed rows of the second start at a
  // multiple of 16, so they are a contiguous part of the buffer).
  if (rounds >= 1 && rounds < 4 && rest > 0 && rest * 4 < 3 * kCUs) {
    const int64_t tm_big = (M + 255) / 256, tm_half = (M + 127) / 128;
    int64_t nA = (rounds * kCUs / tm_big) * 256;
    while (nA > 0 && tm_half * ((N - nA + 255) / 256) > kCUs) nA -= 256;
    if (nA > 0 && nA < N) {
      hipError_t e = launch_tile<256, 256, 4, 2>(Xq, gamma_a, rowsum, M, Kp, packed, nA, N, gamma, Y,
                                                 acc, relu2, stream);
      if (e != hipSuccess) return e;
      return launch_tile<128, 256, 2, 4>(Xq, gamma_a, rowsum, M, Kp, packed + nA * (Kp / 16), N - nA, N,
                                         gamma, Y + nA, acc ? acc + nA : nullptr, relu2, stream);
    }
  }
  if (big >= 192)
    return launch_tile<256, 256, 4, 2>(Xq, gamma_a, rowsum, M, Kp, packed, N, N, gamma, Y, acc, relu2, stream);
  if (tiles(128, 256) >= 192)
    return launch_tile<128, 256, 2, 4>(Xq, gamma_a, rowsum, M, Kp, packed, N, N, gamma, Y, acc, relu2, stream);
  return launch_tile<128, 128, 2, 2>(Xq, gamma_a, rowsum, M, Kp, packed, N, N, gamma, Y, acc, relu2, stream);
}

}  // namespace bitlinear
