// Decode path (M <= 16 tokens): one fused kernel per call.
//
//   phase A  each workgroup quantises the (few) tokens into LDS with the
//            per-token AbsMax quantiser (one wave per token, a wave with two
//            tokens loading both rows at once), or copies codes quantised
//            beforehand (the FFN block's down projection, whose input rows
//            are long and shared by all its workgroups);
//   phase B  each wave streams the packed codes of 16 weight rows once from
//            HBM (16 bytes per lane per load; the rows' interleaved order
//            makes one load instruction one contiguous KiB), unpacks them in
//            registers and contracts them against the LDS codes with
//            v_mfma_i32_16x16x64_i8;
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
// packed codes and token l%16 from the same 16 k of the LDS codes, so every k
// is paired consistently.
//
// Two weight formats share the kernel; a row is a run of 16-byte units either
// way:
//   2-bit    a unit is 64 weights (four words of 16); one word unpacks with
//            shifts and masks into one B operand, four MFMAs per unit;
//   radix-3  a unit is 80 weights (four words of 20, five weights per byte,
//            the Radix-3 packing of the article's bitnet.cpp section); byte b
//            of word j holds k = 20j + 4t + b for t = 0..4 as
//            ceil(256 v / 243) with v = sum_t c_t 3^(4-t).  Multiplying the
//            byte by 3 puts digit t = 0 in bits 8-9 and the rest, which yields
//            the next digit the same way, in bits 0-7.  The four bytes of a
//            word sit in the four 16-bit lanes of a register pair, so one
//            64-bit shift-add (x + 2x), one byte permute and two masks give
//            four codes.  The twenty code dwords of a unit, in (word, digit)
//            order, are k = 4f .. 4f+3 of the unit: five B operands for five
//            MFMAs.
#include <type_traits>

#include "kernels.hpp"
#include "quant_act.hpp"

namespace bitlinear {

namespace {

constexpr int kRowsPerWave = 16;   // one MFMA column block of weight rows
constexpr int kDecodeThreads = 256;
constexpr int kWaves = kDecodeThreads / kWave;
constexpr int kNontemporal = 2;    // cache-policy bits of a buffer load: streaming

// Radix-3 unpack of one word (20 weights): d[t] holds the offset codes of
// k = 20j + 4t + b in byte b.  Radix-3 decode is bound by the vector ALU, so
// the times-3 step is one 64-bit shift-add over all four 16-bit lanes
// (v_lshl_add_u64, written out: the compiler splits a 64-bit multiply of
// masked lanes into two 32-bit ones).  A lane stays below 768, so no carry
// crosses into the next lane.
__device__ __forceinline__ void unpack_r3_word(uint32_t w, int* d) {
  uint32_t lo = __builtin_amdgcn_perm(w, w, 0x0c010c00u);   // bytes 0, 1 in 16-bit lanes (selector 12 gives 0)
  uint32_t hi = __builtin_amdgcn_perm(w, w, 0x0c030c02u);   // bytes 2, 3
#pragma unroll
  for (int t = 0; t < 5; ++t) {
    uint64_t v = (static_cast<uint64_t>(hi) << 32) | lo;
    asm volatile("v_lshl_add_u64 %0, %1, 1, %1" : "=v"(v) : "v"(v));  // v = 3 v
    lo = static_cast<uint32_t>(v);
    hi = static_cast<uint32_t>(v >> 32);
    // digits in bits 8-9 of each lane: bytes {lo.1, lo.3, hi.1, hi.3} are
    // the codes of bytes 0, 1, 2, 3 of the word
    d[t] = static_cast<int>(__builtin_amdgcn_perm(hi, lo, 0x07050301u));
    lo &= 0x00ff00ffu;  // the rest, for the next digit
    hi &= 0x00ff00ffu;
  }
}

template <int FMT>
struct Format;
template <>
struct Format<2> {
  static constexpr int kPerUnit = 64;  // weights per 16-byte unit
  static constexpr int kMfma = 4;      // MFMAs per unit
  static constexpr int kUnroll = 8;    // 16-byte loads per lane per batch (8 KiB per wave)
};
template <>
struct Format<3> {
  static constexpr int kPerUnit = 80;
  static constexpr int kMfma = 5;
  // 7 loads per batch: rows of 2048 and 11008 weights (26 and 138 units, 7
  // and 35 load instructions) fill their batches exactly
  static constexpr int kUnroll = 7;
};

// B operands of one 16-byte unit, in k order.  Unit slots past a row's end
// were loaded as zero bytes, which decode to all-zero operands in both formats.
template <int FMT>
__device__ __forceinline__ void unit_operands(const uint4& r, v4i (&bop)[Format<FMT>::kMfma]) {
  const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
  if constexpr (FMT == 2) {
#pragma unroll
    for (int t = 0; t < 4; ++t) bop[t] = unpack_word(wd[t]);
  } else {
    int d[20];
#pragma unroll
    for (int q = 0; q < 4; ++q) unpack_r3_word(wd[q], d + 5 * q);
#pragma unroll
    for (int i = 0; i < 5; ++i) bop[i] = v4i{d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]};
  }
}

// A wave owns `groups` blocks of 16 weight rows and walks them in batches of
// kUnroll 16-byte loads per lane (each load instruction covers four
// consecutive units of 16 rows); the loads of batch b+1 are issued before
// batch b is contracted, and the first batch is in flight while phase A
// quantises X.  Kp is the LDS row length in codes (units * kPerUnit).
// Epilogues: Y only, Y and the INT32 accumulators, or ReLU^2 of Y (the hidden
// activation of a BitNet FFN block).
enum Epilogue { kEpiY = 0, kEpiAcc = 1, kEpiRelu2 = 2 };

// Outputs of a wave (M tokens x 16 * groups rows, 4 bytes each, twice with
// the accumulators) are staged in LDS and stored once at the end when they
// take at most 4 KiB per wave and the workgroup's LDS stays within 64 KiB;
// otherwise each row group stores directly.
__host__ __device__ inline int stage_bytes(int M, int groups, bool with_acc, int64_t code_bytes) {
  const int b = M * groups * kRowsPerWave * 4 * (with_acc ? 2 : 1);
  return (M * groups * kRowsPerWave * 4 <= 4096 && code_bytes + kWaves * b <= 65536) ? b : 0;
}

// DT: 0 = float32 tokens, 1 = bfloat16 tokens, both quantised in phase A;
// 2 = int8 codes [L, M, Kp] quantised beforehand, with gamma_A and the code
// sums in ga_in / rs_in [L, M] (phase A only copies them into LDS).
// SPLIT: for calls with too few weight rows to give every CU a workgroup (a
// single layer, token by token): a workgroup owns one block of 16 weight
// rows and its four waves each walk a quarter of the rows' load chunks; the
// exact INT32 partial sums are added in LDS (in any order: they are
// integers) and one wave rescales and stores them.  SPLIT is then the loads
// per lane per batch, 2 or 4 (a quarter of a 2048-weight row is two chunks,
// and forming the addresses of unused slots costs time on the critical
// path); 0 is the streaming form.
// Radix-3 is held to 128 registers (four waves per SIMD instead of three):
// more waves keep its vector ALU busier.  The 2-bit form is bound by memory
// and keeps the compiler's choice.
template <int FMT, int DT, bool VEC, int EPI, int SPLIT>
__global__ __launch_bounds__(kDecodeThreads) __attribute__((amdgpu_waves_per_eu(FMT == 3 ? 4 : 1))) void decode_kernel(
    const void* __restrict__ X, int M, int64_t K, int64_t Kp, int64_t units,
    const uint32_t* __restrict__ packed, int64_t N, const float* __restrict__ gamma,
    float* __restrict__ Y, int32_t* __restrict__ acc, int blocks_per_layer, int groups, int interleave,
    const float* __restrict__ ga_in, const int32_t* __restrict__ rs_in) {
  extern __shared__ __align__(16) int8_t sxq[];
  __shared__ float s_ga[kDecodeMaxM];
  __shared__ int s_rs[kDecodeMaxM];
  __shared__ float s_sc[kDecodeMaxM];  // (split form) gamma * gamma_A / 127 per token

  constexpr int esize = DT == 0 ? 4 : DT == 1 ? 2 : 1;
  constexpr int kPerUnit = Format<FMT>::kPerUnit;
  constexpr int kMfma = Format<FMT>::kMfma;
  constexpr int kUnroll = SPLIT ? SPLIT : Format<FMT>::kUnroll;
  // Workgroups are dealt round-robin to the 8 XCDs, each with its own L2:
  // give each XCD a contiguous run of (layer, row block) pairs, so that the
  // workgroups of one layer share one L2 (its tokens, or the FFN hidden
  // layer, are fetched from memory once) and each XCD streams one region.
  const uint32_t G = gridDim.x, G8 = G >> 3;
  const uint32_t v = blockIdx.x < 8u * G8 ? (blockIdx.x & 7u) * G8 + (blockIdx.x >> 3) : blockIdx.x;
  const int64_t layer = v / blocks_per_layer;
  const int rb = static_cast<int>(v - layer * blocks_per_layer);
  const int64_t lds_stride = Kp + 16;  // +16 bytes: token rows start on different banks
  // per wave, 0: direct stores (always in the SPLIT form)
  const int stage = SPLIT ? 0 : stage_bytes(M, groups, EPI == kEpiAcc, M * lds_stride);
  X = static_cast<const char*>(X) + layer * M * (DT == 2 ? Kp : K * esize);
  packed += layer * N * units * 4;
  Y += layer * M * N;
  if constexpr (EPI == kEpiAcc) acc += layer * M * N;
  gamma += layer;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar address math
  const int lane = threadIdx.x & (kWave - 1);
  const int j = lane & 15;
  const int g = lane >> 4;
  // Row group gi of this wave starts at row n_base + gi * g_step.  A
  // workgroup owns 4 * groups consecutive blocks of 16 rows; each wave takes
  // a contiguous quarter of them, or (interleave) every fourth block, so that
  // the four waves stream adjacent KiB chunks of one region.
  const int64_t wg_rows = static_cast<int64_t>(kWaves) * groups * kRowsPerWave;
  const int64_t n_base = SPLIT ? static_cast<int64_t>(rb) * kRowsPerWave
                               : static_cast<int64_t>(rb) * wg_rows +
                                     static_cast<int64_t>(wave) * (interleave ? kRowsPerWave : groups * kRowsPerWave);
  const int64_t g_step = interleave ? kWaves * kRowsPerWave : kRowsPerWave;
  const int chunks = static_cast<int>((units + 3) >> 2);  // load instructions per row
  // the wave's load chunks of a row: all of them, or (SPLIT) its quarter
  const int c_lo = SPLIT ? wave * chunks / kWaves : 0;
  const int c_hi = SPLIT ? (wave + 1) * chunks / kWaves : chunks;
  const int bpg = (c_hi - c_lo + kUnroll - 1) / kUnroll;  // batches per row group
  const int nbatch = groups * bpg;

  // Packed rows are read, and outputs written, through buffer resources over
  // this layer's arrays.  Every load and store is unconditional: offsets that
  // must not touch memory (rows past N, units past a row's end, batches past
  // the last, outputs that are not due yet) are set past the resource and the
  // hardware bounds check turns them into zeros / dropped stores.  Without
  // branches the compiler keeps the next batch of loads in flight while the
  // current one is contracted.
  constexpr uint32_t kOff = 0xfffffff0u;  // past every resource
  const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(packed), 0, static_cast<int>(N * units * 16), 0x00020000);
  const __amdgpu_buffer_rsrc_t ysrc = __builtin_amdgcn_make_buffer_rsrc(
      Y, 0, static_cast<int>(static_cast<int64_t>(M) * N * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t asrc = __builtin_amdgcn_make_buffer_rsrc(
      (EPI == kEpiAcc) ? static_cast<void*>(acc) : static_cast<void*>(Y), 0,
      (EPI == kEpiAcc) ? static_cast<int>(static_cast<int64_t>(M) * N * 4) : 0, 0x00020000);
  const uint32_t units32 = static_cast<uint32_t>(units);
  const uint32_t N32 = static_cast<uint32_t>(N);
  // A group's 16 rows are one block of the interleaved row order: load
  // instruction cs reads chunk cs of the block, one contiguous KiB when the
  // block and the chunk are full (unit_offset in closed form).  The loads are
  // nontemporal: every byte is used once.
  auto load_batch = [&](int b, bool valid, uint4 (&r)[kUnroll]) {
    const int gi = b / bpg;
    const int cb = b - gi * bpg;
    const uint32_t n0 = static_cast<uint32_t>(n_base + gi * g_step);
    const uint32_t R = N32 > n0 ? min(16u, N32 - n0) : 0u;  // rows of the block
    const uint32_t blk = n0 * units32 * 16u;
    const bool row_ok = valid && static_cast<uint32_t>(j) < R;
    if constexpr (FMT == 3) {
      // Radix-3 is bound by the vector ALU, so its offsets are formed with
      // fewer operations: chunks before the last hold 4 units, so chunk cs of
      // lane (j, g) is at blk + 64 R cs + 16 (4 j + g), linear in cs; the last
      // chunk holds W = units - 4 last units (lanes j W + g, none for g >= W).
      // The block part is wave-uniform (scalar), the lane part is one of two
      // per-batch values: two vector operations per load.  (For the
      // memory-bound 2-bit decode the general form below streams faster, so
      // it keeps it.)
      const uint32_t cs0 = static_cast<uint32_t>(c_lo + cb * kUnroll);
      const uint32_t last = (units32 - 1u) >> 2;
      const uint32_t Wl = units32 - 4u * last;
      // lane part of the offset: invalid lanes get the resource size, so
      // that any valid block offset added to it stays past the end
      const uint32_t nrec = static_cast<uint32_t>(N * units * 16);
      const bool jr = static_cast<uint32_t>(j) < R;
      const uint32_t l_full = jr ? (4u * j + g) * 16u : nrec;
      const uint32_t l_last = jr && static_cast<uint32_t>(g) < Wl ? (j * Wl + g) * 16u : nrec;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t cs = cs0 + static_cast<uint32_t>(u);
        const bool in = valid && cs <= last && (!SPLIT || cs < static_cast<uint32_t>(c_hi));
        // block part 2^31 when not due: past every resource, and with a lane
        // part below 2^31 the sum does not wrap around
        const uint32_t ub = in ? blk + cs * R * 64u : 0x80000000u;
        const uint32_t off = ub + (cs == last ? l_last : l_full);
        const v4u v = __builtin_amdgcn_raw_buffer_load_b128(wsrc, off, 0, kNontemporal);
        r[u] = make_uint4(v[0], v[1], v[2], v[3]);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t cs = static_cast<uint32_t>(c_lo + cb * kUnroll + u);
      const uint32_t un = cs * 4u + g;
      const uint32_t W = min(4u, units32 - min(units32, 4u * cs));  // units of chunk cs
      const bool ok = row_ok && un < units32 && (!SPLIT || cs < static_cast<uint32_t>(c_hi));
      const uint32_t off = ok ? blk + (cs * R * 4u + j * W + g) * 16u : kOff;
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(wsrc, off, 0, kNontemporal);
      r[u] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };

  uint4 buf0[kUnroll], buf1[kUnroll];
  // Split form with at most two tokens per wave (M <= 8) whose rows fit in
  // registers (at most 4 16-byte chunks per lane): each wave's token rows
  // (token 0's for a wave past M) are requested before the weights, so their
  // quantisation starts as soon as they arrive (a single 1 x 2048 x 2048
  // layer replayed from a graph: 3.50 -> 3.23 us).
  constexpr int kRc = 4;
  uint4 xv[kRc], xv2[kRc];
  const int64_t xnc = K / (DT == 0 ? 4 : 8);
  const bool early = SPLIT && DT != 2 && VEC && M <= 2 * kWaves && xnc <= kRc * kWave;
  // One token (the split form's usual case): every wave has the row in
  // registers, forms its maximum itself and quantises only the codes that its
  // own quarter of K reads, so no wave waits for another before its MFMAs;
  // each subtracts its quarter's code sum from its partial sums (1 x 2048 x
  // 2048 replayed from a graph: 3.08 -> 3.00 us, outputs bitwise unchanged).
  const bool qtr = early && M == 1;
  int q_sum = 0;         // (qtr) code sum of this wave's quarter
  float q_scale = 0.0f;  // (qtr) gamma * gamma_A / 127
  if constexpr (SPLIT && DT != 2 && VEC) {
    if (early) {
      const int m2 = wave + kWaves < M ? wave + kWaves : 0;
      load_row_chunks<DT, kRc>(static_cast<const char*>(X) + (wave < M ? wave : 0) * K * esize, xnc, lane, xv);
      if (M > kWaves) load_row_chunks<DT, kRc>(static_cast<const char*>(X) + m2 * K * esize, xnc, lane, xv2);
    }
  }
  load_batch(0, true, buf0);
  // gamma is needed only by the epilogue; asked for now, its latency hides
  // behind the weights' (a single-layer call has little else to hide it)
  const float gm = gamma[0];
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (DT == 2) {
    // phase A: copy the layer's codes (M rows of Kp bytes, contiguous) into
    // the LDS rows, eight 16-byte loads per thread in flight
    const uint4* src = static_cast<const uint4*>(X);
    const int per_row = static_cast<int>(Kp >> 4);
    const int total = M * per_row;
    for (int i0 = threadIdx.x; i0 < total; i0 += 8 * kDecodeThreads) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[min(i0 + u * kDecodeThreads, total - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kDecodeThreads;
        const int m = i / per_row;
        if (i < total) *reinterpret_cast<uint4*>(sxq + m * lds_stride + 16 * (i - m * per_row)) = v[u];
      }
    }
    if (threadIdx.x < M) {
      const float ga = ga_in[layer * M + threadIdx.x];
      s_ga[threadIdx.x] = ga;
      s_rs[threadIdx.x] = rs_in[layer * M + threadIdx.x];
      if constexpr (SPLIT) s_sc[threadIdx.x] = __fdiv_rn(__fmul_rn(gm, ga), 127.0f);
    }
  } else {
    // phase A: AbsMax INT8 codes of every token into LDS (one wave per token;
    // a wave with two or more tokens takes them two at a time, their loads
    // in flight together)
    auto keep = [&](int m, float ga, int rs) {
      if (lane == 0) {
        s_ga[m] = ga;
        s_rs[m] = rs;
        if constexpr (SPLIT) s_sc[m] = __fdiv_rn(__fmul_rn(gm, ga), 127.0f);
      }
    };
    const char* xb = static_cast<const char*>(X);
    int m = wave;
    if constexpr (SPLIT && DT != 2 && VEC) {
      if (qtr) {
        constexpr int P = ActTraits<DT>::kPerChunk;
        float mx = 0.0f;
#pragma unroll
        for (int u = 0; u < kRc; ++u) {
          float f[P];
          chunk_to_f32<DT>(xv[u], f);
          float mu = 0.0f;
#pragma unroll
          for (int i = 0; i < P; ++i) mu = fmaxf(mu, fabsf(f[i]));
          mx = (lane + u * kWave < xnc) ? fmaxf(mx, mu) : mx;
        }
        mx = quant_wave_max(mx);
        const float sc = __fdiv_rn(127.0f, __fadd_rn(mx, kEps));
        // the codes this wave's load chunks pair with (a chunk is 4 units)
        const int64_t k_lo = static_cast<int64_t>(c_lo) * 4 * kPerUnit;
        const int64_t k_hi = min(static_cast<int64_t>(c_hi) * 4 * kPerUnit, Kp);
        int sum = 0;
#pragma unroll
        for (int u = 0; u < kRc; ++u) {
          const int64_t c = lane + u * kWave;
          if (c < xnc && c * P >= k_lo && c * P < k_hi) sum += quantize_chunk<DT>(xv[u], sc, sxq + c * P);
        }
        for (int64_t k = max(K, k_lo) + lane; k < k_hi; k += kWave) sxq[k] = 0;
        q_sum = quant_wave_sum(sum);
        q_scale = __fdiv_rn(__fmul_rn(gm, mx), 127.0f);
        m = M;
      } else if (early) {
        if (wave < M) {
          float ga;
          int rs;
          quantize_loaded_row<DT, kRc>(xv, xnc, K, Kp, lane, sxq + wave * lds_stride, ga, rs);
          keep(wave, ga, rs);
        }
        if (wave + kWaves < M) {
          float ga;
          int rs;
          quantize_loaded_row<DT, kRc>(xv2, xnc, K, Kp, lane, sxq + (wave + kWaves) * lds_stride, ga, rs);
          keep(wave + kWaves, ga, rs);
        }
        m = M;  // every token done
      }
    }
    for (; m + kWaves < M; m += 2 * kWaves) {
      float ga[2];
      int rs[2];
      quantize_two_rows_wave<DT, VEC>(xb + m * K * esize, xb + (m + kWaves) * K * esize, K, Kp, lane,
                                      sxq + m * lds_stride, sxq + (m + kWaves) * lds_stride, ga, rs);
      keep(m, ga[0], rs[0]);
      keep(m + kWaves, ga[1], rs[1]);
    }
    for (; m < M; m += kWaves) {
      float ga;
      int rs;
      quantize_row_wave<DT, VEC>(xb + m * K * esize, K, Kp, lane, sxq + m * lds_stride, ga, rs);
      keep(m, ga, rs);
    }
  }
  if (qtr) {
    // each wave reads only codes it wrote: one wave's LDS operations complete
    // in order.  (Slots past a row's end may pair with another wave's codes;
    // their weight operands are zero.)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  } else {
    __syncthreads();
  }

  // Lanes of tokens j >= M read token 0's codes: they only feed accumulator
  // rows that are never stored.
  const int8_t* arow = sxq + (j < M ? j : 0) * lds_stride;
  const v4i zero = {0, 0, 0, 0};
  v4i c = zero;
  // the lane's output tokens 4g + r are fixed: their code sums and rescale
  // factors gamma * gamma_A / 127 are formed once, not per row group
  int tok_rs[4];
  float tok_scale[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * g + r;
    const int ic = i < M ? i : M - 1;
    // (the split form forms the scales in phase A, off its critical path;
    // with one token each wave holds them)
    tok_rs[r] = qtr ? 0 : s_rs[ic];
    tok_scale[r] = qtr ? q_scale : SPLIT ? s_sc[ic] : __fdiv_rn(__fmul_rn(gm, s_ga[ic]), 127.0f);
  }

  auto mfma_batch = [&](int b, const uint4 (&r)[kUnroll]) {
    const int cb = b - (b / bpg) * bpg;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      // (split form: slots past the wave's quarter were loaded as zeros and
      // contribute nothing; contracting them keeps the batch one block)
      const int cs = c_lo + cb * kUnroll + u;
      // units past the row end give all-zero operands, so any in-bounds
      // activation codes may pair with them (radix-3: the row's last unit,
      // with one minimum and no multiply)
      uint32_t abase;
      if constexpr (FMT == 3) {
        abase = min(static_cast<uint32_t>(cs) * (4u * kPerUnit) + kPerUnit * g, kPerUnit * (units32 - 1u));
      } else {
        const uint32_t un = static_cast<uint32_t>(cs) * 4u + g;
        abase = un < units32 ? kPerUnit * un : 0u;
      }
      v4i bop[kMfma];
      unit_operands<FMT>(r[u], bop);
#pragma unroll
      for (int t = 0; t < kMfma; ++t) {
        const v4i a = *reinterpret_cast<const v4i*>(arow + abase + 16u * t);
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bop[t], c, 0, 0, 0);
      }
    }
  };

  // Staging area of this wave: out_y[i][x] (token i, row x of the wave's
  // 16 * groups rows), then out_acc likewise.
  const int wave_rows = groups * kRowsPerWave;
  float* out_y = reinterpret_cast<float*>(sxq + M * lds_stride) + wave * (stage / 4);
  int* out_acc = reinterpret_cast<int*>(out_y + M * wave_rows);

  // After the last batch of a row group: rescale (lane holds tokens 4g + r
  // of weight row n), stage or store, and clear the accumulator.  Reading
  // the accumulator waits for the group's chain of MFMAs; the caller issues
  // the next loads first, so two batches stay in flight meanwhile.
  auto epilogue = [&](int b) {
    if constexpr (SPLIT) return;  // once, after the waves' partial sums are added
    const int gi = b / bpg;
    if (b - gi * bpg != bpg - 1) return;
    const int x = gi * kRowsPerWave + j;
    const uint32_t n = static_cast<uint32_t>(n_base + gi * g_step + j);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * g + r;
      const int v = c[r] - tok_rs[r];
      float y = __fmul_rn(static_cast<float>(v), tok_scale[r]);
      if constexpr (EPI == kEpiRelu2) {
        const float rl = fmaxf(y, 0.0f);
        y = __fmul_rn(rl, rl) + 0.0f;  // + 0: no negative zero
      }
      if (stage) {
        if (i < M) {
          out_y[i * wave_rows + x] = y;
          if constexpr (EPI == kEpiAcc) out_acc[i * wave_rows + x] = v;
        }
      } else {
        const uint32_t off = (i < M && n < N32) ? (static_cast<uint32_t>(i) * N32 + n) * 4u : kOff;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), ysrc, off, 0, 0);
        if constexpr (EPI == kEpiAcc) __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(v), asrc, off, 0, 0);
      }
    }
    c = zero;
  };

  // Batch b is in buf(b % 2); batch b + 1 is in flight while b is contracted,
  // and the loads of b + 2 go out (into b's buffer, whose codes are already
  // unpacked) before b's epilogue.  sched_barrier keeps the scheduler from
  // sinking loads into the work that follows them.
  // A single-layer call (SPLIT) often has one batch: skip the second's
  // loads.  The streaming form keeps them unconditional: behind a branch the
  // compiler no longer knows how many loads are in flight in the loop and
  // waits for all of them.
  if (!SPLIT || nbatch > 1) load_batch(1, 1 < nbatch, buf1);
  __builtin_amdgcn_sched_barrier(0);
  int b = 0;
  for (; b + 1 < nbatch; b += 2) {
    mfma_batch(b, buf0);
    load_batch(b + 2, b + 2 < nbatch, buf0);
    __builtin_amdgcn_sched_barrier(0);
    epilogue(b);
    mfma_batch(b + 1, buf1);
    load_batch(b + 3, b + 3 < nbatch, buf1);
    __builtin_amdgcn_sched_barrier(0);
    epilogue(b + 1);
  }
  if (b < nbatch) {
    mfma_batch(b, buf0);
    epilogue(b);
  }
  if constexpr (SPLIT) {
    // add the four waves' partial sums of the block's 16 rows, then rescale
    // and store them from wave 0 (lane holds tokens 4g + r of row j)
    v4i* red = reinterpret_cast<v4i*>(sxq + M * lds_stride);
    if (qtr && g == 0) c[0] -= q_sum;  // lanes 0..15 hold token 0
    red[threadIdx.x] = c;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 1; w < kWaves; ++w) c += red[w * kWave + lane];
      const uint32_t n = static_cast<uint32_t>(n_base + j);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * g + r;
        const int v = c[r] - tok_rs[r];
        float y = __fmul_rn(static_cast<float>(v), tok_scale[r]);
        if constexpr (EPI == kEpiRelu2) {
          const float rl = fmaxf(y, 0.0f);
          y = __fmul_rn(rl, rl) + 0.0f;  // + 0: no negative zero
        }
        const uint32_t off = (i < M && n < N32) ? (static_cast<uint32_t>(i) * N32 + n) * 4u : kOff;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), ysrc, off, 0, 0);
        if constexpr (EPI == kEpiAcc) __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(v), asrc, off, 0, 0);
      }
    }
  }
  if (stage) {
    // the wave's outputs, row-contiguous per token; LDS operations of one
    // wave complete in order, so the staged values are visible here
    for (int i = 0; i < M; ++i) {
      for (int x = lane; x < wave_rows; x += kWave) {
        const uint32_t n = static_cast<uint32_t>(n_base + (x >> 4) * g_step + (x & 15));
        const uint32_t off = n < N32 ? (static_cast<uint32_t>(i) * N32 + n) * 4u : kOff;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out_y[i * wave_rows + x]), ysrc, off, 0, 0);
        if constexpr (EPI == kEpiAcc)
          __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(out_acc[i * wave_rows + x]), asrc, off, 0, 0);
      }
    }
  }
}

// Rows per workgroup = 64 * groups.  Larger blocks quantise X less often and
// stream longer runs (every workgroup quantises all M tokens, which for long
// rows costs as much as a few hundred weight rows); the choice keeps >= 512
// workgroups (2 per CU) when the work allows and wastes at most 1/16 of a
// layer in its last block.
int pick_groups(int64_t L, int64_t N) {
  for (int gsz = 64; gsz > 1; gsz >>= 1) {
    const int64_t rows = int64_t(kWaves) * kRowsPerWave * gsz;
    const int64_t bpl = (N + rows - 1) / rows;
    if (L * bpl >= 512 && (bpl * rows - N) * 16 <= N) return gsz;
  }
  return 1;
}

// Calls whose normal grid would leave most CUs without a workgroup (a
// single layer of a few thousand rows, say) take the SPLIT form instead: one
// 16-row block per workgroup, K split over its waves.
constexpr int64_t kSplitBelow = 256;

template <int FMT, int DT, bool VEC>
hipError_t launch_v(const void* X, int64_t M, int64_t K, const uint32_t* packed, int64_t N,
                    const float* gamma, float* Y, int32_t* acc, int64_t L, bool relu2,
                    hipStream_t stream, const float* ga_in = nullptr, const int32_t* rs_in = nullptr) {
  const int64_t Kp = FMT == 2 ? padded_k(K) : r3_padded_k(K);
  const int64_t units = Kp / Format<FMT>::kPerUnit;
  const int groups = pick_groups(L, N);
  const int64_t rows = int64_t(kWaves) * kRowsPerWave * groups;
  const int64_t blocks16 = (N + kRowsPerWave - 1) / kRowsPerWave;  // 16-row blocks per layer
  int bpl = static_cast<int>((N + rows - 1) / rows);
  const bool split = L * bpl < kSplitBelow && blocks16 > bpl;
  if (split) bpl = static_cast<int>(blocks16);
  const unsigned blocks = static_cast<unsigned>(L * bpl);
  // 2-bit weights, one workgroup per layer: the waves take interleaved row
  // groups (1 x 2048 x 2048 layers in a batch: +1.0-1.5%, measured on four
  // boxes; where several workgroups share a layer the contiguous quarters
  // measured as fast or faster)
  const int ilv = FMT == 2 && !split && bpl == 1 && groups > 1;
  const int m = static_cast<int>(M);
  const bool with_acc = acc != nullptr && !relu2;
  const int64_t code_bytes = M * (Kp + 16);
  // after the codes: the waves' staged outputs, or (SPLIT) their partial sums
  const size_t lds = static_cast<size_t>(code_bytes) +
                     (split ? static_cast<size_t>(kDecodeThreads) * sizeof(v4i)
                            : static_cast<size_t>(kWaves) * stage_bytes(m, groups, with_acc, code_bytes));
  auto go = [&](auto split_tag) {
    constexpr int S = decltype(split_tag)::value;
    if constexpr (DT == 2) {
      decode_kernel<FMT, DT, VEC, kEpiY, S><<<blocks, kDecodeThreads, lds, stream>>>(
          X, m, K, Kp, units, packed, N, gamma, Y, nullptr, bpl, groups, ilv, ga_in, rs_in);
    } else {
      if (FMT == 2 && relu2)
        decode_kernel<FMT, DT, VEC, FMT == 2 ? kEpiRelu2 : kEpiY, S><<<blocks, kDecodeThreads, lds, stream>>>(
            X, m, K, Kp, units, packed, N, gamma, Y, nullptr, bpl, groups, ilv, nullptr, nullptr);
      else if (acc)
        decode_kernel<FMT, DT, VEC, kEpiAcc, S><<<blocks, kDecodeThreads, lds, stream>>>(
            X, m, K, Kp, units, packed, N, gamma, Y, acc, bpl, groups, ilv, nullptr, nullptr);
      else
        decode_kernel<FMT, DT, VEC, kEpiY, S><<<blocks, kDecodeThreads, lds, stream>>>(
            X, m, K, Kp, units, packed, N, gamma, Y, acc, bpl, groups, ilv, nullptr, nullptr);
    }
  };
  // split form: 2 loads per batch when a wave's quarter of a row is at most
  // eight load chunks, else 4 (measured on single layers: K = 2048 and 8192
  // are faster with 2, K = 11008 with 4)
  const int64_t chunks = (units + 3) / 4;
  if (split && (chunks + kWaves - 1) / kWaves <= 8) go(std::integral_constant<int, 2>());
  else if (split) go(std::integral_constant<int, 4>());
  else go(std::integral_constant<int, 0>());
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const void* X, int x_dtype, int64_t M, int64_t K, const uint32_t* packed,
                      int64_t N, const float* gamma, float* Y, int32_t* acc, int64_t L, bool relu2,
                      hipStream_t stream) {
  const int esize = x_dtype == 0 ? 4 : 2;
  const bool vec = (reinterpret_cast<uintptr_t>(X) % 16 == 0) && ((K * esize) % 16 == 0);
  if (x_dtype == 0)
    return vec ? launch_v<FMT, 0, true>(X, M, K, packed, N, gamma, Y, acc, L, relu2, stream)
               : launch_v<FMT, 0, false>(X, M, K, packed, N, gamma, Y, acc, L, relu2, stream);
  return vec ? launch_v<FMT, 1, true>(X, M, K, packed, N, gamma, Y, acc, L, relu2, stream)
             : launch_v<FMT, 1, false>(X, M, K, packed, N, gamma, Y, acc, L, relu2, stream);
}

}  // namespace

hipError_t launch_decode(const void* X, int x_dtype, int64_t M, int64_t K, const uint32_t* packed,
                         int64_t N, const float* gamma, float* Y, int32_t* acc, int64_t L,
                         hipStream_t stream, bool relu2) {
  return launch_fmt<2>(X, x_dtype, M, K, packed, N, gamma, Y, acc, L, relu2, stream);
}

hipError_t launch_decode_codes(const int8_t* Xq, const float* gamma_a, const int32_t* rowsum, int64_t M,
                              int64_t K, const uint32_t* packed, int64_t N, const float* gamma, float* Y,
                              int64_t L, hipStream_t stream) {
  return launch_v<2, 2, true>(Xq, M, K, packed, N, gamma, Y, nullptr, L, false, stream, gamma_a, rowsum);
}

hipError_t launch_decode_r3(const void* X, int x_dtype, int64_t M, int64_t K, const uint8_t* packed,
                            int64_t N, const float* gamma, float* Y, int32_t* acc, int64_t L,
                            hipStream_t stream) {
  return launch_fmt<3>(X, x_dtype, M, K, reinterpret_cast<const uint32_t*>(packed), N, gamma, Y,
                       acc, L, false, stream);
}

}  // namespace bitlinear
