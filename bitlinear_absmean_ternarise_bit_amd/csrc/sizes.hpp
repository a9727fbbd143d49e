// Buffer sizes shared by the C ABI's checks and the kernels' launchers.  Plain
// host C++ (no HIP), so the argument checks can also be built and tested
// without a GPU toolchain's device pass.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace bitlinear {

constexpr int kAbsmeanBlocks = 1024;  // fixed grid of the gamma reduction
constexpr int kAbsmeanDigits = 10;    // base-2^32 digits of each block's exact partial sum

// Largest M, N, K or L a size query takes (larger arguments give size 0), so
// no size arithmetic below can overflow int64.
constexpr int64_t kSizeArgMax = int64_t(1) << 40;
inline bool size_args_ok(int64_t a) { return a >= 1 && a <= kSizeArgMax; }

inline int64_t padded_k(int64_t K) { return ((K + 63) / 64) * 64; }
// radix-3 rows: a multiple of 80 weights (16 bytes)
inline int64_t r3_padded_k(int64_t K) { return ((K + 79) / 80) * 80; }
// 32-bit words of one row of the STE range mask
inline int64_t mask_words(int64_t K) { return (K + 31) / 32; }

// Size arithmetic saturates to 0 ("no valid size") on overflow, so a size
// query with absurd arguments returns 0 instead of a wrapped value.
inline size_t size_mul(size_t a, size_t b) {
  size_t r;
  return __builtin_mul_overflow(a, b, &r) ? 0 : r;
}
inline size_t size_add(size_t a, size_t b) {
  size_t r;
  return (a == 0 || b == 0 || __builtin_add_overflow(a, b, &r)) ? 0 : r;
}
inline size_t align256(size_t v) { return v > SIZE_MAX - 255 ? 0 : (v + 255) & ~size_t(255); }

// Workspace of the weight quantiser: every block's digit table.
inline size_t quantize_workspace_bytes() { return size_t(kAbsmeanBlocks) * kAbsmeanDigits * 8; }

// Prefill workspace: int8 codes [M, Kp], gamma_A float32 [M], code sums int32
// [M], each part 256-byte aligned (0 for arguments out of range).
inline size_t prefill_ws_bytes(int64_t M, int64_t K) {
  if (!size_args_ok(M) || !size_args_ok(K)) return 0;
  const size_t codes = align256(size_mul(size_t(M), size_t(padded_k(K))));
  const size_t vec = align256(size_mul(size_t(M), 4));
  return size_add(size_add(codes, vec), vec);
}

// Workspace of the STE backward: dY zero-padded to [M, Np] bf16, then dY^T
// and A_hat^T with M padded to a multiple of 64 ([N, Mp] and [K, Mp] bf16).
inline size_t backward_ws_part(int64_t rows, int64_t cols) {
  return align256(size_mul(size_mul(size_t(rows), size_t(cols)), 2));
}
inline size_t backward_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!size_args_ok(M) || !size_args_ok(N) || !size_args_ok(K)) return 0;
  const int64_t Mp = ((M + 63) / 64) * 64, Np = padded_k(N);
  return size_add(size_add(backward_ws_part(M, Np), backward_ws_part(N, Mp)), backward_ws_part(K, Mp));
}

}  // namespace bitlinear
