// C ABI of the BitLinear library: argument checks, path choice, launches.
// Every check runs on the host before anything is enqueued.
#include <stdint.h>

#include "../../include/bitlinear.h"
#include "kernels.hpp"

using namespace bitlinear;

namespace {

constexpr int64_t kMaxK = int64_t(1) << 20;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_mnk(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return BITLINEAR_ERR_SHAPE;
  if (K > kMaxK) return BITLINEAR_ERR_SHAPE;
  if (N > (int64_t(1) << 31) || M > (int64_t(1) << 31)) return BITLINEAR_ERR_SHAPE;
  if (static_cast<uint64_t>(N) * static_cast<uint64_t>(K) >= (uint64_t(1) << 32)) return BITLINEAR_ERR_SHAPE;
  // the kernels address a packed matrix (N * Kp / 4 bytes; the radix-3 form,
  // N * Kp3 / 5, is never larger) with 32-bit signed byte counts
  if (static_cast<uint64_t>(N) * static_cast<uint64_t>(padded_k(K)) / 4 >= (uint64_t(1) << 31))
    return BITLINEAR_ERR_SHAPE;
  if (static_cast<uint64_t>(M) * static_cast<uint64_t>(N) >= (uint64_t(1) << 40)) return BITLINEAR_ERR_SHAPE;
  if (static_cast<uint64_t>(M) * static_cast<uint64_t>(K) >= (uint64_t(1) << 40)) return BITLINEAR_ERR_SHAPE;
  return BITLINEAR_OK;
}

int check_x(const void* X, int x_dtype) {
  if (x_dtype != BITLINEAR_F32 && x_dtype != BITLINEAR_BF16) return BITLINEAR_ERR_DTYPE;
  if (!aligned(X, x_dtype == BITLINEAR_F32 ? 4 : 2)) return BITLINEAR_ERR_ALIGN;
  return BITLINEAR_OK;
}

// The decode kernel keeps all token codes in LDS and addresses a layer's
// outputs with 32-bit offsets.
bool decode_fits(int64_t M, int64_t K, int64_t N) {
  return M <= kDecodeMaxM && M * (padded_k(K) + 16) <= kDecodeMaxCodes && M * N < (int64_t(1) << 29);
}

bool decode_fits_r3(int64_t M, int64_t K, int64_t N) {
  return M <= kDecodeMaxM && M * (r3_padded_k(K) + 16) <= kDecodeMaxCodes && M * N < (int64_t(1) << 29);
}

struct PrefillWs {
  int8_t* xq;
  float* ga;
  int32_t* rs;
};

PrefillWs prefill_ws(void* ws, int64_t M, int64_t K) {
  char* p = static_cast<char*>(ws);
  PrefillWs w;
  w.xq = reinterpret_cast<int8_t*>(p);
  p += align256(static_cast<size_t>(M) * static_cast<size_t>(padded_k(K)));
  w.ga = reinterpret_cast<float*>(p);
  p += align256(static_cast<size_t>(M) * 4);
  w.rs = reinterpret_cast<int32_t*>(p);
  return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? BITLINEAR_OK : BITLINEAR_ERR_HIP; }

}  // namespace

namespace bitlinear {

int check_forward_args(const void* X, int x_dtype, int64_t M, int64_t K, const uint32_t* packed, int64_t N,
                       const float* gamma, const float* Y, const int32_t* acc, int path, bool* decode) {
  if (!X || !packed || !gamma || !Y) return BITLINEAR_ERR_NULL;
  int st = check_mnk(M, N, K);
  if (st) return st;
  st = check_x(X, x_dtype);
  if (st) return st;
  if (path != BITLINEAR_PATH_AUTO && path != BITLINEAR_PATH_DECODE && path != BITLINEAR_PATH_PREFILL)
    return BITLINEAR_ERR_ARG;
  if (!aligned(packed, 16) || !aligned(gamma, 4) || !aligned(Y, 4) || (acc && !aligned(acc, 4)))
    return BITLINEAR_ERR_ALIGN;
  const bool fits = decode_fits(M, K, N);
  if (path == BITLINEAR_PATH_DECODE && !fits) return BITLINEAR_ERR_SHAPE;
  *decode = path == BITLINEAR_PATH_DECODE || (path == BITLINEAR_PATH_AUTO && fits);
  return BITLINEAR_OK;
}

}  // namespace bitlinear

extern "C" {

int64_t bitlinear_padded_k(int64_t K) { return size_args_ok(K) ? padded_k(K) : 0; }

size_t bitlinear_packed_bytes(int64_t N, int64_t K) {
  if (!size_args_ok(N) || !size_args_ok(K)) return 0;
  return size_mul(static_cast<size_t>(N), static_cast<size_t>(padded_k(K) / 4));
}

size_t bitlinear_quantize_workspace_bytes(void) { return quantize_workspace_bytes(); }

size_t bitlinear_forward_workspace_bytes(int64_t M, int64_t K) { return prefill_ws_bytes(M, K); }

int bitlinear_max_decode_m(void) { return kDecodeMaxM; }

int64_t bitlinear_max_decode_codes(void) { return kDecodeMaxCodes; }

int bitlinear_quantize_weights(const float* W, int64_t N, int64_t K, uint32_t* packed, float* gamma,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!W || !packed || !gamma) return BITLINEAR_ERR_NULL;
  int st = check_mnk(1, N, K);
  if (st) return st;
  if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(gamma, 4)) return BITLINEAR_ERR_ALIGN;
  if (!workspace || workspace_bytes < quantize_workspace_bytes()) return BITLINEAR_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return BITLINEAR_ERR_ALIGN;
  return hip_status(launch_quantize_weights(W, N, K, packed, gamma, workspace,
                                            static_cast<hipStream_t>(stream)));
}

int bitlinear_quantize_activations(const void* X, int x_dtype, int64_t M, int64_t K, int8_t* Xq,
                                   float* gamma_a, int32_t* rowsum, void* stream) {
  if (!X || !Xq || !gamma_a || !rowsum) return BITLINEAR_ERR_NULL;
  int st = check_mnk(M, 1, K);
  if (st) return st;
  st = check_x(X, x_dtype);
  if (st) return st;
  if (!aligned(Xq, 16) || !aligned(gamma_a, 4) || !aligned(rowsum, 4)) return BITLINEAR_ERR_ALIGN;
  return hip_status(launch_act_quant(X, x_dtype, M, K, Xq, gamma_a, rowsum,
                                     static_cast<hipStream_t>(stream)));
}

int bitlinear_forward_ex(const void* X, int x_dtype, int64_t M, int64_t K, const uint32_t* packed,
                         int64_t N, const float* gamma, float* Y, int32_t* acc, int path,
                         void* workspace, size_t workspace_bytes, void* stream) {
  bool decode = false;
  const int st = bitlinear::check_forward_args(X, x_dtype, M, K, packed, N, gamma, Y, acc, path, &decode);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (decode) return hip_status(launch_decode(X, x_dtype, M, K, packed, N, gamma, Y, acc, 1, s));
  if (!workspace || workspace_bytes < prefill_ws_bytes(M, K)) return BITLINEAR_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BITLINEAR_ERR_ALIGN;
  PrefillWs w = prefill_ws(workspace, M, K);
  hipError_t e = launch_act_quant(X, x_dtype, M, K, w.xq, w.ga, w.rs, s);
  if (e != hipSuccess) return BITLINEAR_ERR_HIP;
  return hip_status(launch_prefill_gemm(w.xq, w.ga, w.rs, M, K, packed, N, gamma, Y, acc, s));
}

int bitlinear_forward(const void* X, int x_dtype, int64_t M, int64_t K, const uint32_t* packed,
                      int64_t N, const float* gamma, float* Y, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return bitlinear_forward_ex(X, x_dtype, M, K, packed, N, gamma, Y, nullptr, BITLINEAR_PATH_AUTO,
                              workspace, workspace_bytes, stream);
}

int bitlinear_forward_quantized(const int8_t* Xq, const float* gamma_a, const int32_t* rowsum,
                                int64_t M, int64_t K, const uint32_t* packed, int64_t N,
                                const float* gamma, float* Y, int32_t* acc, void* stream) {
  if (!Xq || !gamma_a || !rowsum || !packed || !gamma || !Y) return BITLINEAR_ERR_NULL;
  int st = check_mnk(M, N, K);
  if (st) return st;
  if (!aligned(Xq, 16) || !aligned(gamma_a, 4) || !aligned(rowsum, 4) || !aligned(packed, 16) ||
      !aligned(gamma, 4) || !aligned(Y, 4) || (acc && !aligned(acc, 4)))
    return BITLINEAR_ERR_ALIGN;
  return hip_status(launch_prefill_gemm(Xq, gamma_a, rowsum, M, K, packed, N, gamma, Y, acc,
                                        static_cast<hipStream_t>(stream)));
}

int bitlinear_forward_batched(int64_t L, const void* X, int x_dtype, int64_t M, int64_t K,
                              const uint32_t* packed, int64_t N, const float* gamma, float* Y,
                              void* stream) {
  if (!X || !packed || !gamma || !Y) return BITLINEAR_ERR_NULL;
  if (L < 1 || L > (int64_t(1) << 20)) return BITLINEAR_ERR_SHAPE;
  int st = check_mnk(M, N, K);
  if (st) return st;
  st = check_x(X, x_dtype);
  if (st) return st;
  if (!decode_fits(M, K, N)) return BITLINEAR_ERR_SHAPE;
  const int64_t bpl = (N + 63) / 64;
  if (L * bpl >= (int64_t(1) << 31)) return BITLINEAR_ERR_SHAPE;
  if (!aligned(packed, 16) || !aligned(gamma, 4) || !aligned(Y, 4)) return BITLINEAR_ERR_ALIGN;
  return hip_status(launch_decode(X, x_dtype, M, K, packed, N, gamma, Y, nullptr, L,
                                  static_cast<hipStream_t>(stream)));
}

size_t bitlinear_ffn_workspace_bytes(int64_t L, int64_t M, int64_t D, int64_t F) {
  if (!size_args_ok(L) || !size_args_ok(M) || !size_args_ok(D) || !size_args_ok(F) ||
      L > (int64_t(1) << 20) || M > (int64_t(1) << 20))
    return 0;
  const size_t hidden = align256(size_mul(size_mul(size_t(L) * size_t(M), size_t(F)), 4));
  // codes of one layer's tokens (prefill path, both projections) or of all
  // layers' hidden rows (decode path)
  const size_t one = prefill_ws_bytes(M, D), all = prefill_ws_bytes(L * M, F);
  if (one == 0 || all == 0) return 0;
  return size_add(hidden, one > all ? one : all);
}

int bitlinear_ffn_forward(int64_t L, const void* X, int x_dtype, int64_t M, int64_t D, int64_t F,
                          int64_t D_out, const uint32_t* packed_up, const float* gamma_up,
                          const uint32_t* packed_down, const float* gamma_down, float* Y,
                          float* hidden, int path, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!X || !packed_up || !gamma_up || !packed_down || !gamma_down || !Y) return BITLINEAR_ERR_NULL;
  if (L < 1 || L > (int64_t(1) << 20)) return BITLINEAR_ERR_SHAPE;
  int st = check_mnk(M, F, D);
  if (st) return st;
  st = check_mnk(M, D_out, F);
  if (st) return st;
  if (static_cast<uint64_t>(L) * static_cast<uint64_t>(M) * static_cast<uint64_t>(F > D_out ? F : D_out) >=
      (uint64_t(1) << 40))
    return BITLINEAR_ERR_SHAPE;
  st = check_x(X, x_dtype);
  if (st) return st;
  if (path != BITLINEAR_PATH_AUTO && path != BITLINEAR_PATH_DECODE && path != BITLINEAR_PATH_PREFILL)
    return BITLINEAR_ERR_ARG;
  if (!aligned(packed_up, 16) || !aligned(packed_down, 16) || !aligned(gamma_up, 4) ||
      !aligned(gamma_down, 4) || !aligned(Y, 4) || (hidden && !aligned(hidden, 16)))
    return BITLINEAR_ERR_ALIGN;
  const bool fits = decode_fits(M, D, F) && decode_fits(M, F, D_out) &&
                    L * ((F > D_out ? F : D_out) + 63) / 64 < (int64_t(1) << 31);
  if (path == BITLINEAR_PATH_DECODE && !fits) return BITLINEAR_ERR_SHAPE;
  const bool decode = path == BITLINEAR_PATH_DECODE || (path == BITLINEAR_PATH_AUTO && fits);
  const size_t hidden_bytes = align256(static_cast<size_t>(L) * static_cast<size_t>(M) * static_cast<size_t>(F) * 4);
  const size_t codes_bytes = decode ? prefill_ws_bytes(L * M, F)
                                    : (prefill_ws_bytes(M, D) > prefill_ws_bytes(M, F) ? prefill_ws_bytes(M, D)
                                                                                       : prefill_ws_bytes(M, F));
  const size_t need = (hidden ? 0 : hidden_bytes) + codes_bytes;
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return BITLINEAR_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return BITLINEAR_ERR_ALIGN;
  }
  char* ws = static_cast<char*>(workspace);
  float* A = hidden ? hidden : reinterpret_cast<float*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t up_words = F * (padded_k(D) / 16), down_words = D_out * (padded_k(F) / 16);
  if (decode) {
    // all layers' hidden activations in one launch, their codes in one
    // quantiser launch (each hidden row once, instead of once in every
    // workgroup of the down projection), then all down projections
    PrefillWs w = prefill_ws(ws + (hidden ? 0 : hidden_bytes), L * M, F);
    hipError_t e = launch_decode(X, x_dtype, M, D, packed_up, F, gamma_up, A, nullptr, L, s, true);
    if (e == hipSuccess) e = launch_act_quant(A, BITLINEAR_F32, L * M, F, w.xq, w.ga, w.rs, s);
    if (e != hipSuccess) return BITLINEAR_ERR_HIP;
    return hip_status(launch_decode_codes(w.xq, w.ga, w.rs, M, F, packed_down, D_out, gamma_down, Y, L, s));
  }
  PrefillWs w = prefill_ws(ws + (hidden ? 0 : hidden_bytes), M, D > F ? D : F);
  const int esize = x_dtype == BITLINEAR_F32 ? 4 : 2;
  for (int64_t l = 0; l < L; ++l) {
    const char* Xl = static_cast<const char*>(X) + l * M * D * esize;
    float* Al = A + l * M * F;
    hipError_t e = launch_act_quant(Xl, x_dtype, M, D, w.xq, w.ga, w.rs, s);
    if (e == hipSuccess)
      e = launch_prefill_gemm(w.xq, w.ga, w.rs, M, D, packed_up + l * up_words, F, gamma_up + l, Al, nullptr, s,
                              true);
    if (e == hipSuccess) e = launch_act_quant(Al, BITLINEAR_F32, M, F, w.xq, w.ga, w.rs, s);
    if (e == hipSuccess)
      e = launch_prefill_gemm(w.xq, w.ga, w.rs, M, F, packed_down + l * down_words, D_out, gamma_down + l,
                              Y + l * M * D_out, nullptr, s);
    if (e != hipSuccess) return BITLINEAR_ERR_HIP;
  }
  return BITLINEAR_OK;
}

size_t bitlinear_ste_mask_bytes(int64_t N, int64_t K) {
  if (!size_args_ok(N) || !size_args_ok(K)) return 0;
  return size_mul(static_cast<size_t>(N), static_cast<size_t>(mask_words(K)) * 4);
}

int bitlinear_pack_transposed(const float* W, int64_t N, int64_t K, const float* gamma, uint32_t* packedT,
                              uint32_t* mask, void* stream) {
  if (!W || !gamma || (!packedT && !mask)) return BITLINEAR_ERR_NULL;
  int st = check_mnk(1, N, K);
  if (st) return st;
  st = check_mnk(1, K, N);
  if (st) return st;
  if (!aligned(W, 4) || !aligned(gamma, 4) || (packedT && !aligned(packedT, 16)) || (mask && !aligned(mask, 4)))
    return BITLINEAR_ERR_ALIGN;
  return hip_status(launch_pack_transposed(W, N, K, gamma, packedT, mask, static_cast<hipStream_t>(stream)));
}

size_t bitlinear_backward_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return backward_workspace_bytes(M, N, K);
}

int bitlinear_backward(const uint16_t* dY, int64_t M, int64_t N, int64_t K, const uint32_t* packedT,
                       const float* gamma, const int8_t* Xq, const float* gamma_a, const uint32_t* mask,
                       float* dX, float* dW, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dY || !gamma || (!dX && !dW)) return BITLINEAR_ERR_NULL;
  if (dX && !packedT) return BITLINEAR_ERR_NULL;
  if (dW && (!Xq || !gamma_a || !mask)) return BITLINEAR_ERR_NULL;
  int st = check_mnk(M, N, K);
  if (st) return st;
  st = check_mnk(M, K, N);
  if (st) return st;
  // bf16 operands are addressed with 32-bit byte offsets
  const int64_t Mp = ((M + 63) / 64) * 64;
  const int64_t lim = int64_t(1) << 31;
  if (M * padded_k(N) * 2 >= lim || N * Mp * 2 >= lim || K * Mp * 2 >= lim) return BITLINEAR_ERR_SHAPE;
  if (!aligned(dY, 2) || !aligned(gamma, 4) || (packedT && !aligned(packedT, 16)) ||
      (gamma_a && !aligned(gamma_a, 4)) || (mask && !aligned(mask, 4)) || (dX && !aligned(dX, 4)) ||
      (dW && !aligned(dW, 4)))
    return BITLINEAR_ERR_ALIGN;
  if (!workspace || workspace_bytes < backward_workspace_bytes(M, N, K)) return BITLINEAR_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BITLINEAR_ERR_ALIGN;
  return hip_status(launch_backward(dY, M, N, K, packedT, gamma, Xq, gamma_a, mask, dX, dW, workspace,
                                    static_cast<hipStream_t>(stream)));
}

int64_t bitlinear_r3_padded_k(int64_t K) { return size_args_ok(K) ? r3_padded_k(K) : 0; }

size_t bitlinear_r3_packed_bytes(int64_t N, int64_t K) {
  if (!size_args_ok(N) || !size_args_ok(K)) return 0;
  return size_mul(static_cast<size_t>(N), static_cast<size_t>(r3_padded_k(K) / 5));
}

int bitlinear_quantize_weights_r3(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!W || !packed || !gamma) return BITLINEAR_ERR_NULL;
  int st = check_mnk(1, N, K);
  if (st) return st;
  if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(gamma, 4)) return BITLINEAR_ERR_ALIGN;
  if (!workspace || workspace_bytes < quantize_workspace_bytes()) return BITLINEAR_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return BITLINEAR_ERR_ALIGN;
  return hip_status(launch_quantize_weights_r3(W, N, K, packed, gamma, workspace,
                                               static_cast<hipStream_t>(stream)));
}

int bitlinear_forward_r3(int64_t L, const void* X, int x_dtype, int64_t M, int64_t K,
                         const uint8_t* packed, int64_t N, const float* gamma, float* Y,
                         int32_t* acc, void* stream) {
  if (!X || !packed || !gamma || !Y) return BITLINEAR_ERR_NULL;
  if (L < 1 || L > (int64_t(1) << 20)) return BITLINEAR_ERR_SHAPE;
  int st = check_mnk(M, N, K);
  if (st) return st;
  st = check_x(X, x_dtype);
  if (st) return st;
  if (!decode_fits_r3(M, K, N)) return BITLINEAR_ERR_SHAPE;
  const int64_t bpl = (N + 63) / 64;
  if (L * bpl >= (int64_t(1) << 31)) return BITLINEAR_ERR_SHAPE;
  if (!aligned(packed, 16) || !aligned(gamma, 4) || !aligned(Y, 4) || (acc && !aligned(acc, 4)))
    return BITLINEAR_ERR_ALIGN;
  return hip_status(launch_decode_r3(X, x_dtype, M, K, packed, N, gamma, Y, acc, L,
                                     static_cast<hipStream_t>(stream)));
}

size_t bitlinear_lut_workspace_bytes(int64_t L, int64_t M, int64_t K) {
  if (L < 1 || M < 1 || K < 1 || L > (int64_t(1) << 20) || M > kDecodeMaxM) return 0;
  return prefill_ws_bytes(L * M, K);
}

int bitlinear_forward_lut(int64_t L, const void* X, int x_dtype, int64_t M, int64_t K,
                          const uint32_t* packed, int64_t N, const float* gamma, float* Y, int32_t* acc,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!X || !packed || !gamma || !Y) return BITLINEAR_ERR_NULL;
  if (L < 1 || L > (int64_t(1) << 20)) return BITLINEAR_ERR_SHAPE;
  if (M < 1 || M > kDecodeMaxM) return BITLINEAR_ERR_SHAPE;
  int st = check_mnk(L * M, N, K);
  if (st) return st;
  if (L * ((N + 255) / 256) >= (int64_t(1) << 31)) return BITLINEAR_ERR_SHAPE;
  st = check_x(X, x_dtype);
  if (st) return st;
  if (!aligned(packed, 16) || !aligned(gamma, 4) || !aligned(Y, 4) || (acc && !aligned(acc, 4)))
    return BITLINEAR_ERR_ALIGN;
  if (!workspace || workspace_bytes < prefill_ws_bytes(L * M, K)) return BITLINEAR_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BITLINEAR_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  PrefillWs w = prefill_ws(workspace, L * M, K);
  hipError_t e = launch_act_quant(X, x_dtype, L * M, K, w.xq, w.ga, w.rs, s);
  if (e != hipSuccess) return BITLINEAR_ERR_HIP;
  return hip_status(launch_lut_gemv(w.xq, w.ga, M, K, packed, N, gamma, Y, acc, L, s));
}

const char* bitlinear_status_string(int status) {
  switch (status) {
    case BITLINEAR_OK: return "ok";
    case BITLINEAR_ERR_NULL: return "a required pointer is NULL";
    case BITLINEAR_ERR_SHAPE: return "M, N, K or L out of the supported range";
    case BITLINEAR_ERR_DTYPE: return "unknown activation dtype";
    case BITLINEAR_ERR_ALIGN: return "a pointer is not aligned as required";
    case BITLINEAR_ERR_WORKSPACE: return "workspace missing or too small";
    case BITLINEAR_ERR_HIP: return "a HIP call or kernel launch failed";
    case BITLINEAR_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

}  // extern "C"
