// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "sizes.hpp"

namespace bitlinear {

constexpr int kDecodeMaxM = 16;            // one MFMA row block of tokens
constexpr int64_t kDecodeMaxCodes = 65536; // M * Kp int8 codes held in LDS

// The forward's argument checks (null pointers, sizes, dtype, path,
// alignment): a BITLINEAR_* status, and in *decode whether the decode path
// runs.  Shared by the forward entry points (api.hip, noalloc.hip).
int check_forward_args(const void* X, int x_dtype, int64_t M, int64_t K, const uint32_t* packed, int64_t N,
                       const float* gamma, const float* Y, const int32_t* acc, int path, bool* decode);

// a1 + a2
hipError_t launch_quantize_weights(const float* W, int64_t N, int64_t K, uint32_t* packed,
                                   float* gamma, void* workspace, hipStream_t stream);
// a1 + radix-3 pack (same workspace)
hipError_t launch_quantize_weights_r3(const float* W, int64_t N, int64_t K, uint8_t* packed,
                                      float* gamma, void* workspace, hipStream_t stream);

// a3
hipError_t launch_act_quant(const void* X, int x_dtype, int64_t M, int64_t K, int8_t* Xq,
                            float* gamma_a, int32_t* rowsum, hipStream_t stream);

// a3 + a4 + a6 fused (decode, M <= kDecodeMaxM), L layers of one shape;
// relu2: Y receives ReLU^2 of the output (a BitNet FFN block's hidden layer)
hipError_t launch_decode(const void* X, int x_dtype, int64_t M, int64_t K, const uint32_t* packed,
                         int64_t N, const float* gamma, float* Y, int32_t* acc, int64_t L,
                         hipStream_t stream, bool relu2 = false);

// a4 + a6 (decode kernel) on codes from launch_act_quant: L layers of M
// tokens, rows l * M .. l * M + M - 1 of Xq / gamma_a / rowsum
hipError_t launch_decode_codes(const int8_t* Xq, const float* gamma_a, const int32_t* rowsum, int64_t M,
                               int64_t K, const uint32_t* packed, int64_t N, const float* gamma, float* Y,
                               int64_t L, hipStream_t stream);

// a3 + a4 + a6 fused, radix-3 weights
hipError_t launch_decode_r3(const void* X, int x_dtype, int64_t M, int64_t K, const uint8_t* packed,
                            int64_t N, const float* gamma, float* Y, int32_t* acc, int64_t L,
                            hipStream_t stream);

// a5 + a6 (prefill): codes from launch_act_quant
hipError_t launch_prefill_gemm(const int8_t* Xq, const float* gamma_a, const int32_t* rowsum,
                               int64_t M, int64_t K, const uint32_t* packed, int64_t N,
                               const float* gamma, float* Y, int32_t* acc, hipStream_t stream,
                               bool relu2 = false);

// LUT contraction (comparison variant): codes from launch_act_quant for L
// layers of M <= kDecodeMaxM tokens (rows l * M .. l * M + M - 1), 2-bit weights
hipError_t launch_lut_gemv(const int8_t* Xq, const float* gamma_a, int64_t M, int64_t K, const uint32_t* packed,
                           int64_t N, const float* gamma, float* Y, int32_t* acc, int64_t L, hipStream_t stream);

// STE backward: codes of W^T (2-bit format, rows k) and the range mask of W
// (bits, mask_words(K) 32-bit words per row), then the two bf16 GEMMs
hipError_t launch_pack_transposed(const float* W, int64_t N, int64_t K, const float* gamma, uint32_t* packedT,
                                  uint32_t* mask, hipStream_t stream);
hipError_t launch_backward(const uint16_t* dY, int64_t M, int64_t N, int64_t K, const uint32_t* packedT,
                           const float* gamma, const int8_t* Xq, const float* gamma_a, const uint32_t* mask,
                           float* dX, float* dW, void* workspace, hipStream_t stream);

}  // namespace bitlinear
