// Stand-in for the kernel launchers of the BitLinear library, for a host-only
// build of the C ABI's argument checks (csrc/api.hip) under AddressSanitizer
// and UndefinedBehaviorSanitizer.  Every launcher records its call (name and
// sizes, the buffers it was handed) and returns the status the test sets; no
// HIP runtime call is made and nothing touches a GPU.
#include <string.h>

#include "../../bitlinear_absmean_ternarise_bit_amd/csrc/kernels.hpp"
#include "stub.h"

namespace {
StubCall g_calls[kStubMaxCalls];
int g_count = 0;
int g_fail_at = -1;  // index of the call that fails (-1: none)

hipError_t record(const char* name, int64_t M, int64_t N, int64_t K, int64_t L, const void* p0 = nullptr,
                  const void* p1 = nullptr, const void* p2 = nullptr, const void* p3 = nullptr, int flag = 0) {
  const int i = g_count++;
  if (i < kStubMaxCalls) {
    StubCall& c = g_calls[i];
    strncpy(c.name, name, sizeof(c.name) - 1);
    c.name[sizeof(c.name) - 1] = 0;
    c.M = M;
    c.N = N;
    c.K = K;
    c.L = L;
    c.p[0] = p0;
    c.p[1] = p1;
    c.p[2] = p2;
    c.p[3] = p3;
    c.flag = flag;
  }
  return i == g_fail_at ? hipErrorLaunchFailure : hipSuccess;
}
}  // namespace

extern "C" {
void stub_reset(int fail_at) {
  g_count = 0;
  g_fail_at = fail_at;
  memset(g_calls, 0, sizeof(g_calls));
}
int stub_count(void) { return g_count; }
const StubCall* stub_call(int i) { return (i >= 0 && i < g_count && i < kStubMaxCalls) ? &g_calls[i] : nullptr; }
}

namespace bitlinear {

hipError_t launch_quantize_weights(const float* W, int64_t N, int64_t K, uint32_t* packed, float* gamma,
                                   void* workspace, hipStream_t) {
  return record("quantize_weights", 0, N, K, 1, W, packed, gamma, workspace);
}
hipError_t launch_quantize_weights_r3(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                                      void* workspace, hipStream_t) {
  return record("quantize_weights_r3", 0, N, K, 1, W, packed, gamma, workspace);
}
hipError_t launch_act_quant(const void* X, int x_dtype, int64_t M, int64_t K, int8_t* Xq, float* gamma_a,
                            int32_t* rowsum, hipStream_t) {
  return record("act_quant", M, 0, K, 1, X, Xq, gamma_a, rowsum, x_dtype);
}
hipError_t launch_decode(const void* X, int x_dtype, int64_t M, int64_t K, const uint32_t* packed, int64_t N,
                         const float* gamma, float* Y, int32_t*, int64_t L, hipStream_t, bool relu2) {
  return record(relu2 ? "decode_relu2" : "decode", M, N, K, L, X, packed, gamma, Y, x_dtype);
}
hipError_t launch_decode_codes(const int8_t* Xq, const float* gamma_a, const int32_t* rowsum, int64_t M,
                               int64_t K, const uint32_t* packed, int64_t N, const float*, float* Y, int64_t L,
                               hipStream_t) {
  return record("decode_codes", M, N, K, L, Xq, gamma_a, rowsum, packed, Y != nullptr);
}
hipError_t launch_decode_r3(const void* X, int x_dtype, int64_t M, int64_t K, const uint8_t* packed, int64_t N,
                            const float* gamma, float* Y, int32_t*, int64_t L, hipStream_t) {
  return record("decode_r3", M, N, K, L, X, packed, gamma, Y, x_dtype);
}
hipError_t launch_prefill_gemm(const int8_t* Xq, const float* gamma_a, const int32_t* rowsum, int64_t M,
                               int64_t K, const uint32_t* packed, int64_t N, const float*, float* Y, int32_t*,
                               hipStream_t, bool relu2) {
  (void)Y;
  return record(relu2 ? "prefill_relu2" : "prefill", M, N, K, 1, Xq, gamma_a, rowsum, packed);
}
hipError_t launch_lut_gemv(const int8_t* Xq, const float* gamma_a, int64_t M, int64_t K, const uint32_t* packed,
                           int64_t N, const float*, float* Y, int32_t*, int64_t L, hipStream_t) {
  return record("lut", M, N, K, L, Xq, gamma_a, packed, Y);
}
hipError_t launch_pack_transposed(const float* W, int64_t N, int64_t K, const float* gamma, uint32_t* packedT,
                                  uint32_t* mask, hipStream_t) {
  return record("pack_transposed", 0, N, K, 1, W, gamma, packedT, mask);
}
hipError_t launch_backward(const uint16_t* dY, int64_t M, int64_t N, int64_t K, const uint32_t* packedT,
                           const float*, const int8_t* Xq, const float*, const uint32_t*, float* dX, float* dW,
                           void* workspace, hipStream_t) {
  (void)dY;
  (void)packedT;
  (void)Xq;
  return record("backward", M, N, K, 1, dX, dW, workspace, nullptr);
}

}  // namespace bitlinear
