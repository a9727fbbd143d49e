// Standalone per-token AbsMax INT8 quantiser (the prefill path's first
// kernel): one wavefront per token, four tokens per 256-thread workgroup.
#include "kernels.hpp"
#include "quant_act.hpp"

namespace bitlinear {

namespace {

// RC: 16-byte chunks per lane kept in registers (rows of up to RC * 64 chunks
// are read once)
template <int DT, bool VEC, int RC>
__global__ __launch_bounds__(256) void act_quant_kernel(const void* __restrict__ X, int64_t M, int64_t K,
                                                        int64_t Kp, int8_t* __restrict__ Xq,
                                                        float* __restrict__ gamma_a,
                                                        int32_t* __restrict__ rowsum) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (m >= M) return;  // whole wave leaves together
  constexpr int esize = DT == 0 ? 4 : 2;
  const char* row = static_cast<const char*>(X) + m * K * esize;
  float ga;
  int rs;
  quantize_row_wave<DT, VEC, RC>(row, K, Kp, lane, Xq + m * Kp, ga, rs);
  if (lane == 0) {
    gamma_a[m] = ga;
    rowsum[m] = rs;
  }
}

template <int DT>
hipError_t launch_dt(const void* X, int64_t M, int64_t K, int8_t* Xq, float* gamma_a,
                     int32_t* rowsum, hipStream_t stream) {
  const int64_t Kp = padded_k(K);
  const int blocks = static_cast<int>((M + 3) / 4);
  constexpr int esize = DT == 0 ? 4 : 2;
  const bool vec = (reinterpret_cast<uintptr_t>(X) % 16 == 0) && ((K * esize) % 16 == 0);
  const int64_t chunks_per_lane = (K * esize / 16 + kWave - 1) / kWave;
  if (!vec)
    act_quant_kernel<DT, false, 4><<<blocks, 256, 0, stream>>>(X, M, K, Kp, Xq, gamma_a, rowsum);
  else if (chunks_per_lane <= 4)
    act_quant_kernel<DT, true, 4><<<blocks, 256, 0, stream>>>(X, M, K, Kp, Xq, gamma_a, rowsum);
  else if (chunks_per_lane <= 8)
    act_quant_kernel<DT, true, 8><<<blocks, 256, 0, stream>>>(X, M, K, Kp, Xq, gamma_a, rowsum);
  else
    act_quant_kernel<DT, true, 16><<<blocks, 256, 0, stream>>>(X, M, K, Kp, Xq, gamma_a, rowsum);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_act_quant(const void* X, int x_dtype, int64_t M, int64_t K, int8_t* Xq,
                            float* gamma_a, int32_t* rowsum, hipStream_t stream) {
  if (x_dtype == 0) return launch_dt<0>(X, M, K, Xq, gamma_a, rowsum, stream);
  return launch_dt<1>(X, M, K, Xq, gamma_a, rowsum, stream);
}

}  // namespace bitlinear
