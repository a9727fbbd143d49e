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

// Rows too long for one wave's registers: one 256-thread workgroup per
// token, RC 16-byte chunks per thread kept in registers between the max and
// the codes, so X is read once (the wave-per-token kernel would read such a
// row twice, and with many rows in flight the second read misses L2).
template <int DT, int RC>
__global__ __launch_bounds__(256) void act_quant_row_kernel(const void* __restrict__ X, int64_t K, int64_t Kp,
                                                            int8_t* __restrict__ Xq, float* __restrict__ gamma_a,
                                                            int32_t* __restrict__ rowsum) {
  constexpr int P = ActTraits<DT>::kPerChunk;
  constexpr int esize = DT == 0 ? 4 : 2;
  __shared__ float s_max[4];
  __shared__ int s_sum[4];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int64_t m = blockIdx.x;
  const uint4* r4 = reinterpret_cast<const uint4*>(static_cast<const char*>(X) + m * K * esize);
  const int64_t nc = K / P;
  uint4 v[RC];
#pragma unroll
  for (int u = 0; u < RC; ++u) {
    const int64_t c = tid + u * 256;
    v[u] = r4[c < nc ? c : nc - 1];
  }
  float mx = 0.0f;
#pragma unroll
  for (int u = 0; u < RC; ++u) {
    float f[P];
    chunk_to_f32<DT>(v[u], f);
    float mu = 0.0f;
#pragma unroll
    for (int i = 0; i < P; ++i) mu = fmaxf(mu, fabsf(f[i]));
    mx = (tid + u * 256 < nc) ? fmaxf(mx, mu) : mx;
  }
  mx = wave_max(mx);
  if (lane == 0) s_max[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float s = __fdiv_rn(127.0f, __fadd_rn(mx, kEps));
  int8_t* dst = Xq + m * Kp;
  int sum = 0;
#pragma unroll
  for (int u = 0; u < RC; ++u) {
    const int64_t c = tid + u * 256;
    if (c < nc) sum += quantize_chunk<DT>(v[u], s, dst + c * P);
  }
  for (int64_t k = K + tid; k < Kp; k += 256) dst[k] = 0;
  sum = wave_sum(sum);
  if (lane == 0) s_sum[wave] = sum;
  __syncthreads();
  if (tid == 0) {
    gamma_a[m] = mx;
    rowsum[m] = s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3];
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
  else if (chunks_per_lane <= 16)
    act_quant_kernel<DT, true, 16><<<blocks, 256, 0, stream>>>(X, M, K, Kp, Xq, gamma_a, rowsum);
  else if (chunks_per_lane <= 32)  // a workgroup per token: at most 8 chunks per thread
    act_quant_row_kernel<DT, 8><<<static_cast<unsigned>(M), 256, 0, stream>>>(X, K, Kp, Xq, gamma_a, rowsum);
  else if (chunks_per_lane <= 64)
    act_quant_row_kernel<DT, 16><<<static_cast<unsigned>(M), 256, 0, stream>>>(X, K, Kp, Xq, gamma_a, rowsum);
  else  // rows over 64 KiB: two passes, the second from L2
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
