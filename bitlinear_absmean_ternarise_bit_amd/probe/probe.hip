// Attainable-peak probes: what the chip delivers to plain kernels, reported
// beside the published peaks (8 TB/s HBM3E, 5 POPS dense INT8).  They are a
// measurement aid of the benchmark, built into their own library with their
// own header (include/bitlinear_probe.h); they are not part of the BitLinear
// library or its ABI.
//
//  - stream_read_kernel: every lane reads 16-byte vectors with the streaming
//    (nontemporal) cache policy, in batches of eight per lane, each batch one
//    contiguous KiB per wave per load, and folds them into one word;
//  - stream_copy_kernel: the same reads, each vector written to the
//    destination;
//  - mfma_i8_kernel: every wave issues v_mfma_i32_32x32x32_i8 back to back on
//    eight independent accumulators (no memory traffic inside the loop).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bitlinear_probe.h"

namespace bitlinear {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kStreamnt = 2;  // cache-policy bits of a buffer access: streaming

// Each workgroup owns one contiguous slice of the buffer (a multiple of
// 32 KiB: the host checks), read in batches of eight 16-byte loads per lane
// (8 KiB per wave per batch); offsets past the slice would read zeros.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint32_t* __restrict__ src, int64_t per_block,
                                                          uint32_t* __restrict__ out) {
  const char* base = reinterpret_cast<const char*>(src) + static_cast<int64_t>(blockIdx.x) * per_block;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0,
                                                                      static_cast<int>(per_block), 0x00020000);
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t acc = 0;
  for (uint32_t off = wave * 8192u + lane * 16u; off < static_cast<uint32_t>(per_block); off += 4u * 8192u) {
    v4u v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + u * 1024u, 0, kStreamnt);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void stream_copy_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                                          int64_t per_block) {
  const int64_t shift = static_cast<int64_t>(blockIdx.x) * per_block;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(reinterpret_cast<const char*>(src) + shift), 0, static_cast<int>(per_block), 0x00020000);
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char*>(dst) + shift, 0,
                                                                      static_cast<int>(per_block), 0x00020000);
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (uint32_t off = wave * 8192u + lane * 16u; off < static_cast<uint32_t>(per_block); off += 4u * 8192u) {
    v4u v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + u * 1024u, 0, kStreamnt);
#pragma unroll
    for (int u = 0; u < 8; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], ws, off + u * 1024u, 0, kStreamnt);
  }
}

// Two 256-thread workgroups per CU (two waves per SIMD); the operands depend
// on the lane so that nothing is folded, and the accumulators are summed into
// `out` so that nothing is dropped.
__global__ __launch_bounds__(256, 2) void mfma_i8_kernel(int iters, int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const v4i a = {lane, lane + 1, lane + 2, lane + 3};
  const v4i b = {3 * lane, 1, 2 * lane, 5};
  v16i c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[i][r] = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[i], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[i][r];
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = s;
}

// The same with v_mfma_f32_32x32x16_bf16 (32768 flops each) on eight
// independent float accumulators.  The operands are small integers, so every
// product and partial sum is exact and the result does not depend on the
// accumulation order.
typedef __bf16 probe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x16 __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(256, 2) void mfma_bf16_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  probe_bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(static_cast<float>((lane + i) & 3));
    b[i] = static_cast<__bf16>(static_cast<float>((3 * lane + i) & 1));
  }
  probe_f32x16 c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[i][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[i][r];
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = s;
}

}  // namespace

}  // namespace bitlinear

namespace {
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
int hip_status(hipError_t e) { return e == hipSuccess ? BITLINEAR_PROBE_OK : BITLINEAR_PROBE_ERR_HIP; }
}  // namespace

extern "C" {

int bitlinear_probe_stream(const void* src, void* dst, int64_t bytes, int blocks, uint32_t* out, void* stream) {
  if (!src || (!dst && !out)) return BITLINEAR_PROBE_ERR_NULL;
  if (blocks < 1 || blocks > (1 << 20) || bytes < 1 || bytes % (int64_t(blocks) * 32768) != 0 ||
      bytes / blocks >= (int64_t(1) << 31))
    return BITLINEAR_PROBE_ERR_SHAPE;
  if (!aligned(src, 16) || (dst && !aligned(dst, 16)) || (out && !aligned(out, 4))) return BITLINEAR_PROBE_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t per_block = bytes / blocks;
  if (dst)
    bitlinear::stream_copy_kernel<<<blocks, 256, 0, s>>>(static_cast<const uint32_t*>(src),
                                                         static_cast<uint32_t*>(dst), per_block);
  else
    bitlinear::stream_read_kernel<<<blocks, 256, 0, s>>>(static_cast<const uint32_t*>(src), per_block, out);
  return hip_status(hipGetLastError());
}

int bitlinear_probe_mfma_i8(int iters, int blocks, int32_t* out, void* stream) {
  if (!out) return BITLINEAR_PROBE_ERR_NULL;
  if (iters < 1 || blocks < 1 || blocks > (1 << 20)) return BITLINEAR_PROBE_ERR_SHAPE;
  if (!aligned(out, 4)) return BITLINEAR_PROBE_ERR_ALIGN;
  bitlinear::mfma_i8_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, out);
  return hip_status(hipGetLastError());
}

int bitlinear_probe_mfma_bf16(int iters, int blocks, float* out, void* stream) {
  if (!out) return BITLINEAR_PROBE_ERR_NULL;
  if (iters < 1 || iters > (1 << 20) || blocks < 1 || blocks > (1 << 20)) return BITLINEAR_PROBE_ERR_SHAPE;
  if (!aligned(out, 4)) return BITLINEAR_PROBE_ERR_ALIGN;
  bitlinear::mfma_bf16_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, out);
  return hip_status(hipGetLastError());
}

}  // extern "C"
