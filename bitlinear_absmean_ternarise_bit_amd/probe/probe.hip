// Attainable-peak probes: what the chip delivers to plain kernels, reported
// beside the published peaks (8 TB/s HBM3E, 5 POPS dense INT8).  Not part of
// the method; the benchmark calls them through the C ABI.
//
//  - stream_read_kernel: every lane reads 16-byte vectors with the streaming
//    (nontemporal) cache policy, in batches of eight per lane, each batch one
//    contiguous KiB per wave per load, and folds them into one word;
//  - stream_copy_kernel: the same reads, each vector written to the
//    destination;
//  - mfma_i8_kernel: every wave issues v_mfma_i32_32x32x32_i8 back to back on
//    eight independent accumulators (no memory traffic inside the loop).
#include "kernels.hpp"

namespace bitlinear {

namespace {

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

}  // namespace

hipError_t launch_probe_read(const void* src, int64_t bytes, int blocks, uint32_t* out, hipStream_t stream) {
  stream_read_kernel<<<blocks, 256, 0, stream>>>(static_cast<const uint32_t*>(src), bytes / blocks, out);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, int64_t bytes, int blocks, hipStream_t stream) {
  stream_copy_kernel<<<blocks, 256, 0, stream>>>(static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst),
                                                 bytes / blocks);
  return hipGetLastError();
}

hipError_t launch_probe_mfma_i8(int iters, int blocks, int32_t* out, hipStream_t stream) {
  mfma_i8_kernel<<<blocks, 256, 0, stream>>>(iters, out);
  return hipGetLastError();
}

}  // namespace bitlinear
