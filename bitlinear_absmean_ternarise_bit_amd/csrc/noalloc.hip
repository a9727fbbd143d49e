// bitlinear_forward_noalloc: the forward for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid allocation).  It runs the same kernels as bitlinear_forward; the
// prefill path's workspace (activation codes, gamma_A, code sums) is a
// file-scope device array instead of a caller buffer.
//
// The array is one per GPU, created when the library's code is loaded on that
// GPU and held until the process ends.  Host code never uses the array's name
// as an address (in host code it names a host-side stand-in): on the first
// call on a device, with that device current, hipGetSymbolAddress gives the
// device address, which is kept per device and passed to the kernels.  Every
// call on a GPU shares that GPU's array, so calls that overlap on one GPU
// (on different streams, or from different host threads without ordering)
// race on it.  Nothing in it needs clearing: the activation quantiser writes
// every byte the GEMM reads.
#include <mutex>

#include "../../include/bitlinear.h"
#include "kernels.hpp"

namespace {

static_assert(BITLINEAR_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size is a multiple of 256 bytes");
static __device__ __align__(256) char scratch[BITLINEAR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];

// The device address of this device's scratch array (looked up once per
// device, with that device current), or nullptr with *err set.
void* scratch_of(int dev, hipError_t* err) {
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_once[dev], [dev] {
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess && prev != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev >= 0 && prev != dev) {
      const hipError_t r = hipSetDevice(prev);
      if (e == hipSuccess) e = r;
    }
    g_status[dev] = e;
    g_scratch[dev] = e == hipSuccess ? p : nullptr;
  });
  *err = g_status[dev];
  return g_scratch[dev];
}

}  // namespace

extern "C" int bitlinear_forward_noalloc(const void* X, int x_dtype, int64_t M, int64_t K, const uint32_t* packed,
                                         int64_t N, const float* gamma, float* Y, void* stream) {
  bool decode = false;
  const int st = bitlinear::check_forward_args(X, x_dtype, M, K, packed, N, gamma, Y, nullptr,
                                               BITLINEAR_PATH_AUTO, &decode);
  if (st) return st;
  if (decode)  // the fused decode kernel needs no workspace
    return bitlinear_forward_ex(X, x_dtype, M, K, packed, N, gamma, Y, nullptr, BITLINEAR_PATH_AUTO, nullptr, 0,
                                stream);
  if (bitlinear::prefill_ws_bytes(M, K) > BITLINEAR_NOALLOC_SCRATCH_BYTES) return BITLINEAR_ERR_WORKSPACE;
  // the device the work runs on: the stream's, or the current one for the null stream
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = -1;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return BITLINEAR_ERR_HIP;
  void* ws = scratch_of(dev, &e);
  if (!ws) return BITLINEAR_ERR_HIP;
  return bitlinear_forward_ex(X, x_dtype, M, K, packed, N, gamma, Y, nullptr, BITLINEAR_PATH_AUTO, ws,
                              BITLINEAR_NOALLOC_SCRATCH_BYTES, stream);
}
