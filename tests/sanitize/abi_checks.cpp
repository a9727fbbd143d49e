// The C ABI's host-side argument checks, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (every report is fatal) against a launch stub
// (launch_stub.hip): each entry point is called with bad arguments (which must
// fail before any launch) and with good ones (which must reach the expected
// launchers, with workspace parts inside the workspace), including sizes at
// the limits where the size arithmetic could overflow, and with a failing
// launch (which must come back as BITLINEAR_ERR_HIP).  Prints one line per
// failed check and exits non-zero if any failed.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/bitlinear.h"
#include "stub.h"

namespace {

int g_failed = 0, g_checked = 0;

#define CHECK(cond)                                                      \
  do {                                                                   \
    ++g_checked;                                                         \
    if (!(cond)) {                                                       \
      ++g_failed;                                                        \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
    }                                                                    \
  } while (0)
#define CHECK_EQ(a, b) CHECK((a) == (b))

// Non-null, 256-byte aligned stand-ins for device pointers: only their
// values are used (the stub never dereferences them).
char* const F = reinterpret_cast<char*>(uintptr_t(1) << 20);
const int64_t I64MAX = INT64_MAX, I64MIN = INT64_MIN;

struct Workspace {
  char* p;
  size_t n;
  char* data() { return p; }
  size_t size() const { return n; }
};

bool called(int i, const char* name) {
  const StubCall* c = stub_call(i);
  return c && strcmp(c->name, name) == 0;
}

bool inside(const void* p, const void* base, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(base);
  return a >= b && a < b + bytes;
}

void size_queries() {
  const int64_t bad[] = {0, -1, I64MIN, I64MAX, (int64_t(1) << 40) + 1};
  for (int64_t v : bad) {
    CHECK_EQ(bitlinear_padded_k(v), 0);
    CHECK_EQ(bitlinear_r3_padded_k(v), 0);
    CHECK_EQ(bitlinear_packed_bytes(v, 64), 0u);
    CHECK_EQ(bitlinear_packed_bytes(64, v), 0u);
    CHECK_EQ(bitlinear_r3_packed_bytes(v, 80), 0u);
    CHECK_EQ(bitlinear_forward_workspace_bytes(v, 64), 0u);
    CHECK_EQ(bitlinear_forward_workspace_bytes(64, v), 0u);
    CHECK_EQ(bitlinear_ste_mask_bytes(v, 7), 0u);
    CHECK_EQ(bitlinear_backward_workspace_bytes(v, 8, 8), 0u);
    CHECK_EQ(bitlinear_backward_workspace_bytes(8, 8, v), 0u);
    CHECK_EQ(bitlinear_ffn_workspace_bytes(v, 1, 64, 64), 0u);
    CHECK_EQ(bitlinear_ffn_workspace_bytes(1, 1, 64, v), 0u);
    CHECK_EQ(bitlinear_lut_workspace_bytes(1, v, 64), 0u);
  }
  const int64_t t = int64_t(1) << 40;
  CHECK_EQ(bitlinear_padded_k(t), t);
  CHECK_EQ(bitlinear_packed_bytes(t, t), 0u);  // 2^78 bytes
  CHECK_EQ(bitlinear_packed_bytes(t, 64), size_t(t) * 16);
  CHECK_EQ(bitlinear_backward_workspace_bytes(t, t, t), 0u);
  CHECK_EQ(bitlinear_ffn_workspace_bytes(int64_t(1) << 20, int64_t(1) << 20, t, t), 0u);
  CHECK_EQ(bitlinear_padded_k(1), 64);
  CHECK_EQ(bitlinear_r3_padded_k(81), 160);
  CHECK_EQ(bitlinear_packed_bytes(3, 100), size_t(3 * 128 / 4));
  CHECK_EQ(bitlinear_forward_workspace_bytes(10, 100) % 256, 0u);
  CHECK(bitlinear_quantize_workspace_bytes() > 0);
  for (int s = -8; s <= 1; ++s) CHECK(bitlinear_status_string(s) != nullptr && strlen(bitlinear_status_string(s)) > 0);
  CHECK(strcmp(bitlinear_status_string(-99), "unknown status") == 0);
  CHECK(strcmp(bitlinear_status_string(INT32_MIN), "unknown status") == 0);
}

void quantize_weights(Workspace& host_ws) {
  const size_t ws = bitlinear_quantize_workspace_bytes();
  auto q = [&](int64_t N, int64_t K, void* W = F, void* packed = F, void* gamma = F, void* w = F,
               size_t wsb = 0) {
    return bitlinear_quantize_weights(static_cast<const float*>(W), N, K, static_cast<uint32_t*>(packed),
                                      static_cast<float*>(gamma), w, wsb ? wsb : ws, nullptr);
  };
  stub_reset(-1);
  CHECK_EQ(q(4, 4, nullptr), BITLINEAR_ERR_NULL);
  CHECK_EQ(q(4, 4, F, nullptr), BITLINEAR_ERR_NULL);
  CHECK_EQ(q(4, 4, F, F, nullptr), BITLINEAR_ERR_NULL);
  const int64_t shapes[][2] = {{0, 4}, {4, 0}, {-1, 4}, {I64MAX, 4}, {4, I64MAX}, {I64MIN, I64MIN},
                               {4, (int64_t(1) << 20) + 1}, {int64_t(1) << 13, int64_t(1) << 19},
                               {int64_t(1) << 28, 1}, {int64_t(1) << 27, 1}, {int64_t(1) << 27, 64},
                               {(int64_t(1) << 31) + 1, 1}};
  for (auto& s : shapes) CHECK_EQ(q(s[0], s[1]), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(q(4, 4, F + 4), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(q(4, 4, F, F + 8), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(q(4, 4, F, F, F + 2), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(q(4, 4, F, F, F, nullptr), BITLINEAR_ERR_WORKSPACE);
  CHECK_EQ(q(4, 4, F, F, F, F, ws - 1), BITLINEAR_ERR_WORKSPACE);
  CHECK_EQ(q(4, 4, F, F, F, F + 4), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(stub_count(), 0);  // nothing launched on any bad argument
  // the largest packed matrix below 2 GiB, and a valid call
  CHECK_EQ(q((int64_t(1) << 27) - 1, 1, F, F, F, host_ws.data()), BITLINEAR_OK);
  CHECK(called(0, "quantize_weights") && stub_call(0)->N == (int64_t(1) << 27) - 1);
  stub_reset(0);
  CHECK_EQ(q(4, 4), BITLINEAR_ERR_HIP);
  // radix-3
  stub_reset(-1);
  auto r3 = [&](int64_t N, int64_t K, void* packed = F) {
    return bitlinear_quantize_weights_r3(reinterpret_cast<const float*>(F), N, K, static_cast<uint8_t*>(packed),
                                         reinterpret_cast<float*>(F), F, ws, nullptr);
  };
  CHECK_EQ(r3(int64_t(1) << 27, 1), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(r3(4, I64MAX), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(r3(4, 4, F + 8), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(r3(100, 300), BITLINEAR_OK);
  CHECK(called(0, "quantize_weights_r3"));
}

void activations() {
  auto a = [&](int dt, int64_t M, int64_t K, void* X = F, void* Xq = F) {
    return bitlinear_quantize_activations(X, dt, M, K, static_cast<int8_t*>(Xq), reinterpret_cast<float*>(F),
                                          reinterpret_cast<int32_t*>(F), nullptr);
  };
  stub_reset(-1);
  CHECK_EQ(a(0, 2, 8, nullptr), BITLINEAR_ERR_NULL);
  CHECK_EQ(a(2, 2, 8), BITLINEAR_ERR_DTYPE);
  CHECK_EQ(a(-1, 2, 8), BITLINEAR_ERR_DTYPE);
  CHECK_EQ(a(0, 0, 8), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(a(0, I64MAX, 8), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(a(0, int64_t(1) << 31, int64_t(1) << 20), BITLINEAR_ERR_SHAPE);  // M * K >= 2^40... checked
  CHECK_EQ(a(0, 2, 8, F + 2), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(a(1, 2, 8, F + 1), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(a(0, 2, 8, F, F + 4), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(stub_count(), 0);
  CHECK_EQ(a(1, 3, 100), BITLINEAR_OK);
  CHECK(called(0, "act_quant") && stub_call(0)->M == 3 && stub_call(0)->K == 100 && stub_call(0)->flag == 1);
}

void forward(Workspace& host_ws) {
  char* ws = host_ws.data();
  auto fx = [&](int64_t M, int64_t K, int64_t N, int path, size_t wsb, void* w, int dt = 1, void* acc = nullptr) {
    return bitlinear_forward_ex(F, dt, M, K, reinterpret_cast<const uint32_t*>(F), N, reinterpret_cast<const float*>(F),
                                reinterpret_cast<float*>(F), static_cast<int32_t*>(acc), path, w, wsb, nullptr);
  };
  stub_reset(-1);
  CHECK_EQ(fx(1, 64, 16, 3, 0, nullptr), BITLINEAR_ERR_ARG);
  CHECK_EQ(fx(1, 64, 16, -1, 0, nullptr), BITLINEAR_ERR_ARG);
  CHECK_EQ(fx(1, 64, 16, 0, 0, nullptr, 9), BITLINEAR_ERR_DTYPE);
  CHECK_EQ(fx(1, 64, 16, 0, 0, nullptr, 0, F + 2), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(fx(int64_t(1) << 31, 64, int64_t(1) << 10, 0, 0, nullptr), BITLINEAR_ERR_SHAPE);  // M*N >= 2^40
  CHECK_EQ(fx(1, 1, int64_t(1) << 28, 0, 0, nullptr), BITLINEAR_ERR_SHAPE);                  // packed >= 2 GiB
  CHECK_EQ(fx(17, 64, 16, BITLINEAR_PATH_DECODE, 0, nullptr), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(fx(16, 4096, 16, BITLINEAR_PATH_DECODE, 0, nullptr), BITLINEAR_ERR_SHAPE);  // 16 * (4096 + 16) > 65536
  CHECK_EQ(fx(2, 64, int64_t(1) << 28, BITLINEAR_PATH_DECODE, 0, nullptr), BITLINEAR_ERR_SHAPE);  // M*N >= 2^29
  CHECK_EQ(stub_count(), 0);
  // decode: one fused launch, no workspace needed
  CHECK_EQ(fx(16, 4000, 129, 0, 0, nullptr), BITLINEAR_OK);
  CHECK(stub_count() == 1 && called(0, "decode") && stub_call(0)->L == 1 && stub_call(0)->M == 16);
  // prefill: the quantiser, then the GEMM on the codes it wrote; the parts
  // of the workspace lie inside it and are 256-byte aligned
  const int64_t M = 300, K = 1000, N = 77;
  const size_t need = bitlinear_forward_workspace_bytes(M, K);
  CHECK(need <= host_ws.size());
  stub_reset(-1);
  CHECK_EQ(fx(M, K, N, 0, need, nullptr), BITLINEAR_ERR_WORKSPACE);
  CHECK_EQ(fx(M, K, N, 0, need - 1, ws), BITLINEAR_ERR_WORKSPACE);
  CHECK_EQ(fx(M, K, N, 0, need, ws + 16), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(stub_count(), 0);
  CHECK_EQ(fx(M, K, N, 0, need, ws), BITLINEAR_OK);
  CHECK(stub_count() == 2 && called(0, "act_quant") && called(1, "prefill"));
  if (stub_count() == 2) {
    const StubCall *aq = stub_call(0), *gm = stub_call(1);
    for (int i = 1; i < 4; ++i) {
      CHECK(inside(aq->p[i], ws, need));
      CHECK(reinterpret_cast<uintptr_t>(aq->p[i]) % 256 == 0);
      CHECK(aq->p[i] == gm->p[i - 1]);  // the GEMM reads what the quantiser wrote
    }
    // the code block [M, Kp] ends before gamma_A, gamma_A before the code sums
    CHECK(reinterpret_cast<const char*>(aq->p[1]) + M * bitlinear_padded_k(K) <= aq->p[2]);
    CHECK(reinterpret_cast<const char*>(aq->p[2]) + M * 4 <= aq->p[3]);
    CHECK(reinterpret_cast<const char*>(aq->p[3]) + M * 4 <= ws + need);
  }
  // a failing quantiser launch stops the call before the GEMM
  stub_reset(0);
  CHECK_EQ(fx(M, K, N, 0, need, ws), BITLINEAR_ERR_HIP);
  CHECK_EQ(stub_count(), 1);
  stub_reset(1);
  CHECK_EQ(fx(M, K, N, 0, need, ws), BITLINEAR_ERR_HIP);
  // bitlinear_forward takes the same route
  stub_reset(-1);
  CHECK_EQ(bitlinear_forward(F, 0, 1, 64, reinterpret_cast<const uint32_t*>(F), 16, reinterpret_cast<const float*>(F),
                             reinterpret_cast<float*>(F), nullptr, 0, nullptr),
           BITLINEAR_OK);
  CHECK(called(0, "decode"));
  // forward_quantized: the GEMM alone
  stub_reset(-1);
  auto fq = [&](int64_t M2, int64_t K2, void* Xq) {
    return bitlinear_forward_quantized(static_cast<const int8_t*>(Xq), reinterpret_cast<const float*>(F),
                                       reinterpret_cast<const int32_t*>(F), M2, K2, reinterpret_cast<const uint32_t*>(F),
                                       8, reinterpret_cast<const float*>(F), reinterpret_cast<float*>(F), nullptr, nullptr);
  };
  CHECK_EQ(fq(4, 64, nullptr), BITLINEAR_ERR_NULL);
  CHECK_EQ(fq(4, 64, F + 8), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(fq(0, 64, F), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(fq(4, I64MAX, F), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(fq(4, 64, F), BITLINEAR_OK);
  CHECK(stub_count() == 1 && called(0, "prefill"));
}

void batched_and_r3_and_lut(Workspace& host_ws) {
  auto fb = [&](int64_t L, int64_t M, int64_t K, int64_t N) {
    return bitlinear_forward_batched(L, F, 1, M, K, reinterpret_cast<const uint32_t*>(F), N,
                                     reinterpret_cast<const float*>(F), reinterpret_cast<float*>(F), nullptr);
  };
  stub_reset(-1);
  CHECK_EQ(fb(0, 1, 2048, 2048), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(fb((int64_t(1) << 20) + 1, 1, 2048, 2048), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(fb(I64MAX, 1, 2048, 2048), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(fb(4, 17, 2048, 2048), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(fb(int64_t(1) << 20, 1, 64, int64_t(1) << 17), BITLINEAR_ERR_SHAPE);  // L * row blocks >= 2^31
  CHECK_EQ(stub_count(), 0);
  CHECK_EQ(fb(1024, 1, 2048, 2048), BITLINEAR_OK);
  CHECK(called(0, "decode") && stub_call(0)->L == 1024);

  auto r3 = [&](int64_t L, int64_t M, int64_t K, int64_t N) {
    return bitlinear_forward_r3(L, F, 0, M, K, reinterpret_cast<const uint8_t*>(F), N, reinterpret_cast<const float*>(F),
                                reinterpret_cast<float*>(F), nullptr, nullptr);
  };
  stub_reset(-1);
  CHECK_EQ(r3(1, 16, 4081, 8), BITLINEAR_ERR_SHAPE);  // 16 * (4160 + 16) > 65536
  CHECK_EQ(r3(1, 1, 1, int64_t(1) << 28), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(r3(-5, 1, 64, 8), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(stub_count(), 0);
  CHECK_EQ(r3(3, 8, 2048, 5632), BITLINEAR_OK);
  CHECK(called(0, "decode_r3") && stub_call(0)->L == 3);

  auto lut = [&](int64_t L, int64_t M, int64_t K, int64_t N, size_t wsb, void* w) {
    return bitlinear_forward_lut(L, F, 1, M, K, reinterpret_cast<const uint32_t*>(F), N,
                                 reinterpret_cast<const float*>(F), reinterpret_cast<float*>(F), nullptr, w, wsb, nullptr);
  };
  const size_t need = bitlinear_lut_workspace_bytes(4, 8, 2048);
  CHECK(need > 0 && need <= host_ws.size());
  stub_reset(-1);
  CHECK_EQ(lut(4, 17, 2048, 64, need, host_ws.data()), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(lut(I64MAX, 8, 2048, 64, need, host_ws.data()), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(lut(4, 8, 2048, 64, need - 1, host_ws.data()), BITLINEAR_ERR_WORKSPACE);
  CHECK_EQ(stub_count(), 0);
  CHECK_EQ(lut(4, 8, 2048, 64, need, host_ws.data()), BITLINEAR_OK);
  CHECK(stub_count() == 2 && called(0, "act_quant") && called(1, "lut") && stub_call(0)->M == 32);
}

void ffn(Workspace& host_ws) {
  char* ws = host_ws.data();
  auto call = [&](int64_t L, int64_t M, int64_t D, int64_t Fh, int64_t Do, float* hidden, int path, size_t wsb,
                  void* w) {
    return bitlinear_ffn_forward(L, F, 1, M, D, Fh, Do, reinterpret_cast<const uint32_t*>(F),
                                 reinterpret_cast<const float*>(F), reinterpret_cast<const uint32_t*>(F),
                                 reinterpret_cast<const float*>(F), reinterpret_cast<float*>(F), hidden, path, w,
                                 wsb, nullptr);
  };
  // decode path: up (ReLU^2), the quantiser over all L*M hidden rows, down on those codes
  const int64_t L = 3, M = 8, D = 256, Fh = 704, Do = 256;
  const size_t need = bitlinear_ffn_workspace_bytes(L, M, D, Fh);
  CHECK(need > 0 && need <= host_ws.size());
  stub_reset(-1);
  CHECK_EQ(call(0, M, D, Fh, Do, nullptr, 0, need, ws), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(call(L, M, D, Fh, -1, nullptr, 0, need, ws), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(call(L, M, D, I64MAX, Do, nullptr, 0, need, ws), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(call(L, M, D, Fh, Do, nullptr, 5, need, ws), BITLINEAR_ERR_ARG);
  CHECK_EQ(call(L, 17, D, Fh, Do, nullptr, BITLINEAR_PATH_DECODE, need, ws), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(call(L, M, D, Fh, Do, nullptr, 0, need - 1, ws), BITLINEAR_ERR_WORKSPACE);
  CHECK_EQ(call(L, M, D, Fh, Do, reinterpret_cast<float*>(F + 4), 0, need, ws), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(stub_count(), 0);
  CHECK_EQ(call(L, M, D, Fh, Do, nullptr, 0, need, ws), BITLINEAR_OK);
  CHECK(stub_count() == 3 && called(0, "decode_relu2") && called(1, "act_quant") && called(2, "decode_codes"));
  if (stub_count() == 3) {
    CHECK(stub_call(1)->M == L * M && stub_call(1)->K == Fh);
    CHECK(inside(stub_call(0)->p[3], ws, need));  // the hidden layer in the workspace
    for (int i = 1; i < 4; ++i) CHECK(inside(stub_call(1)->p[i], ws, need));
  }
  stub_reset(1);
  CHECK_EQ(call(L, M, D, Fh, Do, nullptr, 0, need, ws), BITLINEAR_ERR_HIP);
  CHECK_EQ(stub_count(), 2);
  // prefill path: per layer, quantise X, GEMM (ReLU^2), quantise A, GEMM
  stub_reset(-1);
  CHECK_EQ(call(2, 40, D, Fh, Do, nullptr, BITLINEAR_PATH_PREFILL, bitlinear_ffn_workspace_bytes(2, 40, D, Fh), ws),
           BITLINEAR_OK);
  CHECK(stub_count() == 8 && called(0, "act_quant") && called(1, "prefill_relu2") && called(2, "act_quant") &&
        called(3, "prefill") && called(7, "prefill"));
  stub_reset(5);
  CHECK_EQ(call(2, 40, D, Fh, Do, nullptr, BITLINEAR_PATH_PREFILL, bitlinear_ffn_workspace_bytes(2, 40, D, Fh), ws),
           BITLINEAR_ERR_HIP);
  CHECK_EQ(stub_count(), 6);
}

void backward(Workspace& host_ws) {
  char* ws = host_ws.data();
  stub_reset(-1);
  auto pt = [&](int64_t N, int64_t K, void* packedT, void* mask) {
    return bitlinear_pack_transposed(reinterpret_cast<const float*>(F), N, K, reinterpret_cast<const float*>(F),
                                     static_cast<uint32_t*>(packedT), static_cast<uint32_t*>(mask), nullptr);
  };
  CHECK_EQ(pt(4, 4, nullptr, nullptr), BITLINEAR_ERR_NULL);
  CHECK_EQ(pt(0, 4, F, F), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(pt(1, int64_t(1) << 28, F, F), BITLINEAR_ERR_SHAPE);  // W^T packed >= 2 GiB
  CHECK_EQ(pt(4, 4, F + 8, F), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(stub_count(), 0);
  CHECK_EQ(pt(11008, 4096, F, nullptr), BITLINEAR_OK);
  CHECK(called(0, "pack_transposed"));

  auto bw = [&](int64_t M, int64_t N, int64_t K, void* dX, void* dW, size_t wsb, void* w) {
    return bitlinear_backward(reinterpret_cast<const uint16_t*>(F), M, N, K, reinterpret_cast<const uint32_t*>(F),
                              reinterpret_cast<const float*>(F), reinterpret_cast<const int8_t*>(F),
                              reinterpret_cast<const float*>(F), reinterpret_cast<const uint32_t*>(F),
                              static_cast<float*>(dX), static_cast<float*>(dW), w, wsb, nullptr);
  };
  const int64_t M = 200, N = 300, K = 100;
  const size_t need = bitlinear_backward_workspace_bytes(M, N, K);
  CHECK(need > 0 && need <= host_ws.size());
  stub_reset(-1);
  CHECK_EQ(bw(M, N, K, nullptr, nullptr, need, ws), BITLINEAR_ERR_NULL);
  CHECK_EQ(bw(0, N, K, F, F, need, ws), BITLINEAR_ERR_SHAPE);
  CHECK_EQ(bw(int64_t(1) << 20, int64_t(1) << 11, 64, F, F, need, ws), BITLINEAR_ERR_SHAPE);  // 32-bit operand offsets
  CHECK_EQ(bw(M, N, K, F, F, need - 1, ws), BITLINEAR_ERR_WORKSPACE);
  CHECK_EQ(bw(M, N, K, F + 2, F, need, ws), BITLINEAR_ERR_ALIGN);
  CHECK_EQ(stub_count(), 0);
  CHECK_EQ(bw(M, N, K, F, F, need, ws), BITLINEAR_OK);
  CHECK(called(0, "backward") && stub_call(0)->p[2] == ws);
}

}  // namespace

int main() {
  // a host buffer standing in for workspaces: its addresses are compared with
  // what the launchers receive, its bytes are never read or written
  const size_t bytes = size_t(4) << 20;
  char* ws = static_cast<char*>(aligned_alloc(256, bytes));
  if (!ws) return 2;
  Workspace w{ws, bytes};
  size_queries();
  quantize_weights(w);
  activations();
  forward(w);
  batched_and_r3_and_lut(w);
  ffn(w);
  backward(w);
  free(ws);
  printf("%d checks, %d failed\n", g_checked, g_failed);
  return g_failed ? 1 : 0;
}
