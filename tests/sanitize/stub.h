/* The launch stub's record of calls (see launch_stub.hip). */
#ifndef BITLINEAR_TEST_STUB_H
#define BITLINEAR_TEST_STUB_H

#include <stdint.h>

#define kStubMaxCalls 64

typedef struct {
  char name[32];
  int64_t M, N, K, L;
  const void* p[4];
  int flag;
} StubCall;

#ifdef __cplusplus
extern "C" {
#endif
/* Forget every recorded call; the call with index fail_at (0-based, -1 for
 * none) returns a launch failure. */
void stub_reset(int fail_at);
int stub_count(void);
const StubCall* stub_call(int i);
#ifdef __cplusplus
}
#endif

#endif
