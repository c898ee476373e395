/* A C caller of libspec_verify: plain device buffers from the HIP runtime, no Python and
 * no torch.  Greedy verification of two requests and chain verification of two requests
 * whose rows are one-hot (so every emitted token is determined), each checked against the
 * answer worked out by hand; prints "ok" and returns 0 when all match.
 * Built by __graft_entry__.build() and run by tests/test_gpu_abi_c.py. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spec_verify.h"

#define HIP_OK(x)                                                                      \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                   \
      return 2;                                                                        \
    }                                                                                  \
  } while (0)

#define SPEC_OK_OR_FAIL(x)                                                             \
  do {                                                                                 \
    spec_status s_ = (x);                                                              \
    if (s_ != SPEC_OK) {                                                               \
      fprintf(stderr, "%s returned %s\n", #x, spec_status_string(s_));                 \
      return 3;                                                                        \
    }                                                                                  \
  } while (0)

static int same(const int32_t* got, const int32_t* want, int n, const char* what) {
  for (int i = 0; i < n; ++i)
    if (got[i] != want[i]) {
      fprintf(stderr, "%s[%d] = %d, expected %d\n", what, i, got[i], want[i]);
      return 0;
    }
  return 1;
}

/* device copy of n bytes of host data */
static void* to_device(const void* host, size_t n) {
  void* d = NULL;
  if (hipMalloc(&d, n) != hipSuccess) return NULL;
  if (hipMemcpy(d, host, n, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

static int greedy_case(void) {
  enum { B = 2, G = 2, R = 3, V = 5 };
  /* row argmaxes: request 0 -> 1, 3, 4; request 1 -> 2, 0, 1 */
  float logits[B][R][V] = {{{0, 5, 1, 2, 0}, {1, 0, 2, 9, 3}, {0, 1, 2, 3, 4}},
                           {{0, 1, 7, 2, 0}, {6, 0, 2, 1, 3}, {0, 8, 2, 3, 4}}};
  int32_t tokens[B][G] = {{1, 3}, {2, 4}};
  /* request 0 matches both drafts and adds the bonus argmax; request 1 fails at draft 1 */
  const int32_t want_len[B] = {2, 1}, want_out[B * R] = {1, 3, 4, 2, 0, -1}, want_st[B] = {0, 0};
  void *dl = to_device(logits, sizeof logits), *dt = to_device(tokens, sizeof tokens);
  int32_t *d_len = NULL, *d_out = NULL, *d_st = NULL;
  void* ws = NULL;
  const size_t wsb = spec_greedy_workspace_bytes(B, G, V);
  if (!dl || !dt || wsb == 0) return 4;
  HIP_OK(hipMalloc((void**)&d_len, sizeof(int32_t) * B));
  HIP_OK(hipMalloc((void**)&d_out, sizeof(int32_t) * B * R));
  HIP_OK(hipMalloc((void**)&d_st, sizeof(int32_t) * B));
  HIP_OK(hipMalloc(&ws, wsb));
  HIP_OK(hipMemset(ws, 0, wsb));
  SPEC_OK_OR_FAIL(spec_verify_greedy(dl, SPEC_F32, (const int32_t*)dt, B, G, V, d_len, d_out, d_st, ws, wsb, NULL));
  HIP_OK(hipDeviceSynchronize());
  int32_t len[B], out[B * R], st[B];
  HIP_OK(hipMemcpy(len, d_len, sizeof len, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(st, d_st, sizeof st, hipMemcpyDeviceToHost));
  hipFree(dl); hipFree(dt); hipFree(d_len); hipFree(d_out); hipFree(d_st); hipFree(ws);
  return same(len, want_len, B, "greedy accepted_len") && same(out, want_out, B * R, "greedy out_tokens") &&
                 same(st, want_st, B, "greedy req_status")
             ? 0
             : 1;
}

static int chain_case(void) {
  enum { B = 2, G = 2, R = 3, V = 4 };
  /* one-hot target rows (-inf elsewhere): row i of both requests puts all mass on token
   * (i + 1) % V; draft rows are one-hot at the draft token */
  float logits[B][R][V], q[B][G][V];
  int32_t tokens[B][G] = {{1, 2}, {1, 3}};
  float u[B][R] = {{0.5f, 0.5f, 0.5f}, {0.5f, 0.5f, 0.5f}};
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < R; ++i)
      for (int x = 0; x < V; ++x) logits[b][i][x] = x == (i + 1) % V ? 0.0f : -INFINITY;
  memset(q, 0, sizeof q);
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < G; ++i) q[b][i][tokens[b][i]] = 1.0f;
  /* request 0: both drafts are the target's tokens (p / q = 1), bonus token 3 from row 2;
   * request 1: draft 1 (token 3) has p = 0, so it is rejected and the residual
   * max(p - q, 0) is the target's row 1: token 2 */
  const int32_t want_len[B] = {2, 1}, want_out[B * R] = {1, 2, 3, 1, 2, -1}, want_st[B] = {0, 0};
  void *dl = to_device(logits, sizeof logits), *dq = to_device(q, sizeof q);
  void *dt = to_device(tokens, sizeof tokens), *du = to_device(u, sizeof u);
  int32_t *d_len = NULL, *d_out = NULL, *d_st = NULL;
  void* ws = NULL;
  const size_t wsb = spec_chain_workspace_bytes(B, G, V);
  if (!dl || !dq || !dt || !du || wsb == 0) return 4;
  HIP_OK(hipMalloc((void**)&d_len, sizeof(int32_t) * B));
  HIP_OK(hipMalloc((void**)&d_out, sizeof(int32_t) * B * R));
  HIP_OK(hipMalloc((void**)&d_st, sizeof(int32_t) * B));
  HIP_OK(hipMalloc(&ws, wsb));
  HIP_OK(hipMemset(ws, 0, wsb));
  SPEC_OK_OR_FAIL(spec_verify_chain(dl, SPEC_F32, dq, SPEC_F32, (const int32_t*)dt, (const float*)du, B, G, V, 1.0f,
                                    d_len, d_out, d_st, NULL, ws, wsb, NULL));
  HIP_OK(hipDeviceSynchronize());
  int32_t len[B], out[B * R], st[B];
  HIP_OK(hipMemcpy(len, d_len, sizeof len, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(st, d_st, sizeof st, hipMemcpyDeviceToHost));
  /* the workspace is back to zero */
  unsigned char* host_ws = (unsigned char*)calloc(wsb, 1);
  int dirty = 0;
  if (host_ws && hipMemcpy(host_ws, ws, wsb, hipMemcpyDeviceToHost) == hipSuccess)
    for (size_t k = 0; k < wsb; ++k) dirty |= host_ws[k] != 0;
  free(host_ws);
  hipFree(dl); hipFree(dq); hipFree(dt); hipFree(du); hipFree(d_len); hipFree(d_out); hipFree(d_st); hipFree(ws);
  if (dirty) {
    fprintf(stderr, "chain workspace not returned to zero\n");
    return 1;
  }
  return same(len, want_len, B, "chain accepted_len") && same(out, want_out, B * R, "chain out_tokens") &&
                 same(st, want_st, B, "chain req_status")
             ? 0
             : 1;
}

int main(void) {
  if (spec_abi_version() != SPEC_ABI_VERSION) {
    fprintf(stderr, "library ABI %d, header ABI %d\n", spec_abi_version(), SPEC_ABI_VERSION);
    return 5;
  }
  int rc = greedy_case();
  if (rc == 0) rc = chain_case();
  if (rc == 0) printf("ok\n");
  return rc;
}
