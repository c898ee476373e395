// Target logit processors applied where the verifiers read logits: additive bias (fp32),
// allowed-token mask, and the per-row keep threshold that top-k / top-p leave.
//
// Method: [M7.1] "M7.1 - Speculative Decoding: Draft, Verify, Accept, Reject" §0x06J
// (p and q are the processed rows) and §0x04G (temperature and additive-bias processors);
// [Tiny] "Exact Speculative and Assisted Decoding for TinyRustLM", "Grammar and
// deterministic opportunities" (a grammar mask renormalizes over the valid tokens).
#pragma once

#include "device_common.h"
#include "internal.h"

namespace sv {

// s = l + b; a token outside the allowed set or below the threshold tau becomes -inf.  NaN
// and +inf pass through, so a faulty row stays invalid whatever the mask.
__device__ __forceinline__ float proc_elem(float l, float b, bool allowed, float tau) {
  const float s = l + b;
  if (s != s || s == INFINITY) return s;
  return (allowed && s >= tau) ? s : -INFINITY;
}

// Processors over this lane's 8 elements [e0, e0 + 8) of row `row` (e0 a multiple of 8, so
// the 8 mask bits lie in one word).  Elements at or past V are left as they are.
template <bool VEC>
__device__ __forceinline__ void proc8(const ProcSpec& pr, size_t row, float tau, long e0, long V, float (&v)[8]) {
  float b[8];
  if (pr.bias) {
    if (VEC && e0 + 8 <= V) {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(pr.bias + e0);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(pr.bias + e0 + 4);
      b[0] = lo.x; b[1] = lo.y; b[2] = lo.z; b[3] = lo.w;
      b[4] = hi.x; b[5] = hi.y; b[6] = hi.z; b[7] = hi.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = e0 + j < V ? pr.bias[e0 + j] : 0.0f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = 0.0f;
  }
  unsigned bits = 0xffu;
  if (pr.allowed && e0 < V) bits = (pr.allowed[row * pr.W + (e0 >> 5)] >> (e0 & 31)) & 0xffu;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (e0 + j < V) v[j] = proc_elem(v[j], b[j], (bits >> j) & 1u, tau);
}

// The processed value of one element x of row `row`.
__device__ __forceinline__ float proc1(const ProcSpec& pr, size_t row, float tau, long x, float l) {
  const float b = pr.bias ? pr.bias[x] : 0.0f;
  const bool ok = pr.allowed ? ((pr.allowed[row * pr.W + (x >> 5)] >> (x & 31)) & 1u) != 0u : true;
  return proc_elem(l, b, ok, tau);
}

__device__ __forceinline__ float row_tau(const ProcSpec& pr, size_t row) {
  return pr.thresh ? pr.thresh[row] : -INFINITY;
}

}  // namespace sv
