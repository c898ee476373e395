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
  // NaN and +inf pass through (!(s < inf) holds for exactly those two)
  return (!(s < INFINITY) || (allowed && s >= tau)) ? s : -INFINITY;
}

// The processor inputs of 8 elements [e0, e0 + 8) of row `row` (e0 a multiple of 8, so the
// 8 mask bits lie in one word): the bias values and the allowed bits.
struct Proc8In {
  float b[8];
  unsigned bits;
};
template <bool VEC>
__device__ __forceinline__ void proc8_load(const ProcSpec& pr, size_t row, long e0, long V, Proc8In& in) {
  if (pr.bias) {
    if (VEC && e0 + 8 <= V) {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(pr.bias + e0);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(pr.bias + e0 + 4);
      in.b[0] = lo.x; in.b[1] = lo.y; in.b[2] = lo.z; in.b[3] = lo.w;
      in.b[4] = hi.x; in.b[5] = hi.y; in.b[6] = hi.z; in.b[7] = hi.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) in.b[j] = e0 + j < V ? pr.bias[e0 + j] : 0.0f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) in.b[j] = 0.0f;
  }
  in.bits = 0xffu;
  if (pr.allowed && e0 < V) in.bits = (pr.allowed[row * pr.W + (e0 >> 5)] >> (e0 & 31)) & 0xffu;
}

// Processors applied to 8 loaded logits; elements at or past V are left as they are.
// VEC (V % 8 == 0): the 8 positions are all inside the row or all past it, and a vector
// past it holds -inf with a zero bias, which the transform leaves at -inf, so no position
// needs a bounds test.
template <bool VEC>
__device__ __forceinline__ void proc8_apply(const Proc8In& in, float tau, long e0, long V, float (&v)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (VEC || e0 + j < V) v[j] = proc_elem(v[j], in.b[j], (in.bits >> j) & 1u, tau);
}

// Processors over this lane's 8 elements [e0, e0 + 8) of row `row`.
template <bool VEC>
__device__ __forceinline__ void proc8(const ProcSpec& pr, size_t row, float tau, long e0, long V, float (&v)[8]) {
  Proc8In in;
  proc8_load<VEC>(pr, row, e0, V, in);
  proc8_apply<VEC>(in, tau, e0, V, v);
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
