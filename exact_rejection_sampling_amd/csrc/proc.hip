// Keep thresholds of top-k and top-p (the pre-pass of spec_verify_chain_ex).
//
// One block per row.  A token is a candidate when it is allowed and s = l + b (fp32) is
// finite; a candidate's key is an order-preserving map of s to 32 bits.
//  * top-k (k >= 1, fewer than k candidates: off): tau_k = the k-th largest key, with
//    multiplicity -- the largest key t with #{candidates with key >= t} >= k.
//  * top-p (0 < p < 1): among the candidates with key >= tau_k, with weights
//    w = 2^((s - max) * c2), tau_p = the largest key t whose mass {key >= t} reaches
//    p * (total mass): the smallest tie-closed set of top tokens whose probability reaches p.
// Both are found by 16-way bisection over the key range: a pass streams the row once and
// accumulates, per thread and in registers, the count (or fp64 mass) of candidates at or
// above each of 16 boundaries; one block reduction, in a fixed order, picks the
// sub-interval.  Eight passes resolve a 32-bit key; there are no atomics and the result is
// the same on every run.  The row's threshold is the larger of the two, or -inf.
//
// Method: [M7.1] "M7.1 - Speculative Decoding: Draft, Verify, Accept, Reject" §0x06J (the
// verified p is the row after top-k and top-p); [Tiny] "Exact Speculative and Assisted
// Decoding for TinyRustLM", "Exactness tests" (transformed distributions after top-k and
// top-p).
#include "device_common.h"
#include "internal.h"
#include "proc.h"

namespace sv {

namespace {

constexpr int kWays = 16;

__device__ __forceinline__ unsigned key_of(float s) {
  if (s == 0.0f) s = 0.0f;                       // -0 and +0 are one value
  const unsigned u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float value_of(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// The candidates of this thread's 8 elements at e0: processed values (mask applied, no
// threshold), validity bits.
template <int DT, bool VEC>
__device__ __forceinline__ unsigned cand8(const ThreshParams& p, const void* lrow, size_t row, long e0, float (&s)[8]) {
  load8<DT, VEC, false>(lrow, e0, p.V, s, -INFINITY);
  ProcSpec pr{};
  pr.bias = p.bias;
  pr.allowed = p.allowed;
  pr.W = p.W;
  proc8<VEC>(pr, row, -INFINITY, e0, p.V, s);
  unsigned ok = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (e0 + j < p.V && s[j] > -INFINITY && s[j] < INFINITY) ok |= 1u << j;   // false for NaN
  return ok;
}

// Block-wide fp64 sums of 16 per-thread accumulators (fixed order: DPP tree per wave, waves
// in index order).  Every thread receives the totals.
__device__ void block_sums16(double (&acc)[kWays], double* scratch /* [kWavesPerBlock * kWays] */) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
#pragma unroll
  for (int j = 0; j < kWays; ++j) {
    const double t = wave_sum_d(acc[j]);
    if (lane == 0) scratch[wave * kWays + j] = t;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kWays; ++j) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) t += scratch[w * kWays + j];
    acc[j] = t;
  }
  __syncthreads();
}

// 16-way bisection for the largest key t in [lo, hi] with F(t) >= target, where F(t) is
// the count (MASS false) or the mass (MASS true) of candidates with key >= t, and
// F(lo) >= target.  The target is target_of(F(lo)), F(lo) coming from the first pass.
template <int DT, bool VEC, bool MASS, class TargetOf>
__device__ unsigned bisect(const ThreshParams& p, const void* lrow, size_t row, unsigned lo, unsigned hi, float M,
                           TargetOf target_of, double* scratch) {
  double target = 0.0;
  bool first = true;
  while (lo < hi) {
    const unsigned long long width = ((unsigned long long)(hi - lo) + kWays) / kWays;   // ceil((hi-lo+1)/16)
    unsigned bnd[kWays];
#pragma unroll
    for (int j = 0; j < kWays; ++j) {
      const unsigned long long b = (unsigned long long)lo + (unsigned long long)j * width;
      bnd[j] = b > hi ? 0xffffffffu : static_cast<unsigned>(b);   // past hi: never reached below
    }
    double acc[kWays];
#pragma unroll
    for (int j = 0; j < kWays; ++j) acc[j] = 0.0;
    for (long e0 = (long)threadIdx.x * kVec; e0 < p.V; e0 += (long)kBlock * kVec) {
      float s[8];
      const unsigned ok = cand8<DT, VEC>(p, lrow, row, e0, s);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (!((ok >> e) & 1u)) continue;
        const unsigned k = key_of(s[e]);
        if (k < lo) continue;
        const double w = MASS ? (double)__builtin_amdgcn_exp2f((s[e] - M) * p.c2) : 1.0;
#pragma unroll
        for (int j = 0; j < kWays; ++j)
          if (k >= bnd[j] && (j == 0 || (unsigned long long)lo + (unsigned long long)j * width <= hi)) acc[j] += w;
      }
    }
    block_sums16(acc, scratch);
    if (first) {
      target = target_of(acc[0]);
      first = false;
    }
    int jbest = 0;
#pragma unroll
    for (int j = 1; j < kWays; ++j)
      if ((unsigned long long)lo + (unsigned long long)j * width <= hi && acc[j] >= target) jbest = j;
    const unsigned long long nlo = (unsigned long long)lo + (unsigned long long)jbest * width;
    const unsigned long long nhi = nlo + width - 1;
    lo = static_cast<unsigned>(nlo);
    hi = nhi < hi ? static_cast<unsigned>(nhi) : hi;
  }
  return lo;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void thresh_kernel(ThreshParams p) {
  __shared__ double s_scratch[kWavesPerBlock * kWays];
  __shared__ float s_m[kWavesPerBlock], s_mn[kWavesPerBlock];
  __shared__ int s_fault;
  const size_t row = blockIdx.x;
  const int b = static_cast<int>(row / p.R);
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const int k = p.top_k ? p.top_k[b] : 0;
  const float tp = p.top_p ? p.top_p[b] : 1.0f;
  const bool use_k = k >= 1, use_p = tp > 0.0f && tp < 1.0f;   // false for NaN
  if (!use_k && !use_p) {
    if (threadIdx.x == 0) p.thresh[row] = -INFINITY;
    return;
  }
  const void* lrow = row_ptr<DT>(p.logits, row, p.V);
  if (threadIdx.x == 0) s_fault = 0;
  __syncthreads();
  // pass 0: the candidates' maximum, minimum and count; NaN / +inf anywhere makes the row
  // invalid for the verifier, and then no threshold is needed
  float m = -INFINITY, mn = INFINITY;
  double cnt = 0.0;
  bool fault = false;
  for (long e0 = (long)threadIdx.x * kVec; e0 < p.V; e0 += (long)kBlock * kVec) {
    float s[8];
    const unsigned ok = cand8<DT, VEC>(p, lrow, row, e0, s);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e0 + e < p.V && (s[e] != s[e] || s[e] == INFINITY)) fault = true;
      if ((ok >> e) & 1u) {
        m = fmaxf(m, s[e]);
        mn = fminf(mn, s[e]);
        cnt += 1.0;
      }
    }
  }
  if (fault) s_fault = 1;
  const float wm = wave_max(m);
  const float wmn = -wave_max(-mn);
  const double wc = wave_sum_d(cnt);
  if (lane == 0) {
    s_m[wave] = wm;
    s_mn[wave] = wmn;
    s_scratch[wave] = wc;
  }
  __syncthreads();
  float M = -INFINITY, MN = INFINITY;
  double C = 0.0;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) {
    M = fmaxf(M, s_m[w]);
    MN = fminf(MN, s_mn[w]);
    C += s_scratch[w];
  }
  __syncthreads();
  float tau = -INFINITY;
  if (!s_fault && C > 0.0) {
    unsigned lo = key_of(MN), hi = key_of(M);
    if (use_k && (double)k < C) {
      const double kk = (double)k;
      lo = bisect<DT, VEC, false>(p, lrow, row, lo, hi, M, [kk](double) { return kk; }, s_scratch);
      tau = value_of(lo);
    }
    if (use_p) {
      const double pp = (double)tp;
      const unsigned t = bisect<DT, VEC, true>(p, lrow, row, lo, hi, M, [pp](double z) { return pp * z; }, s_scratch);
      tau = value_of(t);
    }
  }
  if (threadIdx.x == 0) p.thresh[row] = tau;
}

template <int DT, bool VEC>
hipError_t launch_typed(const ThreshParams& p, hipStream_t s) {
  thresh_kernel<DT, VEC><<<dim3((unsigned)p.rows), dim3(kBlock), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_thresholds(const ThreshParams& p, int logit_dtype, bool vec, hipStream_t s) {
  if (logit_dtype == kBF16) return vec ? launch_typed<kBF16, true>(p, s) : launch_typed<kBF16, false>(p, s);
  return vec ? launch_typed<kF32, true>(p, s) : launch_typed<kF32, false>(p, s);
}

}  // namespace sv
