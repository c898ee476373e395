// Keep thresholds of top-k and top-p (the pre-pass of spec_verify_chain_ex).
//
// One block per row.  A token is a candidate when it is allowed and s = l + b (fp32) is
// finite; a candidate's key is an order-preserving map of s to 32 bits.
//  * top-k (k >= 1, fewer than k candidates: off): tau_k = the k-th largest key, with
//    multiplicity -- the largest key t with #{candidates with key >= t} >= k.
//  * top-p (0 < p < 1): among the candidates with key >= tau_k, with weights
//    w = 2^((s - max) * c2), tau_p = the largest key t whose mass {key >= t} reaches
//    p * (total mass): the smallest tie-closed set of top tokens whose probability reaches p.
// Both are found by radix selection over the bits in which the row's candidate keys differ,
// 12 bits per pass: a pass streams the row once and adds each candidate whose higher bits
// match the prefix found so far into one of 4096 LDS bins -- a count (top-k) or a mass in
// fixed point, 2^-32 of the largest weight, rounded to nearest (top-p).  Integer sums do not
// depend on the order of the additions, so the result is the same on every run.  The row's
// threshold is the larger of the two, or -inf.
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

// 1024 threads (16 waves) per row: enough waves per SIMD to hide the per-element chain.
constexpr int kTB = 1024;
constexpr int kTW = kTB / kWave;
constexpr int kDigit = 12;
constexpr int kBins = 1 << kDigit;
constexpr int kBinsPerThread = kBins / kTB;

struct RadixLds {
  unsigned long long bin[kBins];        // counts, or masses in fixed point
  double scan[kTW];
  int digit;
  double f_above;
};

// Block-wide exclusive prefix (fp64) over the kTB threads; *total gets the block sum.
__device__ double tb_excl_scan(double v, double* scratch, double* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const double incl = wave_incl_scan_d(v, lane);
  const double excl = wave_shr1_d(incl);
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  double off = 0.0, tot = 0.0;
#pragma unroll
  for (int w = 0; w < kTW; ++w) {
    if (w < wave) off += scratch[w];
    tot += scratch[w];
  }
  __syncthreads();
  *total = tot;
  return off + excl;
}

// Radix selection of the largest key t >= klo with F(t) >= target, where F(t) is the count
// (MASS false) or the fixed-point mass (MASS true; weights scaled by `fix`) of the
// candidates with key >= t; keys below klo are ignored.  [klo, khi] bounds the keys; the
// bits above their highest differing bit are shared.  `param` is the count target k, or the
// fraction p of the total mass F(klo) that the target is.  Every value stays an integer
// below 2^53, so the fp64 scans are exact.
template <int DT, bool VEC, bool MASS>
__device__ unsigned radix_select(const ThreshParams& p, const void* lrow, size_t row, unsigned klo, unsigned khi,
                                 double param, float M, double fix, RadixLds& L) {
  const int tid = threadIdx.x;
  const int nb = (klo == khi) ? 0 : 32 - __clz(klo ^ khi);   // the varying low bits
  unsigned prefix = nb == 32 ? 0u : (klo >> nb);             // the digits chosen so far
  double above = 0.0;                                        // F just above the prefix's range
  double target = MASS ? -1.0 : param;
  for (int done = 0; done < nb;) {
    const int width = min(kDigit, nb - done), shift = nb - done - width;
    for (int j = tid; j < kBins; j += kTB) L.bin[j] = 0ull;
    __syncthreads();
    for (long e0 = (long)tid * kVec; e0 < p.V; e0 += (long)kTB * kVec) {
      float s[8];
      const unsigned ok = cand8<DT, VEC>(p, lrow, row, e0, s);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (!((ok >> e) & 1u)) continue;
        const unsigned k = key_of(s[e]);
        if (k < klo) continue;
        const unsigned high = shift + width == 32 ? 0u : (k >> (shift + width));
        if (high != prefix) continue;
        unsigned long long v = 1ull;
        if constexpr (MASS) v = __double2ull_rn((double)__builtin_amdgcn_exp2f((s[e] - M) * p.c2) * fix);
        atomicAdd(&L.bin[(k >> shift) & ((1u << width) - 1u)], v);
      }
    }
    __syncthreads();
    // thread t owns kBinsPerThread consecutive digits, highest digits to thread 0
    const int d_hi = (1 << width) - 1 - tid * kBinsPerThread;
    double run = 0.0;
#pragma unroll
    for (int i = 0; i < kBinsPerThread; ++i)
      if (d_hi - i >= 0) run += (double)L.bin[d_hi - i];
    double tot;
    const double before = tb_excl_scan(run, L.scan, &tot);   // F of the digits above this run
    if (target < 0.0) target = param * (above + tot);             // MASS: p * total mass
    if (tid == 0) L.digit = -1;
    __syncthreads();
    // the largest digit whose F reaches the target: the first hit going down; only one
    // thread's run holds it (F rises as the digit falls)
    double f = above + before;
    for (int i = 0; i < kBinsPerThread; ++i) {
      const int d = d_hi - i;
      if (d < 0) break;
      const double b = (double)L.bin[d];
      if (f < target && f + b >= target) {
        L.digit = d;
        L.f_above = f;
      }
      f += b;
    }
    __syncthreads();
    const int d = L.digit;
    above = L.f_above;
    __syncthreads();
    prefix = (prefix << width) | static_cast<unsigned>(d < 0 ? 0 : d);
    done += width;
  }
  return nb == 0 ? klo : prefix;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kTB) void thresh_kernel(ThreshParams p) {
  __shared__ double s_scratch[kTW];
  __shared__ RadixLds s_radix;
  __shared__ float s_m[kTW], s_mn[kTW];
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
  for (long e0 = (long)threadIdx.x * kVec; e0 < p.V; e0 += (long)kTB * kVec) {
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
  for (int w = 0; w < kTW; ++w) {
    M = fmaxf(M, s_m[w]);
    MN = fminf(MN, s_mn[w]);
    C += s_scratch[w];
  }
  __syncthreads();
  float tau = -INFINITY;
  if (!s_fault && C > 0.0) {
    unsigned lo = key_of(MN);
    const unsigned hi = key_of(M);
    if (use_k && (double)k < C) {
      lo = radix_select<DT, VEC, false>(p, lrow, row, lo, hi, (double)k, M, 1.0, s_radix);
      tau = value_of(lo);
    }
    if (use_p) {
      // the largest scale that keeps every sum of fixed-point weights (each <= 1) below 2^53
      const double fix = ldexp(1.0, 52 - (64 - __clzll(static_cast<unsigned long long>(C))));
      const unsigned t = radix_select<DT, VEC, true>(p, lrow, row, lo, hi, (double)tp, M, fix, s_radix);
      tau = value_of(t);
    }
  }
  if (threadIdx.x == 0) p.thresh[row] = tau;
}

template <int DT, bool VEC>
hipError_t launch_typed(const ThreshParams& p, hipStream_t s) {
  thresh_kernel<DT, VEC><<<dim3((unsigned)p.rows), dim3(kTB), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_thresholds(const ThreshParams& p, int logit_dtype, bool vec, hipStream_t s) {
  if (logit_dtype == kBF16) return vec ? launch_typed<kBF16, true>(p, s) : launch_typed<kBF16, false>(p, s);
  return vec ? launch_typed<kF32, true>(p, s) : launch_typed<kF32, false>(p, s);
}

}  // namespace sv
