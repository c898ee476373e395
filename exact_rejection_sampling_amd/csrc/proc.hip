// Keep thresholds of top-k and top-p (the pre-pass of spec_verify_chain_ex).
//
// One 512-thread block per row.  A token is a candidate when it is allowed and s = l + b (fp32) is
// finite; a candidate's key is an order-preserving map of s to 32 bits.
//  * top-k (k >= 1, fewer than k candidates: off): tau_k = the k-th largest key, with
//    multiplicity -- the largest key t with #{candidates with key >= t} >= k.
//  * top-p (0 < p < 1): among the candidates with key >= tau_k, with weights
//    w = 2^((s - max) * c2), tau_p = the largest key t whose mass {key >= t} reaches
//    p * (total mass): the smallest tie-closed set of top tokens whose probability reaches p.
// Counts are integers; masses are fp64 sums of fp32 weights 2^((s - ref) c2) (ref a value of
// the row, which cancels in every ratio), whose rounding (about 1e-16 relative per add) is
// far inside the 1e-5 relative window around a top-p boundary that parity tests exclude.
// First a sample of the row (one batch per thread, spread over it).  Window path (the usual
// one): from the sample, a value t_lo with about 2k candidates above it in the row (top-k),
// or about 3300 (top-p alone); one pass collects every candidate at or above t_lo, with its
// weight, into LDS and keeps only the count and weight of the rest; the thresholds are
// resolved inside the window (bins over it, then the deciding bin's candidates), which is
// used only when it provably holds them.  Full path (top-1, k above about 1600, or a window
// that overflows or misses): the sample fixes the range of 4096
// LDS bins linear in s; (1) one pass adds every candidate's count and weight to its bin
// (values outside the range go to the end bins) and finds the row's max, min and count; then
// for each selection the bin where the count or mass from the top reaches its target, (2) a
// pass that collects that bin's candidates into LDS, and an exact resolution among them.
// With both selections on, one collecting pass serves both whenever the top-p bin is fixed
// before tau_k is.  Top-1 keeps the maximum's ties whatever top-p is.  A bin with more than
// 1024 candidates (values piled on a few points) falls back to radix selection over the bits
// in which the candidate keys differ, 12 bits per pass, with fixed-point masses (each weight
// scaled by the largest power of two that keeps every sum below 2^53).  The row's threshold
// is tau_p when top-p is on (it is at least tau_k), else tau_k, or -inf.
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

// Elements per thread and loop step: kU vectors of 8, kTB * 8 elements apart, whose loads
// (logits, bias, mask words) are all issued before any is used -- one memory latency per
// step instead of one per vector.  (Deeper batches fit the 128 registers per thread but
// measured slower: the pass is bound by its per-element arithmetic and LDS atomics as much
// as by memory latency.)
#ifndef SPEC_THRESH_U
#define SPEC_THRESH_U 2
#endif
constexpr int kU = SPEC_THRESH_U;

// The candidates of this thread's kU vectors at e0, e0 + stride, ...: processed values
// (bias and mask applied, no threshold) and validity bits.
template <int DT, bool VEC>
__device__ __forceinline__ void cand_batch(const ThreshParams& p, const void* lrow, size_t row, long e0, long stride,
                                           float (&s)[kU][8], unsigned (&ok)[kU]) {
  Proc8In in[kU];
  if (VEC && e0 + (kU - 1) * stride + 8 <= p.V) {
    // every vector inside the row: raw loads only (the bias and mask branches are uniform),
    // then the arithmetic
    u32x4 w[kU];
    f32x4 f[kU][2], bl[kU], bh[kU];
    unsigned mw[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const long e = e0 + u * stride;
      if constexpr (DT == kBF16) {
        w[u] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(lrow) + e);
      } else {
        f[u][0] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(lrow) + e);
        f[u][1] = *(reinterpret_cast<const f32x4*>(static_cast<const float*>(lrow) + e) + 1);
      }
    }
    if (p.bias) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        bl[u] = *reinterpret_cast<const f32x4*>(p.bias + e0 + u * stride);
        bh[u] = *reinterpret_cast<const f32x4*>(p.bias + e0 + u * stride + 4);
      }
    }
    if (p.allowed) {
#pragma unroll
      for (int u = 0; u < kU; ++u) mw[u] = p.allowed[row * p.W + ((e0 + u * stride) >> 5)];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if constexpr (DT == kBF16) {
        s[u][0] = __uint_as_float(w[u].x << 16); s[u][1] = __uint_as_float(w[u].x & 0xffff0000u);
        s[u][2] = __uint_as_float(w[u].y << 16); s[u][3] = __uint_as_float(w[u].y & 0xffff0000u);
        s[u][4] = __uint_as_float(w[u].z << 16); s[u][5] = __uint_as_float(w[u].z & 0xffff0000u);
        s[u][6] = __uint_as_float(w[u].w << 16); s[u][7] = __uint_as_float(w[u].w & 0xffff0000u);
      } else {
        s[u][0] = f[u][0].x; s[u][1] = f[u][0].y; s[u][2] = f[u][0].z; s[u][3] = f[u][0].w;
        s[u][4] = f[u][1].x; s[u][5] = f[u][1].y; s[u][6] = f[u][1].z; s[u][7] = f[u][1].w;
      }
      // s = l + b in fp32 (b = 0 without a bias, as the verifier computes it); a candidate is
      // an allowed token with a finite s.  Masked tokens keep their raw value here: every
      // use of s other than the NaN / +inf fault test is guarded by the candidate bits.
      const float b[8] = {p.bias ? bl[u].x : 0.0f, p.bias ? bl[u].y : 0.0f, p.bias ? bl[u].z : 0.0f,
                          p.bias ? bl[u].w : 0.0f, p.bias ? bh[u].x : 0.0f, p.bias ? bh[u].y : 0.0f,
                          p.bias ? bh[u].z : 0.0f, p.bias ? bh[u].w : 0.0f};
      const long e = e0 + u * stride;
      const unsigned bits = p.allowed ? (mw[u] >> (e & 31)) & 0xffu : 0xffu;
      unsigned m = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        s[u][j] += b[j];
        if (__builtin_isfinite(s[u][j])) m |= 1u << j;
      }
      ok[u] = m & bits;
    }
    return;
  } else {
    ProcSpec pr{};
    pr.bias = p.bias;
    pr.allowed = p.allowed;
    pr.W = p.W;
#pragma unroll
    for (int u = 0; u < kU; ++u) load8<DT, VEC, false>(lrow, e0 + u * stride, p.V, s[u], -INFINITY);
#pragma unroll
    for (int u = 0; u < kU; ++u) proc8_load<VEC>(pr, row, e0 + u * stride, p.V, in[u]);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const long e = e0 + u * stride;
    proc8_apply<VEC>(in[u], -INFINITY, e, p.V, s[u]);
    unsigned m = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (e + j < p.V && s[u][j] > -INFINITY && s[u][j] < INFINITY) m |= 1u << j;   // false for NaN
    ok[u] = m;
  }
}

// 512 threads (8 waves) per row, at most 128 registers and about 73 KB of LDS, so that two
// blocks share a CU and a batch's rows (384 at the headline shape) run in one round on 256
// CUs rather than two (measured 4% faster than one 1024-thread block per CU).
#ifndef SPEC_THRESH_TB
#define SPEC_THRESH_TB 512
#endif
constexpr int kTB = SPEC_THRESH_TB;
constexpr int kTW = kTB / kWave;
constexpr int kDigit = 12;
constexpr int kBins = 1 << kDigit;
constexpr int kBinsPerThread = kBins / kTB;

// ------------------------------------------------------------------ lean streaming passes
// One thread's kU vectors of a batch lying wholly inside the row, loaded and not yet used:
// the logits (one 16-byte vector per 8 bf16, two per 8 fp32), the bias and the mask word.
template <int DT>
struct RawBatch {
  u32x4 l[kU][DT == kBF16 ? 1 : 2];
  f32x4 b[kU][2];
  unsigned m[kU];
};

// The loads of the batch at row position eb + lane * 8 (eb, a multiple of 32, is uniform over
// the wave): addresses are a uniform base plus a 32-bit lane offset, so that no load needs a
// 64-bit address register of its own.
template <int DT, bool BIAS, bool MASK>
__device__ __forceinline__ void load_raw(const ThreshParams& p, const void* lrow, size_t row, long eb, unsigned lane,
                                         long stride, RawBatch<DT>& r) {
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const long e = eb + u * stride;
    if constexpr (DT == kBF16) {
      r.l[u][0] = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(lrow) + e)[lane];
    } else {
      const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const float*>(lrow) + e);
      r.l[u][0] = q[2 * lane];
      r.l[u][1] = q[2 * lane + 1];
    }
    if constexpr (BIAS) {
      const f32x4* q = reinterpret_cast<const f32x4*>(p.bias + e);
      r.b[u][0] = q[2 * lane];
      r.b[u][1] = q[2 * lane + 1];
    }
    if constexpr (MASK) r.m[u] = (p.allowed + row * p.W + (e >> 5))[lane >> 2];
  }
}

// s = l + b of a loaded batch, and each vector's 8 allowed bits (all set without a mask).
// Nothing is tested here: NaN, +inf and masked tokens keep their values.
template <int DT, bool BIAS, bool MASK>
__device__ __forceinline__ void unpack_raw(const RawBatch<DT>& r, long e0, float (&s)[kU][8], unsigned (&al)[kU]) {
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    if constexpr (DT == kBF16) {
      const u32x4 w = r.l[u][0];
      s[u][0] = __uint_as_float(w.x << 16); s[u][1] = __uint_as_float(w.x & 0xffff0000u);
      s[u][2] = __uint_as_float(w.y << 16); s[u][3] = __uint_as_float(w.y & 0xffff0000u);
      s[u][4] = __uint_as_float(w.z << 16); s[u][5] = __uint_as_float(w.z & 0xffff0000u);
      s[u][6] = __uint_as_float(w.w << 16); s[u][7] = __uint_as_float(w.w & 0xffff0000u);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        s[u][4 * h + 0] = __uint_as_float(r.l[u][h].x); s[u][4 * h + 1] = __uint_as_float(r.l[u][h].y);
        s[u][4 * h + 2] = __uint_as_float(r.l[u][h].z); s[u][4 * h + 3] = __uint_as_float(r.l[u][h].w);
      }
    }
    if constexpr (BIAS) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        s[u][4 * h + 0] += r.b[u][h].x; s[u][4 * h + 1] += r.b[u][h].y;
        s[u][4 * h + 2] += r.b[u][h].z; s[u][4 * h + 3] += r.b[u][h].w;
      }
    }
    // e0 is a multiple of 8 and the vectors of a batch lie a multiple of 32 apart, so every
    // vector's 8 bits sit at the same place in its mask word
    al[u] = MASK ? (r.m[u] >> (e0 & 31)) & 0xffu : 0xffu;
  }
}

// v when bit j of the allowed bits is set, else -inf (two bit operations, no compare).
__device__ __forceinline__ float masked_value(float v, unsigned al, int j) {
  const unsigned t = static_cast<unsigned>(static_cast<int>(al << (31 - j)) >> 31);   // all ones if allowed
  return __uint_as_float((__float_as_uint(v) & t) | (0xff800000u & ~t));
}

// Streams the row once, wave w taking the batches at w * 512 + i * kTB * kU * 8.  Batches
// wholly inside the row go to fast(s, al, e0) -- s = l + b untested, al the allowed bits --
// from a ring of NBUF register buffers, each reloaded with the batch NBUF ahead as soon as it
// has been used, so that NBUF - 1 batches stay in flight while one is used; the rest go to
// slow(s, ok, e0) with cand_batch's candidate bits.
template <int DT, bool VEC, bool BIAS, bool MASK, int NBUF, class Fast, class Slow>
__device__ __forceinline__ void row_pass(const ThreshParams& p, const void* lrow, size_t row, Fast&& fast, Slow&& slow) {
  static_assert(NBUF >= 2, "at least one batch in flight");
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const unsigned ulane = static_cast<unsigned>(lane);
  const long stride = (long)kTB * kVec, step = stride * kU;
  long base = (long)wave * kWave * kVec;
  // a batch at `base` is wholly inside the row when base <= last_fast (uniform over the wave)
  const long last_fast = VEC ? (long)p.V - ((kWave - 1) * kVec + (kU - 1) * stride + kVec) : -1;
  // nf batches wholly inside the row, at base + t * step; the main loop takes NBUF of them per
  // trip with no exit in between (every trip runs the same straight line, so the compiler's
  // waits are exact), and the last nf mod NBUF follow it
  const int nf = base <= last_fast ? static_cast<int>((last_fast - base) / step) + 1 : 0;
  if (nf > 0) {
    const long first = base;
    // Rows start their walk at different batches (the shared bias row is read at different
    // places at once rather than every block on the same lines), and loads past the last
    // batch re-read it, which stays in bounds.
    const int rot = static_cast<int>((row * 7) % static_cast<size_t>(nf));
    auto pos = [&](int t) {
      int i = min(t, nf - 1) + rot;
      i = i >= nf ? i - nf : i;
      return first + static_cast<long>(i) * step;
    };
    RawBatch<DT> buf[NBUF];
    float s[kU][8];
    unsigned al[kU];
#pragma unroll
    for (int i = 0; i < NBUF; ++i) load_raw<DT, BIAS, MASK>(p, lrow, row, pos(i), ulane, stride, buf[i]);
    int t = 0;
    for (; t + NBUF <= nf; t += NBUF) {
#pragma unroll
      for (int i = 0; i < NBUF; ++i) {
        const long e0 = pos(t + i) + lane * kVec;
        unpack_raw<DT, BIAS, MASK>(buf[i], e0, s, al);
        fast(s, al, e0);
        // the buffer just used takes the batch NBUF ahead
        load_raw<DT, BIAS, MASK>(p, lrow, row, pos(t + i + NBUF), ulane, stride, buf[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < NBUF; ++i) {
      if (t + i < nf) {
        const long e0 = pos(t + i) + lane * kVec;
        unpack_raw<DT, BIAS, MASK>(buf[i], e0, s, al);
        fast(s, al, e0);
      }
    }
    base = first + static_cast<long>(nf) * step;
  }
  for (; base < p.V; base += step) {
    float s[kU][8];
    unsigned ok[kU];
    cand_batch<DT, VEC>(p, lrow, row, base + lane * kVec, stride, s, ok);
    slow(s, ok, base + lane * kVec);
  }
}

// Batches in flight per wave in the window pass and in the top-1 pass.
#ifndef SPEC_THRESH_NBUF_WIN
#define SPEC_THRESH_NBUF_WIN 2
#endif
#ifndef SPEC_THRESH_NBUF_TOP1
#define SPEC_THRESH_NBUF_TOP1 2
#endif

struct RadixLds {
  unsigned long long bin[kBins];        // counts, or masses in fixed point
  double scan[kTW];
  int digit;
  double f_above;
};

// The weight 2^((s - M) c2) in fixed point with 2^fe units, rounded to the nearest integer
// (ties to even).  w * 2^fe is exact in fp32 (a power-of-two scaling of a value in [0, 1],
// fe <= 52), so rounding it in fp32 and splitting it into two exact 32-bit halves gives
// the same integer as rounding the product in fp64.
__device__ __forceinline__ unsigned long long fixed_weight(float s, float M, float c2, int fe) {
  const float w = __builtin_amdgcn_exp2f((s - M) * c2);
  const float v = rintf(ldexpf(w, fe));
  const float hi = truncf(v * 0x1p-32f);
  const float lo = fmaf(hi, -0x1p32f, v);
  return (static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) | static_cast<unsigned>(lo);
}

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
// (MASS false) or the fixed-point mass (MASS true; weights in units of 2^-fe) of the
// candidates with key >= t; keys below klo are ignored.  [klo, khi] bounds the keys; the
// bits above their highest differing bit are shared.  `param` is the count target k, or the
// fraction p of the total mass F(klo) that the target is.  Every value stays an integer
// below 2^53, so the fp64 scans are exact.
template <int DT, bool VEC, bool MASS>
__device__ __forceinline__ unsigned radix_select(const ThreshParams& p, const void* lrow, size_t row, unsigned klo, unsigned khi,
                                 double param, float M, int fe, RadixLds& L) {
  const int tid = threadIdx.x;
  const int nb = (klo == khi) ? 0 : 32 - __clz(klo ^ khi);   // the varying low bits
  unsigned prefix = nb == 32 ? 0u : (klo >> nb);             // the digits chosen so far
  double above = 0.0;                                        // F just above the prefix's range
  double target = MASS ? -1.0 : param;
  for (int done = 0; done < nb;) {
    const int width = min(kDigit, nb - done), shift = nb - done - width;
    for (int j = tid; j < kBins; j += kTB) L.bin[j] = 0ull;
    __syncthreads();
    for (long e0 = (long)tid * kVec; e0 < p.V; e0 += (long)kTB * kVec * kU) {
      float s[kU][8];
      unsigned ok[kU];
      cand_batch<DT, VEC>(p, lrow, row, e0, (long)kTB * kVec, s, ok);
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (!((ok[u] >> e) & 1u)) continue;
          const unsigned k = key_of(s[u][e]);
          if (k < klo) continue;
          const unsigned high = shift + width == 32 ? 0u : (k >> (shift + width));
          if (high != prefix) continue;
          unsigned long long v = 1ull;
          if constexpr (MASS) v = fixed_weight(s[u][e], M, p.c2, fe);
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

// ------------------------------------------------------------------ value-bin selection
// The usual path: one pass adds every candidate into one of kBins bins linear in its value
// over [min, max] (counts, and fixed-point masses for top-p); the bin where the count or
// mass from the top reaches the target holds the threshold, and a second pass collects that
// bin's candidates into LDS, where the threshold is resolved exactly.  Linear bins spread a
// row's values evenly, so the LDS adds rarely collide (the first radix digit of the keys
// piles most of a row into a few dozen bins).  bin(s) is monotone in s, ties share a bin,
// and every count and mass is an integer sum, so the result is the radix selection's.  A
// bin with more than kCap candidates falls back to the radix selection.
constexpr int kCap = kTB >= 1024 ? 2048 : 1024;

struct BinLds {
  unsigned cnt[kBins];
  double mass[kBins];                   // fp64 sums of fp32 weights relative to the bins' reference
};
// The window path (below): every candidate at or above a value t_lo estimated from the
// sample, with its weight, collected in one pass; then bins over the window alone.
constexpr int kWinCap = 4096;
constexpr int kWinBins = 1024;
struct WinLds {
  float v[kWinCap];
  float w[kWinCap];                     // fp32 weights relative to the bins' reference (or 1)
  unsigned cnt[kWinBins];               // the sample's, then the window's, bin counts
  double mass[kWinBins];                // the window's bin masses
  int n;
};
union SelectLds {
  BinLds bins;
  RadixLds radix;
  WinLds win;
};
struct Collected {
  float v[kCap];
  double w[kCap];                       // the weights, relative to the bins' reference (or 1)
  int n;
};

// Bins linear in the value over [lo, lo + kBins / scale]; values outside fall into the end
// bins, so bin(s) stays monotone in s and ties share a bin.
struct ValueBins {
  float lo, scale;
  __device__ __forceinline__ int of(float s) const {
    return static_cast<int>(fminf(fmaxf((s - lo) * scale, 0.0f), static_cast<float>(kBins - 1)));
  }
};

// A candidate's top-p weight relative to the reference value ref: 2^((s - ref) c2) in fp32,
// accumulated in fp64.  The reference cancels in every mass ratio.
__device__ __forceinline__ double rel_weight(float s, float ref, float c2) {
  return (double)__builtin_amdgcn_exp2f((s - ref) * c2);
}

// Block-wide fp64 sum (every thread receives it).
__device__ __forceinline__ double block_sum_d(double v, double* scratch) {
  double tot;
  tb_excl_scan(v, scratch, &tot);
  return tot;
}

// The largest bin d whose F(d) = above + sum of val over bins >= d reaches `target` (block-
// wide; -1 if none): returns d and, in *f_above, F(d + 1).  Thread t owns kBinsPerThread
// consecutive bins, the highest to thread 0.
template <class Val, int NB = kBins>
__device__ __forceinline__ int find_bin(Val val, double above, double target, double* scratch, int* s_d, double* s_f, double* f_above) {
  constexpr int kBinsPerThread = NB / kTB;
  static_assert(NB % kTB == 0, "whole bins per thread");
  const int tid = threadIdx.x;
  const int d_hi = NB - 1 - tid * kBinsPerThread;
  double run = 0.0;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) run += val(d_hi - i);
  double tot;
  const double before = tb_excl_scan(run, scratch, &tot);
  if (tid == 0) *s_d = -1;
  __syncthreads();
  double f = above + before;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) {
    const double v = val(d_hi - i);
    if (f < target && f + v >= target) {   // one thread's run holds the crossing
      *s_d = d_hi - i;
      *s_f = f;
    }
    f += v;
  }
  __syncthreads();
  const int d = *s_d;
  *f_above = *s_f;
  __syncthreads();
  return d;
}

// Collects the candidates of bin d with their weights (fixed-point masses when fe >= 0);
// returns the number found (which may exceed kCap: then only kCap are stored).
template <int DT, bool VEC>
__device__ __forceinline__ int collect(const ThreshParams& p, const void* lrow, size_t row, const ValueBins& vb, int d, float ref,
                       bool weights, Collected& L) {
  if (threadIdx.x == 0) L.n = 0;
  __syncthreads();
  for (long e0 = (long)threadIdx.x * kVec; e0 < p.V; e0 += (long)kTB * kVec * kU) {
    float s[kU][8];
    unsigned ok[kU];
    cand_batch<DT, VEC>(p, lrow, row, e0, (long)kTB * kVec, s, ok);
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (!((ok[u] >> e) & 1u)) continue;
        if (s[u][e] < vb.lo || vb.of(s[u][e]) != d) continue;   // below the bins: in none
        const int i = atomicAdd(&L.n, 1);
        if (i < kCap) {
          L.v[i] = s[u][e];
          L.w[i] = weights ? rel_weight(s[u][e], ref, p.c2) : 1.0;
        }
      }
  }
  __syncthreads();
  const int n = L.n;
  __syncthreads();
  return n;
}

// collect() for two bins in one pass: d1's candidates into L1, d2's into L2; returns the
// count of d1 and leaves d2's in *n2.
template <int DT, bool VEC>
__device__ __forceinline__ int collect2(const ThreshParams& p, const void* lrow, size_t row, const ValueBins& vb, int d1, int d2,
                        float ref, Collected& L1, Collected& L2, int* n2) {
  if (threadIdx.x == 0) {
    L1.n = 0;
    L2.n = 0;
  }
  __syncthreads();
  for (long e0 = (long)threadIdx.x * kVec; e0 < p.V; e0 += (long)kTB * kVec * kU) {
    float s[kU][8];
    unsigned ok[kU];
    cand_batch<DT, VEC>(p, lrow, row, e0, (long)kTB * kVec, s, ok);
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (!((ok[u] >> e) & 1u) || s[u][e] < vb.lo) continue;
        const int d = vb.of(s[u][e]);
        if (d != d1 && d != d2) continue;
        Collected& L = d == d1 ? L1 : L2;
        const int i = atomicAdd(&L.n, 1);
        if (i < kCap) {
          L.v[i] = s[u][e];
          L.w[i] = rel_weight(s[u][e], ref, p.c2);
        }
      }
  }
  __syncthreads();
  const int n = L1.n;
  *n2 = L2.n;
  __syncthreads();
  return n;
}

// Among the n collected candidates (one bin) with value >= floor_v: the largest value t with
// above + the sum of w (mass) or the count over those with value >= t reaching `target`
// (-inf if none).  Ties share their sum, so the threshold never splits them.
__device__ __forceinline__ float resolve(const Collected& L, int n, float floor_v, bool mass, double above, double target,
                         float* scratch) {
  float best = -INFINITY;
  for (int i = threadIdx.x; i < n; i += kTB) {
    const float t = L.v[i];
    if (t < floor_v) continue;
    double f = above;
    for (int j = 0; j < n; ++j)
      if (L.v[j] >= t) f += mass ? L.w[j] : 1.0;
    if (f >= target) best = fmaxf(best, t);
  }
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const float wb = wave_max(best);
  if (lane == 0) scratch[wave] = wb;
  __syncthreads();
  float r = -INFINITY;
#pragma unroll
  for (int w = 0; w < kTW; ++w) r = fmaxf(r, scratch[w]);
  __syncthreads();
  return r;
}

// An empty asm hides a value from the compiler.
__device__ __forceinline__ float opaque(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// v[j] for a lane-varying j in [0, 8), by a select tree (no branch, no indexed registers:
// the values are hidden from the compiler first, which would otherwise turn the tree back
// into an indexed load from a stack copy of v).
__device__ __forceinline__ float pick8(const float (&v)[8], int j) {
  const bool b0 = j & 1, b1 = j & 2, b2 = j & 4;
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = opaque(v[i]);
  const float a0 = b0 ? x[1] : x[0], a1 = b0 ? x[3] : x[2], a2 = b0 ? x[5] : x[4], a3 = b0 ? x[7] : x[6];
  const float c0 = b1 ? a1 : a0, c1 = b1 ? a3 : a2;
  return b2 ? c1 : c0;
}

// Inclusive prefix sum of an int over the lanes of a wave (lanes that do not run add 0).
__device__ __forceinline__ int wave_incl_scan_i(int v) {
  v += dpp_i<0x111>(0, v);        // row_shr:1
  v += dpp_i<0x112>(0, v);        // row_shr:2
  v += dpp_i<0x114>(0, v);        // row_shr:4
  v += dpp_i<0x118>(0, v);        // row_shr:8
  v += dpp_i<0x142, 0xa>(0, v);   // row_bcast:15 into rows 1, 3
  v += dpp_i<0x143, 0xc>(0, v);   // row_bcast:31 into rows 2, 3
  return v;
}

// The window path's pass over the row: every candidate with s >= t_cmp (t_cmp finite, so -inf
// and NaN never qualify) is appended to the window with its weight (1 without top-p); with
// PALONE, the weights of the allowed tokens below t_cmp are summed into *low.  A NaN or +inf
// anywhere in the row sets *fault.  Per element the fast batches spend the bf16 unpack, the
// bias add, one class test and one compare (with PALONE also the mask applied to the value,
// and the weight): the mask is applied to a vector's 8 hit bits at once.
template <int DT, bool VEC, bool BIAS, bool MASK, bool PALONE>
__device__ __forceinline__ void window_pass(const ThreshParams& p, const void* lrow, size_t row, float t_cmp, float ref,
                                            bool use_p, WinLds& W, bool* fault_out, double* low_out) {
  const int lane = threadIdx.x & (kWave - 1);
  // weights 2^(s c2 - fp32(ref c2)): the rounding of ref c2 scales every weight of the row
  // alike, so it cancels in every mass ratio; one fma per weight
  const float c2 = p.c2, rc2 = ref * c2;
  bool fault = false;
  double low_mass = 0.0;
  // this thread's hits (bit 8u + j: element j of vector u) appended to the window, the
  // wave's places taken with one LDS atomic
  auto append = [&](const float (&s)[kU][8], unsigned hit) {
    const int mine = __popc(hit);
    if (!__ballot(mine > 0)) return;
    const int incl = wave_incl_scan_i(mine);
    int at = 0;
    if (lane == kWave - 1) at = atomicAdd(&W.n, incl);
    at = __builtin_amdgcn_readlane(at, kWave - 1) + incl - mine;
    // the lanes' few hits (usually none or one per lane), each value picked out of its
    // vector by a select tree rather than one branch per position
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      unsigned h = (hit >> (8 * u)) & 0xffu;
      while (h) {
        const int j = __builtin_ctz(h);
        h &= h - 1u;
        const float v = pick8(s[u], j);
        if (at < kWinCap) {
          W.v[at] = v;
          W.w[at] = use_p ? __builtin_amdgcn_exp2f(fmaf(v, c2, -rc2)) : 1.0f;
        }
        ++at;
      }
    }
  };
  row_pass<DT, VEC, BIAS, MASK, SPEC_THRESH_NBUF_WIN>(
      p, lrow, row,
      [&](const float (&s)[kU][8], const unsigned (&al)[kU], long) {
        unsigned hit = 0u;
        float lw = 0.0f;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          unsigned hb = 0u;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            fault |= !(s[u][j] < INFINITY);   // NaN or +inf, masked or not
            if constexpr (PALONE) {
              const float v = MASK ? masked_value(s[u][j], al[u], j) : s[u][j];
              const bool in = v >= t_cmp;
              hb |= (in ? 1u : 0u) << j;
              lw += in ? 0.0f : __builtin_amdgcn_exp2f(fmaf(v, c2, -rc2));   // 0 for -inf
            } else {
              hb |= (s[u][j] >= t_cmp ? 1u : 0u) << j;
            }
          }
          if constexpr (!PALONE && MASK) hb &= al[u];
          hit |= hb << (8 * u);
        }
        if constexpr (PALONE) low_mass += (double)lw;
        append(s, hit);
      },
      [&](const float (&s)[kU][8], const unsigned (&ok)[kU], long) {
        unsigned hit = 0u;
        float lw = 0.0f;
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            fault |= !(s[u][j] < INFINITY);   // positions past the row read as -inf
            const bool c = (ok[u] >> j) & 1u;
            const bool in = c && s[u][j] >= t_cmp;
            hit |= (in ? 1u : 0u) << (8 * u + j);
            if (PALONE && c && !in) lw += __builtin_amdgcn_exp2f(fmaf(s[u][j], c2, -rc2));
          }
        if constexpr (PALONE) low_mass += (double)lw;
        append(s, hit);
      });
  *fault_out = fault;
  *low_out = low_mass;
}

template <int DT, bool VEC>
__device__ __forceinline__ void window_pass_any(const ThreshParams& p, const void* lrow, size_t row, float t_cmp,
                                                float ref, bool use_p, bool p_alone, WinLds& W, bool* fault,
                                                double* low) {
  if (p.bias) {
    if (p.allowed) {
      if (p_alone) window_pass<DT, VEC, true, true, true>(p, lrow, row, t_cmp, ref, use_p, W, fault, low);
      else window_pass<DT, VEC, true, true, false>(p, lrow, row, t_cmp, ref, use_p, W, fault, low);
    } else {
      if (p_alone) window_pass<DT, VEC, true, false, true>(p, lrow, row, t_cmp, ref, use_p, W, fault, low);
      else window_pass<DT, VEC, true, false, false>(p, lrow, row, t_cmp, ref, use_p, W, fault, low);
    }
  } else {
    if (p.allowed) {
      if (p_alone) window_pass<DT, VEC, false, true, true>(p, lrow, row, t_cmp, ref, use_p, W, fault, low);
      else window_pass<DT, VEC, false, true, false>(p, lrow, row, t_cmp, ref, use_p, W, fault, low);
    } else {
      if (p_alone) window_pass<DT, VEC, false, false, true>(p, lrow, row, t_cmp, ref, use_p, W, fault, low);
      else window_pass<DT, VEC, false, false, false>(p, lrow, row, t_cmp, ref, use_p, W, fault, low);
    }
  }
}

// The window path.  It wants the top 2k candidates (at least k + 256) for top-k (top-p then
// works among the top-k survivors), or the largest window (about 3300) for top-p alone, and
// from the sample (each thread's batch smp at smp_e0) takes t_lo, a value with about that
// many candidates above it in the row.  One pass collects every candidate at or above t_lo,
// with its weight, into LDS (wave-aggregated appends) and keeps only the count and weight of
// the rest.  The thresholds are then resolved over the window exactly as the full path
// resolves them over the row (bins, then the deciding bin's candidates), and the window is
// used only when it provably holds them: at least k candidates for top-k, the target mass
// reached inside it for top-p.  Returns false -- the full path then runs -- when the window
// cannot hold 2k, overflows, or misses.  On true, *tau_out is the row's threshold (-inf for
// a faulty row or no candidates).
template <int DT, bool VEC>
__device__ __forceinline__ bool window_select(const ThreshParams& p, const void* lrow, size_t row, int k, float tp, bool use_k,
                              bool use_p, const float (&smp)[kU][8], const unsigned (&smp_ok)[kU], long smp_e0,
                              long smp_stride, float SM, float SMN, WinLds& W, Collected& C1, Collected& C2, double* s_scratch,
                              float* s_m, float* s_mn, int* s_fault, int* s_d, double* s_f, float* tau_out) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
  const float ref = SM;                 // the weights' reference value
  // 1. the sample's counts in bins linear over [SMN, SM]
  const float sscale = static_cast<float>(kWinBins) / (SM - SMN);
  if (!(isfinite(sscale) && sscale > 0.0f)) return false;
  auto sbin = [&](float v) {
    return static_cast<int>(fminf(fmaxf((v - SMN) * sscale, 0.0f), static_cast<float>(kWinBins - 1)));
  };
  const bool p_alone = use_p && !use_k;
  for (int j = tid; j < kWinBins; j += kTB) W.cnt[j] = 0u;
  __syncthreads();
  int npos = 0;                         // sampled positions inside the row
#pragma unroll
  for (int u = 0; u < kU; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (smp_e0 + u * smp_stride + e < p.V) ++npos;
      if ((smp_ok[u] >> e) & 1u) atomicAdd(&W.cnt[sbin(smp[u][e])], 1u);
    }
  const double S_pos = block_sum_d(static_cast<double>(npos), s_scratch);   // (its barriers end the adds)
  double fa;
  // 2. candidates wanted from the top of the row: for top-k, 2k (at least k + 256); for
  //    top-p alone the largest window, since an estimate of the nucleus from the sample rests
  //    on the few sampled values that carry its mass and errs either way by large factors
  //    (a window that misses is detected after the pass and falls back)
  const double room = 0.8 * kWinCap;
  const double want = p_alone ? room : fmax(2.0 * k, k + 256.0);
  if (!(want <= room)) return false;
  // 3. t_lo: the lower edge of the sample bin where the sample's count from the top reaches
  //    want scaled to the sample (every candidate when the sample has fewer)
  {
    auto scnt = [&](int d) { return d >= 0 ? (double)W.cnt[d] : 0.0; };
    const double r = fmax(1.0, ceil(want * S_pos / (double)p.V));
    const int bw = find_bin<decltype(scnt), kWinBins>(scnt, 0.0, r, s_scratch, s_d, s_f, &fa);
    const float t_lo = bw <= 0 ? -INFINITY : SMN + static_cast<float>(bw) / sscale;
    // 4. the pass: the window into LDS, the rest weighed in registers (top-p alone)
    if (tid == 0) W.n = 0;
    __syncthreads();
    SPEC_STAMP(p, 4, 2);   // window chosen
    bool fault = false;
    double low_mass = 0.0;
    window_pass_any<DT, VEC>(p, lrow, row, fmaxf(t_lo, -0x1.fffffep127f), ref, use_p, p_alone, W, &fault, &low_mass);
    if (fault) *s_fault = 1;
    __syncthreads();
    const int n = W.n;
    SPEC_STAMP(p, 4, 3);   // window pass done
    const double W_low = p_alone ? block_sum_d(low_mass, s_scratch) : 0.0;   // (its barriers order n's read)
    if (*s_fault) {                     // the verifier reports the row; no threshold is needed
      *tau_out = -INFINITY;
      return true;
    }
    // With t_lo = -inf the window holds every candidate; otherwise the row may hold more.
    const bool all_in = !(t_lo > -INFINITY);
    if (n == 0) {
      if (!all_in) return false;
      *tau_out = -INFINITY;             // no candidate at all
      return true;
    }
    if (n > kWinCap) return false;
    // top-k selects when the row has more than k candidates: known when the window holds them
    // all; otherwise a window of at least k holds the top k (fewer: the full path decides)
    if (use_k && !all_in && n < k) return false;
    const bool sel_k = use_k && (!all_in || k < n);
    // 5. bins linear over the window [wlo, M] (M, the row's largest candidate, is in it: the
    //    window path runs only when the sample holds two distinct values, so t_lo <= SM <= M)
    float lo_v = INFINITY, hi_v = -INFINITY;
    for (int j = tid; j < n; j += kTB) {
      lo_v = fminf(lo_v, W.v[j]);
      hi_v = fmaxf(hi_v, W.v[j]);
    }
    const float wlo_w = -wave_max(-lo_v), whi_w = wave_max(hi_v);
    if (lane == 0) {
      s_mn[wave] = wlo_w;
      s_m[wave] = whi_w;
    }
    __syncthreads();
    float wlo = INFINITY, M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kTW; ++w) {
      wlo = fminf(wlo, s_mn[w]);
      M = fmaxf(M, s_m[w]);
    }
    __syncthreads();
    if (!((M - ref) * p.c2 < 64.0f)) return false;
    const float wscale = static_cast<float>(kWinBins) / (M - wlo);
    if (!(n > 0 && M > wlo && isfinite(wscale) && wscale > 0.0f)) return false;
    auto wbin = [&](float v) {
      return static_cast<int>(fminf(fmaxf((v - wlo) * wscale, 0.0f), static_cast<float>(kWinBins - 1)));
    };
    for (int j = tid; j < kWinBins; j += kTB) {
      W.cnt[j] = 0u;
      W.mass[j] = 0.0;
    }
    __syncthreads();
    for (int j = tid; j < n; j += kTB) {
      const int d = wbin(W.v[j]);
      atomicAdd(&W.cnt[d], 1u);
      if (use_p) atomicAdd(&W.mass[d], (double)W.w[j]);
    }
    __syncthreads();
    SPEC_STAMP(p, 4, 4);   // window binned
    // the candidates of window bin d into L (n_d of them; false if more than kCap)
    auto gather = [&](int d, Collected& L) -> int {
      if (tid == 0) L.n = 0;
      __syncthreads();
      for (int j = tid; j < n; j += kTB) {
        if (wbin(W.v[j]) != d) continue;
        const int i = atomicAdd(&L.n, 1);
        if (i < kCap) {
          L.v[i] = W.v[j];
          L.w[i] = (double)W.w[j];
        }
      }
      __syncthreads();
      const int nd = L.n;
      __syncthreads();
      return nd;
    };
    float tau = -INFINITY, tau_k = -INFINITY;
    int dk = -1, nk = 0;
    if (sel_k) {
      double fk = 0.0;
      auto wcnt = [&](int d) { return d >= 0 ? (double)W.cnt[d] : 0.0; };
      dk = find_bin<decltype(wcnt), kWinBins>(wcnt, 0.0, (double)k, s_scratch, s_d, s_f, &fk);
      if (dk < 0) return false;
      nk = gather(dk, C1);
      if (nk > kCap) return false;
      tau_k = resolve(C1, nk, -INFINITY, false, fk, (double)k, s_m);
      tau = tau_k;
    }
    SPEC_STAMP(p, 4, 5);   // top-k resolved
    if (use_p) {
      // survivors of top-k: every window candidate above bin dk and those of bin dk at or
      // above tau_k; without top-k every candidate, those below the window too
      double part = 0.0;
      if (sel_k)
        for (int i = tid; i < nk; i += kTB)
          if (C1.v[i] >= tau_k) part += C1.w[i];
      part = block_sum_d(part, s_scratch);
      auto valp = [&](int d) -> double {
        if (d < 0 || (sel_k && d < dk)) return 0.0;
        return (sel_k && d == dk) ? part : W.mass[d];
      };
      double t = 0.0;
      for (int d = tid; d < kWinBins; d += kTB) t += valp(d);
      const double total = block_sum_d(t, s_scratch) + W_low;
      const double target = (double)tp * total;
      double fp = 0.0;
      const int dp = find_bin<decltype(valp), kWinBins>(valp, 0.0, target, s_scratch, s_d, s_f, &fp);
      if (dp < 0) return false;         // the target mass lies below the window
      if (sel_k && dp == dk) {
        tau = resolve(C1, nk, tau_k, true, fp, target, s_m);
      } else {
        const int np = gather(dp, C2);
        if (np > kCap) return false;
        tau = resolve(C2, np, -INFINITY, true, fp, target, s_m);
      }
    }
    SPEC_STAMP(p, 4, 6);   // top-p resolved
    // every kept token (a candidate with s >= tau, tau a window value) is in the window:
    // its summary spares the statistics pass the row
    if (p.summ && tau > -INFINITY) {
      const float R = M * p.c2;
      double z = 0.0;
      for (int j = tid; j < n; j += kTB)
        if (W.v[j] >= tau) z += (double)__builtin_amdgcn_exp2f(fmaf(W.v[j], p.c2, -R));
      z = block_sum_d(z, s_scratch);
      if (tid == 0) p.summ[row] = make_float2(M, static_cast<float>(z));
    }
    *tau_out = tau;
    return true;
  }
}

// The full path: bins over the value range near the top of the row, counted and weighed in
// one pass, the deciding bins' candidates collected in another, and radix selection for
// rows the bins cannot decide.  The window path's fallback; kept out of line so that its
// registers do not add to the window path's.
template <int DT, bool VEC>
__attribute__((noinline)) __device__ float full_select(const ThreshParams p, const void* lrow, size_t row, int k,
                                                       float tp, bool use_k, bool use_p, float SM, float SMN,
                                                       SelectLds& s_sel, Collected& s_col, Collected& s_col2,
                                                       double* s_scratch, float* s_m, float* s_mn, int* s_fault_p,
                                                       int* s_d_p, double* s_f_p) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const long step = (long)kTB * kVec * kU;
  const float ref = SM;                 // the weights' reference value
  int& s_fault = *s_fault_p;
  int& s_d = *s_d_p;
  double& s_f = *s_f_p;
  float tau = -INFINITY;
  // Only values near the top can hold a threshold: the bins cover [lo, SM] with lo the
  // sample's minimum or, if higher, the cut SM - cut / c2, below which a weight is under
  // 2^-cut.  Top-p keeps a set whose mass reaches p of the total, and the candidates below
  // the cut weigh less than V 2^-cut <= (1 - p) / 8 of a total of at least 1 (the sample's
  // maximum weighs 1), so its threshold lies above the cut; the k-th largest for top-k lies
  // there whenever at least k candidates do.  Candidates below lo go to two running sums
  // (count and weight) instead of the bins; a row whose threshold falls below lo after all
  // takes the radix selection.
  const float q1 = use_p ? 1.0f - tp : 1.0f;
  const float cut = fmaxf(24.0f, ceilf(log2f(8.0f * static_cast<float>(p.V) / q1)));
  ValueBins vb;
  vb.lo = fmaxf(SMN, SM - cut / p.c2);
  vb.scale = static_cast<float>(kBins) / (SM - vb.lo);
  // (top-1 keeps the maximum's ties whatever top-p is: no bins needed)
  const bool binned = !(use_k && k == 1) && SM > vb.lo && isfinite(SM - vb.lo) && isfinite(vb.scale) &&
                      vb.scale > 0.0f;
  BinLds& L = s_sel.bins;
  if (binned) {
    for (int j = threadIdx.x; j < kBins; j += kTB) {
      L.cnt[j] = 0u;
      L.mass[j] = 0.0;
    }
  }
  __syncthreads();
  float m = -INFINITY, mn = INFINITY;
  unsigned cnt = 0u;
  double low_mass = 0.0;
  bool fault = false;
  for (long e0 = (long)threadIdx.x * kVec; e0 < p.V; e0 += step) {
    float s[kU][8];
    unsigned ok[kU];
    cand_batch<DT, VEC>(p, lrow, row, e0, (long)kTB * kVec, s, ok);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        fault |= !(s[u][e] < INFINITY);      // NaN or +inf; positions past the row read as -inf
        const bool c = (ok[u] >> e) & 1u;
        m = fmaxf(m, c ? s[u][e] : -INFINITY);
        mn = fminf(mn, c ? s[u][e] : INFINITY);
        if (binned && c) {
          if (s[u][e] >= vb.lo) {
            const int d = vb.of(s[u][e]);
            if (use_k) atomicAdd(&L.cnt[d], 1u);
            if (use_p) atomicAdd(&L.mass[d], rel_weight(s[u][e], ref, p.c2));
          } else {
            if (use_p) low_mass += rel_weight(s[u][e], ref, p.c2);
          }
        }
      }
      cnt += __popc(ok[u]);
    }
  }
  if (fault) s_fault = 1;
  const float wm = wave_max(m);
  const float wmn = -wave_max(-mn);
  const double wc = wave_sum_d(static_cast<double>(cnt));
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
  // the weight of the candidates below the bins
  const double W_low = use_p ? block_sum_d(low_mass, s_scratch) : 0.0;
  SPEC_STAMP(p, 4, 2);   // sample and fused pass done
  SPEC_STAMP(p, 4, 3);
  if (!s_fault && C > 0.0) {
    const bool sel_k = use_k && (double)k < C;
    // the radix fallback's fixed point: the largest scale that keeps every sum of weights
    // (each <= 1) below 2^53
    const int fe = use_p ? 52 - (64 - __clzll(static_cast<unsigned long long>(C))) : -1;
    // a candidate far above the sample's maximum would overflow its fp32 weight
    bool fast = binned && (!use_p || (M - ref) * p.c2 < 64.0f);
    float tau_k = -INFINITY;
    if (M == MN || (sel_k && k == 1)) {
      // one distinct value, or top-1: the kept set is the maximum's ties whatever top-p is
      tau = M;
      fast = true;
    } else if (fast) {
      int dk = -1, n = 0, dpf = -1, n2 = 0;
      double fk = 0.0;
      if (sel_k) {
        // (dk < 0 when fewer than k candidates lie in the bins: then the radix selection)
        dk = find_bin([&](int d) { return d >= 0 ? (double)L.cnt[d] : 0.0; }, 0.0, (double)k, s_scratch, &s_d, &s_f, &fk);
        if (dk >= 0 && use_p) {
          // The top-p target is p * (A + part), A the mass of the bins above dk and part the
          // mass of bin dk's survivors (0 <= part <= mass[dk], known only after tau_k).  When
          // the targets for both ends fall in the same bin above dk, that bin is collected in
          // the same pass as dk (the running mass is monotone in the bin, so the true
          // target's bin lies between the two).
          double A = 0.0;
          for (int d = threadIdx.x; d < kBins; d += kTB)
            if (d > dk) A += (double)L.mass[d];
          A = block_sum_d(A, s_scratch);
          const double mdk = (double)L.mass[dk];
          double f0 = 0.0, f1 = 0.0;
          const int d0 = find_bin([&](int d) { return d > dk ? (double)L.mass[d] : 0.0; }, 0.0, (double)tp * A,
                                  s_scratch, &s_d, &s_f, &f0);
          const int d1 = find_bin([&](int d) { return d > dk ? (double)L.mass[d] : (d == dk ? mdk : 0.0); }, 0.0,
                                  (double)tp * (A + mdk), s_scratch, &s_d, &s_f, &f1);
          if (d0 > dk && d1 == d0) dpf = d0;
        }
        if (dk >= 0) {
          if (dpf >= 0) n = collect2<DT, VEC>(p, lrow, row, vb, dk, dpf, ref, s_col, s_col2, &n2);
          else n = collect<DT, VEC>(p, lrow, row, vb, dk, ref, use_p, s_col);
        }
        SPEC_STAMP(p, 4, 4);   // collected
        SPEC_TRACE_ONLY(trace_word(p.trace, 4, blockIdx.x, 10, (unsigned)n | ((unsigned long long)n2 << 32)));
        if (dk < 0 || n > kCap) fast = false;
        else tau_k = resolve(s_col, n, -INFINITY, false, fk, (double)k, s_m);
        tau = tau_k;
        SPEC_STAMP(p, 4, 5);   // top-k resolved
      }
      if (fast && use_p) {
        // survivors of top-k: every candidate above bin dk, and those of bin dk at or above
        // tau_k (collected); their total mass fixes the target
        double part = 0.0, total = 0.0;
        if (sel_k)
          for (int i = threadIdx.x; i < n; i += kTB)
            if (s_col.v[i] >= tau_k) part += s_col.w[i];
        part = block_sum_d(part, s_scratch);
        auto valp = [&](int d) -> double {
          if (d < 0 || (sel_k && d < dk)) return 0.0;
          return (sel_k && d == dk) ? part : (double)L.mass[d];
        };
        {
          double t = 0.0;
          for (int d = threadIdx.x; d < kBins; d += kTB) t += valp(d);
          // without top-k every candidate survives, those below the bins too
          total = block_sum_d(t, s_scratch) + (sel_k ? 0.0 : W_low);
        }
        const double target = (double)tp * total;
        double fp = 0.0;
        const int dp = find_bin(valp, 0.0, target, s_scratch, &s_d, &s_f, &fp);
        if (dp < 0) {
          fast = false;
        } else if (sel_k && dp == dk) {
          tau = resolve(s_col, n, tau_k, true, fp, target, s_m);
        } else if (dp == dpf) {          // collected with bin dk
          if (n2 > kCap) fast = false;
          else tau = resolve(s_col2, n2, -INFINITY, true, fp, target, s_m);
        } else {
          const int n2 = collect<DT, VEC>(p, lrow, row, vb, dp, ref, true, s_col);
          if (n2 > kCap) fast = false;
          else tau = resolve(s_col, n2, -INFINITY, true, fp, target, s_m);
        }
      }
    }
    SPEC_STAMP(p, 4, 6);   // binned path done
    if (!fast) {
      SPEC_TRACE_ONLY(trace_word(p.trace, 4, blockIdx.x, 11, 1ull));   // radix path taken
      // radix selection (also for rows whose values cannot be binned)
      unsigned lo = key_of(MN);
      const unsigned hi = key_of(M);
      if (sel_k) {
        lo = radix_select<DT, VEC, false>(p, lrow, row, lo, hi, (double)k, M, -1, s_sel.radix);
        tau = value_of(lo);
      }
      if (use_p) {
        const unsigned t = radix_select<DT, VEC, true>(p, lrow, row, lo, hi, (double)tp, M, fe, s_sel.radix);
        tau = value_of(t);
      }
    }
  }
  return tau;
}

// Top-1 keeps the row's largest candidate value and its ties, whatever top-p is: one pass
// for the largest allowed value and any NaN / +inf.
template <int DT, bool VEC, bool BIAS, bool MASK>
__device__ __forceinline__ void top1_pass(const ThreshParams& p, const void* lrow, size_t row, float* m_out,
                                          float* m2_out, bool* fault_out) {
  // the lane's two largest values with multiplicity: m2 == m when its largest is tied
  float m = -INFINITY, m2 = -INFINITY;
  bool fault = false;
  auto see = [&](float v) {
    m2 = fmaxf(m2, fminf(v, m));
    m = fmaxf(m, v);
  };
  row_pass<DT, VEC, BIAS, MASK, SPEC_THRESH_NBUF_TOP1>(
      p, lrow, row,
      [&](const float (&s)[kU][8], const unsigned (&al)[kU], long) {
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            fault |= !(s[u][j] < INFINITY);
            see(MASK ? masked_value(s[u][j], al[u], j) : s[u][j]);
          }
      },
      [&](const float (&s)[kU][8], const unsigned (&ok)[kU], long) {
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            fault |= !(s[u][j] < INFINITY);
            see(((ok[u] >> j) & 1u) ? s[u][j] : -INFINITY);
          }
      });
  *m_out = m;
  *m2_out = m2;
  *fault_out = fault;
}

// The top-1 threshold: the largest candidate, or -inf for a faulty row or one without
// candidates.  The kept set is the largest value's ties; when the largest value is unique
// its summary (M, 2^(M c2 - fp32(M c2))) is written for the statistics pass (a row with a
// tied maximum is left to that pass).
template <int DT, bool VEC>
__device__ __forceinline__ float top1_select(const ThreshParams& p, const void* lrow, size_t row, float* s_m,
                                             double* s_scratch, int* s_fault) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  float m, m2;
  bool fault;
  if (p.bias) {
    if (p.allowed) top1_pass<DT, VEC, true, true>(p, lrow, row, &m, &m2, &fault);
    else top1_pass<DT, VEC, true, false>(p, lrow, row, &m, &m2, &fault);
  } else {
    if (p.allowed) top1_pass<DT, VEC, false, true>(p, lrow, row, &m, &m2, &fault);
    else top1_pass<DT, VEC, false, false>(p, lrow, row, &m, &m2, &fault);
  }
  if (fault) *s_fault = 1;
  const float wm = wave_max(m);
  if (lane == 0) s_m[wave] = wm;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kTW; ++w) M = fmaxf(M, s_m[w]);
  const bool none = *s_fault || !(M > -INFINITY);
  if (p.summ && !none) {                // block-uniform
    // copies of M: 2 stands for "two or more" in a lane
    const double c = block_sum_d(m == M ? (m2 == M ? 2.0 : 1.0) : 0.0, s_scratch);
    if (threadIdx.x == 0 && c == 1.0)
      p.summ[row] = make_float2(M, __builtin_amdgcn_exp2f(fmaf(M, p.c2, -(M * p.c2))));
  }
  return none ? -INFINITY : M;
}

// Rows in order of cost, heaviest first: 0 top-p alone (a weight per element), 1 top-k
// with k >= 2, 2 top-1, 3 neither (nothing to do).
__device__ __forceinline__ int row_cost_class(const ThreshParams& p, int b) {
  const int k = p.top_k ? p.top_k[b] : 0;
  const float tp = p.top_p ? p.top_p[b] : 1.0f;
  const bool use_k = k >= 1, use_p = tp > 0.0f && tp < 1.0f;
  if (!use_k) return use_p ? 0 : 3;
  return k == 1 ? 2 : 1;
}

// The row block j takes when there are more rows than CUs but at most two per CU.  Sorted by
// cost class, then request, then row, the rows are dealt so that the blocks that share a CU
// (those below rows - CUs, and those from CUs up, as the dispatcher fills each CU once before
// any twice) take the rows after the heaviest CUs - (rows - CUs): the heaviest rows run alone
// and a shared CU pairs a middle row with one of the lightest.  A
// bijection on [0, rows): any row order gives the same thresholds.  Wave 0 computes it
// from every request's top-k and top-p; the others wait at the barrier.
__device__ size_t balanced_row(const ThreshParams& p, unsigned j, long* s_row) {
  if (threadIdx.x < kWave) {
    constexpr int kKept = 4;          // the classes of the first 4 * 64 requests stay in registers
    const int lane = threadIdx.x;
    const int R = p.R, B = p.rows / R;
    int kept[kKept];
    long cnt[4] = {0, 0, 0, 0};       // requests per class
#pragma unroll
    for (int t = 0; t < kKept; ++t) {
      const int b = t * kWave + lane;
      kept[t] = b < B ? row_cost_class(p, b) : 4;
    }
    for (int b0 = 0; b0 < B; b0 += kWave) {
      const int t = b0 / kWave, b = b0 + lane;
      int c = 4;
#pragma unroll
      for (int u = 0; u < kKept; ++u)
        if (t == u) c = kept[u];
      if (t >= kKept && b < B) c = row_cost_class(p, b);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) cnt[cc] += __popcll(__ballot(c == cc));
    }
    const long rows = p.rows, cus = p.cus, d = rows - cus;   // d: CUs that hold two rows
    long srt = j;                     // j's place in the sorted order (the second of a pair)
    if (j >= d && j < cus) srt = j - d;              // alone on a CU: the heaviest rows
    else if (j < d) srt = cus - d + j;               // first of a pair
    int c = 0;
    long base = 0;
    while (c < 3 && srt >= base + cnt[c] * R) {
      base += cnt[c] * R;
      ++c;
    }
    const long q = srt - base, want = q / R;          // the want-th request of class c
    long seen = 0, req = 0;
    for (int b0 = 0; b0 < B; b0 += kWave) {
      const int t = b0 / kWave, b = b0 + lane;
      int cb = 4;
#pragma unroll
      for (int u = 0; u < kKept; ++u)
        if (t == u) cb = kept[u];
      if (t >= kKept && b < B) cb = row_cost_class(p, b);
      unsigned long long m = __ballot(cb == c);
      const long n = __popcll(m);
      if (seen + n > want) {
        for (long i = seen; i < want; ++i) m &= m - 1ull;   // drop the set bits before it
        req = b0 + __ffsll(static_cast<long long>(m)) - 1;
        break;
      }
      seen += n;
    }
    if (lane == 0) *s_row = req * R + q % R;
  }
  __syncthreads();
  return static_cast<size_t>(*s_row);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kTB, kTB >= 1024 ? 1 : 4) void thresh_kernel(ThreshParams p) {
  __shared__ double s_scratch[kTW];
  __shared__ SelectLds s_sel;
  __shared__ Collected s_col, s_col2;
  __shared__ float s_m[kTW], s_mn[kTW];
  __shared__ int s_fault, s_d;
  __shared__ double s_f;
  __shared__ long s_row;
  SPEC_STAMP(p, 4, 1);
  // the shared-CU order only where some CUs hold two rows (then at most 2 * CUs rows, so the
  // mapping reads at most that many requests' top-k and top-p)
  const size_t row =
      p.cus > 0 && p.rows > p.cus && p.rows <= 2 * p.cus ? balanced_row(p, blockIdx.x, &s_row) : blockIdx.x;
  const int b = static_cast<int>(row / p.R);
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const void* lrow = row_ptr<DT>(p.logits, row, p.V);
  // This thread's sample batch, for the window path's estimate, is read first, with the
  // request's top-k and top-p in flight beside it: eight consecutive threads read one stretch
  // of 64 tokens (whole 128-byte lines of bf16 logits), and the block's kTB / 8 * kU stretches
  // are spread evenly over the row, at a row-dependent offset (so that the rows' reads of the
  // shared bias row spread over its lines).  Rows that need no sample waste one batch.
  const long stretches = (p.V + 63) / 64;
  const long gap = max(1L, stretches / ((long)(kTB / 8) * kU));
  const long smp_e0 =
      ((long)(threadIdx.x >> 3) * gap + (long)(row % (size_t)gap)) * 64 + (long)(threadIdx.x & 7) * kVec;
  const long smp_stride = (long)(kTB / 8) * gap * 64;
  float smp[kU][8];
  unsigned smp_ok[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) smp_ok[u] = 0u;
  if (smp_e0 < p.V) cand_batch<DT, VEC>(p, lrow, row, smp_e0, smp_stride, smp, smp_ok);
  const int k = p.top_k ? p.top_k[b] : 0;
  const float tp = p.top_p ? p.top_p[b] : 1.0f;
  const bool use_k = k >= 1, use_p = tp > 0.0f && tp < 1.0f;   // false for NaN
  SPEC_TAG(p, 4, SPEC_TRACE_TAG((use_k ? 1 : 0) | (use_p ? 2 : 0), row, k));
  SPEC_TRACE_ONLY(trace_word(p.trace, 4, blockIdx.x, 9, __float_as_uint(tp)));
  // where the block runs: XCC, then shader engine, shader array and CU (a register read)
  SPEC_TRACE_ONLY({
    unsigned hw;
    unsigned xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    trace_word(p.trace, 4, blockIdx.x, 12, ((unsigned long long)(xcc & 0xfu) << 16) | ((hw >> 8) & 0xffu));
  });
  if (!use_k && !use_p) {
    if (threadIdx.x == 0) p.thresh[row] = -INFINITY;
    return;
  }
  if (threadIdx.x == 0) s_fault = 0;
  __syncthreads();
  if (use_k && k == 1) {
    const float t1 = top1_select<DT, VEC>(p, lrow, row, s_m, s_scratch, &s_fault);
    if (threadIdx.x == 0) p.thresh[row] = t1;
    SPEC_STAMP(p, 4, 7);
    return;
  }
  // The sample's range [SMN, SM]: the window path's bins over the sample, or the full path's
  // bins over the row (values outside it fall into the end bins).
  {
    float sm = -INFINITY, smn = INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool c = (smp_ok[u] >> e) & 1u;
        sm = fmaxf(sm, c ? smp[u][e] : -INFINITY);
        smn = fminf(smn, c ? smp[u][e] : INFINITY);
      }
    const float wm = wave_max(sm), wmn = -wave_max(-smn);
    if (lane == 0) {
      s_m[wave] = wm;
      s_mn[wave] = wmn;
    }
  }
  __syncthreads();
  float SM = -INFINITY, SMN = INFINITY;
#pragma unroll
  for (int w = 0; w < kTW; ++w) {
    SM = fmaxf(SM, s_m[w]);
    SMN = fminf(SMN, s_mn[w]);
  }
  __syncthreads();
  float tau = -INFINITY;
  bool decided = false;
  const bool windowed = SM > SMN && isfinite(SM - SMN);
  if (windowed)
    decided = window_select<DT, VEC>(p, lrow, row, k, tp, use_k, use_p, smp, smp_ok, smp_e0, smp_stride, SM, SMN, s_sel.win,
                                     s_col, s_col2, s_scratch, s_m, s_mn, &s_fault, &s_d, &s_f, &tau);
  SPEC_TRACE_ONLY(if (windowed && !decided) trace_word(p.trace, 4, blockIdx.x, 11, 2ull));   // window fell back
  if (!decided)
    tau = full_select<DT, VEC>(p, lrow, row, k, tp, use_k, use_p, SM, SMN, s_sel, s_col, s_col2, s_scratch, s_m,
                               s_mn, &s_fault, &s_d, &s_f);
  if (threadIdx.x == 0) p.thresh[row] = tau;
  SPEC_STAMP(p, 4, 7);
}

template <int DT, bool VEC>
hipError_t launch_typed(ThreshParams p, hipStream_t s) {
  static int s_cus[64] = {0};        // per device ordinal: CUs if two blocks share each, -1 if not
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (s_cus[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, thresh_kernel<DT, VEC>, kTB, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidValue;
    s_cus[dev] = (per_cu == 2 && cus > 0) ? cus : -1;
  }
  p.cus = s_cus[dev] > 0 ? s_cus[dev] : 0;
  thresh_kernel<DT, VEC><<<dim3((unsigned)p.rows), dim3(kTB), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_thresholds(const ThreshParams& p, int logit_dtype, bool vec, hipStream_t s) {
  if (logit_dtype == kBF16) return vec ? launch_typed<kBF16, true>(p, s) : launch_typed<kBF16, false>(p, s);
  return vec ? launch_typed<kF32, true>(p, s) : launch_typed<kF32, false>(p, s);
}

}  // namespace sv
