// Chain verification by rejection sampling (spec_verify_chain).
//
// Two kernels on the caller's stream:
//  1. chain_stats_kernel -- one block per (row, 8192-element slice): every wave streams a
//     2048-element chunk of a target row once and writes its online-softmax summary
//     (max, sum of exponentials).  The last block to finish a request combines the
//     summaries of all gamma+1 rows, evaluates the accept tests of the draft tokens in
//     order, and records the terminal row A (the first rejection, or the bonus row).
//  2. chain_terminal_kernel -- one block per (request, 4096-element chunk) of the
//     terminal row: chunk masses of the terminal weights w = max(p_A - q_A, 0) (or p_gamma
//     when every draft was accepted).  The last block of a request finds the chunk where
//     the running mass passes u_gamma * W and rescans that chunk in vocabulary order.
//
// Method: [M7.1] "M7.1 - Speculative Decoding: Draft, Verify, Accept, Reject" §0x03A
// (accept test), §0x03C (positive residual), §0x03G (stop at the first rejection),
// §0x03H (bonus row), §0x04J (online (m, l) merge over vocabulary blocks); [M16]
// "Module 16: Speculative Decoding", "The Math: Speculative Sampling" (u < min(1, p/q)).
#include "device_common.h"
#include "internal.h"
#include "spec_verify.h"

namespace sv {

namespace {

constexpr double kLn2 = 0.69314718055994530942;

template <int DT>
__device__ __forceinline__ float gather(const void* base, size_t idx) { return load_scalar<DT>(base, idx); }

__device__ __forceinline__ float gather_q(const ChainParams& p, size_t idx) {
  return p.q_dtype == kBF16 ? load_scalar<kBF16>(p.q, idx) : load_scalar<kF32>(p.q, idx);
}

__device__ void write_failed(const ChainParams& p, int b, int code) {
  for (int i = threadIdx.x; i < p.R; i += blockDim.x) p.out_tokens[(size_t)b * p.R + i] = -1;
  if (p.stats)
    for (int i = threadIdx.x; i < p.R * 4; i += blockDim.x) p.stats[(size_t)b * p.R * 4 + i] = NAN;
  if (threadIdx.x == 0) {
    p.accepted_len[b] = -1;
    p.req_status[b] = code;
  }
}

// Last block of request b in the statistics pass: combine, accept scan, decision.
template <int DT>
__device__ void chain_decide(const ChainParams& p, int b) {
  __shared__ float s_r[SPEC_MAX_GAMMA + 1];     // reference exponent per row
  __shared__ float s_m[SPEC_MAX_GAMMA + 1];     // raw max per row
  __shared__ double s_z[SPEC_MAX_GAMMA + 1];    // sum 2^(l c2 - r) per row
  __shared__ int s_bad[SPEC_MAX_GAMMA + 1];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const float c2 = p.c2;

  for (int i = wave; i < p.R; i += kWavesPerBlock) {
    const float2* part = p.part + ((size_t)b * p.R + i) * p.P;
    float m = -INFINITY;
    for (int j = lane; j < p.P; j += kWave) m = fmaxf(m, fetch_f2(part + j).x);
    m = wave_max(m);
    const float r = m * c2;
    double z = 0.0;
    for (int j = lane; j < p.P; j += kWave) {
      const float2 s = fetch_f2(part + j);
      const float rj = s.x * c2;
      z += (double)s.y * exp2((double)rj - (double)r);
    }
    z = wave_sum_d(z);
    if (lane == 0) {
      s_r[i] = r;
      s_m[i] = m;
      s_z[i] = z;
      // all -inf (r = -inf gives NaN above), NaN or +inf anywhere: z is not finite
      s_bad[i] = !(isfinite(z) && z > 0.0);
    }
  }
  __syncthreads();
  // the summaries are consumed: return them to zero (every call leaves the workspace zeroed)
  {
    float2* part = p.part + (size_t)b * p.R * p.P;
    for (int j = threadIdx.x; j < p.R * p.P; j += kBlock) part[j] = make_float2(0.0f, 0.0f);
  }
  if (wave != 0) return;

  // lane i < G: draft position i, checked in the order a round reaches it
  int code = 0;
  bool reject = false;
  double px = NAN, a = NAN;
  const int G = p.G;
  if (lane < G) {
    const int x = p.tokens[(size_t)b * G + lane];
    if (s_bad[lane]) {
      code = SPEC_REQ_NONFINITE;
    } else if (x < 0 || x >= p.V) {
      code = SPEC_REQ_BADTOKEN;
    } else {
      const float qx = gather_q(p, ((size_t)b * G + lane) * p.V + x);
      if (!(isfinite(qx) && qx > 0.0f)) {
        code = SPEC_REQ_QZERO;
      } else {
        const float ui = p.u[(size_t)b * p.R + lane];
        if (!(ui >= 0.0f && ui < 1.0f)) {
          code = SPEC_REQ_BADUNIFORM;
        } else {
          const float lx = gather<DT>(p.logits, ((size_t)b * p.R + lane) * p.V + x);
          px = exp2((double)lx * (double)c2 - (double)s_r[lane]) / s_z[lane];
          a = fmin(1.0, px / (double)qx);
          reject = !((double)ui < a);
        }
      }
    }
  }
  const unsigned long long stop = __ballot(lane < G && (code != 0 || reject));
  int A = stop ? (__ffsll((long long)stop) - 1) : G;
  int status = __shfl(code, A < G ? A : 0, kWave);
  if (A == G) {
    status = s_bad[G] ? SPEC_REQ_NONFINITE : 0;
  }
  if (status == 0) {
    const float ut = p.u[(size_t)b * p.R + G];
    if (!(ut >= 0.0f && ut < 1.0f)) status = SPEC_REQ_BADUNIFORM;
  }

  if (status != 0) {
    // whole wave writes the failure record
    for (int i = lane; i < p.R; i += kWave) p.out_tokens[(size_t)b * p.R + i] = -1;
    if (p.stats)
      for (int i = lane; i < p.R * 4; i += kWave) p.stats[(size_t)b * p.R * 4 + i] = NAN;
    if (lane == 0) {
      p.accepted_len[b] = -1;
      p.req_status[b] = status;
      p.dec[b] = ChainDecision{-1, status, 0.0f, 0.0f};
    }
    return;
  }

  if (p.stats) {
    float* st = p.stats + (size_t)b * p.R * 4;
    // rows 0..A (< G) reached: (m, log Z, p(x), a); later draft rows NaN
    if (lane < G) {
      const bool reached = lane <= A;
      const double m_nat = (double)s_m[lane] * p.inv_t;
      const double logz = log(s_z[lane]) + (double)s_r[lane] * kLn2 - m_nat;
      st[lane * 4 + 0] = reached ? (float)m_nat : NAN;
      st[lane * 4 + 1] = reached ? (float)logz : NAN;
      st[lane * 4 + 2] = reached ? (float)px : NAN;
      st[lane * 4 + 3] = reached ? (float)a : NAN;
    }
    if (lane == 0) {
      const bool bonus = (A == G);
      const double m_nat = (double)s_m[G] * p.inv_t;
      const double logz = log(s_z[G]) + (double)s_r[G] * kLn2 - m_nat;
      st[G * 4 + 0] = bonus ? (float)m_nat : NAN;
      st[G * 4 + 1] = bonus ? (float)logz : NAN;
      st[G * 4 + 2] = NAN;   // W, written by the terminal pass
      st[G * 4 + 3] = NAN;
    }
  }
  if (lane == 0) {
    p.dec[b] = ChainDecision{A, 0, s_r[A], (float)(1.0 / s_z[A])};
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void chain_stats_kernel(ChainParams p) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const size_t rowid = blockIdx.x / p.WG1;
  const int slice = blockIdx.x % p.WG1;
  const int b = (int)(rowid / p.R);
  const int chunk = slice * kWavesPerBlock + wave;
  if (chunk < p.P) {
    float m, z;
    chunk_summary<DT, VEC>(row_ptr<DT>(p.logits, rowid, p.V), p.V, chunk, lane, p.c2, m, z);
    if (lane == 0) publish_f2(p.part + rowid * p.P + chunk, make_float2(m, z));
  }
  __syncthreads();   // every wave's summary store has completed
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    const unsigned prev = arrive(&p.counters[(size_t)b * kCounterSlots + 0]);
    s_last = (prev == (unsigned)(p.R * p.WG1 - 1));
  }
  __syncthreads();
  if (!s_last) return;
  chain_decide<DT>(p, b);
  if (threadIdx.x == 0) reset_counter(&p.counters[(size_t)b * kCounterSlots + 0]);
}

// Terminal weight of one element: p(x) = 2^(l c2 - r) / Z; residual rows subtract q and
// clamp at zero.  A negative or non-finite q entry poisons the mass with NaN.
template <bool RESID>
__device__ __forceinline__ float term_weight(float l, float qv, float c2, float r, float inv_z,
                                             bool& bad) {
  const float pv = scaled_exp(l, c2, r) * inv_z;
  if constexpr (RESID) {
    bad |= !(qv >= 0.0f && qv < INFINITY);
    const float d = pv - qv;
    return d > 0.0f ? d : 0.0f;
  } else {
    return pv;
  }
}

template <int DT, int QT, bool VEC, bool RESID>
__device__ __forceinline__ void term_load8(const void* lrow, const void* qrow, long e0, long V, float c2,
                                           float r, float inv_z, float (&w)[8], bool& bad) {
  float lv[8], qv[8];
  load8<DT, VEC, false>(lrow, e0, V, lv, -INFINITY);
  if constexpr (RESID) {
    load8<QT, VEC, false>(qrow, e0, V, qv, 0.0f);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) qv[k] = 0.0f;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k] = term_weight<RESID>(lv[k], qv[k], c2, r, inv_z, bad);
}

// Last block of request b in the terminal pass: pick the chunk, rescan it, emit.
template <int DT, int QT, bool VEC, bool RESID>
__device__ void chain_select(const ChainParams& p, int b, const ChainDecision& d, const void* lrow,
                             const void* qrow) {
  __shared__ double s_scan[kWavesPerBlock];
  __shared__ int s_pick;
  __shared__ double s_before;
  __shared__ double s_total;
  const int tid = threadIdx.x;
  const double* tm = p.tmass + (size_t)b * p.S2;

  // 1. running mass over the chunks in order: thread t owns a contiguous run of chunks
  //    and extends the block-exclusive prefix sequentially over it.  W is the running
  //    value after the last chunk, computed the same way, so u * W < W always finds a
  //    chunk whose running value exceeds the target.
  const int per = (p.S2 + kBlock - 1) / kBlock;
  const int c_lo = min(tid * per, p.S2), c_hi = min(c_lo + per, p.S2);
  double mine = 0.0;
  for (int c = c_lo; c < c_hi; ++c) mine += fetch_d(tm + c);
  double tot;
  const double excl = block_excl_scan_d(mine, s_scan, &tot);
  double run_end = excl;
  for (int c = c_lo; c < c_hi; ++c) run_end += fetch_d(tm + c);
  if (c_lo < c_hi && c_hi == p.S2) s_total = run_end;
  if (tid == 0) s_pick = 0x7fffffff;
  __syncthreads();
  const double W = s_total;
  const int G = p.G;
  if (!(isfinite(W) && W > 0.0)) {
    write_failed(p, b, SPEC_REQ_RESIDUAL_EMPTY);
    return;
  }
  const double t = (double)p.u[(size_t)b * p.R + G] * W;
  {
    double run = excl;
    for (int c = c_lo; c < c_hi; ++c) {
      const double nxt = run + fetch_d(tm + c);
      if (nxt > t) {
        atomicMin(&s_pick, c);
        break;
      }
      run = nxt;
    }
  }
  __syncthreads();
  // a chunk is always found (t < W and the last running value is W); clamp regardless
  const int cstar = s_pick == 0x7fffffff ? p.S2 - 1 : s_pick;
  if (tid == 0) s_before = 0.0;
  __syncthreads();
  if (cstar >= c_lo && cstar < c_hi) {       // the owner of cstar records the mass before it
    double run = excl;
    for (int c = c_lo; c < cstar; ++c) run += fetch_d(tm + c);
    s_before = run;
  }
  __syncthreads();
  if (tid == 0) s_pick = 0x7fffffff;
  __syncthreads();
  double rem = t - s_before;   // target mass inside chunk cstar

  // 2. rescan cstar in vocabulary order, slab by slab
  const float c2 = p.c2, r = d.r_ref, inv_z = d.inv_z;
  int last_pos = -1;
  for (int s = 0; s < kTermSlabs; ++s) {
    const long e0 = ((long)cstar * kTermSlabs + s) * kSlab + (long)tid * kVec;
    float w[8];
    bool bad = false;
    term_load8<DT, QT, VEC, RESID>(lrow, qrow, e0, p.V, c2, r, inv_z, w, bad);
    double incl[8];
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc += (double)w[k];
      incl[k] = acc;
      if (w[k] > 0.0f) last_pos = (int)(e0 + k);
    }
    double slab_total;
    const double off = block_excl_scan_d(acc, s_scan, &slab_total);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (off + incl[k] > rem && w[k] > 0.0f) { atomicMin(&s_pick, (int)(e0 + k)); break; }
    }
    __syncthreads();
    if (s_pick != 0x7fffffff) break;
    rem -= slab_total;
    __syncthreads();
  }
  __shared__ int s_last_pos;
  if (tid == 0) s_last_pos = -1;
  __syncthreads();
  if (s_pick == 0x7fffffff) atomicMax(&s_last_pos, last_pos);   // rounding left the target past the chunk
  __syncthreads();
  const int k = (s_pick != 0x7fffffff) ? s_pick : s_last_pos;

  // 3. emit
  const int A = d.A;
  for (int i = tid; i < p.R; i += kBlock) {
    int v;
    if (i < A) v = p.tokens[(size_t)b * G + i];
    else if (i == A) v = k;
    else v = -1;
    p.out_tokens[(size_t)b * p.R + i] = v;
  }
  if (tid == 0) {
    p.accepted_len[b] = A;
    p.req_status[b] = 0;
    if (p.stats) p.stats[((size_t)b * p.R + G) * 4 + 2] = (float)W;
  }
}

template <int DT, int QT, bool VEC, bool RESID>
__device__ void chain_terminal_body(const ChainParams& p, int b, int c, const ChainDecision& d) {
  const int tid = threadIdx.x;
  const int A = d.A;
  const void* lrow = row_ptr<DT>(p.logits, (size_t)b * p.R + A, p.V);
  const void* qrow = RESID ? row_ptr<QT>(p.q, (size_t)b * p.G + A, p.V) : nullptr;
  double acc = 0.0;
  bool bad = false;
#pragma unroll
  for (int s = 0; s < kTermSlabs; ++s) {
    const long e0 = ((long)c * kTermSlabs + s) * kSlab + (long)tid * kVec;
    float w[8];
    term_load8<DT, QT, VEC, RESID>(lrow, qrow, e0, p.V, p.c2, d.r_ref, d.inv_z, w, bad);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += (double)w[k];
  }
  if (bad) acc = NAN;
  __shared__ double s_red[kWavesPerBlock];
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const double ws = wave_sum_d(acc);
  if (lane == 0) s_red[wave] = ws;
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0) {
    const double m = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    publish_d(p.tmass + (size_t)b * p.S2 + c, m);
    vmem_wait();
    const unsigned prev = arrive(&p.counters[(size_t)b * kCounterSlots + 1]);
    s_last = (prev == (unsigned)(p.S2 - 1));
  }
  __syncthreads();
  if (!s_last) return;
  chain_select<DT, QT, VEC, RESID>(p, b, d, lrow, qrow);
  __syncthreads();
  for (int j = tid; j < p.S2; j += kBlock) p.tmass[(size_t)b * p.S2 + j] = 0.0;
  if (tid == 0) {
    p.dec[b] = ChainDecision{0, 0, 0.0f, 0.0f};
    reset_counter(&p.counters[(size_t)b * kCounterSlots + 1]);
  }
}

template <int DT, int QT, bool VEC>
__global__ __launch_bounds__(kBlock) void chain_terminal_kernel(ChainParams p) {
  const int b = blockIdx.x / p.S2;
  const int c = blockIdx.x % p.S2;
  const ChainDecision d = p.dec[b];
  if (d.status != 0) {
    // failed in the statistics pass (outputs already written): only count the arrival,
    // so that the last block can clear the decision record
    __shared__ int s_last;
    if (threadIdx.x == 0) {
      const unsigned prev = arrive(&p.counters[(size_t)b * kCounterSlots + 1]);
      s_last = (prev == (unsigned)(p.S2 - 1));
    }
    __syncthreads();
    if (s_last && threadIdx.x == 0) {
      p.dec[b] = ChainDecision{0, 0, 0.0f, 0.0f};
      reset_counter(&p.counters[(size_t)b * kCounterSlots + 1]);
    }
    return;
  }
  if (d.A < p.G) chain_terminal_body<DT, QT, VEC, true>(p, b, c, d);
  else chain_terminal_body<DT, QT, VEC, false>(p, b, c, d);
}

template <int DT, int QT, bool VEC>
hipError_t launch_typed(const ChainParams& p, hipStream_t s) {
  const unsigned g1 = (unsigned)((size_t)p.B * p.R * p.WG1);
  chain_stats_kernel<DT, VEC><<<dim3(g1), dim3(kBlock), 0, s>>>(p);
  const unsigned g2 = (unsigned)((size_t)p.B * p.S2);
  chain_terminal_kernel<DT, QT, VEC><<<dim3(g2), dim3(kBlock), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chain(const ChainParams& p, int logit_dtype, bool vec, hipStream_t s) {
  const bool lb = logit_dtype == kBF16, qb = p.q_dtype == kBF16;
  if (vec) {
    if (lb) return qb ? launch_typed<kBF16, kBF16, true>(p, s) : launch_typed<kBF16, kF32, true>(p, s);
    return qb ? launch_typed<kF32, kBF16, true>(p, s) : launch_typed<kF32, kF32, true>(p, s);
  }
  if (lb) return qb ? launch_typed<kBF16, kBF16, false>(p, s) : launch_typed<kBF16, kF32, false>(p, s);
  return qb ? launch_typed<kF32, kBF16, false>(p, s) : launch_typed<kF32, kF32, false>(p, s);
}

}  // namespace sv
