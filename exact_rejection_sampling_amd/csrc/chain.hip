// Chain verification by rejection sampling (spec_verify_chain).
//
// One launch, one block per work item, the item chosen by blockIdx.  The first B*(gamma+1)*SL
// blocks are statistics items, request-major; the B*S2 blocks after them are terminal
// items, also request-major:
//  * statistics item (row, slice): the block's four waves stream a slice of one target
//    row with 16-byte non-temporal loads, keep an online (max, sum of exponentials) per
//    lane and publish one summary per wave.  The last item of a request to finish
//    combines the summaries of all gamma+1 rows, runs the accept tests of the draft
//    tokens in order and publishes the decision: the first rejection A (or gamma).
//  * terminal item (request, 4096-element chunk): waits for the request's decision,
//    then sums the terminal weights w = max(p_A - q_A, 0) (or p_gamma when every draft
//    was accepted) over its chunk.  The last chunk to finish finds the chunk where the
//    running mass passes u_gamma * W and rescans that chunk in vocabulary order.
// Statistics items never wait for another block (the last arriver's reads of the other
// summaries only bridge the time until their stores are visible).  Terminal items wait only
// for statistics items, whose block indices are all lower; the hardware dispatches the
// workgroups of a launch in index order, so those blocks are running or done, and every
// wait ends.  The wait is bounded all the same: a decision that does not arrive within the
// bound is reported as SPEC_REQ_INTERNAL rather than waited for.
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

constexpr int kSlotStats = 0, kSlotTerm = 1;

__device__ __forceinline__ unsigned* slot(const ChainParams& p, int b, int k) {
  return p.counters + (size_t)b * kCounterSlots + k;
}

// A request's decision as two self-validating words for the terminal items of the same
// launch: word 0 = A | status << 32 with the top bit set; word 1 = r_ref | inv_z << 32,
// where inv_z is positive (failed requests carry 1.0).
__device__ __forceinline__ void publish_decision(const ChainParams& p, int b, const ChainDecision& d) {
  unsigned long long* w = reinterpret_cast<unsigned long long*>(p.dec + b);
  const float inv_z = d.status == 0 ? d.inv_z : 1.0f;
  publish_u64(w + 1, (static_cast<unsigned long long>(__float_as_uint(inv_z)) << 32) |
                         __float_as_uint(d.r_ref));
  publish_u64(w, (1ull << 63) | (static_cast<unsigned long long>(static_cast<unsigned>(d.status)) << 32) |
                     static_cast<unsigned>(d.A));
}

// Wait (bounded) for request b's decision; a decision that never arrives is reported
// as an internal error.
__device__ __forceinline__ ChainDecision await_decision(const ChainParams& p, int b) {
  const unsigned long long* w = reinterpret_cast<const unsigned long long*>(p.dec + b);
  const unsigned long long a = await_u64(w);
  unsigned long long c = await_u64(w + 1);
  for (unsigned spins = 0; (c >> 32) == 0ull && spins < kSpinLimit; ++spins) c = fetch_u64(w + 1);
  if (!(a >> 63) || (c >> 32) == 0ull) return ChainDecision{-1, SPEC_REQ_INTERNAL, 0.0f, 0.0f};
  return ChainDecision{static_cast<int32_t>(static_cast<unsigned>(a)),
                       static_cast<int32_t>(static_cast<unsigned>(a >> 32) & 0x7fffffffu),
                       __uint_as_float(static_cast<unsigned>(c)),
                       __uint_as_float(static_cast<unsigned>(c >> 32))};
}

// Gather record of draft row i, published by the block that streams the row's first
// slice while it streams: three words (token, its logit, its draft probability), each
// with bit 63 set so that a published word is never zero.
__device__ __forceinline__ unsigned long long* gather_rec(const ChainParams& p, int b, int i) {
  return p.gath + ((size_t)b * p.G + i) * 3;
}

template <int DT>
__device__ __forceinline__ void gather_issue(const ChainParams& p, int b, int i, unsigned& x, unsigned& lb,
                                             unsigned& qb) {
  const int t = p.tokens[(size_t)b * p.G + i];
  x = static_cast<unsigned>(t);
  lb = qb = 0u;
  if (t >= 0 && t < p.V) {
    lb = __float_as_uint(load_scalar<DT>(p.logits, ((size_t)b * p.R + i) * p.V + t));
    qb = __float_as_uint(gather_q(p, ((size_t)b * p.G + i) * p.V + t));
  }
}

__device__ __forceinline__ void gather_publish(const ChainParams& p, int b, int i, unsigned x, unsigned lb,
                                               unsigned qb) {
  unsigned long long* g = gather_rec(p, b, i);
  publish_u64(g + 0, (1ull << 63) | x);
  publish_u64(g + 1, (1ull << 63) | lb);
  publish_u64(g + 2, (1ull << 63) | qb);
}

constexpr int kDecideStage = 2048;                    // summaries the deciding block stages in LDS
constexpr int kStagePerThread = kDecideStage / kBlock;

// Last block of request b in the statistics pass: combine, accept scan, decision.  All of
// its global reads (summaries, gathered draft values, uniforms) are issued together.
template <int DT>
__device__ void chain_decide(const ChainParams& p, int b) {
  __shared__ float2 s_part[kDecideStage];
  __shared__ float s_r[SPEC_MAX_GAMMA + 1];     // reference exponent per row
  __shared__ float s_m[SPEC_MAX_GAMMA + 1];     // raw max per row
  __shared__ double s_z[SPEC_MAX_GAMMA + 1];    // sum 2^(l c2 - r) per row
  __shared__ int s_bad[SPEC_MAX_GAMMA + 1];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
  const float c2 = p.c2;
  const int G = p.G;
  const int total = p.R * p.PP;
  const float2* part_b = p.part + (size_t)b * p.R * p.PP;
  const bool staged = total <= kDecideStage;

  // wave 0, lane i < G: draft position i -- its gather record and uniform
  unsigned long long g[3] = {0ull, 0ull, 0ull};
  float ui = 0.0f;
  if (wave == 0 && lane < G) {
    const unsigned long long* rec = gather_rec(p, b, lane);
    g[0] = fetch_u64(rec);
    g[1] = fetch_u64(rec + 1);
    g[2] = fetch_u64(rec + 2);
    ui = p.u[(size_t)b * p.R + lane];
  }
  if (staged) {
    unsigned long long v[kStagePerThread];
#pragma unroll
    for (int k = 0; k < kStagePerThread; ++k) {
      const int j = tid + k * kBlock;
      v[k] = j < total ? fetch_u64(reinterpret_cast<const unsigned long long*>(part_b + j)) : 1ull;
    }
#pragma unroll
    for (int k = 0; k < kStagePerThread; ++k) {
      const int j = tid + k * kBlock;
      if (j < total) {
        if (v[k] == 0ull) v[k] = await_u64(reinterpret_cast<const unsigned long long*>(part_b + j));
        s_part[j] = make_float2(__uint_as_float(static_cast<unsigned>(v[k])),
                                __uint_as_float(static_cast<unsigned>(v[k] >> 32)));
      }
    }
  }
  if (wave == 0 && lane < G) {
    const unsigned long long* rec = gather_rec(p, b, lane);
#pragma unroll
    for (int k = 0; k < 3; ++k)
      if (g[k] == 0ull) g[k] = await_u64(rec + k);
  }
  __syncthreads();

  for (int i = wave; i < p.R; i += kWavesPerBlock) {
    const float2* row_part = part_b + (size_t)i * p.PP;
    float m = -INFINITY;
    for (int j = lane; j < p.PP; j += kWave)
      m = fmaxf(m, staged ? s_part[i * p.PP + j].x : await_f2(row_part + j).x);
    m = wave_max(m);
    const float r = m * c2;
    double z = 0.0;
    for (int j = lane; j < p.PP; j += kWave) {
      const float2 s = staged ? s_part[i * p.PP + j] : await_f2(row_part + j);
      // 2^(r_j - r) <= 1; an all -inf row gives (-inf) - (-inf) = NaN, flagged below
      z += (double)s.y * (double)__builtin_amdgcn_exp2f(s.x * c2 - r);
    }
    z = wave_sum_d(z);
    if (lane == 0) {
      s_r[i] = r;
      s_m[i] = m;
      s_z[i] = z;
      // all -inf, NaN or +inf anywhere: z is not a positive finite number
      s_bad[i] = !(isfinite(z) && z > 0.0);
    }
  }
  __syncthreads();
  // the summaries and gather records are consumed: return them to zero (every call
  // leaves the workspace zeroed)
  for (int j = tid; j < total; j += kBlock) clear_f2(const_cast<float2*>(part_b) + j);
  for (int j = tid; j < 3 * G; j += kBlock) clear_u64(gather_rec(p, b, 0) + j);
  if (wave != 0) return;

  // lane i < G: draft position i, checked in the order a round reaches it
  int code = 0;
  bool reject = false;
  double px = NAN, a = NAN;
  if (lane < G) {
    const int x = static_cast<int>(static_cast<unsigned>(g[0]));
    if (s_bad[lane]) {
      code = SPEC_REQ_NONFINITE;
    } else if (x < 0 || x >= p.V) {
      code = SPEC_REQ_BADTOKEN;
    } else {
      const float qx = __uint_as_float(static_cast<unsigned>(g[2]));
      if (!(isfinite(qx) && qx > 0.0f)) {
        code = SPEC_REQ_QZERO;
      } else if (!(ui >= 0.0f && ui < 1.0f)) {
        code = SPEC_REQ_BADUNIFORM;
      } else {
        const float lx = __uint_as_float(static_cast<unsigned>(g[1]));
        px = exp2((double)lx * (double)c2 - (double)s_r[lane]) / s_z[lane];
        a = fmin(1.0, px / (double)qx);
        reject = !((double)ui < a);
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
      publish_decision(p, b, ChainDecision{-1, status, 0.0f, 0.0f});
    }
    return;
  }

  if (p.stats) {
    // Written through to memory before the decision is published: the terminal items'
    // last block writes W (or, on failure, NaN over everything) afterwards.
    float* st = p.stats + (size_t)b * p.R * 4;
    // rows 0..A (< G) reached: (m, log Z, p(x), a); later draft rows NaN
    if (lane < G) {
      const bool reached = lane <= A;
      const double m_nat = (double)s_m[lane] * p.inv_t;
      const double logz = log(s_z[lane]) + (double)s_r[lane] * kLn2 - m_nat;
      store_wt(st + lane * 4 + 0, reached ? (float)m_nat : NAN);
      store_wt(st + lane * 4 + 1, reached ? (float)logz : NAN);
      store_wt(st + lane * 4 + 2, reached ? (float)px : NAN);
      store_wt(st + lane * 4 + 3, reached ? (float)a : NAN);
    }
    if (lane == 0) {
      const bool bonus = (A == G);
      const double m_nat = (double)s_m[G] * p.inv_t;
      const double logz = log(s_z[G]) + (double)s_r[G] * kLn2 - m_nat;
      store_wt(st + G * 4 + 0, bonus ? (float)m_nat : NAN);
      store_wt(st + G * 4 + 1, bonus ? (float)logz : NAN);
      store_wt(st + G * 4 + 3, NAN);   // column 2 (W) belongs to the terminal items
    }
  }
  if (lane == 0) publish_decision(p, b, ChainDecision{A, 0, s_r[A], (float)(1.0 / s_z[A])});
}

// Statistics item: slice `slice` of row i of request b.
template <int DT, bool VEC>
__device__ void stats_item(const ChainParams& p, int b, int i, int slice) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const size_t rowid = (size_t)b * p.R + i;
  // the first slice of a draft row also fetches the draft token, its logit and its draft
  // probability for the decision, overlapped with the streaming below
  const bool gathers = slice == 0 && i < p.G && threadIdx.x == 0;
  unsigned gx = 0, gl = 0, gq = 0;
  if (gathers) gather_issue<DT>(p, b, i, gx, gl, gq);
  {
    // wave w streams chunks first + 4k of this slice (k < CPW); always one summary per wave
    const long first = (long)slice * kWavesPerBlock * p.CPW + wave;
    float m, z;
    wave_row_summary<DT, VEC>(row_ptr<DT>(p.logits, rowid, p.V), p.V, p.P, first, kWavesPerBlock, p.CPW,
                              lane, p.c2, m, z);
    if (lane == 0) publish_f2(p.part + rowid * p.PP + slice * kWavesPerBlock + wave, make_float2(m, z));
  }
  if (gathers) gather_publish(p, b, i, gx, gl, gq);
  __syncthreads();   // every wave's summary store has completed
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    const unsigned prev = arrive(slot(p, b, kSlotStats));
    s_last = (prev == (unsigned)(p.R * p.SL - 1));
  }
  __syncthreads();
  if (!s_last) return;
  chain_decide<DT>(p, b);
  if (threadIdx.x == 0) reset_counter(slot(p, b, kSlotStats));
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
  for (int c = c_lo; c < c_hi; ++c) mine += await_mass(tm + c);
  double tot;
  const double excl = block_excl_scan_d(mine, s_scan, &tot);
  double run_end = excl;
  for (int c = c_lo; c < c_hi; ++c) run_end += await_mass(tm + c);
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
      const double nxt = run + await_mass(tm + c);
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
    for (int c = c_lo; c < cstar; ++c) run += await_mass(tm + c);
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

// Every terminal item of request b has arrived: clear the request's workspace state.
__device__ __forceinline__ void finish_request(const ChainParams& p, int b) {
  unsigned long long* w = reinterpret_cast<unsigned long long*>(p.dec + b);
  clear_u64(w);
  clear_u64(w + 1);
  reset_counter(slot(p, b, kSlotTerm));
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
  const int lane = tid & (kWave - 1), wave = wave_id();
  const double ws = wave_sum_d(acc);
  if (lane == 0) s_red[wave] = ws;
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0) {
    const double m = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    publish_mass(p.tmass + (size_t)b * p.S2 + c, m);
    vmem_wait();
    const unsigned prev = arrive(slot(p, b, kSlotTerm));
    s_last = (prev == (unsigned)(p.S2 - 1));
  }
  __syncthreads();
  if (!s_last) return;
  chain_select<DT, QT, VEC, RESID>(p, b, d, lrow, qrow);
  __syncthreads();
  for (int j = tid; j < p.S2; j += kBlock) clear_mass(p.tmass + (size_t)b * p.S2 + j);
  if (tid == 0) finish_request(p, b);
}

// Terminal item: chunk c of request b's terminal row.
template <int DT, int QT, bool VEC>
__device__ void terminal_item(const ChainParams& p, int b, int c) {
  __shared__ ChainDecision s_dec;
  if (threadIdx.x == 0) s_dec = await_decision(p, b);
  __syncthreads();
  const ChainDecision d = s_dec;
  if (d.status != 0) {
    // the request failed (its outputs are written): only count the arrival, so that
    // the last item can clear the request's state
    __shared__ int s_last;
    if (threadIdx.x == 0) {
      if (d.status == SPEC_REQ_INTERNAL) {   // wait bound hit: report instead of guessing
        p.accepted_len[b] = -1;
        p.req_status[b] = SPEC_REQ_INTERNAL;
      }
      const unsigned prev = arrive(slot(p, b, kSlotTerm));
      s_last = (prev == (unsigned)(p.S2 - 1));
    }
    __syncthreads();
    if (s_last && threadIdx.x == 0) finish_request(p, b);
    return;
  }
  if (d.A < p.G) chain_terminal_body<DT, QT, VEC, true>(p, b, c, d);
  else chain_terminal_body<DT, QT, VEC, false>(p, b, c, d);
}

// Statistics items first, then terminal items, each request-major.
template <int DT, int QT, bool VEC>
__global__ __launch_bounds__(kBlock) void chain_kernel(ChainParams p) {
  const long t = blockIdx.x, Sb = (long)p.R * p.SL, n_stats = (long)p.B * Sb;
  if (t < n_stats) {
    const int b = (int)(t / Sb), o = (int)(t % Sb);
    stats_item<DT, VEC>(p, b, o / p.SL, o % p.SL);
  } else {
    const long u = t - n_stats;
    terminal_item<DT, QT, VEC>(p, (int)(u / p.S2), (int)(u % p.S2));
  }
}

template <int DT, int QT, bool VEC>
hipError_t launch_typed(const ChainParams& p, hipStream_t s) {
  const unsigned long long blocks = (unsigned long long)p.B * ((unsigned long long)p.R * p.SL + p.S2);  // == chain_blocks
  chain_kernel<DT, QT, VEC><<<dim3((unsigned)blocks), dim3(kBlock), 0, s>>>(p);
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
