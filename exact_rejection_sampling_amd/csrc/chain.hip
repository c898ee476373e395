// Chain verification by rejection sampling (spec_verify_chain).
//
// One launch, one block per work item, the item chosen by blockIdx (block_item): B*(gamma+1)*SL
// statistics items and B*S2 terminal items, each request's terminal items placed a fixed
// lag of blocks after its statistics items:
//  * statistics item (row, slice): the block's four waves stream a slice of one target
//    row with 16-byte non-temporal loads, keep an online (max, sum of exponentials) per
//    lane, merge lanes and waves, and publish one summary for the slice.  The block that
//    streams a draft row's first slice also publishes the draft token, its logit and its
//    draft probability.  A statistics item never counts arrivals, and waits only as
//    the gate of a lazy row group (below).
//  * lazy rows (lazy_rows = LK): the rows come in groups of LK, ordered group by group
//    (lazy_item).  An item of a group after the first first takes the request's decision
//    over the previous group's published words; if the round never reaches its group it
//    publishes a marker (an empty-range summary, a zero gather record) instead of
//    streaming.  Markers read as invalid rows, so they only ever follow an earlier event
//    and never change the decision.
//  * terminal item (request, 4096-element chunk): reads every summary of its request as
//    soon as it is published, combines them into each row's normalizer, runs the accept
//    tests in order and so finds the first rejection A (or gamma) -- every terminal item of
//    a request computes the same decision from the same words -- then sums the terminal
//    weights w = max(p_A - q_A, 0) (or p_gamma when every draft was accepted) over its
//    chunk and publishes the chunk's mass.  The request's last terminal item (its
//    selector) waits for the other chunks' masses, finds the chunk where the running mass
//    passes u_gamma * W, rescans that chunk in vocabulary order, writes the outputs and
//    returns every workspace word the request used to zero.
// Waits: a terminal item waits only for its request's statistics items, whose block
// indices are all lower (see block_item), a lazy gate only for the previous group's items
// (lower, see lazy_item), and a selector only for its request's other terminal items,
// whose indices are lower too.  The hardware dispatches the workgroups of a launch in index order, so a
// waiting block never holds a slot that one of the blocks it waits for still needs, and
// every wait ends.  Each wait is bounded all the same: a word that does not arrive within
// the bound makes the request report SPEC_REQ_INTERNAL rather than wait on.
//
// Method: [M7.1] "M7.1 - Speculative Decoding: Draft, Verify, Accept, Reject" §0x03A
// (accept test), §0x03C (positive residual), §0x03G (stop at the first rejection),
// §0x03H (bonus row), §0x04J (online (m, l) merge over vocabulary blocks); [M16]
// "Module 16: Speculative Decoding", "The Math: Speculative Sampling" (u < min(1, p/q)).
#include "device_common.h"
#include "internal.h"
#include "proc.h"
#include "spec_verify.h"

namespace sv {

namespace {

constexpr double kLn2 = 0.69314718055994530942;

// Item kinds in a trace record's tag (trace builds only).
enum : int { kTraceStats = 0, kTraceSkipped = 1, kTraceTerminal = 2, kTraceSelector = 3,
             kTraceExactIdle = 4, kTraceExact = 5 };

__device__ __forceinline__ float gather_q(const ChainParams& p, size_t idx) {
  return p.q_dtype == kBF16 ? load_scalar<kBF16>(p.q, idx) : load_scalar<kF32>(p.q, idx);
}

// Gather record of draft row i, published by the block that streams the row's first
// slice while it streams: three words (token, its logit, its draft probability), each
// with bit 63 set so that a published word is never zero.
__device__ __forceinline__ unsigned long long* gather_rec(const ChainParams& p, int b, int i) {
  return p.gath + ((size_t)b * p.G + i) * 3;
}

template <int DT, int QT, bool PROC>
__device__ __forceinline__ void gather_issue(const ChainParams& p, int b, int i, unsigned& x, unsigned& lb,
                                             unsigned& qb) {
  const int t = p.tokens[(size_t)b * p.G + i];
  x = static_cast<unsigned>(t);
  lb = qb = 0u;
  if (t >= 0 && t < p.V) {
    const size_t rowid = (size_t)b * p.R + i;
    float l = load_scalar<DT>(p.logits, rowid * p.V + t);
    if constexpr (PROC) l = proc1(p.pr, rowid, row_tau(p.pr, rowid), t, l);
    lb = __float_as_uint(l);
    if constexpr (QT != kSparseQ) qb = __float_as_uint(gather_q(p, ((size_t)b * p.G + i) * p.V + t));
  }
}

// q_i(x) of a sparse draft row, block-wide: the sum of the values listed at index x (each
// thread sums its share of the entries in order, then a fixed-order block sum); every
// thread receives it.  Contains two barriers.
// The thread's first entry (x0, v0; has0 when it exists) was loaded by the caller before
// streaming the row.
__device__ float sparse_q_lookup(const ChainParams& p, int b, int i, int x, float* scratch, bool has0, int x0,
                                 float v0) {
  const size_t base = ((size_t)b * p.G + i) * p.q_k;
  const float* val = static_cast<const float*>(p.q) + base;
  const int32_t* idx = p.q_index + base;
  float acc = (has0 && x0 == x) ? v0 : 0.0f;
  for (int j = threadIdx.x + kBlock; j < p.q_k; j += kBlock)
    if (idx[j] == x) acc += val[j];
  const float w = wave_sum(acc);
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[wave_id()] = w;
  __syncthreads();
  const float t = (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
  __syncthreads();
  return t;
}

__device__ __forceinline__ void gather_publish(const ChainParams& p, int b, int i, unsigned x, unsigned lb,
                                               unsigned qb) {
  unsigned long long* g = gather_rec(p, b, i);
  publish_u64(g + 0, (1ull << 63) | x);
  publish_u64(g + 1, (1ull << 63) | lb);
  publish_u64(g + 2, (1ull << 63) | qb);
}

// Online-softmax summary of the chunks a wave visits, the processors applied to every
// element first.
template <int DT, bool VEC>
__device__ __forceinline__ void wave_row_summary_proc(const ChainParams& p, size_t rowid, long first, int lane,
                                                      float& m_out, float& z_out) {
  const float tau = row_tau(p.pr, rowid);
  LaneSoftmax st;
  stream_chunks<DT, VEC>(row_ptr<DT>(p.logits, rowid, p.V), p.V, p.P, first, kWavesPerBlock, p.CPW, lane,
                         [&](const ChunkRegs<DT>& r, long c) {
                           float v[kStatVecs][8];
                           chunk_values<DT>(r, v);
#pragma unroll
                           for (int j = 0; j < kStatVecs; ++j)
                             proc8<VEC>(p.pr, rowid, tau, c * kWaveChunk + static_cast<long>(j * kWave + lane) * kVec,
                                        p.V, v[j]);
                           lane_softmax_update(st, v, p.c2);
                         });
  wave_softmax_merge(st, p.c2, m_out, z_out);
}

// Per-row results of a terminal item's decision, kept for the selector's outputs.
struct RowState {
  float r[SPEC_MAX_GAMMA + 1];    // reference exponent per row
  float m[SPEC_MAX_GAMMA + 1];    // raw max per row
  double z[SPEC_MAX_GAMMA + 1];   // sum 2^(l c2 - r) per row
  int bad[SPEC_MAX_GAMMA + 1];    // row is all -inf, or holds NaN / +inf
  double px[SPEC_MAX_GAMMA];      // p_i(x_i) of the reached draft rows
  double a[SPEC_MAX_GAMMA];       // a_i of the reached draft rows
};

// Statistics item: slice `slice` of row i of request b.
// Lazy rows: an item of a row the round never reaches publishes an empty-range summary
// (-inf, 0) and a zero gather record, which say only that the item is done; the decision
// never uses them, because an earlier event ends the round.
__device__ __forceinline__ void stats_skip(const ChainParams& p, int b, int i, int slice) {
  if (threadIdx.x == 0) {
    publish_f2(p.part + ((size_t)b * p.R + i) * p.SL + slice, make_float2(-INFINITY, 0.0f));
    if (slice == 0 && i < p.G) gather_publish(p, b, i, 0u, 0u, 0u);
  }
}

template <int DT, int QT, bool VEC, bool PROC>
__device__ void stats_item(const ChainParams& p, int b, int i, int slice) {
  __shared__ float s_wm[kWavesPerBlock], s_wz[kWavesPerBlock];
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const size_t rowid = (size_t)b * p.R + i;
  // the first slice of a draft row also fetches the draft token, its logit and its draft
  // probability for the decision, overlapped with the streaming below
  const bool gathers = slice == 0 && i < p.G && threadIdx.x == 0;
  unsigned gx = 0, gl = 0, gq = 0;
  if (gathers) gather_issue<DT, QT, PROC>(p, b, i, gx, gl, gq);
  // sparse draft rows: the draft token and this thread's first entry are loaded before the
  // stream too, so the lookup after it costs no further memory round trip
  int sp_t = 0, sp_x0 = 0;
  float sp_v0 = 0.0f;
  bool sp_has0 = false;
  if constexpr (QT == kSparseQ) {
    if (slice == 0 && i < p.G) {
      sp_t = p.tokens[(size_t)b * p.G + i];
      const size_t base = ((size_t)b * p.G + i) * p.q_k;
      sp_has0 = (int)threadIdx.x < p.q_k;
      if (sp_has0) {
        sp_x0 = p.q_index[base + threadIdx.x];
        sp_v0 = static_cast<const float*>(p.q)[base + threadIdx.x];
      }
    }
  }
  // A row whose kept set the threshold pass summarized is not streamed: its first slice
  // publishes that summary and the others an empty range.
  float2 summ = make_float2(0.0f, 0.0f);
  if constexpr (PROC)
    if (p.summ_ws) summ = p.summ_ws[rowid];
  const bool summarized = summ.y > 0.0f;   // block-uniform
  if (!summarized) {
    // wave w streams chunks first + 4k of this slice (k < CPW)
    const long first = (long)slice * kWavesPerBlock * p.CPW + wave;
    float m, z;
    if constexpr (PROC)
      wave_row_summary_proc<DT, VEC>(p, rowid, first, lane, m, z);
    else
      wave_row_summary<DT, VEC>(row_ptr<DT>(p.logits, rowid, p.V), p.V, p.P, first, kWavesPerBlock, p.CPW, lane,
                                p.c2, m, z);
    if (lane == 0) {
      s_wm[wave] = m;
      s_wz[wave] = z;
    }
  }
  if constexpr (QT == kSparseQ) {
    if (slice == 0 && i < p.G) {        // block-uniform: the whole block searches the row
      __shared__ float s_q[kWavesPerBlock];
      const float qx = sparse_q_lookup(p, b, i, sp_t, s_q, sp_has0, sp_x0, sp_v0);
      if (gathers && sp_t >= 0 && sp_t < p.V) gq = __float_as_uint(qx);
    }
  }
  if (gathers) gather_publish(p, b, i, gx, gl, gq);
  __syncthreads();
  SPEC_STAMP(p, 0, 2);
  if (threadIdx.x == 0 && summarized) {
    publish_f2(p.part + rowid * p.SL + slice, slice == 0 ? summ : make_float2(-INFINITY, 0.0f));
  } else if (threadIdx.x == 0) {
    // the slice's summary: M = max of the waves' maxima, Z = sum of their sums rescaled
    // to M (NaN if any wave saw NaN or +inf; (-inf, 0) if every element was -inf).  Z >= 1
    // otherwise (the maximum contributes 2^0), so the published word is never zero.
    float M = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
      M = fmaxf(M, s_wm[w]);
      nan |= (s_wz[w] != s_wz[w]);
    }
    float Z = 0.0f;
    if (M != -INFINITY) {
      const float R = M * p.c2;
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w)
        if (s_wm[w] != -INFINITY) Z += s_wz[w] * __builtin_amdgcn_exp2f(s_wm[w] * p.c2 - R);
    }
    if (nan) Z = NAN;
    publish_f2(p.part + rowid * p.SL + slice, make_float2(M, Z));
  }
}


// The decision of request b from its published summaries and gather records.  Every
// terminal item of the request runs this on the same words and takes the same decision,
// which it leaves in `s_dec` (shared; valid after the final barrier).  Wave 0 does all of
// it with no block barrier until the end: lane l holds the summaries of one (row, slice)
// pair per pass -- rows in groups of S = 2^ceil(log2 SL) lanes (at most 64, lanes then
// looping over slices) -- and a row's maximum and normalizer come from segmented DPP
// reductions over its group.  With [lo, nr) != [0, R) only rows lo..nr-1 and drafts lo..nr-1
// are read (the gate of a lazy row group): then only `ev`, `H` and an INTERNAL status are
// meaningful.
__device__ __forceinline__ int seg_lanes(int SL) {
  int S = 1;
  while (S < SL && S < kWave) S <<= 1;
  return S;
}

template <int DT>
__device__ __forceinline__ void chain_decide(const ChainParams& p, int b, RowState& rs, ChainDecision& s_dec, int lo, int nr) {
  if (wave_id() != 0) {
    __syncthreads();
    return;
  }
  // the decision is a chain of dependent steps on the call's critical path, sharing its SIMD
  // with streaming waves: the highest wave priority lets it issue first (measured 1 us off
  // the headline call; levels 1 and 2 gave less, and raising the selector's waves as well
  // gave nothing)
  __builtin_amdgcn_s_setprio(3);
  constexpr int kPre = 4;                       // slices per lane and pass kept in registers
  const int lane = threadIdx.x & (kWave - 1);
  const float c2 = p.c2;
  const int G = p.G, R = p.R, SL = p.SL;
  const int nd = min(G, nr);                    // drafts decided
  const float2* part_b = p.part + (size_t)b * R * SL;
  const auto* words = reinterpret_cast<const unsigned long long*>(part_b);

  // independent reads first: lane i < G's gather record and uniform, the terminal uniform,
  // the budget, and lane l's stop entries l, l + 64, ...
  unsigned long long g[3] = {0ull, 0ull, 0ull};
  float ui = 0.0f;
  const bool dl = lane >= lo && lane < nd;      // this lane's draft is decided
  if (dl) {
    const unsigned long long* rec = gather_rec(p, b, lane);
#pragma unroll
    for (int k = 0; k < 3; ++k) g[k] = fetch_u64(rec + k);
    ui = p.u[(size_t)b * R + lane];
  }
  const float ut = p.u[(size_t)b * R + G];
  const int H = p.st.budget ? p.st.budget[b] : INT32_MAX;   // remaining output budget
  const float tau_lane = lane < R ? row_tau(p.pr, (size_t)b * R + lane) : -INFINITY;   // keep thresholds
  const int n_stop = p.st.n_stop;
  int stop_e[SPEC_MAX_STOP / kWave];
#pragma unroll
  for (int k = 0; k < SPEC_MAX_STOP / kWave; ++k) {
    const int j = lane + k * kWave;
    stop_e[k] = j < n_stop ? p.st.stop[j] : 0;
  }

  const int S = seg_lanes(SL), rows_per_pass = kWave / S, tpl = (SL + S - 1) / S;
  const int srow = lane / S, sj = lane & (S - 1);
  bool lost = false;
  for (int pass = lo / rows_per_pass; pass * rows_per_pass < nr; ++pass) {
    const int i = pass * rows_per_pass + srow;   // this lane's row
    const bool rv = i >= lo && i < nr;
    auto slice_ok = [&](int t) { return rv && sj + S * t < SL; };
    auto word = [&](int t) { return words + (size_t)i * SL + sj + S * t; };
    unsigned long long v[kPre];
#pragma unroll
    for (int t = 0; t < kPre; ++t) v[t] = t < tpl && slice_ok(t) ? fetch_u64(word(t)) : 1ull;
    // maximum over the row's slices
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < kPre; ++t) {
      if (t < tpl && slice_ok(t)) {
        if (v[t] == 0ull) v[t] = await_u64(word(t));
        lost |= (v[t] == 0ull);
        m = fmaxf(m, __uint_as_float(static_cast<unsigned>(v[t])));
      }
    }
    for (int t = kPre; t < tpl; ++t) {
      if (slice_ok(t)) {
        const unsigned long long w = await_u64(word(t));
        lost |= (w == 0ull);
        m = fmaxf(m, __uint_as_float(static_cast<unsigned>(w)));
      }
    }
    m = seg_max(m, S);
    const float r = m * c2;
    // Z = sum_j Z_j 2^(r_j - r); an all -inf row gives (-inf) - (-inf) = NaN, flagged below
    double z = 0.0;
#pragma unroll
    for (int t = 0; t < kPre; ++t) {
      if (t < tpl && slice_ok(t)) {
        const unsigned long long w = v[t];
        z += (double)__uint_as_float(static_cast<unsigned>(w >> 32)) *
             (double)__builtin_amdgcn_exp2f(__uint_as_float(static_cast<unsigned>(w)) * c2 - r);
      }
    }
    for (int t = kPre; t < tpl; ++t) {
      if (slice_ok(t)) {
        const unsigned long long w = fetch_u64(word(t));
        z += (double)__uint_as_float(static_cast<unsigned>(w >> 32)) *
             (double)__builtin_amdgcn_exp2f(__uint_as_float(static_cast<unsigned>(w)) * c2 - r);
      }
    }
    z = seg_sum_d(z, S);
    if (rv && sj == 0) {
      rs.r[i] = r;
      rs.m[i] = m;
      rs.z[i] = z;
      // all -inf, NaN or +inf anywhere: z is not a positive finite number
      rs.bad[i] = !(isfinite(z) && z > 0.0);
    }
  }
  SPEC_STAMP(p, 0, 8);   // summaries in, rows combined
  if (dl) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      if (g[k] == 0ull) g[k] = await_u64(gather_rec(p, b, lane) + k);
      lost |= (g[k] == 0ull);
    }
  }
  const bool timeout = wave_any(lost);
  SPEC_STAMP(p, 0, 9);   // gather records in
  // the row results travel through LDS within this wave: LDS operations of one wave complete
  // in order, and the fence keeps the compiler from moving the reads above the writes
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // stop tokens: bit i of `hits` is set when draft i is one of them
  const int x = static_cast<int>(static_cast<unsigned>(g[0]));
  unsigned long long hits = 0ull;
  if (n_stop > 0) {
    for (int i = lo; i < nd; ++i) {
      const int xi = __builtin_amdgcn_readlane(x, i);
      bool h = false;
#pragma unroll
      for (int k = 0; k < SPEC_MAX_STOP / kWave; ++k) h |= (lane + k * kWave < n_stop) && stop_e[k] == xi;
      if (wave_any(h)) hits |= 1ull << i;
    }
  }

  // lane i < G: draft position i, checked in the order a round reaches it; an accepted
  // draft that is a stop token, or that uses up the budget, ends the round after itself
  int code = 0, fin = 0;
  bool reject = false;
  double px = NAN, a = NAN;
  if (dl) {
    if (rs.bad[lane]) {
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
        px = exp2((double)lx * (double)c2 - (double)rs.r[lane]) / rs.z[lane];
        a = fmin(1.0, px / (double)qx);
        reject = !((double)ui < a);
        if (!reject) {
          if ((hits >> lane) & 1ull) fin = SPEC_FINISH_STOP;
          else if (lane + 1 == H) fin = SPEC_FINISH_BUDGET;
        }
      }
    }
    rs.px[lane] = px;
    rs.a[lane] = a;
  }
  const unsigned long long ev = __ballot(dl && (code != 0 || reject || fin != 0));
  const int e = ev ? (__ffsll((long long)ev) - 1) : G;   // the first event
  const int code_e = __shfl(code, e < G ? e : 0, kWave);
  const int fin_e = __shfl(fin, e < G ? e : 0, kWave);
  int A = e, status = 0, draw = 1, finish = 0;
  if (e < G && fin_e != 0) {          // the round ends on draft e, with no draw
    A = e + 1;
    draw = 0;
    finish = fin_e;
  } else {
    status = e < G ? code_e : (nr > G && rs.bad[G] ? SPEC_REQ_NONFINITE : 0);
    if (status == 0 && !(ut >= 0.0f && ut < 1.0f)) status = SPEC_REQ_BADUNIFORM;
  }
  if (H <= 0) {                       // no budget left: no round, nothing checked
    A = 0;
    status = 0;
    draw = 0;
    finish = SPEC_FINISH_BUDGET;
  }
  if (timeout) status = SPEC_REQ_INTERNAL;
  const float tau_a = __shfl(tau_lane, A < R ? A : 0, kWave);
  if (lane == 0) {
    const bool drawn = status == 0 && draw && A < nr;
    s_dec.ev = e;
    s_dec.tau = tau_a;
    s_dec.A = status == 0 ? A : -1;
    s_dec.status = status;
    s_dec.draw = drawn ? 1 : 0;
    s_dec.finish = finish;
    s_dec.H = H;
    s_dec.r_ref = drawn ? rs.r[A] : 0.0f;
    s_dec.inv_z = drawn ? (float)(1.0 / rs.z[A]) : 0.0f;
  }
  SPEC_STAMP(p, 0, 10);  // decided (before the block barrier)
  __builtin_amdgcn_s_setprio(0);
  __syncthreads();
}

// An empty asm on an element's input keeps the compiler from widening every element of a
// chunk to fp64 at once.
__device__ __forceinline__ float pin(float x) {
  asm volatile("" : "+v"(x));
  return x;
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

// The inputs of this thread's 8 elements in each slab of terminal chunk c, both slabs'
// loads issued together: the logits with the processors applied and (RESID) the q values
// (a sparse row densified per chunk in LDS).
template <int DT, int QT, bool VEC, bool RESID, bool PROC>
__device__ __forceinline__ void term_inputs(const ChainParams& p, const void* lrow, const void* qrow, int c,
                                            const ChainDecision& d, size_t rowid, float (&lv)[kTermSlabs][8],
                                            float (&qv)[kTermSlabs][8], bool& bad) {
#pragma unroll
  for (int s = 0; s < kTermSlabs; ++s) {
    const long e0 = ((long)c * kTermSlabs + s) * kSlab + (long)threadIdx.x * kVec;
    load8<DT, VEC, false>(lrow, e0, p.V, lv[s], -INFINITY);
    if constexpr (RESID && QT != kSparseQ) load8<QT, VEC, false>(qrow, e0, p.V, qv[s], 0.0f);
  }
  if constexpr (RESID && QT == kSparseQ) {
    // the chunk of the sparse row, densified in LDS: listed values added at their indices
    // (an entry with an index outside [0, V) makes the row invalid, like a negative value)
    __shared__ float s_qd[kTermChunk];
    __shared__ int s_qbad;
    const int tid = threadIdx.x;
    const size_t base = ((rowid / p.R) * p.G + d.A) * p.q_k;
    const float* val = static_cast<const float*>(p.q) + base;
    const int32_t* idx = p.q_index + base;
    const long lo = (long)c * kTermChunk;
    // this thread's first entry is loaded before the barrier, together with the logits
    // (the barrier waits for both), so the row costs one memory round trip, not two
    const bool has0 = tid < p.q_k;
    int x0 = 0;
    float v0 = 0.0f;
    if (has0) {
      x0 = idx[tid];
      v0 = val[tid];
    }
    for (int j = tid; j < kTermChunk; j += kBlock) s_qd[j] = 0.0f;
    if (tid == 0) s_qbad = 0;
    __syncthreads();
    auto add = [&](int x, float v) {
      if (x < 0 || x >= p.V || !(v >= 0.0f && v < INFINITY)) s_qbad = 1;
      else if (x >= lo && x < lo + kTermChunk) atomicAdd(&s_qd[x - lo], v);
    };
    if (has0) add(x0, v0);
    for (int j = tid + kBlock; j < p.q_k; j += kBlock) add(idx[j], val[j]);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kTermSlabs; ++s)
#pragma unroll
      for (int k = 0; k < 8; ++k) qv[s][k] = s_qd[s * kSlab + tid * kVec + k];
    bad |= (s_qbad != 0);
    __syncthreads();                    // s_qd is reused by the next call
  }
  if constexpr (PROC) {
#pragma unroll
    for (int s = 0; s < kTermSlabs; ++s)
      proc8<VEC>(p.pr, rowid, d.tau, ((long)c * kTermSlabs + s) * kSlab + (long)threadIdx.x * kVec, p.V, lv[s]);
  }
}

// The weights of this thread's 8 elements in each slab of terminal chunk c.
template <int DT, int QT, bool VEC, bool RESID, bool PROC>
__device__ __forceinline__ void term_chunk(const ChainParams& p, const void* lrow, const void* qrow, int c,
                                           const ChainDecision& d, size_t rowid, float (&w)[kTermSlabs][8],
                                           bool& bad) {
  float lv[kTermSlabs][8], qv[kTermSlabs][8];
  term_inputs<DT, QT, VEC, RESID, PROC>(p, lrow, qrow, c, d, rowid, lv, qv, bad);
#pragma unroll
  for (int s = 0; s < kTermSlabs; ++s)
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w[s][k] = term_weight<RESID>(lv[s][k], RESID ? qv[s][k] : 0.0f, p.c2, d.r_ref, d.inv_z, bad);
}

// Block sum (fp64) of this thread's weights; NaN if any thread saw a bad q entry.
__device__ __forceinline__ double block_mass(const float (&w)[kTermSlabs][8], bool bad) {
  __shared__ double s_red[kWavesPerBlock];
  double acc = 0.0;
#pragma unroll
  for (int s = 0; s < kTermSlabs; ++s)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += (double)w[s][k];
  if (bad) acc = NAN;
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const double ws = wave_sum_d(acc);
  if (lane == 0) s_red[wave] = ws;
  __syncthreads();
  const double m = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  __syncthreads();
  return m;
}

// Chunk masses are read in runs of up to kMassRegs per thread and kept in registers;
// longer runs (vocabularies beyond 8M) re-read the published words.
constexpr int kMassRegs = 8;

// A rejection whose residual mass (from the fp32 terminal weights) is below this is drawn
// again, exactly, by chain_exact_kernel.
constexpr double kExactBelow = 0.05;
// Terminal chunks each block of chain_exact_kernel covers: the kernel runs after every chain
// call, almost always to find nothing to redraw, and fewer blocks find that sooner.
constexpr int kExactChunks = 8;
__host__ __device__ __forceinline__ int exact_blocks(int S2) { return (S2 + kExactChunks - 1) / kExactChunks; }

// Statistics of row i: (m, log Z, p(x), a) of a reached draft row, (m, log Z, NaN, NaN)
// of the reached bonus row, NaN otherwise.
__device__ __forceinline__ void row_stats(const ChainParams& p, const RowState& rs, int i, bool reached,
                                          float (&v)[4]) {
  v[0] = v[1] = v[2] = v[3] = NAN;
  if (!reached) return;
  v[0] = (float)((double)rs.m[i] * p.inv_t);
  // log Z = log sum 2^((l - m) c2) = log z + (r - m c2) ln 2: relative to the row's own
  // maximum, so that the fp32 rounding of c2 enters only through (l - m) (written as
  // log z + r ln 2 - m / T it would add m (c2 ln 2 - 1/T), about 1e-4 at m / T = 1800)
  v[1] = (float)(log(rs.z[i]) + ((double)rs.r[i] - (double)rs.m[i] * (double)p.c2) * kLn2);
  if (i < p.G) {
    v[2] = (float)rs.px[i];
    v[3] = (float)rs.a[i];
  }
}

// Every other terminal item of request b has published its chunk's mass, and so has
// finished reading the request's summaries and gather records: return them to zero.  xd:
// the decision of a draw that the exact kernel redoes, whose record then takes the
// request's first two summary words (R * SL >= 2 whenever there is a residual); the exact
// kernel clears them.
__device__ void chain_clear_summaries(const ChainParams& p, int b, const ChainDecision* xd) {
  const int tid = threadIdx.x;
  float2* part_b = p.part + (size_t)b * p.R * p.SL;
  for (int j = tid; j < p.R * p.SL; j += kBlock) {
    if (xd && j < 2) {
      const unsigned lo = j == 0 ? static_cast<unsigned>(xd->A + 1) : __float_as_uint(xd->inv_z);
      const unsigned hi = j == 0 ? __float_as_uint(xd->r_ref) : __float_as_uint(xd->tau);
      publish_u64(reinterpret_cast<unsigned long long*>(part_b + j), (unsigned long long)hi << 32 | lo);
    } else {
      clear_f2(part_b + j);
    }
  }
  for (int j = tid; j < 3 * p.G; j += kBlock) clear_u64(gather_rec(p, b, 0) + j);
  if (p.thresh_ws)   // written by the threshold pass, read by this request's blocks only
    for (int j = tid; j < p.R; j += kBlock) store_wt(p.thresh_ws + (size_t)b * p.R + j, 0.0f);
  if (p.summ_ws)
    for (int j = tid; j < p.R; j += kBlock) clear_f2(p.summ_ws + (size_t)b * p.R + j);
}
// ... and the chunk masses, once the selector has read them for the last time.
__device__ void chain_clear_masses(const ChainParams& p, int b) {
  for (int j = threadIdx.x; j < p.S2; j += kBlock) clear_mass(p.tmass + (size_t)b * p.S2 + j);
}

// The selector of request b: every other chunk's mass is awaited; then the chunk where the
// running mass passes u_gamma * W is rescanned in vocabulary order and the outputs are
// written.  `own` is the mass of chunk S2 - 1, which the selector computed itself.
template <int DT, int QT, bool VEC, bool RESID, bool PROC>
__device__ void chain_select(const ChainParams& p, int b, const ChainDecision& d, const RowState& rs,
                             double own, const void* lrow, const void* qrow) {
  __shared__ double s_scan[kWavesPerBlock];
  __shared__ double s_scan2[2 * kWavesPerBlock];
  __shared__ int s_imin[kWavesPerBlock];
  __shared__ int s_imin2[2 * kWavesPerBlock];
  __shared__ int s_timeout, s_cstar;
  __shared__ double s_before, s_total;
  const int tid = threadIdx.x, G = p.G;
  const double* tm = p.tmass + (size_t)b * p.S2;
  const float ut = p.u[(size_t)b * p.R + G];
  // stop-token entry t, fetched while the masses are awaited (tested against the token)
  const int my_stop = tid < p.st.n_stop ? p.st.stop[tid] : 0;
  if (tid == 0) {
    s_timeout = 0;
    s_before = 0.0;
  }
  __syncthreads();

  // 1. running mass over the chunks in order: thread t owns a contiguous run of chunks
  //    and extends the block-exclusive prefix over it.  W is the running value after the
  //    last chunk, computed the same way, so u * W < W always finds a chunk whose running
  //    value exceeds the target.  With at most 64 chunks they all sit in wave 0, one per
  //    lane, whose prefix is the block-wide one (the other waves add zeros), and wave 0
  //    also picks the chunk: one barrier instead of the block scans' five.
  const bool one_wave = p.S2 <= kWave;
  const int per = (p.S2 + kBlock - 1) / kBlock;
  const int c_lo = min(tid * per, p.S2), c_hi = min(c_lo + per, p.S2);
  double mv[kMassRegs];
  bool lost = false;
  auto mass_at = [&](int c) -> double {
    if (c == p.S2 - 1) return own;
    const unsigned long long bits = await_u64(reinterpret_cast<const unsigned long long*>(tm + c));
    lost |= (bits == 0ull);
    return -__longlong_as_double(static_cast<long long>(bits));
  };
  double mine = 0.0, excl = 0.0;
  if (one_wave) {
    if (tid < kWave) {                  // wave 0: lane c holds chunk c (c_lo = c, per = 1)
      mine = c_lo < c_hi ? mass_at(c_lo) : 0.0;
      mv[0] = mine;
      excl = 0.0 + wave_shr1_d(wave_incl_scan_d(mine, tid));   // as block_excl_scan_d forms it
      const double Wl = __shfl(excl + mine, p.S2 - 1, kWave);
      const bool lost_w = wave_any(lost);
      const bool failed_w = lost_w || !(isfinite(Wl) && Wl > 0.0);
      int cs = p.S2 - 1;
      if (!failed_w) {
        const double t = (double)ut * Wl;
        const unsigned long long hit = __ballot(c_lo < c_hi && excl + mine > t);
        if (hit) cs = __ffsll(static_cast<long long>(hit)) - 1;
      }
      const double before = __shfl(excl, cs, kWave);
      if (tid == 0) {
        s_total = Wl;
        s_timeout = lost_w ? 1 : 0;
        s_before = before;
        s_cstar = cs;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kMassRegs; ++k) {
      const int c = c_lo + k;
      mv[k] = c < c_hi ? mass_at(c) : 0.0;
      mine += mv[k];
    }
    for (int c = c_lo + kMassRegs; c < c_hi; ++c) mine += mass_at(c);
    if (lost) s_timeout = 1;
    double tot;
    excl = block_excl_scan_d(mine, s_scan, &tot);
    if (c_lo < c_hi && c_hi == p.S2) s_total = excl + mine;
  }
  __syncthreads();
  const double W = s_total;
  const bool failed = s_timeout || !(isfinite(W) && W > 0.0);   // uniform across the block
  SPEC_STAMP(p, 0, 4);
  // every other terminal item is done with the request's words: clear them now, so that the
  // clears complete under the rescan
  const bool exact = RESID && !failed && W < kExactBelow;
  chain_clear_summaries(p, b, exact ? &d : nullptr);
  double t = 0.0;
  int k = -1;
  if (failed) chain_clear_masses(p, b);
  if (!failed) {
    t = (double)ut * W;
    int cstar = s_cstar;            // (one wave: picked already)
    if (!one_wave) {
      int cand = 0x7fffffff;        // first chunk of this thread's run whose running value passes t
      double run = excl;
      for (int c = c_lo; c < c_hi; ++c) {
        const double mc = c - c_lo < kMassRegs ? mv[c - c_lo] : mass_at(c);
        const double nxt = run + mc;
        if (nxt > t) {
          cand = c;
          break;
        }
        run = nxt;
      }
      // a chunk is always found (t < W and the last running value is W); clamp regardless
      cstar = block_min_i(cand, s_imin);
      if (cstar == 0x7fffffff) cstar = p.S2 - 1;
      if (cstar >= c_lo && cstar < c_hi) {       // the owner of cstar records the mass before it
        double before = excl;
        for (int c = c_lo; c < cstar; ++c) before += c - c_lo < kMassRegs ? mv[c - c_lo] : mass_at(c);
        s_before = before;
      }
      __syncthreads();
    }
    const double rem = t - s_before;   // target mass inside chunk cstar
    chain_clear_masses(p, b);          // every thread has read its masses for the last time
    SPEC_STAMP(p, 0, 11);   // chunk picked

    // 2. rescan cstar in vocabulary order: slab 0 then slab 1, each thread's 8 elements
    //    in order within a slab
    float w[kTermSlabs][8];
    bool bad = false;
    term_chunk<DT, QT, VEC, RESID, PROC>(p, lrow, qrow, cstar, d, (size_t)b * p.R + d.A, w, bad);
    SPEC_STAMP(p, 0, 12);   // chunk reloaded, weights formed
    static_assert(kTermSlabs == 2, "the rescan scans two slabs in one pass");
    double acc[kTermSlabs];
    unsigned pos_mask[kTermSlabs];
#pragma unroll
    for (int s = 0; s < kTermSlabs; ++s) {
      acc[s] = 0.0;
      pos_mask[s] = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[s] += (double)w[s][j];
        pos_mask[s] |= (w[s][j] > 0.0f ? 1u : 0u) << j;
      }
    }
    double off[kTermSlabs], slab_total[kTermSlabs];
    block_excl_scan_d2(acc[0], acc[1], s_scan2, &off[0], &off[1], &slab_total[0], &slab_total[1]);
    off[1] += 0.0 + slab_total[0];
    int last_pos = -1, pick = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < kTermSlabs; ++s) {
      const int e0 = (int)(((long)cstar * kTermSlabs + s) * kSlab + (long)tid * kVec);
      unsigned hit = 0u;
      double run = 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        run += (double)pin(w[s][j]);
        hit |= (off[s] + run > rem ? 1u : 0u) << j;
      }
      hit &= pos_mask[s];
      if (hit) pick = min(pick, e0 + __builtin_ctz(hit));
      if (pos_mask[s]) last_pos = max(last_pos, e0 + 31 - __builtin_clz(pos_mask[s]));
    }
    // the first position whose running value passes the target; rounding may leave the
    // target just past the chunk's last positive weight: then take that weight
    int last_any;
    pick = block_min_max_i(pick, last_pos, s_imin2, &last_any);
    k = pick != 0x7fffffff ? pick : last_any;
  }
  SPEC_STAMP(p, 0, 5);

  // 3. outputs
  const int A = d.A;
  const int status = s_timeout ? SPEC_REQ_INTERNAL : (failed ? SPEC_REQ_RESIDUAL_EMPTY : 0);
  // a terminal token that is a stop token, or that uses up the budget, finishes the request
  int finish = 0;
  if (p.st.n_stop > 0 && __syncthreads_or(tid < p.st.n_stop && my_stop == k)) finish = SPEC_FINISH_STOP;
  else if (A + 1 == d.H) finish = SPEC_FINISH_BUDGET;
  if (status != 0) finish = 0;
  for (int i = tid; i < p.R; i += kBlock) {
    int v = -1;
    if (status == 0) {
      if (i < A) v = p.tokens[(size_t)b * G + i];
      else if (i == A) v = k;
    }
    p.out_tokens[(size_t)b * p.R + i] = v;
  }
  if (p.stats) {
    // rows 0..A (< G) reached: (m, log Z, p(x), a); row G: (m, log Z) when the bonus row
    // is reached, W in column 2; everything else NaN, and everything on failure
    float* st = p.stats + (size_t)b * p.R * 4;
    for (int i = tid; i < p.R; i += kBlock) {
      float v[4];
      row_stats(p, rs, i, status == 0 && (i < G ? i <= A : A == G), v);
      if (i == G && status == 0) v[2] = (float)W;
#pragma unroll
      for (int c = 0; c < 4; ++c) st[i * 4 + c] = v[c];
    }
  }
  if (tid == 0) {
    p.accepted_len[b] = status == 0 ? A : -1;
    p.req_status[b] = status;
    if (p.st.finish) p.st.finish[b] = finish;
  }
  SPEC_STAMP(p, 0, 6);
}

// A request with no terminal draw -- a failed request, or a round that ended on an
// accepted draft (a stop token, or the last token of the budget) or had no budget left:
// the selector writes its record once every other terminal item has signalled that it is
// done with the request.
__device__ void chain_nodraw(const ChainParams& p, int b, const ChainDecision& d, const RowState& rs) {
  const int tid = threadIdx.x;
  __shared__ int s_lost;
  if (tid == 0) s_lost = 0;
  __syncthreads();
  const double* tm = p.tmass + (size_t)b * p.S2;
  for (int c = tid; c < p.S2 - 1; c += kBlock)
    if (await_u64(reinterpret_cast<const unsigned long long*>(tm + c)) == 0ull) s_lost = 1;
  __syncthreads();
  const int code = s_lost ? SPEC_REQ_INTERNAL : d.status;
  const int A = code == 0 ? d.A : 0;   // drafts emitted; their rows are the ones tested
  for (int i = tid; i < p.R; i += kBlock)
    p.out_tokens[(size_t)b * p.R + i] = i < A ? p.tokens[(size_t)b * p.G + i] : -1;
  if (p.stats) {
    float* st = p.stats + (size_t)b * p.R * 4;
    for (int i = tid; i < p.R; i += kBlock) {
      float v[4];
      row_stats(p, rs, i, i < A, v);
#pragma unroll
      for (int c = 0; c < 4; ++c) st[i * 4 + c] = v[c];
    }
  }
  if (tid == 0) {
    p.accepted_len[b] = code == 0 ? A : -1;
    p.req_status[b] = code;
    if (p.st.finish) p.st.finish[b] = code == 0 ? d.finish : 0;
  }
}

// Terminal item with a valid decision: chunk c of request b's terminal row; the last
// chunk's item selects.
template <int DT, int QT, bool VEC, bool RESID, bool PROC>
__device__ void terminal_body(const ChainParams& p, int b, int c, const ChainDecision& d, const RowState& rs) {
  const void* lrow = row_ptr<DT>(p.logits, (size_t)b * p.R + d.A, p.V);
  const void* qrow = nullptr;
  if constexpr (RESID && QT != kSparseQ) qrow = row_ptr<QT>(p.q, (size_t)b * p.G + d.A, p.V);
  float w[kTermSlabs][8];
  bool bad = false;
  term_chunk<DT, QT, VEC, RESID, PROC>(p, lrow, qrow, c, d, (size_t)b * p.R + d.A, w, bad);
  const double m = block_mass(w, bad);
  SPEC_STAMP(p, 0, 3);
  if (c != p.S2 - 1) {
    if (threadIdx.x == 0) publish_mass(p.tmass + (size_t)b * p.S2 + c, m);
    return;
  }
  chain_select<DT, QT, VEC, RESID, PROC>(p, b, d, rs, m, lrow, qrow);
  SPEC_STAMP(p, 0, 7);
}

// Terminal item with the request's decision taken (chain_decide over every row).
template <int DT, int QT, bool VEC, bool PROC>
__device__ void terminal_item(const ChainParams& p, int b, int c, RowState& s_rs, ChainDecision& s_dec) {
  const ChainDecision d = s_dec;
  if (d.status != 0 || !d.draw) {
    if (c != p.S2 - 1) {
      // no mass to contribute: a NaN marker says only that this item is done with the
      // request's words
      if (threadIdx.x == 0) publish_mass(p.tmass + (size_t)b * p.S2 + c, NAN);
      return;
    }
    chain_nodraw(p, b, d, s_rs);
    __syncthreads();
    chain_clear_summaries(p, b, nullptr);
    chain_clear_masses(p, b);
    return;
  }
  if (d.A < p.G) terminal_body<DT, QT, VEC, true, PROC>(p, b, c, d, s_rs);
  else terminal_body<DT, QT, VEC, false, PROC>(p, b, c, d, s_rs);
}

// ------------------------------------------------------------ exact draw of small residuals
// A rejection's terminal token inverts the CDF of max(p - q, 0) normalized by its mass W, so
// every rounding error of the weights reaches that CDF multiplied by 1/W.  The terminal
// items above use fp32 weights (relative errors near 1e-7: the hardware exp2, the fp32
// exponent, the fp32 normalizer), safe while W is large -- the workloads' rejections keep
// W above 0.17 -- but at high acceptance W falls to 1e-3 and below, where such errors can
// move a CDF boundary by more than the 1e-6 that separates an exact draw from a near-tie.
// There the selector leaves a record (A + 1, r, 1/Z, tau) and this kernel, launched after
// the chain kernel, draws again in fp64: e(x) = 2^(l c2d - r) from exp2_acc (c2d = log2(e)/T
// in fp64), and the normalizer Z = sum e over the same e, so that p = e / Z is consistent
// with the weights.  Each block sums its chunk's
//   M = sum max(e / Za - q, 0),   D = sum of e over the elements with a positive weight,
//   E = sum e,
// with Za the statistics stream's normalizer; the request's last block forms Z = sum E and
// the exact chunk masses to first order, M' = M + (1/Z - 1/Za) D (what is left over comes
// from elements whose sign flips between Za and Z, |p - q| within |Z - Za| / Z of p: second
// order, near 1e-12), selects the chunk where the running mass passes u * W, rescans it with
// the weights at 1/Z, and overwrites the request's token, W and finish.  Blocks of requests
// without a record return at once.  It is a kernel of its own so that its fp64 registers
// do not lower the chain kernel's occupancy.

// One element's exact weight at 1/Z = iz; e(x) is returned too.
__device__ __forceinline__ double exact_w(float l, float q, double c2d, double r, double iz, double& e) {
  e = exp2_acc(fma((double)l, c2d, -r));
  const double t = e * iz - (double)q;
  return t > 0.0 ? t : 0.0;
}

// Request b fails with `status`: no tokens, NaN statistics (block-wide).
__device__ void chain_fail(const ChainParams& p, int b, int status) {
  const int tid = threadIdx.x;
  for (int i = tid; i < p.R; i += kBlock) p.out_tokens[(size_t)b * p.R + i] = -1;
  if (p.stats)
    for (int i = tid; i < 4 * p.R; i += kBlock) p.stats[(size_t)b * p.R * 4 + i] = NAN;
  if (tid == 0) {
    p.accepted_len[b] = -1;
    p.req_status[b] = status;
    if (p.st.finish) p.st.finish[b] = 0;
  }
}

// Every workspace word of request b back to zero (block-wide).
__device__ void chain_scrub(const ChainParams& p, int b) {
  const int tid = threadIdx.x;
  float2* part_b = p.part + (size_t)b * p.R * p.SL;
  for (int j = tid; j < p.R * p.SL; j += kBlock) clear_f2(part_b + j);
  for (int j = tid; j < 3 * p.G; j += kBlock) clear_u64(gather_rec(p, b, 0) + j);
  for (int j = tid; j < p.S2; j += kBlock) clear_mass(p.tmass + (size_t)b * p.S2 + j);
  for (int j = tid; j < 3 * p.S2; j += kBlock) clear_mass(p.xmass + (size_t)b * p.S2 * 3 + j);
  if (p.thresh_ws)
    for (int j = tid; j < p.R; j += kBlock) store_wt(p.thresh_ws + (size_t)b * p.R + j, 0.0f);
  if (p.summ_ws)
    for (int j = tid; j < p.R; j += kBlock) clear_f2(p.summ_ws + (size_t)b * p.R + j);
}

__device__ __forceinline__ double* xmass_word(const ChainParams& p, int b, int c, int k) {
  return p.xmass + ((size_t)b * p.S2 + c) * 3 + k;
}

template <int DT, int QT, bool VEC, bool PROC>
__global__ __launch_bounds__(kBlock) void chain_exact_kernel(ChainParams p) {
  __shared__ double s_red[3][kWavesPerBlock];
  __shared__ double s_scan[kWavesPerBlock];
  __shared__ int s_imin[kWavesPerBlock];
  __shared__ int s_lost;
  __shared__ double s_before, s_total;
  __shared__ double s_own[kExactChunks][3];   // the selecting block's own chunks' sums
  const int X = exact_blocks(p.S2);
  const int b = blockIdx.x / X, x = blockIdx.x % X;
  const int c_begin = x * kExactChunks, c_end = min(c_begin + kExactChunks, p.S2);
  const bool selects = x == X - 1;
  SPEC_STAMP(p, 1, 1);
  unsigned* rec = reinterpret_cast<unsigned*>(p.part + (size_t)b * p.R * p.SL);
  const unsigned pend = rec[0];
  const int chain_status = p.req_status[b];
  const unsigned dirty = fetch_u32(dirty_word(p.part));
  SPEC_TAG(p, 1, SPEC_TRACE_TAG(pend ? kTraceExact : kTraceExactIdle, b, x));
  if (dirty != 0u || chain_status == SPEC_REQ_INTERNAL) {
    // A wait of the chain kernel gave up on this request: a word published after its
    // consumer cleared it may be left over.  Every block of the chain kernel has finished
    // now, so zeroing the request's words here leaves them clean for later calls.  On a
    // dirty workspace (a wait of an earlier call gave up) no result of this call can be
    // trusted: every request fails.
    if (x == 0) {
      if (dirty != 0u) chain_fail(p, b, SPEC_REQ_INTERNAL);
      chain_scrub(p, b);
    }
    return;
  }
  if (pend == 0u) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
  ChainDecision d{};
  d.A = static_cast<int>(pend) - 1;
  d.r_ref = __uint_as_float(rec[1]);
  d.inv_z = __uint_as_float(rec[2]);
  d.tau = __uint_as_float(rec[3]);
  const size_t rowid = (size_t)b * p.R + d.A;
  const void* lrow = row_ptr<DT>(p.logits, rowid, p.V);
  const void* qrow = nullptr;
  if constexpr (QT != kSparseQ) qrow = row_ptr<QT>(p.q, (size_t)b * p.G + d.A, p.V);
  const double r = (double)d.r_ref, iza = (double)d.inv_z;

  // 1. the sums of this block's chunks, one chunk at a time
  float lv[kTermSlabs][8], qv[kTermSlabs][8];
  bool bad = false;
  if (tid == 0) {
    s_lost = 0;
    s_before = 0.0;
  }
  for (int c = c_begin; c < c_end; ++c) {
    term_inputs<DT, QT, VEC, true, PROC>(p, lrow, qrow, c, d, rowid, lv, qv, bad);
    double m = 0.0, dm = 0.0, em = 0.0;
#pragma unroll
    for (int s = 0; s < kTermSlabs; ++s)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        double e;
        const double w = exact_w(pin(lv[s][k]), pin(qv[s][k]), p.c2d, r, iza, e);
        m += w;
        em += e;
        dm += w > 0.0 ? e : 0.0;
      }
    if (bad) m = NAN;
    const double wm = wave_sum_d(m), wd = wave_sum_d(dm), we = wave_sum_d(em);
    if (lane == 0) {
      s_red[0][wave] = wm;
      s_red[1][wave] = wd;
      s_red[2][wave] = we;
    }
    __syncthreads();
    if (tid < 3) {
      const double v = (s_red[tid][0] + s_red[tid][1]) + (s_red[tid][2] + s_red[tid][3]);
      if (selects) s_own[c - c_begin][tid] = v;
      else publish_mass(xmass_word(p, b, c, tid), v);
    }
    __syncthreads();
  }
  if (!selects) {
    SPEC_STAMP(p, 1, 3);
    return;
  }

  // 2. the request's last block: every chunk's sums (the others' re-read where needed)
  const int G = p.G, A = d.A;
  const float ut = p.u[(size_t)b * p.R + G];
  const int my_stop = tid < p.st.n_stop ? p.st.stop[tid] : 0;
  auto word = [&](int cc, int k) -> double {
    if (cc >= c_begin) return s_own[cc - c_begin][k];
    const unsigned long long bits = await_u64(reinterpret_cast<const unsigned long long*>(xmass_word(p, b, cc, k)));
    if (bits == 0ull) s_lost = 1;
    return -__longlong_as_double(static_cast<long long>(bits));
  };
  const int per = (p.S2 + kBlock - 1) / kBlock;
  const int c_lo = min(tid * per, p.S2), c_hi = min(c_lo + per, p.S2);
  double e_mine = 0.0;
  for (int cc = c_lo; cc < c_hi; ++cc) e_mine += word(cc, 2);
  double Z;
  block_excl_scan_d(e_mine, s_scan, &Z);          // the same total in every thread
  const double iz = 1.0 / Z, diz = iz - iza;
  auto mass = [&](int cc) { return fma(diz, word(cc, 1), word(cc, 0)); };
  double mine = 0.0;
  for (int cc = c_lo; cc < c_hi; ++cc) mine += mass(cc);
  double tot;
  const double excl = block_excl_scan_d(mine, s_scan, &tot);
  if (c_lo < c_hi && c_hi == p.S2) s_total = excl + mine;
  __syncthreads();
  const double W = s_total;
  const bool failed = s_lost || !(isfinite(W) && W > 0.0);   // uniform across the block
  int k = -1;
  if (!failed) {
    // the chunk where the running mass passes u * W (as in chain_select), then its rescan
    const double t = (double)ut * W;
    int cand = 0x7fffffff;
    double run = excl, prev = excl, before = 0.0;
    for (int cc = c_lo; cc < c_hi; ++cc) {
      const double nxt = run + mass(cc);
      if (nxt > t) {
        cand = cc;
        before = run;
        break;
      }
      prev = run;
      run = nxt;
    }
    int cstar = block_min_i(cand, s_imin);
    if (cstar == 0x7fffffff) {                     // rounding left t past the last chunk
      cstar = p.S2 - 1;
      if (c_lo < c_hi && c_hi == p.S2) s_before = prev;
    } else if (cstar == cand) {
      s_before = before;
    }
    __syncthreads();
    const double rem = t - s_before;
    term_inputs<DT, QT, VEC, true, PROC>(p, lrow, qrow, cstar, d, rowid, lv, qv, bad);
    double before_slab = 0.0;
    int last_pos = -1, pick = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < kTermSlabs; ++s) {
      const long e0 = ((long)cstar * kTermSlabs + s) * kSlab + (long)tid * kVec;
      double w[8];
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        double e;
        w[j] = exact_w(pin(lv[s][j]), pin(qv[s][j]), p.c2d, r, iz, e);
        acc += w[j];
        if (w[j] > 0.0) last_pos = (int)(e0 + j);
      }
      double slab_total;
      const double off = before_slab + block_excl_scan_d(acc, s_scan, &slab_total);
      int cj = 0x7fffffff;
      double incl = 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        incl += w[j];
        if (cj == 0x7fffffff && off + incl > rem && w[j] > 0.0) cj = (int)(e0 + j);
      }
      pick = min(pick, cj);
      before_slab += slab_total;
    }
    pick = block_min_i(pick, s_imin);
    k = pick != 0x7fffffff ? pick : -block_min_i(-last_pos, s_imin);
  }

  // 3. outputs: the drawn token, W and finish; a request with no exact residual mass (or a
  //    sum that never arrived) fails as a whole, as in chain_select
  const int status = s_lost ? SPEC_REQ_INTERNAL : (failed ? SPEC_REQ_RESIDUAL_EMPTY : 0);
  int finish = 0;
  if (p.st.n_stop > 0 && __syncthreads_or(tid < p.st.n_stop && my_stop == k)) finish = SPEC_FINISH_STOP;
  else if (p.st.budget && A + 1 == p.st.budget[b]) finish = SPEC_FINISH_BUDGET;
  if (status == 0) {
    if (tid == 0) {
      p.out_tokens[(size_t)b * p.R + A] = k;
      if (p.stats) p.stats[((size_t)b * p.R + G) * 4 + 2] = (float)W;
      if (p.st.finish) p.st.finish[b] = finish;
    }
  } else {
    chain_fail(p, b, status);
    // this kernel's own words may arrive after the clear below: nothing follows to repair it
    if (status == SPEC_REQ_INTERNAL && tid == 0) publish_u32(dirty_word(p.part), 1u);
  }
  // every other block of the request has published its sums, and so has read the record
  __syncthreads();
  for (int j = tid; j < 3 * p.S2; j += kBlock) clear_mass(p.xmass + (size_t)b * p.S2 * 3 + j);
  if (tid < 4) rec[tid] = 0u;
  SPEC_STAMP(p, 1, 3);
}

// Block order: groups g = 0 .. B + L - 1, group g holding the Sb statistics items of
// request g (if g < B) followed by the Tb terminal items of request g - L (if g >= L), so a
// request's terminal items follow its statistics items by L requests' worth of blocks.
// L = B puts every statistics item first.  32-bit arithmetic: a grid holds fewer than
// 2^24 blocks.
struct Item { int terminal, b, idx; };
__host__ __device__ __forceinline__ Item tail_item(unsigned t, unsigned B, unsigned Sb, unsigned Tb, unsigned L) {
  const unsigned n1 = L * Sb, n2 = (B - L) * (Sb + Tb);
  Item it;
  if (t < n1) {
    it.terminal = 0; it.b = (int)(t / Sb); it.idx = (int)(t - (unsigned)it.b * Sb);
  } else if (t < n1 + n2) {
    const unsigned u = t - n1, k = u / (Sb + Tb), o = u - k * (Sb + Tb);
    if (o < Sb) { it.terminal = 0; it.b = (int)(L + k); it.idx = (int)o; }
    else { it.terminal = 1; it.b = (int)k; it.idx = (int)(o - Sb); }
  } else {
    const unsigned u = t - n1 - n2, k = u / Tb;
    it.terminal = 1; it.b = (int)(B - L + k); it.idx = (int)(u - k * Tb);
  }
  return it;
}

__host__ __device__ __forceinline__ Item block_item(const ChainParams& p, unsigned t) {
  return tail_item(t, p.B, (unsigned)(p.R * p.SL), p.S2, p.LAG);
}

// Lazy-rows order: row group j (rows [j LK, (j + 1) LK)) of every request, for j = 0 .. J-2
// in turn, then the last group interleaved with the terminal items as above.  A group's
// items thus follow every item of the request's earlier groups.  (Interleaving the earlier
// groups with lags as well measured slower: their gates and the terminal items then hold
// slots that the first group's stream needs.)
__host__ __device__ __forceinline__ Item lazy_item(const ChainParams& p, unsigned t) {
  const unsigned B = p.B, SL = p.SL, LK = p.LK, J = p.J;
  const unsigned nG = LK * SL, layer = B * nG, early = (J - 1) * layer;
  Item it;
  if (t < early) {
    const unsigned j = t / layer, u = t - j * layer, b = u / nG;
    it.terminal = 0; it.b = (int)b; it.idx = (int)(j * nG + (u - b * nG));
    return it;
  }
  const unsigned first = (J - 1) * LK;   // the last group's first row
  it = tail_item(t - early, B, ((unsigned)p.R - first) * SL, p.S2, p.LAG);
  if (!it.terminal) it.idx += (int)(first * SL);
  return it;
}

template <int DT, int QT, bool VEC, bool PROC>
// Waves per SIMD the register allocation must allow (0: whatever the code needs).
#ifndef SPEC_CHAIN_WAVES_PER_EU
#define SPEC_CHAIN_WAVES_PER_EU 0
#endif
#if SPEC_CHAIN_WAVES_PER_EU > 0
__global__ __launch_bounds__(kBlock, SPEC_CHAIN_WAVES_PER_EU) void chain_kernel(ChainParams p) {
#else
__global__ __launch_bounds__(kBlock) void chain_kernel(ChainParams p) {
#endif
  __shared__ RowState s_rs;
  __shared__ ChainDecision s_dec;
  SPEC_STAMP(p, 0, 1);
  const Item it = p.J > 1 ? lazy_item(p, blockIdx.x) : block_item(p, blockIdx.x);
  const int row = it.idx / p.SL;
  // the rows whose words this block's decision reads: every row for a terminal item; for
  // a lazy row group after the first, the rows of the group before it, which decide whether
  // the round reaches this group (it does when the group before it was reached and none
  // of that group's drafts ends the round; a skipped group's markers read as invalid rows,
  // an event at its first draft)
  int lo = 0, nr = 0;
  bool reached = true;
  if (it.terminal) {
    nr = p.R;
  } else if (p.J > 1) {
    const int first = (row / p.LK) * p.LK;
    if (first == 0) reached = p.st.budget == nullptr || p.st.budget[it.b] > 0;
    else { lo = first - p.LK; nr = first; }
  }
  if (nr > 0) chain_decide<DT>(p, it.b, s_rs, s_dec, lo, nr);   // one call site: inlined once
  if (it.terminal) {
    SPEC_STAMP(p, 0, 2);
    SPEC_TAG(p, 0, SPEC_TRACE_TAG(it.idx == p.S2 - 1 ? kTraceSelector : kTraceTerminal, it.b, it.idx));
    terminal_item<DT, QT, VEC, PROC>(p, it.b, it.idx, s_rs, s_dec);
    return;
  }
  if (nr > 0) {
    // a gate that timed out answers yes, so that no row the terminal items may need is skipped
    const ChainDecision d = s_dec;
    reached = d.status == SPEC_REQ_INTERNAL || (d.ev >= nr && d.H > 0);
  }
  SPEC_TAG(p, 0, SPEC_TRACE_TAG(reached ? kTraceStats : kTraceSkipped, it.b, it.idx));
  if (reached) stats_item<DT, QT, VEC, PROC>(p, it.b, row, it.idx % p.SL);
  else stats_skip(p, it.b, row, it.idx % p.SL);
  SPEC_STAMP(p, 0, 3);
}

// Lag between a request's statistics and terminal items, in rounds of resident blocks:
// its terminal items start about that many block generations after its statistics
// items, when their summaries are normally published.  0 puts every statistics item
// first.
#ifndef SPEC_CHAIN_LAG_TENTHS
#define SPEC_CHAIN_LAG_TENTHS 16
#endif
constexpr long kLagTenths = SPEC_CHAIN_LAG_TENTHS;   // in tenths of a round
// Lazy rows: lag between a request's last row group and its terminal items, in tenths of
// a round.
#ifndef SPEC_LAZY_LAG_TENTHS
#define SPEC_LAZY_LAG_TENTHS 20
#endif
constexpr long kLazyLagTenths = SPEC_LAZY_LAG_TENTHS;

// Blocks resident per CU: 0 leaves it to the register count; k > 0 reserves LDS so that
// at most k blocks share a CU (fewer loads in flight: shorter queues, so the decision's
// dependent reads come back sooner).
#ifndef SPEC_CHAIN_BLOCKS_PER_CU
#define SPEC_CHAIN_BLOCKS_PER_CU 0
#endif
constexpr int kBlocksPerCU = SPEC_CHAIN_BLOCKS_PER_CU;
constexpr size_t kLdsPerCU = 160 * 1024;
constexpr size_t chain_dyn_lds() { return kBlocksPerCU > 0 ? kLdsPerCU / kBlocksPerCU - 12 * 1024 : 0; }

// A lag of `tenths` tenths of a round of resident blocks, in requests (at most B); a
// non-positive setting gives B (every earlier layer first).
inline long lag_requests(long tenths, long resident, long per_req, long B) {
  if (tenths <= 0) return B;
  const long lag = (tenths * resident / 10 + per_req - 1) / per_req;
  return lag > B ? B : lag;
}

template <int DT, int QT, bool VEC, bool PROC>
hipError_t launch_typed(ChainParams p, hipStream_t s) {
  static int s_resident[64] = {0};   // resident blocks per device ordinal; 0 = not queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (s_resident[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_kernel<DT, QT, VEC, PROC>, kBlock, chain_dyn_lds()) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidValue;
    s_resident[dev] = (per_cu < 1 ? 1 : per_cu) * (cus < 1 ? 1 : cus);
  }
  const long per_req = (long)p.R * p.SL + p.S2;
  p.LAG = (int)lag_requests(p.J > 1 ? kLazyLagTenths : kLagTenths, s_resident[dev], per_req, p.B);
  const unsigned long long blocks = (unsigned long long)p.B * ((unsigned long long)p.R * p.SL + p.S2);  // <= chain_blocks
  chain_kernel<DT, QT, VEC, PROC><<<dim3((unsigned)blocks), dim3(kBlock), chain_dyn_lds(), s>>>(p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the exact redraws of small residuals, and the scrub of requests whose waits gave up
  chain_exact_kernel<DT, QT, VEC, PROC><<<dim3((unsigned)((size_t)p.B * exact_blocks(p.S2))), dim3(kBlock), 0, s>>>(p);
  return hipGetLastError();
}

template <bool PROC>
hipError_t launch_dispatch(const ChainParams& p, int logit_dtype, bool vec, hipStream_t s) {
  const bool lb = logit_dtype == kBF16, qb = p.q_dtype == kBF16;
  if (p.q_index) {
    if (vec) return lb ? launch_typed<kBF16, kSparseQ, true, PROC>(p, s) : launch_typed<kF32, kSparseQ, true, PROC>(p, s);
    return lb ? launch_typed<kBF16, kSparseQ, false, PROC>(p, s) : launch_typed<kF32, kSparseQ, false, PROC>(p, s);
  }
  if (vec) {
    if (lb) return qb ? launch_typed<kBF16, kBF16, true, PROC>(p, s) : launch_typed<kBF16, kF32, true, PROC>(p, s);
    return qb ? launch_typed<kF32, kBF16, true, PROC>(p, s) : launch_typed<kF32, kF32, true, PROC>(p, s);
  }
  if (lb) return qb ? launch_typed<kBF16, kBF16, false, PROC>(p, s) : launch_typed<kBF16, kF32, false, PROC>(p, s);
  return qb ? launch_typed<kF32, kBF16, false, PROC>(p, s) : launch_typed<kF32, kF32, false, PROC>(p, s);
}

}  // namespace

hipError_t launch_chain(const ChainParams& p, int logit_dtype, bool vec, hipStream_t s) {
  return p.pr.on ? launch_dispatch<true>(p, logit_dtype, vec, s) : launch_dispatch<false>(p, logit_dtype, vec, s);
}

}  // namespace sv
