// Tree verification by target-sample membership (spec_verify_tree).
//
// One kernel.  Each request owns ceil(V / 8192) root blocks followed by its helper blocks
// (ceil(V / 16384); ceil(V / 8192) for the residual-update tree), adjacent in block order.
// The root blocks stream the frontier row (node 0) together, one 2048-element chunk per
// wave, and publish the chunks' online-softmax summaries.  The request's first root block,
// once its own chunks are summarized, walks the tree, reading the other summaries as they
// are published:
//   * combine the summaries of the current node's row into (reference, Z) and the chunk
//     masses, pick the chunk where the running mass passes u_v * Z, rescan that chunk in
//     vocabulary order to get the target sample y;
//   * if a child of the node carries token y, accept it and order the request's helper
//     blocks to summarize the child's row (each helper streams 8 chunks of it); otherwise
//     y is the terminal token and the helpers are dismissed.
// In the greedy tree (the argmax in place of the sample) the helpers first stream ahead the
// one root child a walk leaving the root can take, and in the residual-update tree the
// root's first child (the first one tested); the walker reads those summaries instead of
// ordering that row when its walk goes there.  Otherwise only rows on the walked path are
// read.  Waits: the helpers wait for their walker, a
// lower-numbered block; the walker waits for its request's other root blocks and helpers,
// which follow it directly.  Each XCD dispatches the workgroups it is given in index order,
// so once every earlier request has finished, all of a request's workgroups are dispatched
// (a request needs a few slots per XCD) and every wait among them ends; each is bounded all
// the same (a word that does not arrive in time is reported as SPEC_REQ_INTERNAL).
//
// Method: [M7.7] "M7.7 - Draft Sources, Dependent Heads, and Hardware-Aware Trees"
// §0x07E (a node's row scores its children), §0x04B and §0x09 (accept the candidate that
// matches the target's own sample), §0x0F (parent index validity); [M16] "Module 16:
// Speculative Decoding", "Verify the Tree" (walk until no child matches, then emit one
// more target token).
#include "device_common.h"
#include "internal.h"
#include "spec_verify.h"

namespace sv {

namespace {

constexpr int kNoPick = 0x7fffffff;

// Trace records (trace builds only): kernel slot 2 (membership and greedy trees) or 3
// (residual-update tree).  Each block tags its own record as a root block, a helper or, for
// the root block that walks, the walker; the walker also writes one record per hop (a node
// visited, or a residual pass) at record B * (WG1 + WH) + b * kTraceHops + hop.
enum : int { kTraceRoot = 0, kTraceHelper = 1, kTraceWalker = 2, kTraceNode = 8, kTracePass = 9 };
constexpr int kTraceHops = 128;
__device__ __forceinline__ unsigned long long hop_record(const TreeParams& p, int b, int hop) {
  return (unsigned long long)p.B * (p.WG1 + p.WH) + (unsigned long long)b * kTraceHops +
         (unsigned long long)min(hop, kTraceHops - 1);
}

// A failed request.  SPEC_REQ_INTERNAL (a wait that gave up) also marks the workspace dirty.
__device__ void tree_fail(const TreeParams& p, int b, int code) {
  for (int i = threadIdx.x; i < p.N; i += blockDim.x) {
    p.out_tokens[(size_t)b * p.N + i] = -1;
    p.out_nodes[(size_t)b * p.N + i] = -1;
  }
  if (threadIdx.x == 0) {
    p.accepted_len[b] = -1;
    p.req_status[b] = code;
    if (code == SPEC_REQ_INTERNAL) publish_u32(dirty_word(p.counters), 1u);
  }
}

// Chunk summary c of the row being sampled.  PUBLISHED: written by other blocks (read
// with bounded re-reads); otherwise written by this block itself (plain loads after a
// barrier).
template <int DT, bool VEC, bool PUBLISHED>
__device__ __forceinline__ float2 summary(const float2* part, int c) {
  if constexpr (PUBLISHED) return await_f2(part + c);
  else return part[c];
}

// Block-wide: sample one token from softmax(row / T) given the row's chunk summaries.
// Returns the token; a non-finite row or a bad uniform is reported through *status.
template <int DT, bool VEC, bool PUBLISHED>
__device__ int sample_row(const TreeParams& p, const float2* part, const void* row, float uv, int* status) {
  __shared__ double s_scan[kWavesPerBlock];
  __shared__ float s_r;
  __shared__ double s_z;
  __shared__ int s_imin[kWavesPerBlock];
  __shared__ int s_imin2[2 * kWavesPerBlock];
  __shared__ double s_before;
  __shared__ double s_total;
  __shared__ int s_cstar;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
  const float c2 = p.c2;

  // reference exponent: fp32(max raw logit * c2), identical to the chunks' own r_j
  if (wave == 0) {
    float m = -INFINITY;
    for (int j = lane; j < p.P; j += kWave) m = fmaxf(m, summary<DT, VEC, PUBLISHED>(part, j).x);
    m = wave_max(m);
    if (lane == 0) s_r = m * c2;
  }
  __syncthreads();
  const float R = s_r;

  // chunk masses 2^(r_j - R) Z_j in vocabulary order; thread t owns a contiguous run
  auto mass_of = [&](int c) -> double {
    const float2 s = summary<DT, VEC, PUBLISHED>(part, c);
    return (double)s.y * exp2((double)(s.x * c2) - (double)R);
  };
  const bool ok_u = uv >= 0.0f && uv < 1.0f;
  int cstar;
  double Z;
  if (p.P <= 2 * kWave) {
    // At most 128 chunks: wave 0 holds chunks l and 64 + l in lane l and forms the running
    // masses as the block's first two waves would (one chunk per thread, wave 1 offset by
    // wave 0's total), so Z and every running value are the block-wide ones; it also picks
    // the chunk.  One barrier instead of the block scan's, the minimum's and the owner's.
    if (wave == 0) {
      const double ma = lane < p.P ? mass_of(lane) : 0.0;
      const double mb = kWave + lane < p.P ? mass_of(kWave + lane) : 0.0;
      const double ia = wave_incl_scan_d(ma, lane), ib = wave_incl_scan_d(mb, lane);
      const double ea = 0.0 + wave_shr1_d(ia);
      const double eb = (0.0 + __shfl(ia, kWave - 1, kWave)) + wave_shr1_d(ib);
      const int last = p.P - 1;
      const double Zw = last < kWave ? __shfl(ea + ma, last, kWave) : __shfl(eb + mb, last - kWave, kWave);
      int cs = p.P - 1;
      if (isfinite(Zw) && Zw > 0.0 && ok_u) {
        const double t = (double)uv * Zw;
        const unsigned long long ha = __ballot(lane < p.P && ea + ma > t);
        const unsigned long long hb = __ballot(kWave + lane < p.P && eb + mb > t);
        if (ha) cs = __ffsll(static_cast<long long>(ha)) - 1;
        else if (hb) cs = kWave + __ffsll(static_cast<long long>(hb)) - 1;
      }
      const double before = cs < kWave ? __shfl(ea, cs, kWave) : __shfl(eb, cs - kWave, kWave);
      if (lane == 0) {
        s_total = Zw;
        s_before = before;
        s_cstar = cs;
      }
    }
    __syncthreads();
    Z = s_total;
    cstar = s_cstar;
    if (!(isfinite(Z) && Z > 0.0)) { *status = SPEC_REQ_NONFINITE; return -1; }
    if (!ok_u) { *status = SPEC_REQ_BADUNIFORM; return -1; }
  } else {
    const int per = (p.P + kBlock - 1) / kBlock;
    const int c_lo = min(tid * per, p.P), c_hi = min(c_lo + per, p.P);
    double mine = 0.0;
    for (int c = c_lo; c < c_hi; ++c) mine += mass_of(c);
    double tot;
    const double excl = block_excl_scan_d(mine, s_scan, &tot);
    double run_end = excl;
    for (int c = c_lo; c < c_hi; ++c) run_end += mass_of(c);
    if (c_lo < c_hi && c_hi == p.P) s_total = run_end;
    __syncthreads();
    Z = s_total;
    if (!(isfinite(Z) && Z > 0.0)) { *status = SPEC_REQ_NONFINITE; return -1; }
    if (!ok_u) { *status = SPEC_REQ_BADUNIFORM; return -1; }
    const double t = (double)uv * Z;
    int cand = kNoPick;          // first chunk of this thread's run whose running value passes t
    {
      double run = excl;
      for (int c = c_lo; c < c_hi; ++c) {
        const double nxt = run + mass_of(c);
        if (nxt > t) { cand = c; break; }
        run = nxt;
      }
    }
    if (tid == 0) s_before = 0.0;
    // a chunk is always found (t < Z and the last running value is Z); clamp regardless
    cstar = block_min_i(cand, s_imin);
    if (cstar == kNoPick) cstar = p.P - 1;
    if (cstar >= c_lo && cstar < c_hi) {
      double run = excl;
      for (int c = c_lo; c < cstar; ++c) run += mass_of(c);
      s_before = run;
    }
    __syncthreads();
  }
  const double t = (double)uv * Z;

  // rescan chunk cstar (one slab) in the chunk's own units 2^(l c2 - r_c)
  const float rc = summary<DT, VEC, PUBLISHED>(part, cstar).x * c2;
  const double rem = (t - s_before) * exp2((double)R - (double)rc);
  const long e0 = (long)cstar * kWaveChunk + (long)tid * kVec;
  float v[8];
  load8<DT, VEC, false>(row, e0, p.V, v, -INFINITY);
  double incl[8];
  double acc = 0.0;
  int last_pos = -1;
  float e[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    e[k] = scaled_exp(v[k], c2, rc);
    acc += (double)e[k];
    incl[k] = acc;
    if (e[k] > 0.0f) last_pos = (int)(e0 + k);
  }
  double slab_total;
  const double off = block_excl_scan_d(acc, s_scan, &slab_total);
  int pick = kNoPick;
#pragma unroll
  for (int k = 7; k >= 0; --k)
    if (off + incl[k] > rem && e[k] > 0.0f) pick = (int)(e0 + k);
  // the first position whose running value passes the target; rounding may leave the
  // target just past the chunk's last positive weight: then take that weight
  int last_any;
  pick = block_min_max_i(pick, last_pos, s_imin2, &last_any);
  const int y = pick != kNoPick ? pick : last_any;
  *status = 0;
  return y;
}

// Orders from a walking block to its request's helpers, one 64-bit word per request:
// generation << 32 | code, code = row + 1 (summarize that row), kResidualPass | i (chunk
// masses of the residual after i rejected children, residual-update verifier only) or
// kTreeDone (leave).  A generation is never 0, so a published order is never zero.
constexpr unsigned kTreeDone = 0xffffffffu;
// The speculation tag of a request whose root has no child the helpers stream ahead.
constexpr unsigned kNoSpec = 0xffffffffu;
constexpr unsigned kResidualPass = 0x40000000u;

// ------------------------------------------------------------ residual-update verifier
// Descriptor of the residual passes at the current node v: 64-bit words, each tag << 32 |
// value, written through by the walker (one thread) before the pass order that first needs
// it: [0] v, [1] bits of r (reference exponent of row v), [2] bits of 1/Z (base 2), [3 + j]
// the j-th rejected child, [3 + N + j] bits of 1/W_j, W_j the mass of the residual after
// j + 1 rejections.  A node's pass orders carry consecutive generations g1, g1 + 1, ...
// (nothing else is ordered between them), so pass i (order generation g) has g1 = g - i + 1,
// and the tag of words 0..2 is g1 and that of child j and of 1/W_j is g1 + j.  Every word
// thus validates itself: a helper re-reads a word until its tag is the one the order
// implies, in whatever order the stores arrive, and no store of the walker needs to wait
// for another.  Generations only grow within a call and the walker zeroes the descriptor
// before the call ends, so no stale word carries a current tag.
constexpr int kResidStage = 256;   // rejected children a helper keeps in LDS per pass
__device__ __forceinline__ unsigned long long desc_word(unsigned tag, unsigned v) {
  return (static_cast<unsigned long long>(tag) << 32) | v;
}
__device__ __forceinline__ unsigned desc_value(unsigned long long w) { return static_cast<unsigned>(w); }
// A descriptor word re-read until it carries `tag` (bounded: the last read is returned).
__device__ __forceinline__ unsigned long long await_desc(const unsigned long long* w, unsigned tag) {
  unsigned long long v = fetch_u64(w);
  for (unsigned spins = 0; static_cast<unsigned>(v >> 32) != tag && spins < kSpinLimit; ++spins) {
    __builtin_amdgcn_s_sleep(1);
    v = fetch_u64(w);
  }
  return v;
}
// A chunk-mass word meaning "the helper's descriptor never became current": the walker
// reports SPEC_REQ_INTERNAL on it.  (A published mass is a negated fp64 value; this is a
// NaN bit pattern that no negated mass takes.)
constexpr unsigned long long kLostMassWord = 0x7ff4000000000001ull;

// The unnormalized residual after i rejected children c_0..c_{i-1} at node v, for NV
// vectors of eight elements [e0 + n * step, + 8): p(x) = 2^(l c2 - r) / Z, res_0 = p,
// res_{j+1} = [res_j - q_{c_j}]_+ / W_j for j + 1 < i, and g = [res_{i-1} - q_{c_{i-1}}]_+.
// One expression serves the helpers' chunk masses, the walker's single-element accept
// tests and its rescan, so the three agree bit for bit.  The NV vectors' loads of each row
// are issued together, and the first rejected child's q row is fetched with the logits,
// so a call costs max(1, i) dependent memory round trips.  The children and their 1/W come
// from LDS (s_kid, s_invw: the first kResidStage of them) or else from the descriptor.
// bad: an entry of the last rejected child's q row is negative or non-finite.
template <int DT, int QT, bool VEC, int NV>
__device__ __forceinline__ void residualN(const TreeParams& p, int b, const unsigned long long* d, int i,
                                          const int* s_kid,
                                          const float* s_invw, const void* lrow, long e0, long step, float r,
                                          float inv_z, float (&g)[NV][8], bool& bad) {
  auto kid_of = [&](int j) {
    return j < kResidStage && s_kid ? s_kid[j] : static_cast<int>(desc_value(fetch_u64(d + 3 + j)));
  };
  float l[NV][8], q[NV][8];
#pragma unroll
  for (int n = 0; n < NV; ++n) load8<DT, VEC, false>(lrow, e0 + n * step, p.V, l[n], -INFINITY);
  if (i > 0) {
    const void* q0 = row_ptr<QT>(p.q, (size_t)b * p.N + kid_of(0), p.V);
#pragma unroll
    for (int n = 0; n < NV; ++n) load8<QT, VEC, false>(q0, e0 + n * step, p.V, q[n], 0.0f);
  }
#pragma unroll
  for (int n = 0; n < NV; ++n)
#pragma unroll
    for (int k = 0; k < 8; ++k) g[n][k] = scaled_exp(l[n][k], p.c2, r) * inv_z;
  for (int j = 0; j < i; ++j) {
    const float invw = j + 1 == i ? 1.0f
                       : (j < kResidStage && s_invw ? s_invw[j] : __uint_as_float(desc_value(fetch_u64(d + 3 + p.N + j))));
    if (j > 0) {
      const void* qj = row_ptr<QT>(p.q, (size_t)b * p.N + kid_of(j), p.V);
#pragma unroll
      for (int n = 0; n < NV; ++n) load8<QT, VEC, false>(qj, e0 + n * step, p.V, q[n], 0.0f);
    }
#pragma unroll
    for (int n = 0; n < NV; ++n)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float t = g[n][k] - q[n][k];
        const float pos = t > 0.0f ? t : 0.0f;
        if (j + 1 == i) bad |= !(q[n][k] >= 0.0f && q[n][k] < INFINITY);
        g[n][k] = j + 1 == i ? pos : pos * invw;
      }
  }
}

// Helper h's part of residual pass i (order generation gen): the chunk masses (fp64) of g
// over its chunks.  The descriptor words the pass needs -- v, r, 1/Z, the i rejected
// children and the i - 1 values 1/W_j -- are read together, one thread each, and each is
// re-read until it carries the tag the order implies (bounded).
template <int DT, int QT, bool VEC>
__device__ void residual_pass(const TreeParams& p, int b, int h, unsigned gen, int i) {
  __shared__ int s_kid[kResidStage];
  __shared__ float s_invw[kResidStage];
  __shared__ unsigned s_head[3];
  __shared__ int s_stale;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
  const unsigned long long* d = p.desc + (size_t)b * p.desc_words;
  const unsigned g1 = gen - static_cast<unsigned>(i) + 1u;   // the node's first pass order
  if (tid == 0) s_stale = 0;
  __syncthreads();
  const int nwords = 2 + 2 * i;   // 3 head words, i children, i - 1 values 1/W_j
  for (int k = tid; k < nwords; k += kBlock) {
    const int j = k < 3 ? 0 : (k < 3 + i ? k - 3 : k - 3 - i);
    const int idx = k < 3 ? k : (k < 3 + i ? 3 + j : 3 + p.N + j);
    const unsigned tag = g1 + static_cast<unsigned>(j);
    unsigned long long w = fetch_u64(d + idx);
    for (unsigned spins = 0; static_cast<unsigned>(w >> 32) != tag && spins < kSpinLimit; ++spins) {
      __builtin_amdgcn_s_sleep(1);
      w = fetch_u64(d + idx);
    }
    if (static_cast<unsigned>(w >> 32) != tag) s_stale = 1;
    const unsigned val = desc_value(w);
    if (k < 3) s_head[k] = val;
    else if (k < 3 + i) { if (j < kResidStage) s_kid[j] = static_cast<int>(val); }
    else if (j < kResidStage) s_invw[j] = __uint_as_float(val);
  }
  __syncthreads();
  double* dst = reinterpret_cast<double*>(p.deep + ((size_t)b * 2 + (gen & 1u)) * p.P);
  if (s_stale) {   // the wait bound: say so in every chunk mass this helper owns
    for (int k = tid; k < kResidHelperChunks; k += kBlock) {
      const int c = h * kResidHelperChunks + k;
      if (c < p.P) publish_u64(reinterpret_cast<unsigned long long*>(dst + c), kLostMassWord);
    }
    __syncthreads();
    return;
  }
  // every word of the pass has been validated, so re-reads of children past kResidStage
  // (residualN) return the same values: the walker writes each word once per node visit
  const int v = static_cast<int>(s_head[0]);
  const float r = __uint_as_float(s_head[1]), inv_z = __uint_as_float(s_head[2]);
  const void* row = row_ptr<DT>(p.logits, (size_t)b * p.N + v, p.V);
  for (int k = 0; k < kResidHelperBatch; ++k) {
    const int c = h * kResidHelperChunks + k * kWavesPerBlock + wave;
    if (c >= p.P) continue;
    double acc = 0.0;
    bool bad = false;
    float g[kStatVecs][8];
    residualN<DT, QT, VEC, kStatVecs>(p, b, d, i, s_kid, s_invw, row,
                                      (long)c * kWaveChunk + static_cast<long>(lane) * kVec, (long)kWave * kVec,
                                      r, inv_z, g, bad);
#pragma unroll
    for (int jv = 0; jv < kStatVecs; ++jv)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (double)g[jv][e];
    if (bad) acc = NAN;
    const double m = wave_sum_d(acc);
    if (lane == 0) publish_mass(dst + c, m);
  }
  __syncthreads();   // s_kid, s_invw and s_head are rewritten by the next pass
}

__device__ __forceinline__ void publish_order(const TreeParams& p, int b, unsigned gen, unsigned code) {
  publish_u64(p.order + b, (static_cast<unsigned long long>(gen) << 32) | code);
}

// The walker stages a row's summaries in LDS when the row has at most kTreeStage chunks;
// longer rows are read from the workspace directly.

// Read the P published summaries at `src` into `dst` (LDS); sets *lost if one did not arrive.
__device__ void stage_summaries(const float2* src, float2* dst, int P, int* lost) {
  for (int c = threadIdx.x; c < P; c += kBlock) {
    const unsigned long long bits = await_u64(reinterpret_cast<const unsigned long long*>(src + c));
    if (bits == 0ull) *lost = 1;
    dst[c] = make_float2(__uint_as_float(static_cast<unsigned>(bits)), __uint_as_float(static_cast<unsigned>(bits >> 32)));
  }
  __syncthreads();
}

// One target sample from row `row` whose P chunk summaries are published at `src`.
template <int DT, bool VEC>
__device__ int sample_published(const TreeParams& p, const float2* src, const void* row, float uv, int* status,
                                unsigned long long trec) {
  __shared__ float2 s_sum[kTreeStage];
  __shared__ int s_lost;
  if (threadIdx.x == 0) s_lost = 0;
  __syncthreads();
  if (p.P <= kTreeStage) {
    stage_summaries(src, s_sum, p.P, &s_lost);
    SPEC_STAMP_AT(p, 2, trec, 2);
    if (s_lost) { *status = SPEC_REQ_INTERNAL; return -1; }
    return sample_row<DT, VEC, false>(p, s_sum, row, uv, status);
  }
  return sample_row<DT, VEC, true>(p, src, row, uv, status);
}

// The target's greedy token of a row from its P published argmax summaries at `src`
// (greedy mode): the maximum, and the lowest position holding it.  A row holding NaN or
// +inf, or entirely -inf, is reported through *status.
__device__ int argmax_published(const TreeParams& p, const float2* src, int* status) {
  __shared__ float s_m[kWavesPerBlock];
  __shared__ int s_i[kWavesPerBlock];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
  const unsigned long long* words = reinterpret_cast<const unsigned long long*>(src);
  float m = -INFINITY;
  int idx = 0x7fffffff;
  bool nan = false, lost = false;
  for (int c = tid; c < p.P; c += kBlock) {      // a thread's chunks rise with c
    const unsigned long long bits = await_u64(words + c);
    lost |= (bits == 0ull);
    float cm;
    int ci;
    unpack_argmax(bits, cm, ci);
    nan |= (cm != cm);
    if (cm > m) {
      m = cm;
      idx = ci;
    }
  }
  float M;
  int I;
  wave_argmax_merge(m, idx, nan, M, I);
  if (lane == 0) {
    s_m[wave] = M;
    s_i[wave] = I;
  }
  const bool any_lost = __syncthreads_or(lost) != 0;
  float bm = -INFINITY;
  bool bnan = false;
#pragma unroll
  for (int k = 0; k < kWavesPerBlock; ++k) {
    bnan |= (s_m[k] != s_m[k]);
    bm = fmaxf(bm, s_m[k]);
  }
  int bi = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < kWavesPerBlock; ++k)
    if (s_m[k] == bm) bi = min(bi, s_i[k]);
  __syncthreads();                               // s_m and s_i are rewritten by the next row
  if (any_lost) { *status = SPEC_REQ_INTERNAL; return -1; }
  if (bnan || !(bm > -INFINITY && bm < INFINITY)) { *status = SPEC_REQ_NONFINITE; return -1; }
  *status = 0;
  return bi;
}

// Validation of a request's tree ([M7.7] §0x0F: parents[0] = -1, 0 <= parents[v] < v, and
// non-root tokens in [0, V)) and of the workspace (its dirty word), split so that the loads
// overlap the walker's first staging: tree_check_issue loads node 1 + t (and thread 0
// parents[0] and the dirty word) into registers, tree_check_done compares them (and any
// nodes past the first kBlock + 1, directly).  Block-wide; returns 0, SPEC_REQ_INTERNAL (a
// dirty workspace) or SPEC_REQ_BADTREE.
struct TreeCheck { int pv, tv, p0; unsigned dirty; };
__device__ __forceinline__ TreeCheck tree_check_issue(const TreeParams& p, const int32_t* par, const int32_t* tok,
                                                      int N) {
  const int v = 1 + threadIdx.x;
  TreeCheck k{0, 0, -1, 0u};
  if (v < N) {
    k.pv = par[v];
    k.tv = tok[v];
  }
  if (threadIdx.x == 0) {
    k.p0 = par[0];
    k.dirty = fetch_u32(dirty_word(p.counters));
  }
  return k;
}
__device__ int tree_check_done(const int32_t* par, const int32_t* tok, int N, int V, const TreeCheck& k) {
  const int v = 1 + threadIdx.x;
  bool bad = (v < N && (k.pv < 0 || k.pv >= v || k.tv < 0 || k.tv >= V)) || (threadIdx.x == 0 && k.p0 != -1);
  for (int w = 1 + kBlock + threadIdx.x; w < N; w += kBlock) {
    const int pw = par[w], tw = tok[w];
    bad |= pw < 0 || pw >= w || tw < 0 || tw >= V;
  }
  if (__syncthreads_or(threadIdx.x == 0 && k.dirty != 0u)) return SPEC_REQ_INTERNAL;
  return __syncthreads_or(bad) ? SPEC_REQ_BADTREE : 0;
}

// Walk of request b by the last root block.  `gen` counts the orders sent to the helpers.
// ARGMAX: greedy mode, the target's argmax stands in for its sample (no uniforms).
template <int DT, bool VEC, bool ARGMAX>
__device__ void tree_walk(const TreeParams& p, int b, unsigned& gen) {
  __shared__ int s_imin[kWavesPerBlock];
  const int tid = threadIdx.x;
  const int N = p.N;
  const int32_t* par = p.parents + (size_t)b * N;
  const int32_t* tok = p.node_tokens + (size_t)b * N;
  // the tree's validation: loads now, outcome after the root's sample (before any status)
  const TreeCheck check = tree_check_issue(p, par, tok, N);
  // greedy trees: which root child the helpers stream ahead (read now, awaited after the
  // root's argmax)
  unsigned stag = ARGMAX && p.spec && tid == 0 ? fetch_u32(p.stag + b) : 0u;
  __shared__ unsigned s_gen;
  __shared__ int s_ahead;

  int v = 0, depth = 0;
  bool ahead = false;   // this row's summaries are the streamed-ahead ones
  while (true) {
    const unsigned long long trec = hop_record(p, b, depth);
    SPEC_TAG_AT(p, 2, trec, SPEC_TRACE_TAG(kTraceNode, b, v));
    SPEC_STAMP_AT(p, 2, trec, 1);
    const void* row = row_ptr<DT>(p.logits, (size_t)b * N + v, p.V);
    int status = 0;
    const float uv = ARGMAX ? 0.0f : p.u[(size_t)b * N + v];
    int y;
    if (v == 0) {
      if constexpr (ARGMAX) y = argmax_published(p, p.part + (size_t)b * p.P, &status);
      else y = sample_published<DT, VEC>(p, p.part + (size_t)b * p.P, row, uv, &status, trec);
    } else if (ARGMAX && ahead) {
      // the root child's summaries, streamed ahead by the helpers (the last of them to
      // leave returns the words to zero)
      const float2* src = p.spec + (size_t)b * p.P;
      if constexpr (ARGMAX) y = argmax_published(p, src, &status);
      else y = sample_published<DT, VEC>(p, src, row, uv, &status, trec);
    } else {
      // the helpers' summaries of this row; returned to zero once read
      float2* deep = p.deep + ((size_t)b * 2 + (gen & 1u)) * p.P;
      if constexpr (ARGMAX) y = argmax_published(p, deep, &status);
      else y = sample_published<DT, VEC>(p, deep, row, uv, &status, trec);
      for (int c = tid; c < p.P; c += kBlock) clear_f2(deep + c);
      vmem_wait();      // the clears are complete before any later order reuses the words
    }
    SPEC_STAMP_AT(p, 2, trec, 3);
    if (v == 0) {
      const int code = tree_check_done(par, tok, N, p.V, check);
      if (code != 0) { tree_fail(p, b, code); return; }
    }
    if (status != 0) { tree_fail(p, b, status); return; }
    // this thread's lowest matching child: first the node whose parent and token it holds
    // since the validation (1 + tid), then the nodes beyond those (c rises)
    int cand = kNoPick;
    if (1 + tid < N && 1 + tid > v && check.pv == v && check.tv == y) cand = 1 + tid;
    for (int c = 1 + kBlock + tid; c < N; c += kBlock)
      if (cand == kNoPick && c > v && par[c] == v && tok[c] == y) cand = c;
    const int child = block_min_i(cand, s_imin);
    if (child == kNoPick) {
      for (int i = tid; i < N; i += kBlock) {
        if (i > depth) {
          p.out_tokens[(size_t)b * N + i] = -1;
          p.out_nodes[(size_t)b * N + i] = -1;
        } else if (i == depth) {
          p.out_tokens[(size_t)b * N + i] = y;
          p.out_nodes[(size_t)b * N + i] = -1;
        }
      }
      if (tid == 0) {
        p.accepted_len[b] = depth;
        p.req_status[b] = 0;
      }
      SPEC_STAMP_AT(p, 2, trec, 4);
      return;
    }
    if (tid == 0) {
      p.out_tokens[(size_t)b * N + depth] = y;   // the child matched by carrying token y
      p.out_nodes[(size_t)b * N + depth] = child;
      bool hit = false;
      if (ARGMAX && v == 0 && p.spec) {
        for (unsigned spins = 0; stag == 0u && spins < kSpinLimit; ++spins) {
          __builtin_amdgcn_s_sleep(1);
          stag = fetch_u32(p.stag + b);
        }
        hit = stag == static_cast<unsigned>(child) + 1u;   // (a tag that never came: no hit)
      }
      if (!hit) publish_order(p, b, ++gen, static_cast<unsigned>(child) + 1u);   // summarize the child's row
      s_gen = gen;
      s_ahead = hit ? 1 : 0;
    }
    SPEC_STAMP_AT(p, 2, trec, 4);
    ++depth;
    v = child;
    __syncthreads();
    gen = s_gen;
    ahead = ARGMAX && s_ahead != 0;
  }
}

// Next child of v after `after` in index order (children have larger indices than their
// parent), block-wide; kNoPick if there is none.  Thread t holds node 1 + t's parent since
// the validation (k); only the nodes beyond those are read again.
__device__ __forceinline__ int next_child(const TreeCheck& k, const int32_t* par, int N, int v, int after,
                                          int* s_imin) {
  const int tid = threadIdx.x;
  int cand = kNoPick;
  if (1 + tid < N && 1 + tid > after && k.pv == v) cand = 1 + tid;
  for (int c = 1 + kBlock + tid; c < N; c += kBlock)
    if (cand == kNoPick && c > after && par[c] == v) cand = c;
  return block_min_i(cand, s_imin);
}

// Running mass of the P chunk masses in `mass` (LDS), formed the same way wherever it is
// needed: thread t owns a contiguous run of chunks and extends the block-exclusive prefix
// over it.  Returns this thread's exclusive prefix; *total is the running value after the
// last chunk (identical in every thread).
__device__ double mass_prefix(const double* mass, int P, int c_lo, int c_hi, double* total) {
  __shared__ double s_scan[kWavesPerBlock];
  __shared__ double s_total;
  double excl = 0.0;
  if (P <= kWave) {
    // every chunk in wave 0 (one per thread): its prefix is the block-wide one, as the other
    // waves would only add zeros
    if (wave_id() == 0) {
      const int lane = threadIdx.x;
      const double mine = lane < P ? mass[lane] : 0.0;
      excl = 0.0 + wave_shr1_d(wave_incl_scan_d(mine, lane));
      if (lane == P - 1) s_total = excl + mine;
    }
  } else {
    double mine = 0.0;
    for (int c = c_lo; c < c_hi; ++c) mine += mass[c];
    double tot;
    excl = block_excl_scan_d(mine, s_scan, &tot);
    if (c_lo < c_hi && c_hi == P) s_total = excl + mine;
  }
  __syncthreads();
  *total = s_total;
  __syncthreads();
  return excl;
}

// The terminal draw at node v after i >= 1 rejected children: inverse CDF of the residual
// g with u, from the chunk masses of the last pass (in `mass`, total W) and a rescan of
// the chunk holding the target.
template <int DT, int QT, bool VEC>
__device__ int residual_pick(const TreeParams& p, int b, const unsigned long long* d, int i, const int* s_kid,
                             const float* s_invw, const void* row, float r, float inv_z, const double* mass,
                             float u) {
  __shared__ double s_scan[kWavesPerBlock];
  __shared__ int s_imin[kWavesPerBlock];
  __shared__ int s_imin2[2 * kWavesPerBlock];
  __shared__ double s_before, s_w;
  __shared__ int s_cstar;
  const int tid = threadIdx.x;
  int cstar;
  double W;
  if (p.P <= kWave) {
    // every chunk in wave 0: the running masses as mass_prefix forms them, and the pick,
    // with one barrier
    if (wave_id() == 0) {
      const double mine = tid < p.P ? mass[tid] : 0.0;
      const double excl = 0.0 + wave_shr1_d(wave_incl_scan_d(mine, tid));
      const double Ww = __shfl(excl + mine, p.P - 1, kWave);
      const double tw = (double)u * Ww;
      const unsigned long long hit = __ballot(tid < p.P && excl + mine > tw);
      const int cs = hit ? __ffsll(static_cast<long long>(hit)) - 1 : p.P - 1;
      const double before = __shfl(excl, cs, kWave);
      if (tid == 0) {
        s_w = Ww;
        s_before = before;
        s_cstar = cs;
      }
    }
    __syncthreads();
    W = s_w;
    cstar = s_cstar;
  } else {
    const int per = (p.P + kBlock - 1) / kBlock;
    const int c_lo = min(tid * per, p.P), c_hi = min(c_lo + per, p.P);
    const double excl = mass_prefix(mass, p.P, c_lo, c_hi, &W);
    const double t = (double)u * W;
    int cand = kNoPick;
    {
      double run = excl;
      for (int c = c_lo; c < c_hi; ++c) {
        const double nxt = run + mass[c];
        if (nxt > t) { cand = c; break; }
        run = nxt;
      }
    }
    if (tid == 0) s_before = 0.0;
    cstar = block_min_i(cand, s_imin);   // a chunk is always found (t < W); clamp regardless
    if (cstar == kNoPick) cstar = p.P - 1;
    if (cstar >= c_lo && cstar < c_hi) {
      double run = excl;
      for (int c = c_lo; c < cstar; ++c) run += mass[c];
      s_before = run;
    }
    __syncthreads();
  }
  const double t = (double)u * W;
  const double rem = t - s_before;
  const long e0 = (long)cstar * kWaveChunk + (long)tid * kVec;
  float gv[1][8];
  bool bad = false;
  residualN<DT, QT, VEC, 1>(p, b, d, i, s_kid, s_invw, row, e0, 0, r, inv_z, gv, bad);
  const float (&g)[8] = gv[0];
  double incl[8];
  double acc = 0.0;
  int last_pos = -1;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    acc += (double)g[k];
    incl[k] = acc;
    if (g[k] > 0.0f) last_pos = (int)(e0 + k);
  }
  double chunk_total;
  const double off = block_excl_scan_d(acc, s_scan, &chunk_total);
  int pick = kNoPick;
#pragma unroll
  for (int k = 7; k >= 0; --k)
    if (off + incl[k] > rem && g[k] > 0.0f) pick = (int)(e0 + k);
  int last_any;
  pick = block_min_max_i(pick, last_pos, s_imin2, &last_any);
  return pick != kNoPick ? pick : last_any;
}

// Walk of request b by the last root block, residual-update verifier ([M7.7] §0x09A):
// at node v the children are tested in index order against the current residual; an
// accepted child becomes the next node (its row summarized by the helpers), a rejection
// replaces the residual by [res - q_c]_+ / W (W from a helper pass), and a node whose
// children are all rejected (or which has none) emits a draw of the residual.
template <int DT, int QT, bool VEC>
__device__ void tree_walk_residual(const TreeParams& p, int b, unsigned& gen) {
  __shared__ int s_lost, s_status, s_accept;
  __shared__ int s_imin[kWavesPerBlock];
  __shared__ float s_red[kWavesPerBlock];
  __shared__ float s_rz_r;
  __shared__ double s_rz_z;
  __shared__ double s_scan[kWavesPerBlock];
  __shared__ float2 s_sum[kTreeStage];
  __shared__ double s_mass[kTreeStage];
  __shared__ unsigned s_gen;
  // the node's rejected children, the 1/W of their residuals and their q values at the child
  // under test (the first kResidStage; the descriptor holds them all)
  __shared__ int s_kid[kResidStage];
  __shared__ float s_invw[kResidStage];
  __shared__ float s_qx[kResidStage];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
  const int N = p.N, P = p.P;
  const int32_t* par = p.parents + (size_t)b * N;
  const int32_t* tok = p.node_tokens + (size_t)b * N;
  unsigned long long* d = p.desc + (size_t)b * p.desc_words;
  unsigned g1 = 0;   // thread 0: the generation of the current node's first pass order
  // the tree's validation: loads now, outcome once the root's summaries are staged
  const TreeCheck check = tree_check_issue(p, par, tok, N);
  // which root child the helpers stream ahead (read now, awaited once a root child is accepted)
  unsigned stag = p.spec && tid == 0 ? fetch_u32(p.stag + b) : 0u;
  __shared__ int s_ahead;

  int v = 0, depth = 0, hop = 0;
  bool ahead = false;   // this row's summaries are the streamed-ahead ones
  while (true) {
    const unsigned long long trec = hop_record(p, b, hop++);
    SPEC_TAG_AT(p, 3, trec, SPEC_TRACE_TAG(kTraceNode, b, v));
    SPEC_STAMP_AT(p, 3, trec, 1);
    const void* row = row_ptr<DT>(p.logits, (size_t)b * N + v, p.V);
    // 1. the row's chunk summaries: the root items' or, below the root, the helpers'
    if (tid == 0) s_lost = 0;
    __syncthreads();
    float2* src = v == 0 ? p.part + (size_t)b * P
                 : ahead ? p.spec + (size_t)b * P : p.deep + ((size_t)b * 2 + (gen & 1u)) * P;
    stage_summaries(src, s_sum, P, &s_lost);
    SPEC_STAMP_AT(p, 3, trec, 2);
    if (v == 0) {
      const int code = tree_check_done(par, tok, N, p.V, check);
      if (code != 0) { tree_fail(p, b, code); return; }
    }
    if (v != 0 && !ahead) {   // (the streamed-ahead words are cleared by the last helper)
      for (int c = tid; c < P; c += kBlock) clear_f2(src + c);
      vmem_wait();
    }
    if (s_lost) { tree_fail(p, b, SPEC_REQ_INTERNAL); return; }
    // reference exponent r = fp32(max raw logit * c2) and Z = sum 2^(l c2 - r) in fp64
    float r;
    double Z;
    if (P <= kWave) {
      // every summary in wave 0 (one per thread): r and Z as the block-wide reductions form
      // them (the other waves would add -inf to the maximum and zeros to the sum), one barrier
      if (wave == 0) {
        const float mw = wave_max(lane < P ? s_sum[lane].x : -INFINITY);
        const float rw = mw * p.c2;
        const double zt =
            lane < P ? (double)s_sum[lane].y * exp2((double)(s_sum[lane].x * p.c2) - (double)rw) : 0.0;
        const double Zw = 0.0 + __shfl(wave_incl_scan_d(zt, lane), kWave - 1, kWave);
        if (lane == 0) {
          s_rz_r = rw;
          s_rz_z = Zw;
        }
      }
      __syncthreads();
      r = s_rz_r;
      Z = s_rz_z;
    } else {
      float m = -INFINITY;
      for (int c = tid; c < P; c += kBlock) m = fmaxf(m, s_sum[c].x);
      m = wave_max(m);
      if (lane == 0) s_red[wave] = m;
      __syncthreads();
      m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
      r = m * p.c2;
      double zt = 0.0;
      for (int c = tid; c < P; c += kBlock) zt += (double)s_sum[c].y * exp2((double)(s_sum[c].x * p.c2) - (double)r);
      block_excl_scan_d(zt, s_scan, &Z);
    }
    if (!(isfinite(Z) && Z > 0.0)) { tree_fail(p, b, SPEC_REQ_NONFINITE); return; }
    const float inv_z = (float)(1.0 / Z);
    SPEC_STAMP_AT(p, 3, trec, 3);

    // 2. the children, in index order
    int i = 0, accepted = kNoPick, accepted_x = 0;
    int c = next_child(check, par, N, v, v, s_imin);
    while (c != kNoPick) {
      // the accept test's loads, issued together: thread 0 the child's q(x), u and the row's
      // logit at x; threads 1 .. kBlock - 1 the q values at x of the staged rejected children
      // j = tid - 1 and j = tid - 1 + (kBlock - 1) (kResidStage > kBlock - 1: one thread
      // alone would leave the last staged child's value unloaded)
      const int x = tok[c];
      float qx = 0.0f, ua = 0.0f, lx = 0.0f;
      if (tid == 0) {
        qx = load_scalar<QT>(p.q, ((size_t)b * N + c) * p.V + x);
        ua = p.u[(size_t)b * N + c];
        lx = load_scalar<DT>(row, x);
      } else {
        static_assert(kResidStage <= 2 * (kBlock - 1), "two staged children per thread at most");
        const int ns = min(i, kResidStage);
        for (int j = tid - 1; j < ns; j += kBlock - 1)
          s_qx[j] = load_scalar<QT>(p.q, ((size_t)b * N + s_kid[j]) * p.V + x);
      }
      __syncthreads();
      if (tid == 0) {
        int st = 0, acc = 0;
        if (!(isfinite(qx) && qx > 0.0f)) {
          st = SPEC_REQ_QZERO;
        } else if (!(ua >= 0.0f && ua < 1.0f)) {
          st = SPEC_REQ_BADUNIFORM;
        } else {
          // residual at x after the i rejections so far, the same expression as residualN
          float g = scaled_exp(lx, p.c2, r) * inv_z;
          bool stale = false;
          for (int j = 0; j < i; ++j) {
            float qj, invw;
            if (j < kResidStage) {
              qj = s_qx[j];
              invw = s_invw[j];
            } else {
              // this thread wrote both words (tag g1 + j), the 1/W word just before this test:
              // a read that can pass the write-through store is re-read until it is current
              const unsigned tag = g1 + static_cast<unsigned>(j);
              const unsigned long long wk = await_desc(d + 3 + j, tag);
              const unsigned long long ww = await_desc(d + 3 + N + j, tag);
              stale |= static_cast<unsigned>(wk >> 32) != tag || static_cast<unsigned>(ww >> 32) != tag;
              qj = load_scalar<QT>(p.q, ((size_t)b * N + static_cast<int>(desc_value(wk))) * p.V + x);
              invw = __uint_as_float(desc_value(ww));
            }
            const float t = g - qj;
            g = (t > 0.0f ? t : 0.0f) * invw;
          }
          const double a = fmin(1.0, (double)g / (double)qx);
          acc = (double)ua < a;
          if (stale) st = SPEC_REQ_INTERNAL;
        }
        s_status = st;
        s_accept = acc;
      }
      __syncthreads();
      if (s_status) { tree_fail(p, b, s_status); return; }
      if (s_accept) {
        accepted = c;
        accepted_x = x;
        break;
      }
      // rejected: the residual's chunk masses from a helper pass
      if (tid == 0) {
        const unsigned tag = gen + 1u;    // this pass order's generation, g1 + i
        if (i == 0) {
          g1 = tag;
          publish_u64(d, desc_word(g1, static_cast<unsigned>(v)));
          publish_u64(d + 1, desc_word(g1, __float_as_uint(r)));
          publish_u64(d + 2, desc_word(g1, __float_as_uint(inv_z)));
        }
        publish_u64(d + 3 + i, desc_word(tag, static_cast<unsigned>(c)));
        if (i < kResidStage) s_kid[i] = c;
        publish_order(p, b, ++gen, kResidualPass | static_cast<unsigned>(i + 1));
        s_gen = gen;
        s_lost = 0;
      }
      const unsigned long long prec = hop_record(p, b, hop++);
      SPEC_TAG_AT(p, 3, prec, SPEC_TRACE_TAG(kTracePass, b, i));
      SPEC_STAMP_AT(p, 3, prec, 1);
      ++i;
      __syncthreads();
      gen = s_gen;
      double* mw = reinterpret_cast<double*>(p.deep + ((size_t)b * 2 + (gen & 1u)) * P);
      for (int k = tid; k < P; k += kBlock) {
        const unsigned long long bits = await_u64(reinterpret_cast<const unsigned long long*>(mw + k));
        if (bits == 0ull || bits == kLostMassWord) s_lost = 1;
        s_mass[k] = -__longlong_as_double(static_cast<long long>(bits));
        clear_u64(reinterpret_cast<unsigned long long*>(mw + k));
      }
      vmem_wait();                        // cleared before any later order reuses the words
      __syncthreads();
      SPEC_STAMP_AT(p, 3, prec, 2);
      if (s_lost) { tree_fail(p, b, SPEC_REQ_INTERNAL); return; }
      const int per = (P + kBlock - 1) / kBlock;
      const int c_lo = min(tid * per, P), c_hi = min(c_lo + per, P);
      double W;
      mass_prefix(s_mass, P, c_lo, c_hi, &W);
      if (!(isfinite(W) && W > 0.0)) { tree_fail(p, b, SPEC_REQ_RESIDUAL_EMPTY); return; }
      if (tid == 0) {
        const float invw = (float)(1.0 / W);
        publish_u64(d + 3 + N + (i - 1), desc_word(gen, __float_as_uint(invw)));   // tag g1 + i - 1
        if (i - 1 < kResidStage) s_invw[i - 1] = invw;
      }
      SPEC_STAMP_AT(p, 3, prec, 3);
      c = next_child(check, par, N, v, c, s_imin);
    }
    if (accepted != kNoPick) {
      if (tid == 0) {
        p.out_tokens[(size_t)b * N + depth] = accepted_x;
        p.out_nodes[(size_t)b * N + depth] = accepted;
        bool hit = false;
        if (v == 0 && p.spec) {
          for (unsigned spins = 0; stag == 0u && spins < kSpinLimit; ++spins) {
            __builtin_amdgcn_s_sleep(1);
            stag = fetch_u32(p.stag + b);
          }
          hit = stag == static_cast<unsigned>(accepted) + 1u;   // (a tag that never came: no hit)
        }
        if (!hit) publish_order(p, b, ++gen, static_cast<unsigned>(accepted) + 1u);   // summarize its row
        s_gen = gen;
        s_ahead = hit ? 1 : 0;
      }
      SPEC_STAMP_AT(p, 3, trec, 4);
      ++depth;
      v = accepted;
      __syncthreads();
      gen = s_gen;
      ahead = s_ahead != 0;
      continue;
    }

    // 3. no child accepted: the terminal draw at v
    const float ud = p.u_draw[(size_t)b * N + v];
    if (!(ud >= 0.0f && ud < 1.0f)) { tree_fail(p, b, SPEC_REQ_BADUNIFORM); return; }
    int y;
    if (i == 0) {
      int status = 0;
      y = sample_row<DT, VEC, false>(p, s_sum, row, ud, &status);
      if (status != 0) { tree_fail(p, b, status); return; }
    } else {
      y = residual_pick<DT, QT, VEC>(p, b, d, i, s_kid, s_invw, row, r, inv_z, s_mass, ud);
    }
    SPEC_STAMP_AT(p, 3, trec, 5);
    for (int k = tid; k < N; k += kBlock) {
      if (k > depth) {
        p.out_tokens[(size_t)b * N + k] = -1;
        p.out_nodes[(size_t)b * N + k] = -1;
      } else if (k == depth) {
        p.out_tokens[(size_t)b * N + k] = y;
        p.out_nodes[(size_t)b * N + k] = -1;
      }
    }
    if (tid == 0) {
      p.accepted_len[b] = depth;
      p.req_status[b] = 0;
    }
    return;
  }
}

// Helper h's share of the chunk summaries of `row`, published at dst: its groups of HC
// chunks h, h + WH, h + 2 WH, ... (one group unless the request has more chunk groups than
// kMaxTreeHelpers), the same per-chunk summary the root blocks form (one chunk per wave).
template <int DT, bool VEC, bool RESID, bool ARGMAX>
__device__ __forceinline__ void helper_summaries(const TreeParams& p, const void* row, float2* dst, int h) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  constexpr int HB = RESID ? kResidHelperBatch : kTreeHelperBatch;     // chunks per wave
  constexpr int HC = RESID ? kResidHelperChunks : kTreeHelperChunks;   // chunks per helper
  for (int c0 = h * HC; c0 < p.P; c0 += p.WH * HC) {
    ChunkRegs<DT> r[HB];
#pragma unroll
    for (int k = 0; k < HB; ++k) {
      const int c = c0 + k * kWavesPerBlock + wave;
      if (c < p.P) chunk_load<DT, VEC>(row, p.V, c, lane, r[k]);
    }
#pragma unroll
    for (int k = 0; k < HB; ++k) {
      const int c = c0 + k * kWavesPerBlock + wave;
      if (c < p.P) {
        float v[kStatVecs][8];
        chunk_values<DT>(r[k], v);
        if constexpr (ARGMAX) {
          float m = -INFINITY;
          int idx = 0x7fffffff;
          bool nan = false;
          lane_argmax_update(v, (long)c * kWaveChunk, lane, m, idx, nan);
          float M;
          int I;
          wave_argmax_merge(m, idx, nan, M, I);
          if (lane == 0) publish_u64(reinterpret_cast<unsigned long long*>(dst + c), pack_argmax(M, I));
        } else {
          LaneSoftmax st;
          lane_softmax_update(st, v, p.c2);
          float m, z;
          wave_softmax_merge(st, p.c2, m, z);
          if (lane == 0) publish_f2(dst + c, make_float2(m, z));
        }
      }
    }
  }
}

// Before the first order, a greedy tree's helpers stream ahead the row of the root's child
// that a walk leaving the root must take: the walk's root token is the root row's argmax
// (the lowest index holding the maximum), and it moves to the lowest-index child carrying
// that token.  Among nodes 1..kBlock whose parent is the root, the child with the largest
// root logit at its token, then the lowest token, then the lowest index, is that child
// whenever the walk leaves the root.  Every helper of the request picks it from the same
// words; helper 0 publishes which one (the tag).  The walker reads these summaries instead
// of ordering that row; whatever it does, the request's last helper returns the words to
// zero when it leaves.  (For a sampled walk the same guess is only the likeliest child, and
// streaming it ahead measured slower at config 5: 18.3 against 17.3 us.)
template <int DT, bool VEC>
__device__ void helper_speculate(const TreeParams& p, int b, int h) {
  __shared__ float s_m[kWavesPerBlock];
  __shared__ int s_t[kWavesPerBlock], s_c[kWavesPerBlock];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
  const int N = p.N, c = 1 + tid;
  float l = -INFINITY;
  int t = 0x7fffffff;
  if (c < N) {
    const int pc = p.parents[(size_t)b * N + c];
    const int tk = p.node_tokens[(size_t)b * N + c];
    if (pc == 0 && tk >= 0 && tk < p.V) {
      const float x = load_scalar<DT>(p.logits, (size_t)b * N * p.V + (size_t)tk);
      if (x > -INFINITY) {              // NaN and -inf are never taken
        l = x;
        t = tk;
      }
    }
  }
  const float M = wave_max(l);
  const int T = wave_min_i(l == M ? t : 0x7fffffff);
  const int C = wave_min_i(l == M && t == T && T != 0x7fffffff ? c : kNoPick);
  if (lane == 0) {
    s_m[wave] = M;
    s_t[wave] = T;
    s_c[wave] = C;
  }
  __syncthreads();
  float bm = -INFINITY;
  int bt = 0x7fffffff, child = kNoPick;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w)
    if (s_c[w] != kNoPick &&
        (s_m[w] > bm || (s_m[w] == bm && (s_t[w] < bt || (s_t[w] == bt && s_c[w] < child))))) {
      bm = s_m[w];
      bt = s_t[w];
      child = s_c[w];
    }
  if (h == 0 && tid == 0) publish_u32(p.stag + b, child == kNoPick ? kNoSpec : static_cast<unsigned>(child) + 1u);
  if (child == kNoPick) return;
  helper_summaries<DT, VEC, false, true>(p, row_ptr<DT>(p.logits, (size_t)b * N + child, p.V),
                                         p.spec + (size_t)b * p.P, h);
}

// Before the first order, a residual-update tree's helpers stream ahead the row of the
// root's first child (the lowest index among nodes 1..kBlock whose parent is the root): the
// child the walker tests first, whose row it needs next whenever that child is accepted.
// Helper 0 publishes which child it is (the tag), as for the greedy tree.
template <int DT, bool VEC>
__device__ void helper_speculate_first(const TreeParams& p, int b, int h) {
  __shared__ int s_imin[kWavesPerBlock];
  const int tid = threadIdx.x, N = p.N, c = 1 + tid;
  const int cand = c < N && p.parents[(size_t)b * N + c] == 0 ? c : kNoPick;
  const int child = block_min_i(cand, s_imin);
  if (h == 0 && tid == 0) publish_u32(p.stag + b, child == kNoPick ? kNoSpec : static_cast<unsigned>(child) + 1u);
  if (child == kNoPick) return;
  helper_summaries<DT, VEC, true, false>(p, row_ptr<DT>(p.logits, (size_t)b * N + child, p.V),
                                         p.spec + (size_t)b * p.P, h);
}

// Helper h of request b: summarizes its chunks of every row the walker orders, until
// dismissed (in a greedy or residual-update tree, first those of the root child it streams
// ahead); the
// last helper of the request to leave returns the order word, and the streamed-ahead
// words, to zero.
template <int DT, int QT, bool VEC, bool RESID, bool ARGMAX>
__device__ void helper_item(const TreeParams& p, int b, int h) {
  __shared__ unsigned long long s_order;
  __shared__ int s_last;
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const unsigned long long* order = p.order + b;
  unsigned last_gen = 0;
  if constexpr (ARGMAX) {
    if (p.spec) helper_speculate<DT, VEC>(p, b, h);
  } else if constexpr (RESID) {
    if (p.spec) helper_speculate_first<DT, VEC>(p, b, h);
  }
  while (true) {
    if (threadIdx.x == 0) {
      unsigned long long o = fetch_u64(order);
      for (unsigned spins = 0; (o == 0ull || static_cast<unsigned>(o >> 32) == last_gen) && spins < kSpinLimit; ++spins) {
        __builtin_amdgcn_s_sleep(1);
        o = fetch_u64(order);
      }
      s_order = o;
    }
    __syncthreads();
    const unsigned long long o = s_order;
    __syncthreads();                      // every thread has read s_order before it changes
    const unsigned gen = static_cast<unsigned>(o >> 32), code = static_cast<unsigned>(o);
    if (o == 0ull || gen == last_gen || code == kTreeDone) break;   // dismissed (or the wait bound)
    if (last_gen == 0) SPEC_STAMP(p, RESID ? 3 : 2, 2);   // first order
    last_gen = gen;
    if constexpr (RESID) {
      if (code & kResidualPass) {
        residual_pass<DT, QT, VEC>(p, b, h, gen, static_cast<int>(code & ~kResidualPass));
        continue;
      }
    }
    const void* row = row_ptr<DT>(p.logits, (size_t)b * p.N + (code - 1u), p.V);
    helper_summaries<DT, VEC, RESID, ARGMAX>(p, row, p.deep + ((size_t)b * 2 + (gen & 1u)) * p.P, h);
  }
  if constexpr (ARGMAX || RESID) {
    // this block's summary stores are complete before it counts itself out, so that the
    // last helper's clears below follow every helper's stores
    vmem_wait();
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    s_last = (arrive(&p.counters[(size_t)b * kCounterSlots + 1]) == (unsigned)(p.WH - 1));
    if (s_last) {
      clear_u64(p.order + b);
      reset_counter(&p.counters[(size_t)b * kCounterSlots + 1]);
    }
  }
  if constexpr (ARGMAX || RESID) {
    if (p.spec) {           // the streamed-ahead child's words, read (or not) by the walker
      __syncthreads();
      if (s_last) {
        for (int c = threadIdx.x; c < p.P; c += kBlock) clear_f2(p.spec + (size_t)b * p.P + c);
        if (threadIdx.x == 0) publish_u32(p.stag + b, 0u);
      }
    }
  }
}

// Request b's blocks: WG1 root blocks, then WH helpers.  RESID: the residual-update
// verifier (q rows of type QT); ARGMAX: greedy membership (argmax summaries); otherwise
// membership by target sample (QT unused).
template <int DT, int QT, bool VEC, bool RESID, bool ARGMAX>
__global__ __launch_bounds__(kBlock) void tree_kernel(TreeParams p) {
  static_assert(!(RESID && ARGMAX), "the residual verifier samples");
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const int per_req = p.WG1 + p.WH;
  const int b = blockIdx.x / per_req;
  const int slice = blockIdx.x % per_req;
  constexpr int K = RESID ? 3 : 2;   // trace slot
  SPEC_STAMP(p, K, 1);
  if (slice >= p.WG1) {
    SPEC_TAG(p, K, SPEC_TRACE_TAG(kTraceHelper, b, slice - p.WG1));
    helper_item<DT, QT, VEC, RESID, ARGMAX>(p, b, slice - p.WG1);
    SPEC_STAMP(p, K, 3);
    return;
  }
  SPEC_TAG(p, K, SPEC_TRACE_TAG(kTraceRoot, b, slice));
  const int chunk = slice * kWavesPerBlock + wave;
  if (chunk < p.P) {
    const void* row0 = row_ptr<DT>(p.logits, (size_t)b * p.N, p.V);
    if constexpr (ARGMAX) {
      const unsigned long long sum = chunk_argmax<DT, VEC>(row0, p.V, chunk, lane);
      if (lane == 0) publish_u64(reinterpret_cast<unsigned long long*>(p.part + (size_t)b * p.P + chunk), sum);
    } else {
      float m, z;
      chunk_summary<DT, VEC>(row0, p.V, chunk, lane, p.c2, m, z);
      if (lane == 0) publish_f2(p.part + (size_t)b * p.P + chunk, make_float2(m, z));
    }
  }
  __syncthreads();
  SPEC_STAMP(p, K, 2);
  // the request's first root block walks: it reads the other root blocks' summaries as
  // they are published (every summary word validates itself), so no arrival count is kept
  if (slice != 0) return;
  SPEC_TAG(p, K, SPEC_TRACE_TAG(kTraceWalker, b, slice));
  unsigned gen = 0;
  if constexpr (RESID) tree_walk_residual<DT, QT, VEC>(p, b, gen);
  else tree_walk<DT, VEC, ARGMAX>(p, b, gen);
  __syncthreads();
  if (threadIdx.x == 0) publish_order(p, b, gen + 1u, kTreeDone);   // dismiss the helpers
  for (int j = threadIdx.x; j < p.P; j += kBlock) clear_f2(p.part + (size_t)b * p.P + j);
  if constexpr (RESID)   // no helper reads the descriptor once dismissed
    for (int j = threadIdx.x; j < p.desc_words; j += kBlock) publish_u64(p.desc + (size_t)b * p.desc_words + j, 0ull);
  SPEC_STAMP(p, K, 3);
}

template <int DT, int QT, bool VEC, bool RESID, bool ARGMAX = false>
hipError_t launch_typed(const TreeParams& p, hipStream_t s) {
  const unsigned g = (unsigned)((size_t)p.B * (p.WG1 + p.WH));   // == tree_blocks
  tree_kernel<DT, QT, VEC, RESID, ARGMAX><<<dim3(g), dim3(kBlock), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tree(const TreeParams& p, int logit_dtype, bool vec, hipStream_t s) {
  if (logit_dtype == kBF16)
    return vec ? launch_typed<kBF16, kF32, true, false>(p, s) : launch_typed<kBF16, kF32, false, false>(p, s);
  return vec ? launch_typed<kF32, kF32, true, false>(p, s) : launch_typed<kF32, kF32, false, false>(p, s);
}

hipError_t launch_tree_greedy(const TreeParams& p, int logit_dtype, bool vec, hipStream_t s) {
  if (logit_dtype == kBF16)
    return vec ? launch_typed<kBF16, kF32, true, false, true>(p, s) : launch_typed<kBF16, kF32, false, false, true>(p, s);
  return vec ? launch_typed<kF32, kF32, true, false, true>(p, s) : launch_typed<kF32, kF32, false, false, true>(p, s);
}

hipError_t launch_tree_residual(const TreeParams& p, int logit_dtype, bool vec, hipStream_t s) {
  const bool lb = logit_dtype == kBF16, qb = p.q_dtype == kBF16;
  if (vec) {
    if (lb) return qb ? launch_typed<kBF16, kBF16, true, true>(p, s) : launch_typed<kBF16, kF32, true, true>(p, s);
    return qb ? launch_typed<kF32, kBF16, true, true>(p, s) : launch_typed<kF32, kF32, true, true>(p, s);
  }
  if (lb) return qb ? launch_typed<kBF16, kBF16, false, true>(p, s) : launch_typed<kBF16, kF32, false, true>(p, s);
  return qb ? launch_typed<kF32, kBF16, false, true>(p, s) : launch_typed<kF32, kF32, false, true>(p, s);
}

}  // namespace sv
