// Greedy argmax-match verification (spec_verify_greedy).
//
// One launch, one block per work item, the item chosen by blockIdx (block_item): for each
// request, (gamma+1)*SL streaming items and one decider, the decider placed a fixed lag of
// blocks after its request's streaming items.
//  * streaming item (row, slice): the block's four waves stream a slice of one target row
//    with 16-byte non-temporal loads, keeping per lane the maximum and the lowest position
//    holding it; lanes and waves merge, and the block publishes one summary for the slice
//    (max, lowest index attaining it, NaN if the slice holds a NaN).  It waits only as
//    the gate of a lazy row group: with lazy_rows = LK the rows come in groups of LK,
//    ordered group by group, and an item of a later group first decides, from the
//    previous group's summaries, whether the round reaches it; if not it publishes a NaN
//    summary instead of streaming (it reads as an invalid row, after an earlier event).
//  * decider (request): reads every summary of its request as soon as it is published,
//    combines each row's slices (the max, then the lowest index among the slices holding
//    it), compares the argmaxes with the draft tokens in order and emits the matching
//    prefix plus the target argmax at the first mismatch (or at the bonus row).  It then
//    returns the summaries to zero.
// Waits: a decider waits only for its request's streaming items, and a lazy gate only for
// the previous group's items, whose block indices are all lower; the workgroups of a launch are dispatched in index order, so those blocks are
// running or done and the wait ends.  It is bounded all the same: a summary that does not
// arrive in time makes the request report SPEC_REQ_INTERNAL.
//
// Method: [M7.1] "M7.1 - Speculative Decoding: Draft, Verify, Accept, Reject" §0x02D
// (longest-prefix validation is exact for greedy decoding); [Tiny] "Exact Speculative
// and Assisted Decoding for TinyRustLM", "Normative greedy pseudocode" (argmax with a
// declared tie-break -- here the lowest index -- and the target token at the first
// mismatch).
#include "device_common.h"
#include "internal.h"
#include "proc.h"
#include "spec_verify.h"

namespace sv {

namespace {

// Argmax summary of the chunks a wave visits (see stream_chunks): per lane the maximum
// and the lowest position holding it (positions rise with the chunk and, inside a chunk,
// with j and e), then the wave's maximum and the lowest position among its lanes.
// PROC: the processors (bias, allowed set) are applied to every element of row `rowid`
// first; truncations keep the maximum, so they never move an argmax and are not applied.
template <int DT, bool VEC, bool PROC>
__device__ __forceinline__ GreedyPart wave_row_argmax(const ProcSpec& pr, size_t rowid, const void* row, long V,
                                                      long P, long first, long stride, int n, int lane) {
  float m = -INFINITY;
  int idx = 0x7fffffff;
  bool nan = false;
  stream_chunks<DT, VEC>(row, V, P, first, stride, n, lane, [&](const ChunkRegs<DT>& r, long c) {
    float v[kStatVecs][8];
    chunk_values<DT>(r, v);
    if constexpr (PROC) {
#pragma unroll
      for (int j = 0; j < kStatVecs; ++j)
        proc8<VEC>(pr, rowid, -INFINITY, c * kWaveChunk + static_cast<long>(j * kWave + lane) * kVec, V, v[j]);
    }
    lane_argmax_update(v, c * kWaveChunk, lane, m, idx, nan);
  });
  GreedyPart g;
  wave_argmax_merge(m, idx, nan, g.m, g.idx);   // NaN marks a NaN-holding range
  return g;
}

__device__ __forceinline__ unsigned long long pack(const GreedyPart& g) { return pack_argmax(g.m, g.idx); }
__device__ __forceinline__ GreedyPart unpack(unsigned long long b) {
  GreedyPart g;
  unpack_argmax(b, g.m, g.idx);
  return g;
}

// Streaming item: slice `slice` of row i of request b.
template <int DT, bool VEC, bool PROC>
__device__ void stream_item(const GreedyParams& p, int b, int i, int slice) {
  __shared__ GreedyPart s_w[kWavesPerBlock];
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const size_t rowid = (size_t)b * p.R + i;
  const long first = (long)slice * kWavesPerBlock * p.CPW + wave;
  const GreedyPart g = wave_row_argmax<DT, VEC, PROC>(p.pr, rowid, row_ptr<DT>(p.logits, rowid, p.V), p.V, p.P,
                                                      first, kWavesPerBlock, p.CPW, lane);
  if (lane == 0) s_w[wave] = g;
  __syncthreads();
  if (threadIdx.x == 0) {
    // the slice's maximum, then the lowest position among the waves holding it (waves
    // visit interleaved chunks, so positions do not follow wave order); NaN if any wave
    // saw one
    float M = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
      nan |= (s_w[w].m != s_w[w].m);
      M = fmaxf(M, s_w[w].m);
    }
    int idx = 0x7fffffff;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w)
      if (s_w[w].m == M) idx = min(idx, s_w[w].idx);
    GreedyPart out;
    out.m = nan ? __uint_as_float(0x7fc00000u) : M;
    out.idx = idx;
    publish_u64(p.part + rowid * p.SL + slice, pack(out));
  }
}

// Decision of request b over rows [lo, nr) and drafts [lo, min(nr, gamma)).  The decider
// of the request reads every row (lo = 0, nr = gamma + 1), writes the outputs and returns
// the summaries to zero.  With nr < gamma + 1 it is the gate of a lazy row group (rows
// [nr, ...)): it returns, block-uniformly, whether the round reaches row nr -- the rows
// [lo, nr) were read (a skipped group's summaries read as NaN rows, an event at its first
// draft) and none of their drafts ends the round -- and changes nothing.  A gate whose
// words did not arrive answers yes, so that no row the decider may need is skipped.
__device__ bool greedy_decide(const GreedyParams& p, int b, int lo, int nr) {
  __shared__ int s_arg[SPEC_MAX_GAMMA + 1];
  __shared__ int s_bad[SPEC_MAX_GAMMA + 1];
  __shared__ int s_lost;
  __shared__ int s_x[SPEC_MAX_GAMMA];           // the drafts, for the stop-token test
  __shared__ int s_stop[SPEC_MAX_STOP];         // the stop tokens, for the target token's test
  __shared__ unsigned s_hit[2];                 // bit i: draft i is a stop token
  __shared__ int s_reach;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
  const bool gate = nr < p.R;
  const int G = p.G, nd = min(G, nr);
  unsigned long long* part_b = p.part + (size_t)b * p.R * p.SL;
  if (tid == 0) s_lost = 0;
  // the workspace's dirty word (a wait of an earlier call gave up), checked with the summaries
  const unsigned dirty = tid == 0 ? fetch_u32(dirty_word(p.part)) : 0u;
  // wave 0's draft tokens and the remaining budget, fetched while the summaries are awaited
  int x = 0;
  if (wave == 0 && lane < G) x = p.tokens[(size_t)b * G + lane];
  const int H = p.st.budget ? p.st.budget[b] : INT32_MAX;
  const bool stops = p.st.n_stop > 0;
  const int my_stop = stops && tid < p.st.n_stop ? p.st.stop[tid] : 0;
  if (stops) {
    if (wave == 0 && lane < G) s_x[lane] = x;
    if (tid < p.st.n_stop) s_stop[tid] = my_stop;
    if (tid < 2) s_hit[tid] = 0u;
  }
  __syncthreads();
  // stop tokens: thread t < n_stop tests entry t against every decided draft
  if (stops && tid < p.st.n_stop)
    for (int i = lo; i < nd; ++i)
      if (s_x[i] == my_stop) atomicOr(&s_hit[i >> 5], 1u << (i & 31));
  for (int i = lo + wave; i < nr; i += kWavesPerBlock) {
    const unsigned long long* part = part_b + (size_t)i * p.SL;
    float m = -INFINITY;
    int idx = 0x7fffffff;
    bool nan = false, lost = false;
    // lane j takes slices j, j + 64, ...: slices rise with position, so a lane's lowest
    // position at its own maximum is its first slice holding that maximum
    for (int j = lane; j < p.SL; j += kWave) {
      const unsigned long long bits = await_u64(part + j);
      lost |= (bits == 0ull);
      const GreedyPart g = unpack(bits);
      nan |= (g.m != g.m);
      if (g.m > m) {
        m = g.m;
        idx = g.idx;
      }
    }
    const float M = wave_max(m);
    const int arg = wave_min_i(m == M ? idx : 0x7fffffff);
    const bool any_nan = wave_any(nan);
    if (wave_any(lost) && lane == 0) s_lost = 1;
    if (lane == 0) {
      s_arg[i] = arg;
      s_bad[i] = any_nan || !(M > -INFINITY && M < INFINITY);
    }
  }
  if (dirty) s_lost = 1;
  __syncthreads();
  // the summaries are consumed: return them to zero (every call leaves the workspace zeroed)
  if (!gate)
    for (int j = tid; j < p.R * p.SL; j += kBlock) clear_u64(part_b + j);
  // lane i in [lo, nd): draft position i; a matching draft that is a stop token, or that
  // uses up the budget, ends the round after itself ([Tiny] "Normative greedy pseudocode")
  int code = 0, fin = 0;
  bool mismatch = false;
  const bool dl = wave == 0 && lane >= lo && lane < nd;
  if (dl) {
    if (s_bad[lane]) {
      code = SPEC_REQ_NONFINITE;
    } else if (x < 0 || x >= p.V) {
      code = SPEC_REQ_BADTOKEN;
    } else {
      mismatch = (x != s_arg[lane]);
      if (!mismatch) {
        if (stops && ((s_hit[lane >> 5] >> (lane & 31)) & 1u)) fin = SPEC_FINISH_STOP;
        else if (lane + 1 == H) fin = SPEC_FINISH_BUDGET;
      }
    }
  }
  const unsigned long long ev = __ballot(dl && (code != 0 || mismatch || fin != 0));
  const int e = ev ? (__ffsll((long long)ev) - 1) : G;   // the first event
  if (gate) {
    if (tid == 0) s_reach = s_lost || (e >= nr && H > 0);
    __syncthreads();
    return s_reach != 0;
  }
  if (wave != 0) return false;
  const int code_e = __shfl(code, e < G ? e : 0, kWave);
  const int fin_e = __shfl(fin, e < G ? e : 0, kWave);
  int A = e, status = 0, finish = 0;
  bool draw = true;
  if (e < G && fin_e != 0) {           // the round ends on draft e with no target token
    A = e + 1;
    draw = false;
    finish = fin_e;
  } else {
    status = e < G ? code_e : (s_bad[G] ? SPEC_REQ_NONFINITE : 0);
  }
  if (H <= 0) {                        // no budget left: no round, nothing checked
    A = 0;
    status = 0;
    draw = false;
    finish = SPEC_FINISH_BUDGET;
  }
  if (s_lost) status = SPEC_REQ_INTERNAL;
  if (status == 0 && draw) {           // the target token at A
    const int t = s_arg[A];
    bool hit = false;
    for (int j = lane; j < p.st.n_stop; j += kWave) hit |= (s_stop[j] == t);
    finish = wave_any(hit) ? SPEC_FINISH_STOP : (A + 1 == H ? SPEC_FINISH_BUDGET : 0);
  }
  for (int i = lane; i < p.R; i += kWave) {
    int v = -1;
    if (status == 0) {
      if (i < A) v = p.tokens[(size_t)b * G + i];
      else if (i == A && draw) v = s_arg[A];
    }
    p.out_tokens[(size_t)b * p.R + i] = v;
  }
  if (lane == 0) {
    p.accepted_len[b] = status == 0 ? A : -1;
    p.req_status[b] = status;
    if (p.st.finish) p.st.finish[b] = status == 0 ? finish : 0;
    // a summary may arrive after the clear above: the workspace is no longer known to be zero
    if (status == SPEC_REQ_INTERNAL) publish_u32(dirty_word(p.part), 1u);
  }
  return false;
}

// Block order: groups g = 0 .. B + L - 1, group g holding the Sb streaming items of
// request g (if g < B) followed by the decider of request g - L (if g >= L).  32-bit
// arithmetic: a grid holds fewer than 2^24 blocks.
struct Item { int decider, b, idx; };
__host__ __device__ __forceinline__ Item tail_item(unsigned t, unsigned B, unsigned Sb, unsigned L) {
  const unsigned n1 = L * Sb, n2 = (B - L) * (Sb + 1);
  Item it;
  if (t < n1) {
    it.decider = 0; it.b = (int)(t / Sb); it.idx = (int)(t - (unsigned)it.b * Sb);
  } else if (t < n1 + n2) {
    const unsigned u = t - n1, k = u / (Sb + 1), o = u - k * (Sb + 1);
    if (o < Sb) { it.decider = 0; it.b = (int)(L + k); it.idx = (int)o; }
    else { it.decider = 1; it.b = (int)k; it.idx = 0; }
  } else {
    it.decider = 1; it.b = (int)(B - L + (t - n1 - n2)); it.idx = 0;
  }
  return it;
}

// Lazy rows: row group j (rows [j LK, (j + 1) LK)) of every request, for j = 0 .. J-2 in
// turn, then the last group interleaved with the deciders as above; with J = 1 this is the
// order above.  A group's items follow every item of the request's earlier groups.
__host__ __device__ __forceinline__ Item block_item(const GreedyParams& p, unsigned t) {
  const unsigned B = p.B, SL = p.SL, LK = p.LK, J = p.J;
  const unsigned nG = LK * SL, layer = B * nG, early = (J - 1) * layer;
  Item it;
  if (t < early) {
    const unsigned j = t / layer, u = t - j * layer, b = u / nG;
    it.decider = 0; it.b = (int)b; it.idx = (int)(j * nG + (u - b * nG));
    return it;
  }
  const unsigned first = (J - 1) * LK;   // the last group's first row
  it = tail_item(t - early, B, ((unsigned)p.R - first) * SL, p.LAG);
  if (!it.decider) it.idx += (int)(first * SL);
  return it;
}

template <int DT, bool VEC, bool PROC>
__global__ __launch_bounds__(kBlock) void greedy_kernel(GreedyParams p) {
  const Item it = block_item(p, blockIdx.x);
  const int row = it.idx / p.SL;
  // the rows a decision reads: every row for a decider; for a lazy row group after the
  // first, the rows of the group before it (whether the round reaches this group)
  int lo = 0, nr = 0;
  bool reached = true;
  if (it.decider) {
    nr = p.R;
  } else if (p.J > 1) {
    const int first = (row / p.LK) * p.LK;
    if (first == 0) reached = p.st.budget == nullptr || p.st.budget[it.b] > 0;
    else { lo = first - p.LK; nr = first; }
  }
  if (nr > 0) {
    const bool r = greedy_decide(p, it.b, lo, nr);   // one call site: inlined once
    if (it.decider) return;
    reached = r;
  }
  if (reached) {
    stream_item<DT, VEC, PROC>(p, it.b, row, it.idx % p.SL);
  } else if (threadIdx.x == 0) {
    // a row the round never reaches: a NaN summary, which the decision never uses (an
    // earlier event ends the round), says only that this item is done
    publish_u64(p.part + ((size_t)it.b * p.R + row) * p.SL + it.idx % p.SL, pack_argmax(__uint_as_float(0x7fc00000u), 0));
  }
}

// Lag between a request's streaming items and its decider, in tenths of a round of
// resident blocks: the decider starts about that many block generations later, when the
// request's summaries are normally published.
#ifndef SPEC_GREEDY_LAG_TENTHS
#define SPEC_GREEDY_LAG_TENTHS 20
#endif
constexpr long kGreedyLagTenths = SPEC_GREEDY_LAG_TENTHS;

template <int DT, bool VEC, bool PROC>
hipError_t launch_typed(GreedyParams p, hipStream_t s) {
  static int s_resident[64] = {0};   // resident blocks per device ordinal; 0 = not queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (s_resident[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, greedy_kernel<DT, VEC, PROC>, kBlock, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidValue;
    s_resident[dev] = (per_cu < 1 ? 1 : per_cu) * (cus < 1 ? 1 : cus);
  }
  const long per_req = (long)p.R * p.SL + 1;
  long lag = (kGreedyLagTenths * s_resident[dev] / 10 + per_req - 1) / per_req;
  if (lag < 1) lag = 1;
  if (lag > p.B) lag = p.B;
  p.LAG = (int)lag;
  const unsigned long long g = (unsigned long long)p.B * ((unsigned long long)p.R * p.SL + 1);  // == greedy_blocks
  greedy_kernel<DT, VEC, PROC><<<dim3((unsigned)g), dim3(kBlock), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_greedy(const GreedyParams& p, int logit_dtype, bool vec, hipStream_t s) {
  if (p.pr.on) {
    if (logit_dtype == kBF16) return vec ? launch_typed<kBF16, true, true>(p, s) : launch_typed<kBF16, false, true>(p, s);
    return vec ? launch_typed<kF32, true, true>(p, s) : launch_typed<kF32, false, true>(p, s);
  }
  if (logit_dtype == kBF16) return vec ? launch_typed<kBF16, true, false>(p, s) : launch_typed<kBF16, false, false>(p, s);
  return vec ? launch_typed<kF32, true, false>(p, s) : launch_typed<kF32, false, false>(p, s);
}

}  // namespace sv
