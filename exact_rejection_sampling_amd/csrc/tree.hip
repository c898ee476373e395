// Tree verification by target-sample membership (spec_verify_tree).
//
// One kernel.  Each request owns ceil(V / 8192) root blocks followed by ceil(V / 16384)
// helper blocks, adjacent in block order.  The root blocks stream the frontier row (node 0)
// together, one 2048-element chunk per wave, and publish the chunks' online-softmax
// summaries.  The last root block to finish walks the tree:
//   * combine the summaries of the current node's row into (reference, Z) and the chunk
//     masses, pick the chunk where the running mass passes u_v * Z, rescan that chunk in
//     vocabulary order to get the target sample y;
//   * if a child of the node carries token y, accept it and order the request's helper
//     blocks to summarize the child's row (each helper streams 8 chunks of it); otherwise
//     y is the terminal token and the helpers are dismissed.
// Only rows on the walked path are read.  Waits: the helpers wait for their walker, a
// lower-numbered block; the walker waits for its helpers, which follow its request's root
// blocks directly.  The workgroups of a launch are dispatched in index order, so the only
// helpers a walker can wait for before they are dispatched belong to the request being
// dispatched, and every other waiting block's partners are running; every wait ends, and
// each is bounded all the same (a word that does not arrive in time is reported as
// SPEC_REQ_INTERNAL).
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

__device__ void tree_fail(const TreeParams& p, int b, int code) {
  for (int i = threadIdx.x; i < p.N; i += blockDim.x) {
    p.out_tokens[(size_t)b * p.N + i] = -1;
    p.out_nodes[(size_t)b * p.N + i] = -1;
  }
  if (threadIdx.x == 0) {
    p.accepted_len[b] = -1;
    p.req_status[b] = code;
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
  __shared__ double s_before;
  __shared__ double s_total;
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
  const int per = (p.P + kBlock - 1) / kBlock;
  const int c_lo = min(tid * per, p.P), c_hi = min(c_lo + per, p.P);
  double mine = 0.0;
  for (int c = c_lo; c < c_hi; ++c) {
    const float2 s = summary<DT, VEC, PUBLISHED>(part, c);
    mine += (double)s.y * exp2((double)(s.x * c2) - (double)R);
  }
  double tot;
  const double excl = block_excl_scan_d(mine, s_scan, &tot);
  double run_end = excl;
  for (int c = c_lo; c < c_hi; ++c) {
    const float2 s = summary<DT, VEC, PUBLISHED>(part, c);
    run_end += (double)s.y * exp2((double)(s.x * c2) - (double)R);
  }
  if (c_lo < c_hi && c_hi == p.P) s_total = run_end;
  __syncthreads();
  const double Z = s_total;
  if (!(isfinite(Z) && Z > 0.0)) { *status = SPEC_REQ_NONFINITE; return -1; }
  if (!(uv >= 0.0f && uv < 1.0f)) { *status = SPEC_REQ_BADUNIFORM; return -1; }
  const double t = (double)uv * Z;
  int cand = kNoPick;          // first chunk of this thread's run whose running value passes t
  {
    double run = excl;
    for (int c = c_lo; c < c_hi; ++c) {
      const float2 s = summary<DT, VEC, PUBLISHED>(part, c);
      const double nxt = run + (double)s.y * exp2((double)(s.x * c2) - (double)R);
      if (nxt > t) { cand = c; break; }
      run = nxt;
    }
  }
  if (tid == 0) s_before = 0.0;
  // a chunk is always found (t < Z and the last running value is Z); clamp regardless
  int cstar = block_min_i(cand, s_imin);
  if (cstar == kNoPick) cstar = p.P - 1;
  if (cstar >= c_lo && cstar < c_hi) {
    double run = excl;
    for (int c = c_lo; c < cstar; ++c) {
      const float2 s = summary<DT, VEC, PUBLISHED>(part, c);
      run += (double)s.y * exp2((double)(s.x * c2) - (double)R);
    }
    s_before = run;
  }
  __syncthreads();

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
  pick = block_min_i(pick, s_imin);
  const int y = pick != kNoPick ? pick : -block_min_i(-last_pos, s_imin);
  *status = 0;
  return y;
}

// Orders from a walking block to its request's helpers, one 64-bit word per request:
// generation << 32 | code, code = row + 1 (summarize that row) or kTreeDone (leave).  A
// generation is never 0, so a published order is never zero.
constexpr unsigned kTreeDone = 0xffffffffu;

__device__ __forceinline__ void publish_order(const TreeParams& p, int b, unsigned gen, unsigned code) {
  publish_u64(p.order + b, (static_cast<unsigned long long>(gen) << 32) | code);
}

// Summaries of a row staged in LDS by the walker (rows of up to kTreeStage chunks;
// longer rows are read from the workspace directly).
constexpr int kTreeStage = 1024;

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
__device__ int sample_published(const TreeParams& p, const float2* src, const void* row, float uv, int* status) {
  __shared__ float2 s_sum[kTreeStage];
  __shared__ int s_lost;
  if (threadIdx.x == 0) s_lost = 0;
  __syncthreads();
  if (p.P <= kTreeStage) {
    stage_summaries(src, s_sum, p.P, &s_lost);
    if (s_lost) { *status = SPEC_REQ_INTERNAL; return -1; }
    return sample_row<DT, VEC, false>(p, s_sum, row, uv, status);
  }
  return sample_row<DT, VEC, true>(p, src, row, uv, status);
}

// Walk of request b by the last root block.  `gen` counts the orders sent to the helpers.
template <int DT, bool VEC>
__device__ void tree_walk(const TreeParams& p, int b, unsigned& gen) {
  __shared__ int s_bad;
  __shared__ int s_imin[kWavesPerBlock];
  const int tid = threadIdx.x;
  const int N = p.N;
  const int32_t* par = p.parents + (size_t)b * N;
  const int32_t* tok = p.node_tokens + (size_t)b * N;

  if (tid == 0) s_bad = (par[0] != -1);
  __syncthreads();
  for (int v = 1 + tid; v < N; v += kBlock) {
    const int pv = par[v], tv = tok[v];
    if (pv < 0 || pv >= v || tv < 0 || tv >= p.V) s_bad = 1;
  }
  __syncthreads();
  if (s_bad) { tree_fail(p, b, SPEC_REQ_BADTREE); return; }

  int v = 0, depth = 0;
  while (true) {
    const void* row = row_ptr<DT>(p.logits, (size_t)b * N + v, p.V);
    int status = 0;
    const float uv = p.u[(size_t)b * N + v];
    int y;
    if (v == 0) {
      y = sample_published<DT, VEC>(p, p.part + (size_t)b * p.P, row, uv, &status);
    } else {
      // the helpers' summaries of this row; returned to zero once read
      float2* deep = p.deep + ((size_t)b * 2 + (gen & 1u)) * p.P;
      y = sample_published<DT, VEC>(p, deep, row, uv, &status);
      for (int c = tid; c < p.P; c += kBlock) clear_f2(deep + c);
      vmem_wait();      // the clears are complete before any later order reuses the words
    }
    if (status != 0) { tree_fail(p, b, status); return; }
    int cand = kNoPick;           // this thread's lowest matching child (c rises)
    for (int c = v + 1 + tid; c < N; c += kBlock)
      if (cand == kNoPick && par[c] == v && tok[c] == y) cand = c;
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
      return;
    }
    if (tid == 0) {
      p.out_tokens[(size_t)b * N + depth] = tok[child];
      p.out_nodes[(size_t)b * N + depth] = child;
      publish_order(p, b, ++gen, static_cast<unsigned>(child) + 1u);   // summarize the child's row
    }
    ++depth;
    v = child;
    __shared__ unsigned s_gen;
    if (tid == 0) s_gen = gen;
    __syncthreads();
    gen = s_gen;
  }
}

// Helper h of request b: summarizes its chunks of every row the walker orders, until
// dismissed; the last helper of the request to leave returns the order word to zero.
template <int DT, bool VEC>
__device__ void helper_item(const TreeParams& p, int b, int h) {
  __shared__ unsigned long long s_order;
  __shared__ int s_last;
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const unsigned long long* order = p.order + b;
  unsigned last_gen = 0;
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
    last_gen = gen;
    const void* row = row_ptr<DT>(p.logits, (size_t)b * p.N + (code - 1u), p.V);
    float2* dst = p.deep + ((size_t)b * 2 + (gen & 1u)) * p.P;
    ChunkRegs<DT> r[kTreeHelperBatch];
#pragma unroll
    for (int k = 0; k < kTreeHelperBatch; ++k) {
      const int c = h * kTreeHelperChunks + k * kWavesPerBlock + wave;
      if (c < p.P) chunk_load<DT, VEC>(row, p.V, c, lane, r[k]);
    }
#pragma unroll
    for (int k = 0; k < kTreeHelperBatch; ++k) {
      const int c = h * kTreeHelperChunks + k * kWavesPerBlock + wave;
      if (c < p.P) {
        // the same per-chunk summary the root blocks form (one chunk per wave)
        float v[kStatVecs][8];
        chunk_values<DT>(r[k], v);
        LaneSoftmax st;
        lane_softmax_update(st, v, p.c2);
        float m, z;
        wave_softmax_merge(st, p.c2, m, z);
        if (lane == 0) publish_f2(dst + c, make_float2(m, z));
      }
    }
  }
  if (threadIdx.x == 0) {
    s_last = (arrive(&p.counters[(size_t)b * kCounterSlots + 1]) == (unsigned)(p.WH - 1));
    if (s_last) {
      clear_u64(p.order + b);
      reset_counter(&p.counters[(size_t)b * kCounterSlots + 1]);
    }
  }
}

// Request b's blocks: WG1 root blocks, then WH helpers.
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void tree_kernel(TreeParams p) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const int per_req = p.WG1 + p.WH;
  const int b = blockIdx.x / per_req;
  const int slice = blockIdx.x % per_req;
  if (slice >= p.WG1) {
    helper_item<DT, VEC>(p, b, slice - p.WG1);
    return;
  }
  const int chunk = slice * kWavesPerBlock + wave;
  if (chunk < p.P) {
    float m, z;
    chunk_summary<DT, VEC>(row_ptr<DT>(p.logits, (size_t)b * p.N, p.V), p.V, chunk, lane, p.c2, m, z);
    if (lane == 0) publish_f2(p.part + (size_t)b * p.P + chunk, make_float2(m, z));
  }
  __syncthreads();
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    const unsigned prev = arrive(&p.counters[(size_t)b * kCounterSlots + 0]);
    s_last = (prev == (unsigned)(p.WG1 - 1));
  }
  __syncthreads();
  if (!s_last) return;
  unsigned gen = 0;
  tree_walk<DT, VEC>(p, b, gen);
  __syncthreads();
  if (threadIdx.x == 0) publish_order(p, b, gen + 1u, kTreeDone);   // dismiss the helpers
  for (int j = threadIdx.x; j < p.P; j += kBlock) clear_f2(p.part + (size_t)b * p.P + j);
  if (threadIdx.x == 0) reset_counter(&p.counters[(size_t)b * kCounterSlots + 0]);
}

template <int DT, bool VEC>
hipError_t launch_typed(const TreeParams& p, hipStream_t s) {
  const unsigned g = (unsigned)((size_t)p.B * (p.WG1 + p.WH));   // == tree_blocks
  tree_kernel<DT, VEC><<<dim3(g), dim3(kBlock), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tree(const TreeParams& p, int logit_dtype, bool vec, hipStream_t s) {
  if (logit_dtype == kBF16) return vec ? launch_typed<kBF16, true>(p, s) : launch_typed<kBF16, false>(p, s);
  return vec ? launch_typed<kF32, true>(p, s) : launch_typed<kF32, false>(p, s);
}

}  // namespace sv
