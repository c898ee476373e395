// Tree verification by target-sample membership (spec_verify_tree).
//
// One kernel, ceil(V / 8192) blocks per request.  All blocks of a request stream the
// frontier row (node 0) together, one 2048-element chunk per wave, and write the chunks'
// online-softmax summaries.  The last block to finish a request walks the tree:
//   * combine the summaries of the current node's row into (reference, Z) and the
//     chunk masses, pick the chunk where the running mass passes u_v * Z, rescan that
//     chunk in vocabulary order to get the target sample y;
//   * if a child of the node carries token y, accept it and stream the child's row
//     with the same block; otherwise y is the terminal token.
// Only rows on the walked path are read.
//
// Method: [M7.7] "M7.7 - Draft Sources, Dependent Heads, and Hardware-Aware Trees"
// §0x02 (a node's row scores its children; parent index array), §0x04B and §0x09
// (accept the candidate that matches the target's own sample), §0x0F (parent index
// validity); [M16] "Module 16: Speculative Decoding", "Verify the Tree" (walk until no
// child matches, then emit one more target token).
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

// Block-wide: summaries of one full row into `part` (this request's private region for
// rows below the root), written and read by this block alone.
template <int DT, bool VEC>
__device__ void summarize_row(const TreeParams& p, float2* part, const void* row) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  for (int c = wave; c < p.P; c += kWavesPerBlock) {
    float m, z;
    chunk_summary<DT, VEC>(row, p.V, c, lane, p.c2, m, z);
    if (lane == 0) part[c] = make_float2(m, z);
  }
  __syncthreads();
}

template <int DT, bool VEC>
__device__ void tree_walk(const TreeParams& p, int b) {
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
  float2* deep = p.part_deep + (size_t)b * p.P;
  while (true) {
    const void* row = row_ptr<DT>(p.logits, (size_t)b * N + v, p.V);
    int status = 0;
    const float uv = p.u[(size_t)b * N + v];
    const int y = v == 0 ? sample_row<DT, VEC, true>(p, p.part + (size_t)b * p.P, row, uv, &status)
                         : sample_row<DT, VEC, false>(p, deep, row, uv, &status);
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
    }
    ++depth;
    v = child;
    summarize_row<DT, VEC>(p, deep, row_ptr<DT>(p.logits, (size_t)b * N + v, p.V));
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void tree_kernel(TreeParams p) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const int b = blockIdx.x / p.WG1;
  const int slice = blockIdx.x % p.WG1;
  const int chunk = slice * kWavesPerBlock + wave;
  if (chunk < p.P) {
    float m, z;
    chunk_summary<DT, VEC>(row_ptr<DT>(p.logits, (size_t)b * p.N, p.V), p.V, chunk, lane, p.c2, m, z);
    if (lane == 0) publish_f2(p.part + (size_t)b * p.P + chunk, make_float2(m, z));
  }
  __syncthreads();   // every wave's summary store has completed
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    const unsigned prev = arrive(&p.counters[(size_t)b * kCounterSlots + 0]);
    s_last = (prev == (unsigned)(p.WG1 - 1));
  }
  __syncthreads();
  if (!s_last) return;
  tree_walk<DT, VEC>(p, b);
  __syncthreads();
  for (int j = threadIdx.x; j < p.P; j += kBlock) {
    clear_f2(p.part + (size_t)b * p.P + j);
    p.part_deep[(size_t)b * p.P + j] = make_float2(0.0f, 0.0f);
  }
  if (threadIdx.x == 0) reset_counter(&p.counters[(size_t)b * kCounterSlots + 0]);
}

template <int DT, bool VEC>
hipError_t launch_typed(const TreeParams& p, hipStream_t s) {
  const unsigned g = (unsigned)((size_t)p.B * p.WG1);
  tree_kernel<DT, VEC><<<dim3(g), dim3(kBlock), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tree(const TreeParams& p, int logit_dtype, bool vec, hipStream_t s) {
  if (logit_dtype == kBF16) return vec ? launch_typed<kBF16, true>(p, s) : launch_typed<kBF16, false>(p, s);
  return vec ? launch_typed<kF32, true>(p, s) : launch_typed<kF32, false>(p, s);
}

}  // namespace sv
