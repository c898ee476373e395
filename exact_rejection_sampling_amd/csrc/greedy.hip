// Greedy argmax-match verification (spec_verify_greedy).
//
// One kernel: each wave streams a 2048-element chunk of a target row and writes the
// chunk's maximum, the lowest index attaining it, and whether the chunk holds a NaN.
// The last block to finish a request combines the chunks of every row (max, then the
// lowest index among the chunks holding it) and compares the argmaxes with the draft
// tokens in order: the emitted tokens are the matching prefix plus the target argmax at
// the first mismatch (or at the bonus row).
//
// Method: [M7.1] "M7.1 - Speculative Decoding: Draft, Verify, Accept, Reject" §0x02D
// (longest-prefix validation is exact for greedy decoding); [Tiny] "Exact Speculative
// and Assisted Decoding for TinyRustLM", "Normative greedy pseudocode" (argmax with a
// declared tie-break -- here the lowest index -- and the target token at the first
// mismatch).
#include "device_common.h"
#include "internal.h"
#include "spec_verify.h"

namespace sv {

namespace {

template <int DT, bool VEC>
__device__ __forceinline__ GreedyPart greedy_chunk(const void* row, long V, long chunk, int lane) {
  float v[kStatVecs][8];
  const long base = chunk * kWaveChunk;
#pragma unroll
  for (int j = 0; j < kStatVecs; ++j)
    load8<DT, VEC, true>(row, base + static_cast<long>(j * kWave + lane) * kVec, V, v[j], -INFINITY);
  float m = -INFINITY;
  bool nan = false;
#pragma unroll
  for (int j = 0; j < kStatVecs; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      m = fmaxf(m, v[j][k]);
      nan |= (v[j][k] != v[j][k]);
    }
  const float M = wave_max(m);
  // lowest position in this lane holding M: lane vectors ascend with j, elements with k
  int idx = 0x7fffffff;
#pragma unroll
  for (int j = kStatVecs - 1; j >= 0; --j)
#pragma unroll
    for (int k = 7; k >= 0; --k)
      if (v[j][k] == M) idx = static_cast<int>(base + static_cast<long>(j * kWave + lane) * kVec + k);
  GreedyPart g;
  g.m = wave_any(nan) ? __uint_as_float(0x7fc00000u) : M;   // NaN marks a chunk holding NaN
  g.idx = wave_min_i(idx);
  return g;
}

__device__ __forceinline__ unsigned long long pack(const GreedyPart& g) {
  return (static_cast<unsigned long long>(static_cast<unsigned>(g.idx)) << 32) | __float_as_uint(g.m);
}
__device__ __forceinline__ GreedyPart unpack(unsigned long long b) {
  GreedyPart g;
  g.m = __uint_as_float(static_cast<unsigned>(b));
  g.idx = static_cast<int>(static_cast<unsigned>(b >> 32));
  return g;
}

__device__ void greedy_decide(const GreedyParams& p, int b) {
  __shared__ int s_arg[SPEC_MAX_GAMMA + 1];
  __shared__ int s_bad[SPEC_MAX_GAMMA + 1];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  for (int i = wave; i < p.R; i += kWavesPerBlock) {
    const unsigned long long* part = p.part + ((size_t)b * p.R + i) * p.P;
    float m = -INFINITY;
    int nan = 0;
    for (int j = lane; j < p.P; j += kWave) {
      const GreedyPart g = unpack(fetch_u64(part + j));
      m = fmaxf(m, g.m);
      nan |= (g.m != g.m);
    }
    const float M = wave_max(m);
    int idx = 0x7fffffff;
    for (int j = lane; j < p.P; j += kWave) {
      const GreedyPart g = unpack(fetch_u64(part + j));
      if (g.m == M) idx = min(idx, g.idx);
    }
    idx = wave_min_i(idx);
    const bool any_nan = wave_any(nan != 0);
    if (lane == 0) {
      s_arg[i] = idx;
      s_bad[i] = any_nan || !(M > -INFINITY && M < INFINITY);
    }
  }
  __syncthreads();
  {
    unsigned long long* part = p.part + (size_t)b * p.R * p.P;     // consumed: back to zero
    for (int j = threadIdx.x; j < p.R * p.P; j += kBlock) part[j] = 0ull;
  }
  if (wave != 0) return;
  const int G = p.G;
  int code = 0;
  bool mismatch = false;
  if (lane < G) {
    const int x = p.tokens[(size_t)b * G + lane];
    if (s_bad[lane]) code = SPEC_REQ_NONFINITE;
    else if (x < 0 || x >= p.V) code = SPEC_REQ_BADTOKEN;
    else mismatch = (x != s_arg[lane]);
  }
  const unsigned long long stop = __ballot(lane < G && (code != 0 || mismatch));
  const int A = stop ? (__ffsll((long long)stop) - 1) : G;
  int status = __shfl(code, A < G ? A : 0, kWave);
  if (A == G) status = s_bad[G] ? SPEC_REQ_NONFINITE : 0;
  for (int i = lane; i < p.R; i += kWave) {
    int v = -1;
    if (status == 0) {
      if (i < A) v = p.tokens[(size_t)b * G + i];
      else if (i == A) v = s_arg[A];
    }
    p.out_tokens[(size_t)b * p.R + i] = v;
  }
  if (lane == 0) {
    p.accepted_len[b] = status == 0 ? A : -1;
    p.req_status[b] = status;
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void greedy_kernel(GreedyParams p) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const size_t rowid = blockIdx.x / p.WG1;
  const int slice = blockIdx.x % p.WG1;
  const int b = (int)(rowid / p.R);
  const int chunk = slice * kWavesPerBlock + wave;
  if (chunk < p.P) {
    const GreedyPart g = greedy_chunk<DT, VEC>(row_ptr<DT>(p.logits, rowid, p.V), p.V, chunk, lane);
    if (lane == 0) publish_u64(p.part + rowid * p.P + chunk, pack(g));
  }
  __syncthreads();   // every wave's summary store has completed
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    const unsigned prev = arrive(&p.counters[(size_t)b * kCounterSlots + 0]);
    s_last = (prev == (unsigned)(p.R * p.WG1 - 1));
  }
  __syncthreads();
  if (!s_last) return;
  greedy_decide(p, b);
  if (threadIdx.x == 0) reset_counter(&p.counters[(size_t)b * kCounterSlots + 0]);
}

template <int DT, bool VEC>
hipError_t launch_typed(const GreedyParams& p, hipStream_t s) {
  const unsigned g = (unsigned)((size_t)p.B * p.R * p.WG1);
  greedy_kernel<DT, VEC><<<dim3(g), dim3(kBlock), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_greedy(const GreedyParams& p, int logit_dtype, bool vec, hipStream_t s) {
  if (logit_dtype == kBF16) return vec ? launch_typed<kBF16, true>(p, s) : launch_typed<kBF16, false>(p, s);
  return vec ? launch_typed<kF32, true>(p, s) : launch_typed<kF32, false>(p, s);
}

}  // namespace sv
