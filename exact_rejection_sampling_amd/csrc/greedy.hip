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

// Argmax summary of the chunks a wave visits (see stream_chunks): per lane the maximum
// and the lowest position holding it (positions rise with the chunk and, inside a chunk,
// with j and e), then the wave's maximum and the lowest position among its lanes.
template <int DT, bool VEC>
__device__ __forceinline__ GreedyPart wave_row_argmax(const void* row, long V, long P, long first,
                                                      long stride, int n, int lane) {
  float m = -INFINITY;
  int idx = 0x7fffffff;
  bool nan = false;
  stream_chunks<DT, VEC>(row, V, P, first, stride, n, lane, [&](const ChunkRegs<DT>& r, long c) {
    float v[kStatVecs][8];
    chunk_values<DT>(r, v);
    const long base = c * kWaveChunk;
#pragma unroll
    for (int j = 0; j < kStatVecs; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = v[j][e];
        nan |= (x != x);
        if (x > m) {
          m = x;
          idx = static_cast<int>(base + static_cast<long>(j * kWave + lane) * kVec + e);
        }
      }
  });
  const float M = wave_max(m);
  GreedyPart g;
  g.m = wave_any(nan) ? __uint_as_float(0x7fc00000u) : M;   // NaN marks a NaN-holding range
  g.idx = wave_min_i(m == M ? idx : 0x7fffffff);
  return g;
}

// Packed summary: bits of m, and idx with its top bit flipped in the high word, so a
// published summary is never all-zero bits (idx is non-negative).
__device__ __forceinline__ unsigned long long pack(const GreedyPart& g) {
  return (static_cast<unsigned long long>(static_cast<unsigned>(g.idx) ^ 0x80000000u) << 32) |
         __float_as_uint(g.m);
}
__device__ __forceinline__ GreedyPart unpack(unsigned long long b) {
  GreedyPart g;
  g.m = __uint_as_float(static_cast<unsigned>(b));
  g.idx = static_cast<int>(static_cast<unsigned>(b >> 32) ^ 0x80000000u);
  return g;
}

__device__ void greedy_decide(const GreedyParams& p, int b) {
  __shared__ int s_arg[SPEC_MAX_GAMMA + 1];
  __shared__ int s_bad[SPEC_MAX_GAMMA + 1];
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  for (int i = wave; i < p.R; i += kWavesPerBlock) {
    const unsigned long long* part = p.part + ((size_t)b * p.R + i) * p.PP;
    float m = -INFINITY;
    int nan = 0;
    for (int j = lane; j < p.PP; j += kWave) {
      const GreedyPart g = unpack(await_u64(part + j));
      m = fmaxf(m, g.m);
      nan |= (g.m != g.m);
    }
    const float M = wave_max(m);
    int idx = 0x7fffffff;
    for (int j = lane; j < p.PP; j += kWave) {
      const GreedyPart g = unpack(await_u64(part + j));
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
    unsigned long long* part = p.part + (size_t)b * p.R * p.PP;     // consumed: back to zero
    for (int j = threadIdx.x; j < p.R * p.PP; j += kBlock) clear_u64(part + j);
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
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const size_t rowid = blockIdx.x / p.SL;
  const int slice = blockIdx.x % p.SL;
  const int b = (int)(rowid / p.R);
  {
    const long first = (long)slice * kWavesPerBlock * p.CPW + wave;
    const GreedyPart g = wave_row_argmax<DT, VEC>(row_ptr<DT>(p.logits, rowid, p.V), p.V, p.P, first,
                                                  kWavesPerBlock, p.CPW, lane);
    if (lane == 0) publish_u64(p.part + rowid * p.PP + slice * kWavesPerBlock + wave, pack(g));
  }
  __syncthreads();   // every wave's summary store has completed
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    const unsigned prev = arrive(&p.counters[(size_t)b * kCounterSlots + 0]);
    s_last = (prev == (unsigned)(p.R * p.SL - 1));
  }
  __syncthreads();
  if (!s_last) return;
  greedy_decide(p, b);
  if (threadIdx.x == 0) reset_counter(&p.counters[(size_t)b * kCounterSlots + 0]);
}

template <int DT, bool VEC>
hipError_t launch_typed(const GreedyParams& p, hipStream_t s) {
  const unsigned g = (unsigned)((size_t)p.B * p.R * p.SL);
  greedy_kernel<DT, VEC><<<dim3(g), dim3(kBlock), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_greedy(const GreedyParams& p, int logit_dtype, bool vec, hipStream_t s) {
  if (logit_dtype == kBF16) return vec ? launch_typed<kBF16, true>(p, s) : launch_typed<kBF16, false>(p, s);
  return vec ? launch_typed<kF32, true>(p, s) : launch_typed<kF32, false>(p, s);
}

}  // namespace sv
