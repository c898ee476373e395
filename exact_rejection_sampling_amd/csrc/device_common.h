// Device-side building blocks shared by the verification kernels (gfx950, wave64).
//
// Layout conventions used by every kernel:
//  * a "lane vector" is 8 consecutive vocabulary elements; in an aligned row (16-byte
//    aligned base, V % 8 == 0) it is one 16-byte load for bf16 and two for fp32;
//  * a "wave chunk" is 2048 consecutive elements of one row: lane L of the wave holds
//    lane vectors j*64 + L for j = 0..3, so each of the wave's four load instructions
//    reads one contiguous kilobyte (bf16);
//  * a "slab" is 2048 consecutive elements held by a 256-thread block, thread t owning
//    elements [8t, 8t + 8); slabs are used where vocabulary order matters (prefix sums).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

namespace sv {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kVec = 8;
constexpr int kStatVecs = 4;
constexpr int kWaveChunk = kWave * kStatVecs * kVec;   // 2048
constexpr int kSlab = kBlock * kVec;                   // 2048

enum : int { kF32 = 0, kBF16 = 1 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Elt;
template <> struct Elt<kF32> { static constexpr int bytes = 4; };
template <> struct Elt<kBF16> { static constexpr int bytes = 2; };

// Exact widening of one stored element to fp32.
template <int DT>
__device__ __forceinline__ float load_scalar(const void* base, size_t i) {
  if constexpr (DT == kBF16) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16);
  } else {
    return static_cast<const float*>(base)[i];
  }
}

template <int DT>
__device__ __forceinline__ const void* row_ptr(const void* base, size_t row, size_t V) {
  return static_cast<const char*>(base) + row * V * Elt<DT>::bytes;
}

// Eight consecutive elements [e0, e0 + 8) of a row of V elements, e0 % 8 == 0.
// Positions >= V read as `fill`.  VEC: the row is 16-byte aligned and V % 8 == 0, so the
// group is either entirely inside or entirely past the row.  NT: streaming (non-temporal)
// loads for data read exactly once.
template <int DT, bool VEC, bool NT>
__device__ __forceinline__ void load8(const void* row, long e0, long V, float (&v)[8], float fill) {
  if (e0 >= V) {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = fill;
    return;
  }
  if constexpr (VEC) {
    if constexpr (DT == kBF16) {
      const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(row) + e0);
      u32x4 w;
      if constexpr (NT) w = __builtin_nontemporal_load(p); else w = *p;
      v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
      v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
      v[4] = __uint_as_float(w.z << 16); v[5] = __uint_as_float(w.z & 0xffff0000u);
      v[6] = __uint_as_float(w.w << 16); v[7] = __uint_as_float(w.w & 0xffff0000u);
    } else {
      const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + e0);
      f32x4 a, b;
      if constexpr (NT) { a = __builtin_nontemporal_load(p); b = __builtin_nontemporal_load(p + 1); }
      else { a = p[0]; b = p[1]; }
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (e0 + k < V) ? load_scalar<DT>(row, e0 + k) : fill;
  }
}

// ------------------------------------------------------------------ wave reductions
// DPP tree over the 64 lanes; the result is read from lane 63 and is identical in every
// lane.  Rows a DPP step does not write keep `ident`, which the combining op absorbs.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ int dpp_i(int ident, int v) {
  return __builtin_amdgcn_update_dpp(ident, v, CTRL, ROWMASK, 0xf, false);
}
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ float dpp_f(float ident, float v) {
  return __int_as_float(dpp_i<CTRL, ROWMASK>(__float_as_int(ident), __float_as_int(v)));
}

__device__ __forceinline__ float wave_max(float v) {
  const float I = -INFINITY;
  v = fmaxf(v, dpp_f<0xb1>(I, v));         // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4e>(I, v));         // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(I, v));        // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(I, v));        // row_mirror
  v = fmaxf(v, dpp_f<0x142, 0xa>(I, v));   // row_bcast:15 into rows 1, 3
  v = fmaxf(v, dpp_f<0x143, 0xc>(I, v));   // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
  const float I = 0.0f;
  v = v + dpp_f<0xb1>(I, v);
  v = v + dpp_f<0x4e>(I, v);
  v = v + dpp_f<0x141>(I, v);
  v = v + dpp_f<0x140>(I, v);
  v = v + dpp_f<0x142, 0xa>(I, v);
  v = v + dpp_f<0x143, 0xc>(I, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int wave_min_i(int v) {
  const int I = 0x7fffffff;
  v = min(v, dpp_i<0xb1>(I, v));
  v = min(v, dpp_i<0x4e>(I, v));
  v = min(v, dpp_i<0x141>(I, v));
  v = min(v, dpp_i<0x140>(I, v));
  v = min(v, dpp_i<0x142, 0xa>(I, v));
  v = min(v, dpp_i<0x143, 0xc>(I, v));
  return __builtin_amdgcn_readlane(v, 63);
}

// Butterfly sum in fp64: every lane ends with the same bits.
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum in fp64 over the lanes of a wave.
__device__ __forceinline__ double wave_incl_scan_d(double v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    double t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

// Block-wide exclusive prefix (fp64) of one value per thread; returns the exclusive
// prefix and writes the block total to *total.  `scratch` holds >= kWavesPerBlock doubles.
__device__ __forceinline__ double block_excl_scan_d(double v, double* scratch, double* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const double incl = wave_incl_scan_d(v, lane);
  double excl = __shfl_up(incl, 1, kWave);
  if (lane == 0) excl = 0.0;
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  double off = 0.0, tot = 0.0;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) {
    if (w < wave) off += scratch[w];
    tot += scratch[w];
  }
  __syncthreads();
  *total = tot;
  return off + excl;
}

// ------------------------------------------------------------------ softmax pieces
// Online-softmax summary of one wave chunk of a row: m = max of the raw logits, and
// Z = sum_x 2^(l_x * c2 - r) with r = m * c2 (fp32), c2 = log2(e) / T.  The fma keeps
// l_x * c2 - r exact before its single rounding, so the summary is relative to the
// fp32 reference r that any later combine recomputes bit for bit as m * c2.
//  * a chunk whose elements are all -inf gives (m, Z) = (-inf, 0) -- or Z = NaN if the
//    "-inf" maximum hides NaN elements, since fmaxf drops NaN;
//  * NaN or +inf elements make Z NaN (fma gives NaN, exp2 and the adds keep it).
template <int DT, bool VEC>
__device__ __forceinline__ void chunk_summary(const void* row, long V, long chunk, int lane,
                                              float c2, float& m_out, float& z_out) {
  float v[kStatVecs][8];
  const long base = chunk * kWaveChunk;
#pragma unroll
  for (int j = 0; j < kStatVecs; ++j)
    load8<DT, VEC, true>(row, base + static_cast<long>(j * kWave + lane) * kVec, V, v[j], -INFINITY);
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kStatVecs; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, v[j][k]);
  m = wave_max(m);
  float z;
  if (m == -INFINITY) {
    bool nan = false;
#pragma unroll
    for (int j = 0; j < kStatVecs; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) nan |= (v[j][k] != v[j][k]);
    z = wave_any(nan) ? NAN : 0.0f;
  } else {
    const float r = m * c2;
    float s[kStatVecs];
#pragma unroll
    for (int j = 0; j < kStatVecs; ++j) {
      float e[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) e[k] = __builtin_amdgcn_exp2f(fmaf(v[j][k], c2, -r));
      s[j] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    }
    z = wave_sum((s[0] + s[1]) + (s[2] + s[3]));
  }
  m_out = m;
  z_out = z;
}

// 2^(l * c2 - r): the same expression chunk_summary sums, for recomputation of single
// terms in a rescan.
__device__ __forceinline__ float scaled_exp(float l, float c2, float r) {
  return __builtin_amdgcn_exp2f(fmaf(l, c2, -r));
}

// ------------------------------------------------------------------ cross-block traffic
// Values that other blocks read within the same launch (chunk summaries, chunk masses)
// are written and read with device-scope relaxed atomics: on this target those are
// write-through stores and L2-bypassing loads, so they are coherent across the XCDs'
// separate L2 caches without any cache-wide writeback or invalidate.  A block publishes
// them by (1) storing with publish_*, (2) waiting for its own stores to complete
// (__syncthreads, or vmem_wait() in a single thread), and (3) counting its arrival with a
// relaxed device-scope add.  The block that sees the final count reads with fetch_*.
__device__ __forceinline__ void publish_f2(float2* p, float2 v) {
  const unsigned long long bits =
      (static_cast<unsigned long long>(__float_as_uint(v.y)) << 32) | __float_as_uint(v.x);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), bits, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 fetch_f2(const float2* p) {
  const unsigned long long bits = __hip_atomic_load(
      reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<unsigned>(bits)),
                     __uint_as_float(static_cast<unsigned>(bits >> 32)));
}
__device__ __forceinline__ void publish_d(double* p, double v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                     static_cast<unsigned long long>(__double_as_longlong(v)), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double fetch_d(const double* p) {
  return __longlong_as_double(static_cast<long long>(__hip_atomic_load(
      reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
}
__device__ __forceinline__ void publish_u64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long fetch_u64(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this thread's outstanding memory operations have completed (a
// workgroup-scope release: no cache maintenance on this target).
__device__ __forceinline__ void vmem_wait() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup"); }

// Count one arrival; returns the count before this one.
__device__ __forceinline__ unsigned arrive(unsigned* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void reset_counter(unsigned* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace sv
