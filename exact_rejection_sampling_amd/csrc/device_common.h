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
// Draft rows given sparsely: K fp32 values at K listed token indices, zero elsewhere.
constexpr int kSparseQ = 2;

// Index of the calling wave in its block, as a wave-uniform (scalar) value: loop bounds and
// branches derived from it then compile to scalar control flow.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / 64); }

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

// Eight consecutive elements [e0, e0 + 8) of a row whose address is only element-aligned
// (V % 8 != 0, or an offset base): the whole 16-byte granules holding them are loaded and
// the wanted bytes shifted out.  A granule never crosses a page and each one loaded holds
// at least one wanted byte, so it lies in mapped memory; the bytes around the wanted ones
// are never used.  The misalignment is the row's own (e0 * element size is a multiple of
// 16), the same for every lane, so the shift is uniform.
template <int DT>
__device__ __forceinline__ void load8_granules(const void* row, long e0, float (&v)[8]) {
  constexpr unsigned kBytes = DT == kBF16 ? 2u : 4u;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row) + static_cast<uintptr_t>(e0) * kBytes;
  const uintptr_t a0 = addr & ~static_cast<uintptr_t>(15);
  const unsigned off = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(addr - a0));
  const u32x4* g = reinterpret_cast<const u32x4*>(a0);
  constexpr int kGran = DT == kBF16 ? 2 : 3;    // granules spanned when misaligned
  uint32_t w[4 * kGran + 1];
  const u32x4 g0 = g[0];
  w[0] = g0.x; w[1] = g0.y; w[2] = g0.z; w[3] = g0.w;
#pragma unroll
  for (int k = 1; k < kGran; ++k) {
    u32x4 gk = u32x4{0u, 0u, 0u, 0u};
    if (off != 0u) gk = g[k];                   // off = 0: granule 0 (and 1 for fp32) suffice
    if (DT != kBF16 && k == 1) gk = g[1];
    w[4 * k] = gk.x; w[4 * k + 1] = gk.y; w[4 * k + 2] = gk.z; w[4 * k + 3] = gk.w;
  }
  w[4 * kGran] = 0u;
  constexpr int kOut = DT == kBF16 ? 4 : 8;     // dwords wanted
  uint32_t o[kOut];
  const unsigned sh = off & 3u;                 // bytes within a dword (bf16: 0 or 2)
  // the first wanted dword is w[off / 4]; a uniform switch keeps every index constant
  switch (off >> 2) {
#define SPEC_G(D)                                                                        \
  case D:                                                                                \
    _Pragma("unroll") for (int j = 0; j < kOut; ++j) o[j] = __builtin_amdgcn_alignbyte(w[D + j + 1], w[D + j], sh); \
    break;
    SPEC_G(0)
    SPEC_G(1)
    SPEC_G(2)
    SPEC_G(3)
#undef SPEC_G
  }
  if constexpr (DT == kBF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(o[k] << 16);
      v[2 * k + 1] = __uint_as_float(o[k] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __uint_as_float(o[k]);
  }
}

// Eight consecutive elements [e0, e0 + 8) of a row of V elements, e0 % 8 == 0.
// Positions >= V read as `fill`.  VEC: the row is 16-byte aligned and V % 8 == 0, so the
// group is either entirely inside or entirely past the row; a group past the row loads the
// row's first group instead (always mapped) and selects `fill`, with no branch around the
// load, so that a caller's loads of several groups all issue before the first wait.  NT:
// streaming (non-temporal) loads for data read exactly once.
template <int DT, bool VEC, bool NT>
__device__ __forceinline__ void load8(const void* row, long e0, long V, float (&v)[8], float fill) {
  if constexpr (VEC) {
    const bool in = e0 < V;
    const long ea = in ? e0 : 0;
    if constexpr (DT == kBF16) {
      const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(row) + ea);
      u32x4 w;
      if constexpr (NT) w = __builtin_nontemporal_load(p); else w = *p;
      const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = in ? __uint_as_float(d[k] << 16) : fill;
        v[2 * k + 1] = in ? __uint_as_float(d[k] & 0xffff0000u) : fill;
      }
    } else {
      const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + ea);
      f32x4 a, b;
      if constexpr (NT) { a = __builtin_nontemporal_load(p); b = __builtin_nontemporal_load(p + 1); }
      else { a = p[0]; b = p[1]; }
      v[0] = in ? a.x : fill; v[1] = in ? a.y : fill; v[2] = in ? a.z : fill; v[3] = in ? a.w : fill;
      v[4] = in ? b.x : fill; v[5] = in ? b.y : fill; v[6] = in ? b.z : fill; v[7] = in ? b.w : fill;
    }
  } else {
    if (e0 >= V) {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = fill;
    } else if (e0 + 8 <= V) {
      load8_granules<DT>(row, e0, v);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = (e0 + k < V) ? load_scalar<DT>(row, e0 + k) : fill;
    }
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

// fp64 DPP move: both halves through the same DPP pattern; lanes a step does not write
// keep `ident`.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ double dpp_d(double ident, double v) {
  const long long iv = __double_as_longlong(v), ii = __double_as_longlong(ident);
  const int lo = dpp_i<CTRL, ROWMASK>(static_cast<int>(ii), static_cast<int>(iv));
  const int hi = dpp_i<CTRL, ROWMASK>(static_cast<int>(ii >> 32), static_cast<int>(iv >> 32));
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

__device__ __forceinline__ double readlane_d(double v, int lane) {
  const long long iv = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(iv), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(iv >> 32), lane);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

// fp64 sum over the wave (DPP tree, read from lane 63): every lane ends with the same bits.
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<0xb1>(0.0, v);         // quad_perm [1,0,3,2]
  v += dpp_d<0x4e>(0.0, v);         // quad_perm [2,3,0,1]
  v += dpp_d<0x141>(0.0, v);        // row_half_mirror
  v += dpp_d<0x140>(0.0, v);        // row_mirror
  v += dpp_d<0x142, 0xa>(0.0, v);   // row_bcast:15 into rows 1, 3
  v += dpp_d<0x143, 0xc>(0.0, v);   // row_bcast:31 into rows 2, 3
  return readlane_d(v, 63);
}

// Inclusive prefix sum in fp64 over the lanes of a wave: shifts within rows of 16, then
// each row adds the running total of the rows before it.
__device__ __forceinline__ double wave_incl_scan_d(double v, int /*lane*/) {
  v += dpp_d<0x111>(0.0, v);        // row_shr:1
  v += dpp_d<0x112>(0.0, v);        // row_shr:2
  v += dpp_d<0x114>(0.0, v);        // row_shr:4
  v += dpp_d<0x118>(0.0, v);        // row_shr:8
  v += dpp_d<0x142, 0xa>(0.0, v);   // row_bcast:15 into rows 1, 3
  v += dpp_d<0x143, 0xc>(0.0, v);   // row_bcast:31 into rows 2, 3
  return v;
}

// The previous lane's value (0 in lane 0).
__device__ __forceinline__ double wave_shr1_d(double v) { return dpp_d<0x138>(0.0, v); }   // wave_shr:1

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

// Segmented reductions over groups of S consecutive lanes (S a power of two, 1..64, the
// same in every lane): every lane of a group ends with the group's result.  DPP within
// rows of 16 lanes (quad swaps, half-row and row mirrors: each step adds the partner
// half's partial exactly once), xor shuffles across rows.  Call with every lane active.
__device__ __forceinline__ float seg_max(float v, int S) {
  const float I = -INFINITY;
  if (S > 1) v = fmaxf(v, dpp_f<0xb1>(I, v));
  if (S > 2) v = fmaxf(v, dpp_f<0x4e>(I, v));
  if (S > 4) v = fmaxf(v, dpp_f<0x141>(I, v));
  if (S > 8) v = fmaxf(v, dpp_f<0x140>(I, v));
  if (S > 16) v = fmaxf(v, __shfl_xor(v, 16, kWave));
  if (S > 32) v = fmaxf(v, __shfl_xor(v, 32, kWave));
  return v;
}

__device__ __forceinline__ double seg_sum_d(double v, int S) {
  if (S > 1) v += dpp_d<0xb1>(0.0, v);
  if (S > 2) v += dpp_d<0x4e>(0.0, v);
  if (S > 4) v += dpp_d<0x141>(0.0, v);
  if (S > 8) v += dpp_d<0x140>(0.0, v);
  if (S > 16) v += __shfl_xor(v, 16, kWave);
  if (S > 32) v += __shfl_xor(v, 32, kWave);
  return v;
}

// Block-wide minimum of one int per thread, returned to every thread: a DPP tree per
// wave and one LDS word per wave (no contended LDS atomics).  `scratch` holds >=
// kWavesPerBlock ints.  Contains two barriers.
__device__ __forceinline__ int block_min_i(int v, int* scratch) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const int w = wave_min_i(v);
  if (lane == 0) scratch[wave] = w;
  __syncthreads();
  int r = scratch[0];
#pragma unroll
  for (int k = 1; k < kWavesPerBlock; ++k) r = min(r, scratch[k]);
  __syncthreads();
  return r;
}

// Block-wide exclusive prefix (fp64) of one value per thread; returns the exclusive
// prefix and writes the block total to *total.  `scratch` holds >= kWavesPerBlock doubles.
__device__ __forceinline__ double block_excl_scan_d(double v, double* scratch, double* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const double incl = wave_incl_scan_d(v, lane);
  const double excl = wave_shr1_d(incl);
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

// Two independent block-wide exclusive prefixes in one pass (the same sums, in the same
// order, as two calls of block_excl_scan_d); `scratch` holds >= 2 * kWavesPerBlock doubles.
__device__ __forceinline__ void block_excl_scan_d2(double a, double b, double* scratch, double* excl_a,
                                                   double* excl_b, double* total_a, double* total_b) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const double ia = wave_incl_scan_d(a, lane), ib = wave_incl_scan_d(b, lane);
  const double ea = wave_shr1_d(ia), eb = wave_shr1_d(ib);
  if (lane == kWave - 1) {
    scratch[wave] = ia;
    scratch[kWavesPerBlock + wave] = ib;
  }
  __syncthreads();
  double oa = 0.0, ta = 0.0, ob = 0.0, tb = 0.0;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) {
    if (w < wave) {
      oa += scratch[w];
      ob += scratch[kWavesPerBlock + w];
    }
    ta += scratch[w];
    tb += scratch[kWavesPerBlock + w];
  }
  __syncthreads();
  *excl_a = oa + ea;
  *excl_b = ob + eb;
  *total_a = ta;
  *total_b = tb;
}

// Block-wide minimum of `mn` and maximum of `mx` in one pass; `scratch` holds >= 2 *
// kWavesPerBlock ints.
__device__ __forceinline__ int block_min_max_i(int mn, int mx, int* scratch, int* max_out) {
  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const int wmn = wave_min_i(mn), wmx = -wave_min_i(-mx);
  if (lane == 0) {
    scratch[wave] = wmn;
    scratch[kWavesPerBlock + wave] = wmx;
  }
  __syncthreads();
  int r = scratch[0], q = scratch[kWavesPerBlock];
#pragma unroll
  for (int k = 1; k < kWavesPerBlock; ++k) {
    r = min(r, scratch[k]);
    q = max(q, scratch[kWavesPerBlock + k]);
  }
  __syncthreads();
  *max_out = q;
  return r;
}

// ------------------------------------------------------------------ softmax pieces
// Raw lane-vector storage for one wave chunk: 4 lane vectors of 8 elements.
template <int DT> struct ChunkRegs;
template <> struct ChunkRegs<kBF16> { u32x4 w[kStatVecs]; };
template <> struct ChunkRegs<kF32> { f32x4 a[kStatVecs], b[kStatVecs]; };

// Issue the loads of wave chunk `chunk` of a row (non-temporal: read once).  Lane L
// holds lane vectors j*64 + L; vectors past the row end hold -inf.
template <int DT, bool VEC>
__device__ __forceinline__ void chunk_load(const void* row, long V, long chunk, int lane, ChunkRegs<DT>& r) {
  const long base = chunk * kWaveChunk;
#pragma unroll
  for (int j = 0; j < kStatVecs; ++j) {
    const long e0 = base + static_cast<long>(j * kWave + lane) * kVec;
    if constexpr (VEC) {
      if constexpr (DT == kBF16) {
        r.w[j] = e0 < V ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(row) + e0))
                        : u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
      } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + e0);
        const f32x4 ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        r.a[j] = e0 < V ? __builtin_nontemporal_load(p) : ninf;
        r.b[j] = e0 < V ? __builtin_nontemporal_load(p + 1) : ninf;
      }
    } else {
      float v[8];
      load8<DT, false, false>(row, e0, V, v, -INFINITY);
      if constexpr (DT == kBF16) {
        // repack to bf16 bits (exact: the values came from bf16)
        uint32_t t[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          t[k] = (__float_as_uint(v[2 * k]) >> 16) | (__float_as_uint(v[2 * k + 1]) & 0xffff0000u);
        r.w[j] = u32x4{t[0], t[1], t[2], t[3]};
      } else {
        r.a[j] = f32x4{v[0], v[1], v[2], v[3]};
        r.b[j] = f32x4{v[4], v[5], v[6], v[7]};
      }
    }
  }
}

// Loads of a chunk known to lie entirely inside a 16-byte aligned row: unconditional, so
// that the four loads issue back to back.
template <int DT>
__device__ __forceinline__ void chunk_load_full(const void* row, long chunk, int lane, ChunkRegs<DT>& r) {
  const long base = chunk * kWaveChunk;
#pragma unroll
  for (int j = 0; j < kStatVecs; ++j) {
    const long e0 = base + static_cast<long>(j * kWave + lane) * kVec;
    if constexpr (DT == kBF16) {
      r.w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(row) + e0));
    } else {
      const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + e0);
      r.a[j] = __builtin_nontemporal_load(p);
      r.b[j] = __builtin_nontemporal_load(p + 1);
    }
  }
}

// One wave visits chunks first, first + stride, ... (n of them; chunks >= P do not exist)
// of a row and calls f(regs, chunk) for each in order.  It works in batches of kBatch
// chunks: a batch's loads all issue back to back, then the batch is reduced, so no load
// registers live across iterations; the other waves of the CU keep HBM busy meanwhile.
// Chunks entirely inside an aligned row use unconditional loads; a partial last chunk
// (or an unaligned row) the checked loader.
#ifndef SPEC_BATCH
#define SPEC_BATCH 1
#endif
constexpr int kBatch = SPEC_BATCH;

template <int DT, bool VEC, class F>
__device__ __forceinline__ void stream_chunks(const void* row, long V, long P, long first, long stride, int n,
                                              int lane, F&& f) {
  const long p_full = VEC ? V / kWaveChunk : 0;
  for (int k0 = 0; k0 < n; k0 += kBatch) {
    if (first + k0 * stride >= P) break;
    ChunkRegs<DT> r[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const long c = first + (k0 + k) * stride;
      if (k0 + k < n && c < P) {
        if (c < p_full) chunk_load_full<DT>(row, c, lane, r[k]);
        else chunk_load<DT, VEC>(row, V, c, lane, r[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const long c = first + (k0 + k) * stride;
      if (k0 + k < n && c < P) f(r[k], c);
    }
  }
}

template <int DT>
__device__ __forceinline__ void chunk_values(const ChunkRegs<DT>& r, float (&v)[kStatVecs][8]) {
#pragma unroll
  for (int j = 0; j < kStatVecs; ++j) {
    if constexpr (DT == kBF16) {
      const u32x4 w = r.w[j];
      v[j][0] = __uint_as_float(w.x << 16); v[j][1] = __uint_as_float(w.x & 0xffff0000u);
      v[j][2] = __uint_as_float(w.y << 16); v[j][3] = __uint_as_float(w.y & 0xffff0000u);
      v[j][4] = __uint_as_float(w.z << 16); v[j][5] = __uint_as_float(w.z & 0xffff0000u);
      v[j][6] = __uint_as_float(w.w << 16); v[j][7] = __uint_as_float(w.w & 0xffff0000u);
    } else {
      v[j][0] = r.a[j].x; v[j][1] = r.a[j].y; v[j][2] = r.a[j].z; v[j][3] = r.a[j].w;
      v[j][4] = r.b[j].x; v[j][5] = r.b[j].y; v[j][6] = r.b[j].z; v[j][7] = r.b[j].w;
    }
  }
}

// Per-lane online softmax state over the elements a lane has seen: m = max raw logit,
// s = sum 2^(l * c2 - r) with r = m * c2 (fp32), nan = a NaN was seen.
struct LaneSoftmax {
  float m = -INFINITY;
  float s = 0.0f;
  bool nan = false;
};

__device__ __forceinline__ void lane_softmax_update(LaneSoftmax& st, const float (&v)[kStatVecs][8], float c2) {
  float cm = -INFINITY;
#pragma unroll
  for (int j = 0; j < kStatVecs; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) cm = fmaxf(cm, v[j][k]);
  if (cm > st.m) {                       // new maximum: rescale the running sum
    if (st.m != -INFINITY) st.s *= __builtin_amdgcn_exp2f(st.m * c2 - cm * c2);
    st.m = cm;
  }
  if (st.m == -INFINITY) {               // everything so far is -inf (or NaN)
    bool nan = false;
#pragma unroll
    for (int j = 0; j < kStatVecs; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) nan |= (v[j][k] != v[j][k]);
    st.nan |= nan;
    return;
  }
  const float r = st.m * c2;
  float part[kStatVecs];
#pragma unroll
  for (int j = 0; j < kStatVecs; ++j) {
    float e[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = __builtin_amdgcn_exp2f(fmaf(v[j][k], c2, -r));
    part[j] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  }
  st.s += (part[0] + part[1]) + (part[2] + part[3]);
}

// Wave-wide merge of the lanes' states into (m, Z): m = max raw logit seen by the wave,
// Z = sum 2^(l c2 - r), r = m * c2.  Z is NaN if any lane saw NaN or +inf; (m, Z) =
// (-inf, 0) if every element was -inf.
__device__ __forceinline__ void wave_softmax_merge(const LaneSoftmax& st, float c2, float& m_out, float& z_out) {
  const float M = wave_max(st.m);
  const bool nan = wave_any(st.nan);
  float z;
  if (M == -INFINITY) {
    z = nan ? NAN : 0.0f;
  } else {
    const float R = M * c2;
    const float term = st.m == -INFINITY ? (st.nan ? NAN : 0.0f)
                                         : st.s * __builtin_amdgcn_exp2f(st.m * c2 - R);
    z = wave_sum(term);
    if (nan) z = NAN;
  }
  m_out = M;
  z_out = z;
}

// Online-softmax summary of the chunks a wave visits (see stream_chunks).
template <int DT, bool VEC>
__device__ __forceinline__ void wave_row_summary(const void* row, long V, long P, long first, long stride,
                                                 int n, int lane, float c2, float& m_out, float& z_out) {
  LaneSoftmax st;
  stream_chunks<DT, VEC>(row, V, P, first, stride, n, lane, [&](const ChunkRegs<DT>& r, long) {
    float v[kStatVecs][8];
    chunk_values<DT>(r, v);
    lane_softmax_update(st, v, c2);
  });
  wave_softmax_merge(st, c2, m_out, z_out);
}

// Single-chunk summary (one wave, one 2048-element chunk), used where a chunk must be
// summarized exactly as a later rescan recomputes it.
template <int DT, bool VEC>
__device__ __forceinline__ void chunk_summary(const void* row, long V, long chunk, int lane,
                                              float c2, float& m_out, float& z_out) {
  wave_row_summary<DT, VEC>(row, V, chunk + 1, chunk, 1, 1, lane, c2, m_out, z_out);
}

// 2^(l * c2 - r): the same expression chunk_summary sums, for recomputation of single
// terms in a rescan.
__device__ __forceinline__ float scaled_exp(float l, float c2, float r) {
  return __builtin_amdgcn_exp2f(fmaf(l, c2, -r));
}

// 2^t in fp64 with a relative error below 4e-13 for -1020 <= t <= 1 (0 below, and for
// -inf).  t = k + f with k the nearest integer, so |f| <= 1/2; 2^f = e^(f ln 2) is the
// Taylor series of the exponential to degree 10 (coefficients (ln 2)^i / i!; the first
// omitted term is below 3.1e-13 at |f| = 1/2), evaluated by Horner's rule; then the
// exponent is added.  Used where a residual row's weights must carry more precision than
// the hardware fp32 exp2 gives: a residual mass W scales every rounding error by 1/W.
__device__ __forceinline__ double exp2_acc(double t) {
  if (!(t >= -1020.0)) return 0.0;
  const double k = __builtin_rint(t);
  const double f = t - k;
  double s = 0x1.e4cf5158b8ecap-28;             // (ln 2)^10 / 10!
  s = fma(s, f, 0x1.b5253d395e7c4p-24);         // (ln 2)^9 / 9!
  s = fma(s, f, 0x1.62c0223a5c824p-20);
  s = fma(s, f, 0x1.ffcbfc588b0c7p-17);
  s = fma(s, f, 0x1.430912f86c787p-13);
  s = fma(s, f, 0x1.5d87fe78a6731p-10);
  s = fma(s, f, 0x1.3b2ab6fba4e77p-7);
  s = fma(s, f, 0x1.c6b08d704a0c0p-5);
  s = fma(s, f, 0x1.ebfbdff82c58fp-3);
  s = fma(s, f, 0x1.62e42fefa39efp-1);          // ln 2
  s = fma(s, f, 1.0);
  return ldexp(s, static_cast<int>(k));
}

// ------------------------------------------------------------------ argmax pieces
// Per-lane argmax over one chunk's values (a lane's positions base + (j*64 + lane)*8 + e
// rise with j and e): keeps the maximum and the lowest position holding it, notes NaN.
__device__ __forceinline__ void lane_argmax_update(const float (&v)[kStatVecs][8], long base, int lane,
                                                   float& m, int& idx, bool& nan) {
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
}

// Wave-wide merge: the maximum over the lanes and the lowest position among the lanes
// holding it; the maximum reads NaN if any lane saw a NaN.
__device__ __forceinline__ void wave_argmax_merge(float m, int idx, bool nan, float& m_out, int& idx_out) {
  const float M = wave_max(m);
  idx_out = wave_min_i(m == M ? idx : 0x7fffffff);
  m_out = wave_any(nan) ? __uint_as_float(0x7fc00000u) : M;
}

// Argmax summary in one 64-bit word: bits of the maximum, and the position with its top
// bit flipped in the high word, so a published summary is never all-zero bits.
__device__ __forceinline__ unsigned long long pack_argmax(float m, int idx) {
  return (static_cast<unsigned long long>(static_cast<unsigned>(idx) ^ 0x80000000u) << 32) | __float_as_uint(m);
}
__device__ __forceinline__ void unpack_argmax(unsigned long long b, float& m, int& idx) {
  m = __uint_as_float(static_cast<unsigned>(b));
  idx = static_cast<int>(static_cast<unsigned>(b >> 32) ^ 0x80000000u);
}

// Packed argmax summary of one 2048-element chunk of a row (one wave).
template <int DT, bool VEC>
__device__ __forceinline__ unsigned long long chunk_argmax(const void* row, long V, long chunk, int lane) {
  float m = -INFINITY;
  int idx = 0x7fffffff;
  bool nan = false;
  stream_chunks<DT, VEC>(row, V, chunk + 1, chunk, 1, 1, lane, [&](const ChunkRegs<DT>& r, long c) {
    float v[kStatVecs][8];
    chunk_values<DT>(r, v);
    lane_argmax_update(v, c * kWaveChunk, lane, m, idx, nan);
  });
  float M;
  int I;
  wave_argmax_merge(m, idx, nan, M, I);
  return pack_argmax(M, I);
}

// ------------------------------------------------------------------ cross-block traffic
// Values that other blocks read within the same launch (chunk summaries, chunk masses,
// decisions) travel as single 64-bit words written and read with device-scope relaxed
// atomics (write-through stores, L2-bypassing loads: coherent across the XCDs' separate
// L2 caches without cache-wide writeback or invalidate).  Every such word is encoded so
// that a published value is never all-zero bits, and every call returns the words it
// used to zero.  A reader that has learned (through an arrival count) that a word was
// published therefore re-reads it until it is non-zero: a store that is still on its way
// is never mistaken for data.  The re-reading is bounded; a word that never arrives
// reads as zero, which every consumer treats as invalid data.
constexpr unsigned kSpinLimit = 1u << 22;

__device__ __forceinline__ void publish_u64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long fetch_u64(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Re-read until the word is published (non-zero), within the spin bound.
__device__ __forceinline__ unsigned long long await_u64(const unsigned long long* p) {
  unsigned long long v = fetch_u64(p);
  for (unsigned spins = 0; v == 0ull && spins < kSpinLimit; ++spins) {
    __builtin_amdgcn_s_sleep(1);
    v = fetch_u64(p);
  }
  return v;
}
__device__ __forceinline__ void clear_u64(unsigned long long* p) { publish_u64(p, 0ull); }
// 32-bit words read by other blocks after an order that follows them (descriptors).
__device__ __forceinline__ void publish_u32(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned fetch_u32(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// (raw max m, sum Z) of a chunk range: never all-zero bits, because an empty range is
// (-inf, 0) and a non-empty one has Z >= 1 (its maximum contributes 2^0) or NaN.
__device__ __forceinline__ void publish_f2(float2* p, float2 v) {
  publish_u64(reinterpret_cast<unsigned long long*>(p),
              (static_cast<unsigned long long>(__float_as_uint(v.y)) << 32) | __float_as_uint(v.x));
}
__device__ __forceinline__ float2 await_f2(const float2* p) {
  const unsigned long long bits = await_u64(reinterpret_cast<const unsigned long long*>(p));
  return make_float2(__uint_as_float(static_cast<unsigned>(bits)),
                     __uint_as_float(static_cast<unsigned>(bits >> 32)));
}
__device__ __forceinline__ void clear_f2(float2* p) { clear_u64(reinterpret_cast<unsigned long long*>(p)); }

// A non-negative mass (or NaN) is stored negated, so that 0.0 travels as -0.0.
__device__ __forceinline__ void publish_mass(double* p, double v) {
  publish_u64(reinterpret_cast<unsigned long long*>(p),
              static_cast<unsigned long long>(__double_as_longlong(-v)));
}
__device__ __forceinline__ double await_mass(const double* p) {
  return -__longlong_as_double(static_cast<long long>(await_u64(reinterpret_cast<const unsigned long long*>(p))));
}
__device__ __forceinline__ void clear_mass(double* p) { clear_u64(reinterpret_cast<unsigned long long*>(p)); }

// Write-through store of an output word that a later block of the same launch may
// overwrite (after synchronizing on a flag): the later plain store then wins.
__device__ __forceinline__ void store_wt(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every vector memory operation this thread has issued has completed.  A
// write-through store (publish_*, clear_*) has then reached the level every XCD reads
// from, so any store this thread issues afterwards becomes visible to other blocks after
// it.  This is the ordering point of a handoff: data words, vmem_wait(), then the word
// that tells the reader to look.  (A workgroup-scope release fence would not do: with a
// workgroup confined to one CU it compiles to no wait at all.)  The "memory" clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void vmem_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Count one arrival; returns the count before this one.
__device__ __forceinline__ unsigned arrive(unsigned* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void reset_counter(unsigned* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace sv
