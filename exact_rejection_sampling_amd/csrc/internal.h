// Host-side descriptions of the kernels' arguments and workspaces, shared by the
// launchers (chain.hip, greedy.hip, tree.hip) and the C ABI (abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

// Per-request decision of the chain statistics pass, read by the terminal pass.
struct ChainDecision {
  int32_t A;        // first rejected draft (gamma if all accepted); -1 on error
  int32_t status;   // SPEC_REQ_*
  float r_ref;      // reference exponent of the terminal row: fp32(max logit * c2)
  float inv_z;      // 1 / Z of the terminal row (Z relative to r_ref, base 2)
};

struct ChainParams {
  const void* logits;        // [B, R, V]
  const void* q;             // [B, G, V]
  const int32_t* tokens;     // [B, G]
  const float* u;            // [B, R]
  int32_t* accepted_len;     // [B]
  int32_t* out_tokens;       // [B, R]
  int32_t* req_status;       // [B]
  float* stats;              // [B, R, 4] or null
  // workspace
  float2* part;              // [B*R*P] wave-chunk summaries (raw max, Z)
  unsigned* count1;          // [B] statistics-pass arrivals
  ChainDecision* dec;        // [B]
  double* tmass;             // [B*S2] terminal chunk masses
  unsigned* count2;          // [B] terminal-pass arrivals
  int B, G, R, V;
  int P;                     // wave chunks per row = ceil(V / 2048)
  int WG1;                   // blocks per row in the statistics pass = ceil(P / 4)
  int S2;                    // terminal chunks per row = ceil(V / kTermChunk)
  int q_dtype;
  float c2;                  // fp32(log2(e) / T)
  double inv_t;              // 1 / T, T widened exactly from fp32
};

constexpr int kTermSlabs = 2;                 // slabs per terminal chunk
constexpr int kTermChunk = kTermSlabs * 2048;  // elements per terminal chunk

struct GreedyPart {
  float m;      // wave-chunk maximum
  int32_t idx;  // lowest index attaining it (INT32_MAX if none)
  int32_t nan;  // chunk holds a NaN
  int32_t pad;
};

struct GreedyParams {
  const void* logits;
  const int32_t* tokens;
  int32_t* accepted_len;
  int32_t* out_tokens;
  int32_t* req_status;
  GreedyPart* part;          // [B*R*P]
  unsigned* count;           // [B]
  int B, G, R, V, P, WG1;
};

struct TreeParams {
  const void* logits;        // [B, N, V]
  const int32_t* node_tokens;
  const int32_t* parents;
  const float* u;
  int32_t* accepted_len;
  int32_t* out_tokens;
  int32_t* out_nodes;
  int32_t* req_status;
  float2* part;              // [B*P] summaries of the row being walked
  unsigned* count;           // [B]
  int B, N, V, P, WG1;
  float c2;
};

// Workspace carving: each region starts on a 256-byte boundary.
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct ChainLayout {
  size_t part, count1, dec, tmass, count2, total;
};
inline ChainLayout chain_layout(long B, long G, long V) {
  const long R = G + 1, P = (V + 2047) / 2048, S2 = (V + kTermChunk - 1) / kTermChunk;
  ChainLayout L;
  size_t o = 0;
  L.part = o;   o = align256(o + sizeof(float2) * B * R * P);
  L.count1 = o; o = align256(o + sizeof(unsigned) * B);
  L.dec = o;    o = align256(o + sizeof(ChainDecision) * B);
  L.tmass = o;  o = align256(o + sizeof(double) * B * S2);
  L.count2 = o; o = align256(o + sizeof(unsigned) * B);
  L.total = o;
  return L;
}

struct GreedyLayout { size_t part, count, total; };
inline GreedyLayout greedy_layout(long B, long G, long V) {
  const long R = G + 1, P = (V + 2047) / 2048;
  GreedyLayout L;
  size_t o = 0;
  L.part = o;  o = align256(o + sizeof(GreedyPart) * B * R * P);
  L.count = o; o = align256(o + sizeof(unsigned) * B);
  L.total = o;
  return L;
}

struct TreeLayout { size_t part, count, total; };
inline TreeLayout tree_layout(long B, long N, long V) {
  (void)N;
  const long P = (V + 2047) / 2048;
  TreeLayout L;
  size_t o = 0;
  L.part = o;  o = align256(o + sizeof(float2) * B * P);
  L.count = o; o = align256(o + sizeof(unsigned) * B);
  L.total = o;
  return L;
}

// Launchers (return hipGetLastError() after enqueueing).
hipError_t launch_chain(const ChainParams& p, int logit_dtype, bool vec, hipStream_t s);
hipError_t launch_greedy(const GreedyParams& p, int logit_dtype, bool vec, hipStream_t s);
hipError_t launch_tree(const TreeParams& p, int logit_dtype, bool vec, hipStream_t s);

}  // namespace sv
