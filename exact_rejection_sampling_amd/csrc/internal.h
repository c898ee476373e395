// Host-side descriptions of the kernels' arguments and workspaces, shared by the
// launchers (chain.hip, greedy.hip, tree.hip) and the C ABI (abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

// ------------------------------------------------------------ timeline trace
// In a library built with -DSPEC_TRACE (exact_rejection_sampling_amd.build --trace), thread
// 0 of every block of a traced kernel writes a tag and up to 15 stamps of the 100 MHz
// real-time counter (s_memrealtime) into the buffer that spec_trace_set installs: the
// record of block x of kernel slot k is words [(k * cap + x) * 16, + 16), and blocks at or
// past `cap` write nothing.  Other builds compile every mark to nothing and carry no trace
// member in their kernel arguments.
#ifdef SPEC_TRACE
struct TraceSink {
  unsigned long long* buf;   // [kTraceKernels * cap * kTraceWords] words, or null (tracing off)
  unsigned long long cap;    // records per kernel slot
};
constexpr int kTraceKernels = 5;   // slots: 0 chain, 1 chain exact redraw, 2 tree, 3 tree residual,
                                   // 4 top-k / top-p thresholds
constexpr int kTraceWords = 16;    // words per record: the tag, then stamps
extern TraceSink g_trace_sink;     // host copy, set by spec_trace_set
#define SPEC_TRACE_MEMBER TraceSink trace{};
__device__ __forceinline__ void trace_word(const TraceSink& t, int k, unsigned long long rec, int slot,
                                           unsigned long long v) {
  if (threadIdx.x == 0 && t.buf && rec < t.cap) t.buf[((unsigned long long)k * t.cap + rec) * kTraceWords + slot] = v;
}
#define SPEC_STAMP(P, K, SLOT) ::sv::trace_word((P).trace, (K), blockIdx.x, (SLOT), __builtin_amdgcn_s_memrealtime())
#define SPEC_TAG(P, K, TAG) ::sv::trace_word((P).trace, (K), blockIdx.x, 0, (TAG))
// the same into record REC instead of the block's own (per-event records)
#define SPEC_STAMP_AT(P, K, REC, SLOT) \
  ::sv::trace_word((P).trace, (K), (REC), (SLOT), __builtin_amdgcn_s_memrealtime())
#define SPEC_TAG_AT(P, K, REC, TAG) ::sv::trace_word((P).trace, (K), (REC), 0, (TAG))
#define SPEC_TRACE_FILL(P) ((P).trace = ::sv::g_trace_sink)
#define SPEC_TRACE_ONLY(X) X
#else
#define SPEC_TRACE_MEMBER
#define SPEC_STAMP(P, K, SLOT) ((void)0)
#define SPEC_TAG(P, K, TAG) ((void)0)
#define SPEC_STAMP_AT(P, K, REC, SLOT) ((void)0)
#define SPEC_TAG_AT(P, K, REC, TAG) ((void)0)
#define SPEC_TRACE_FILL(P) ((void)0)
#define SPEC_TRACE_ONLY(X) ((void)0)
#endif
// A record's tag: bit 63 set, the item kind in bits 56..62, the request in bits 24..55
// and the item's index within the request in bits 0..23.
#define SPEC_TRACE_TAG(KIND, B, IDX) \
  ((1ull << 63) | ((unsigned long long)(KIND) << 56) | ((unsigned long long)(unsigned)(B) << 24) | \
   (unsigned long long)((IDX) & 0xffffff))

// Per-request decision of the chain verifier: every terminal block of a request computes
// it from the request's published summaries.
struct ChainDecision {
  int32_t A;        // emitted drafts: the first rejected draft (gamma if all accepted), or
                    // the drafts up to the one that ended the round; -1 on error
  int32_t status;   // SPEC_REQ_*
  int32_t draw;     // 1: a terminal token is drawn from row A; 0: the round ended on an
                    // accepted draft (stop token or budget), or the budget was 0
  int32_t finish;   // SPEC_FINISH_* of a round that ends without a draw
  int32_t H;        // remaining output budget (INT32_MAX when none is given)
  float r_ref;      // reference exponent of the terminal row: fp32(max logit * c2)
  float inv_z;      // 1 / Z of the terminal row (Z relative to r_ref, base 2)
  float tau;        // keep threshold of the terminal row (processors; -inf otherwise)
  int32_t ev;       // first event (error, rejection, stop, budget) among the drafts read
                    // (gamma if none)
};

// Stop tokens and output budget of a round (spec_verify_*_stop); n_stop = 0 and a null
// budget give the plain verifiers.
struct StopSpec {
  const int32_t* stop;       // [n_stop] stop tokens (entries outside [0, V) never match)
  const int32_t* budget;     // [B] remaining output budget per request, or null
  int32_t* finish;           // [B] out: SPEC_FINISH_*, or null
  int n_stop;
};

// Target logit processors (spec_verify_*_ex): s = l + bias (fp32), then tokens outside the
// allowed set or below the row's keep threshold are removed (-inf).  NaN and +inf stay,
// so a faulty row still reads as invalid.  With `on` false every row is used as is.
struct ProcSpec {
  const float* bias;         // [V] additive bias, or null
  const uint32_t* allowed;   // [rows, W] allowed-token bitmask (bit x % 32 of word x / 32), or null
  const float* thresh;       // [rows] keep threshold from the top-k / top-p pass, or null
  int W;                     // words per mask row = ceil(V / 32)
  bool on;
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
  StopSpec st;
  ProcSpec pr;
  float* thresh_ws;          // the workspace's threshold words (cleared by the selectors), or null
  float2* summ_ws;           // [B*R] the threshold pass's kept-set summaries (max, Z) (Z > 0; zero
                             //   for a row it leaves to the statistics pass; cleared by the
                             //   selectors), or null
  const int32_t* q_index;    // [B, G, q_k] token indices of sparse draft rows (q then holds
  int q_k;                   //   [B, G, q_k] fp32 values), or null for dense rows
  // workspace
  float2* part;              // [B*R*SL] block summaries (raw max, Z)
  unsigned long long* gath;  // [B*G*3] draft token, its logit, its draft probability
  double* tmass;             // [B*S2] terminal chunk masses
  double* xmass;             // [B*S2*3] exact pass: per chunk residual mass, positive-set
                             // e-mass, e-mass (see chain.hip, chain_exact_kernel)
  int B, G, R, V;
  int P;                     // wave chunks per row = ceil(V / 2048)
  int CPW;                   // wave chunks each wave streams per slice
  int SL;                    // statistics slices (blocks) per row = ceil(P / (4 * CPW))
  int S2;                    // terminal chunks per row = ceil(V / kTermChunk)
  int LAG;                   // requests between a request's statistics and terminal items
  // lazy rows: rows are read in groups of LK (J groups; J = 1: every row read); group j > 0
  // of a request is read only when its drafts before row j * LK were all accepted
  int LK, J;
  int q_dtype;
  float c2;                  // fp32(log2(e) / T)
  double inv_t;              // 1 / T, T widened exactly from fp32
  double c2d;                // log2(e) / T in fp64 (the exact pass's exponent slope)
  SPEC_TRACE_MEMBER
};

#ifndef SPEC_TERM_SLABS
#define SPEC_TERM_SLABS 2
#endif
constexpr int kTermSlabs = SPEC_TERM_SLABS;   // 2048-element slabs per terminal chunk
constexpr int kTermChunk = kTermSlabs * 2048;  // elements per terminal chunk

// Greedy chunk summary, stored packed in 64 bits (idx << 32 | bits of m).
struct GreedyPart {
  float m;      // wave-chunk maximum, or NaN if the chunk holds a NaN
  int32_t idx;  // lowest index attaining it
};

struct GreedyParams {
  const void* logits;
  const int32_t* tokens;
  int32_t* accepted_len;
  int32_t* out_tokens;
  int32_t* req_status;
  StopSpec st;
  ProcSpec pr;               // bias and mask (truncations never move an argmax)
  unsigned long long* part;  // [B*R*SL] packed GreedyPart, one per slice
  int B, G, R, V, P, CPW, SL;
  int LAG;                   // requests between a request's streaming blocks and its decider
  int LK, J;                 // lazy rows: groups of LK rows, J groups (as for the chain)
};

#ifdef SPEC_FORCE_CPW
constexpr int kForceCPW = SPEC_FORCE_CPW;
#else
constexpr int kForceCPW = 0;
#endif

// Slicing of rows among blocks for the streaming passes: a block's 4 waves each stream
// CPW wave chunks (interleaved, 4 KB apart for bf16), so a block covers 4*CPW chunks.
// CPW grows with the total amount of work so that the grid stays near kTargetBlocks.
#ifndef SPEC_TARGET_BLOCKS
#define SPEC_TARGET_BLOCKS 2048
#endif
constexpr long kTargetBlocks = SPEC_TARGET_BLOCKS;
constexpr int kMaxCPW = 16;
struct Slicing { int P, CPW, SL, PP; };
inline Slicing slicing(long rows, long V, long target_blocks = kTargetBlocks) {
  Slicing s;
  s.P = static_cast<int>((V + 2047) / 2048);
  const long total = rows * s.P;
  long cpw = (total + 4 * target_blocks - 1) / (4 * target_blocks);
  if (cpw < 1) cpw = 1;
  if (cpw > kMaxCPW) cpw = kMaxCPW;
  if (kForceCPW > 0) cpw = kForceCPW;
  s.CPW = static_cast<int>(cpw);
  s.SL = static_cast<int>((s.P + 4 * cpw - 1) / (4 * cpw));
  s.PP = 4 * s.SL;
  return s;
}

struct TreeParams {
  const void* logits;        // [B, N, V]
  const int32_t* node_tokens;
  const int32_t* parents;
  const float* u;
  int32_t* accepted_len;
  int32_t* out_tokens;
  int32_t* out_nodes;
  int32_t* req_status;
  float2* part;              // [B*P] root-row summaries, published across blocks
  float2* deep;              // [B*2*P] summaries of deeper rows from the helper blocks,
                             // double-buffered by order generation
  unsigned long long* order; // [B] the walking block's order to its helpers
  unsigned* counters;        // per-request slots: [b*4 + 0] root arrivals, [b*4 + 1] helpers gone
  // greedy and residual-update trees (null for the sampled membership walk): the summaries
  // of the root's child that the helpers stream before the first order [B*P], and that
  // child + 1 per request [B] (kNoSpec when the root has no child to stream; 0 until
  // published)
  float2* spec;
  unsigned* stag;
  int B, N, V, P, WG1, WH;
  float c2;
  // residual-update verifier only
  const void* q;             // [B, N, V] proposal rows: row c = the distribution node c was drawn from
  const float* u_draw;       // [B, N] terminal draw at node v (u holds the child accept uniforms)
  unsigned long long* desc;  // [B * desc_words] residual-pass descriptors (tagged 64-bit words)
  int q_dtype, desc_words;   // desc_words = 3 + 2N
  SPEC_TRACE_MEMBER
};

// Rows the residual-update tree verifier's walking block stages in LDS: at most this many
// 2048-element chunks per row (V <= 2^21).
constexpr int kTreeStage = 1024;

// Helper blocks of a tree request: each summarizes kTreeHelperChunks chunks of an ordered
// row (its four waves two chunks each, loads in flight together).
constexpr int kTreeHelperBatch = 2;
constexpr int kTreeHelperChunks = 4 * kTreeHelperBatch;
// The residual-update tree's helpers take one chunk per wave: a residual pass reads the row
// and every rejected child's q row at each element, so fewer chunks per wave means fewer
// dependent rounds of loads per pass.
constexpr int kResidHelperBatch = 1;
constexpr int kResidHelperChunks = 4 * kResidHelperBatch;
// Helpers per request at most.  Every helper of a request stays resident from the walker's
// first order to its last, and the walker needs all of them, so a request's helpers on one
// XCD (an eighth of them: blocks go to the eight XCDs in turn) plus its
// walker must fit the XCD's slots at once: 256 helpers are 32 per XCD, against 64 slots at
// two blocks per CU on 32 CUs.  Past that (vocabularies beyond 2^22) a helper takes every
// kMaxTreeHelpers-th group of chunks in turn.  The residual tree's V <= 2^21 keeps it at
// P / 4 <= 256 helpers.
constexpr int kMaxTreeHelpers = 256;
inline long tree_helpers(long P, bool residual) {
  const long per = residual ? kResidHelperChunks : kTreeHelperChunks;
  const long h = (P + per - 1) / per;
  return h < kMaxTreeHelpers ? h : kMaxTreeHelpers;
}

// Workspace carving: 256 bytes of global counters, kCounterSlots 32-bit counters per
// request, then the data regions, each on a 256-byte boundary.  Every call returns all
// of it to zero (counters are reset and intermediate results cleared by the blocks that
// consume them), so a zero-filled workspace stays valid for any later call, of any
// entry point and any sizes, issued in order on the same stream.
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

constexpr int kCounterSlots = 4;                 // per request
constexpr size_t kGlobalCounterBytes = 256;
// Word 0 of the global header is the workspace's dirty word: a greedy or tree wait that gave
// up sets it (a word published after its consumer cleared it may be left anywhere), and from
// then on every call on the workspace reports SPEC_REQ_INTERNAL for all its requests until
// the caller zero-fills the workspace.  (A chain call repairs its own give-ups instead: the
// exact-redraw kernel that follows it zeroes those requests' words.)  Every layout starts
// its first region right after the header, so a kernel finds the word from that region.
__host__ __device__ __forceinline__ unsigned* dirty_word(const void* first_region) {
  return reinterpret_cast<unsigned*>(const_cast<char*>(static_cast<const char*>(first_region)) -
                                     kGlobalCounterBytes);
}
inline size_t counter_bytes(long B) { return align256(kGlobalCounterBytes + sizeof(unsigned) * kCounterSlots * B); }
inline unsigned* request_counters(void* ws) {
  return reinterpret_cast<unsigned*>(static_cast<char*>(ws) + kGlobalCounterBytes);
}
// slot s of request b: request_counters(ws)[b * kCounterSlots + s]

struct ChainLayout {
  size_t part, gath, tmass, thresh, summ, xmass, total;
};
// The chain's statistics pass uses finer slices than the other streaming passes: its
// terminal items fill the statistics tail, which shrinks as the slices do.
#ifndef SPEC_CHAIN_TARGET_BLOCKS
#define SPEC_CHAIN_TARGET_BLOCKS 4096
#endif
constexpr long kChainTargetBlocks = SPEC_CHAIN_TARGET_BLOCKS;
// The target counts blocks of bf16 logits: fp32 rows take twice as many blocks, so that a
// statistics item streams the same bytes in either dtype (fp32 calls at config 3 measured
// 53.1 us with one wave chunk per wave against 54.5 us with two; bf16 calls are fastest
// with two).  A larger target never gives fewer slices, so the fp32 slicing bounds both.
inline Slicing chain_slicing(long rows, long V, int logit_bytes) {
  return slicing(rows, V, logit_bytes > 2 ? 2 * kChainTargetBlocks : kChainTargetBlocks);
}
// The chain uses no counters: its regions start after the global header.  The summaries'
// region holds the fp32 slicing, the larger one.
inline ChainLayout chain_layout(long B, long G, long V) {
  const long R = G + 1, S2 = (V + kTermChunk - 1) / kTermChunk;
  const long SL = chain_slicing(B * R, V, 4).SL;
  ChainLayout L;
  size_t o = kGlobalCounterBytes;
  L.part = o;   o = align256(o + sizeof(float2) * B * R * SL);
  L.gath = o;   o = align256(o + sizeof(unsigned long long) * 3 * B * G);
  L.tmass = o;  o = align256(o + sizeof(double) * B * S2);
  L.thresh = o; o = align256(o + sizeof(float) * B * R);
  L.summ = o;   o = align256(o + sizeof(float2) * B * R);
  L.xmass = o;  o = align256(o + sizeof(double) * 3 * B * S2);
  L.total = o;
  return L;
}

// Per-row keep thresholds for top-k / top-p (one block per row): written into `thresh`.
struct ThreshParams {
  const void* logits;        // [rows, V]
  const float* bias;
  const uint32_t* allowed;   // [rows, W] or null
  const int32_t* top_k;      // [B] or null (0: off)
  const float* top_p;        // [B] or null (>= 1: off)
  float* thresh;             // [rows] out: -inf when nothing is truncated
  float2* summ;              // [rows] out: the kept set's (max, Z) where the pass holds every kept
                             //   token (Z = sum of 2^(s c2 - fp32(max c2)), the form the
                             //   statistics pass sums); left zero otherwise
  int rows, R, V, W;
  int cus;                   // compute units when two blocks share each (rows are then taken
                             //   heaviest first, lightest in the blocks that share a CU), or 0
  float c2;                  // fp32(log2(e) / T)
  SPEC_TRACE_MEMBER
};
hipError_t launch_thresholds(const ThreshParams& p, int logit_dtype, bool vec, hipStream_t s);

struct GreedyLayout { size_t part, total; };
// Greedy slicing: finer than the default, since a streaming block no longer waits on
// anything after it has streamed.
#ifndef SPEC_GREEDY_TARGET_BLOCKS
#define SPEC_GREEDY_TARGET_BLOCKS 16384
#endif
constexpr long kGreedyTargetBlocks = SPEC_GREEDY_TARGET_BLOCKS;
inline GreedyLayout greedy_layout(long B, long G, long V) {
  const long R = G + 1;
  const long SL = slicing(B * R, V, kGreedyTargetBlocks).SL;
  GreedyLayout L;
  size_t o = kGlobalCounterBytes;
  L.part = o;  o = align256(o + sizeof(unsigned long long) * B * R * SL);
  L.total = o;
  return L;
}

struct TreeLayout { size_t part, deep, order, desc, spec, stag, total; };
inline TreeLayout tree_layout(long B, long N, long V, bool residual = false) {
  const long P = (V + 2047) / 2048;
  TreeLayout L;
  size_t o = counter_bytes(B);
  L.part = o;   o = align256(o + sizeof(float2) * B * P);
  L.deep = o;   o = align256(o + sizeof(float2) * B * 2 * P);
  L.order = o;  o = align256(o + sizeof(unsigned long long) * B);
  L.desc = o;   if (residual) o = align256(o + sizeof(unsigned long long) * B * (3 + 2 * N));
  L.spec = o;   o = align256(o + sizeof(float2) * B * P);
  L.stag = o;   o = align256(o + sizeof(unsigned) * B);
  L.total = o;
  return L;
}

// Grid sizes of the launches.  A dispatch counts work-items in 32 bits, so a launch
// holds at most floor((2^32 - 1) / kBlock) blocks; grid_fits says whether it does.  The
// chain's is the grid of fp32 logits, the larger one.
inline unsigned long long chain_blocks(long B, long G, long V) {
  const long R = G + 1, S2 = (V + kTermChunk - 1) / kTermChunk;
  return (unsigned long long)B * ((unsigned long long)R * chain_slicing(B * R, V, 4).SL + S2);
}
inline unsigned long long greedy_blocks(long B, long G, long V) {
  const long R = G + 1;
  return (unsigned long long)B * ((unsigned long long)R * slicing(B * R, V, kGreedyTargetBlocks).SL + 1);
}
inline unsigned long long tree_blocks(long B, long V, bool residual = false) {
  const long P = (V + 2047) / 2048;
  return (unsigned long long)B * ((P + kWavesPerBlock - 1) / kWavesPerBlock + tree_helpers(P, residual));
}
inline bool grid_fits(unsigned long long blocks) { return blocks <= 0xffffffffull / kBlock; }

// Launchers (return hipGetLastError() after enqueueing).
hipError_t launch_chain(const ChainParams& p, int logit_dtype, bool vec, hipStream_t s);
hipError_t launch_greedy(const GreedyParams& p, int logit_dtype, bool vec, hipStream_t s);
hipError_t launch_tree(const TreeParams& p, int logit_dtype, bool vec, hipStream_t s);
hipError_t launch_tree_residual(const TreeParams& p, int logit_dtype, bool vec, hipStream_t s);
hipError_t launch_tree_greedy(const TreeParams& p, int logit_dtype, bool vec, hipStream_t s);

}  // namespace sv
