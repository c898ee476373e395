// C ABI of libspec_verify.so: host-side argument checks, workspace carving and launches.
// The entry points and their contracts are declared in include/spec_verify.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "device_common.h"
#include "internal.h"
#include "spec_verify.h"

#ifdef SPEC_TRACE
namespace sv { TraceSink g_trace_sink{}; }
#endif

namespace {

constexpr double kLog2e = 1.44269504088896340736;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }
bool dtype_ok(int d) { return d == SPEC_F32 || d == SPEC_BF16; }
bool temperature_ok(float t) {
  return t >= SPEC_MIN_TEMPERATURE && t <= SPEC_MAX_TEMPERATURE;   // false for NaN
}
bool sizes_ok(int B, int gamma, int V) {
  return B >= 0 && B <= SPEC_MAX_BATCH && gamma >= 0 && gamma <= SPEC_MAX_GAMMA && V >= 1 &&
         V <= SPEC_MAX_VOCAB;
}
int chunks(long V, long per) { return static_cast<int>((V + per - 1) / per); }
bool stop_ok(const int32_t* stop_tokens, int n_stop) {
  return n_stop >= 0 && n_stop <= SPEC_MAX_STOP && (n_stop == 0 || stop_tokens != nullptr);
}
sv::ProcSpec proc_spec(const spec_verify_options& o, int V, const float* thresh) {
  sv::ProcSpec pr{};
  pr.bias = o.bias;
  pr.allowed = o.allowed;
  pr.thresh = thresh;
  pr.W = (V + 31) / 32;
  pr.on = o.bias || o.allowed || thresh;
  return pr;
}
sv::StopSpec stop_spec(const int32_t* stop_tokens, int n_stop, const int32_t* budget, int32_t* finish) {
  sv::StopSpec st;
  st.stop = n_stop > 0 ? stop_tokens : nullptr;
  st.n_stop = n_stop;
  st.budget = budget;
  st.finish = finish;
  return st;
}
}  // namespace

// ------------------------------------------------------------ no-allocation chain call
// Device scratch of spec_verify_chain_static: a file-scope array that each GPU holds for the
// life of the process.  In host code its name stands for no device address; the entry
// point looks the address up once per device (hipGetSymbolAddress, with that device
// current) and passes only that pointer on.
constexpr size_t kStaticScratchBytes = SPEC_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's scratch address, looked up on its first use; null on failure.
void* device_scratch(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Zero-fill of n 64-bit words (a kernel rather than a memset node, so the call can be
// captured in a graph).
__global__ __launch_bounds__(256) void zero_words(unsigned long long* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0ull;
}
}  // namespace

extern "C" {

int spec_abi_version(void) { return SPEC_ABI_VERSION; }

spec_status spec_trace_set(void* buffer, size_t records_per_kernel) {
#ifdef SPEC_TRACE
  if (buffer && records_per_kernel == 0) return SPEC_EINVAL;
  sv::g_trace_sink.buf = static_cast<unsigned long long*>(buffer);
  sv::g_trace_sink.cap = buffer ? records_per_kernel : 0;
  return SPEC_OK;
#else
  (void)buffer;
  (void)records_per_kernel;
  return SPEC_EINVAL;
#endif
}

const char* spec_status_string(int code) {
  switch (code) {
    case SPEC_OK: return "ok";
    case SPEC_EINVAL: return "invalid argument (null pointer, size out of range or bad temperature)";
    case SPEC_EDTYPE: return "unknown dtype";
    case SPEC_EWORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case SPEC_EHIP: return "HIP kernel launch failed";
    case SPEC_ESCRATCH: return "sizes need more device scratch than spec_verify_chain_static holds";
    default: return "unknown status";
  }
}

const char* spec_req_status_string(int code) {
  switch (code) {
    case SPEC_REQ_OK: return "ok";
    case SPEC_REQ_NONFINITE: return "reached logits row has NaN or +inf, or is entirely -inf";
    case SPEC_REQ_BADTOKEN: return "draft token outside [0, V)";
    case SPEC_REQ_BADUNIFORM: return "uniform outside [0, 1)";
    case SPEC_REQ_QZERO: return "draft probability of a proposed token is not positive";
    case SPEC_REQ_RESIDUAL_EMPTY: return "terminal mass not positive or q row invalid";
    case SPEC_REQ_BADTREE: return "invalid parent array or node token";
    case SPEC_REQ_INTERNAL: return "internal wait bound reached (outputs invalid)";
    default: return "unknown request status";
  }
}

size_t spec_chain_workspace_bytes(int B, int gamma, int V) {
  if (!sizes_ok(B, gamma, V) || !sv::grid_fits(sv::chain_blocks(B, gamma, V))) return 0;
  return sv::chain_layout(B, gamma, V).total;
}

size_t spec_greedy_workspace_bytes(int B, int gamma, int V) {
  if (!sizes_ok(B, gamma, V) || !sv::grid_fits(sv::greedy_blocks(B, gamma, V))) return 0;
  return sv::greedy_layout(B, gamma, V).total;
}

bool residual_sizes_ok(int B, int N, int V) {
  return B >= 0 && B <= SPEC_MAX_BATCH && N >= 1 && N <= SPEC_MAX_NODES && V >= 1 &&
         V <= sv::kTreeStage * 2048;
}

size_t spec_tree_residual_workspace_bytes(int B, int N, int V) {
  if (!residual_sizes_ok(B, N, V) || !sv::grid_fits(sv::tree_blocks(B, V, true))) return 0;
  return sv::tree_layout(B, N, V, true).total;
}

size_t spec_tree_workspace_bytes(int B, int N, int V) {
  if (!(B >= 0 && B <= SPEC_MAX_BATCH && N >= 1 && N <= SPEC_MAX_NODES && V >= 1 && V <= SPEC_MAX_VOCAB))
    return 0;
  if (!sv::grid_fits(sv::tree_blocks(B, V))) return 0;
  return sv::tree_layout(B, N, V).total;
}

spec_status spec_verify_chain(const void* target_logits, int logit_dtype, const void* draft_probs,
                              int q_dtype, const int32_t* draft_tokens, const float* uniforms, int B,
                              int gamma, int V, float temperature, int32_t* accepted_len,
                              int32_t* out_tokens, int32_t* req_status, float* stats,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return spec_verify_chain_ex(target_logits, logit_dtype, draft_probs, q_dtype, draft_tokens, uniforms, B, gamma,
                              V, temperature, nullptr, accepted_len, out_tokens, req_status, stats, workspace,
                              workspace_bytes, stream);
}

spec_status spec_verify_chain_stop(const void* target_logits, int logit_dtype, const void* draft_probs,
                                   int q_dtype, const int32_t* draft_tokens, const float* uniforms, int B,
                                   int gamma, int V, float temperature, const int32_t* stop_tokens,
                                   int n_stop, const int32_t* budget, int32_t* accepted_len,
                                   int32_t* out_tokens, int32_t* req_status, int32_t* finish, float* stats,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  spec_verify_options o = {};
  o.stop_tokens = stop_tokens;
  o.n_stop = n_stop;
  o.budget = budget;
  o.finish = finish;
  return spec_verify_chain_ex(target_logits, logit_dtype, draft_probs, q_dtype, draft_tokens, uniforms, B, gamma,
                              V, temperature, &o, accepted_len, out_tokens, req_status, stats, workspace,
                              workspace_bytes, stream);
}

spec_status spec_verify_chain_ex(const void* target_logits, int logit_dtype, const void* draft_probs,
                                 int q_dtype, const int32_t* draft_tokens, const float* uniforms, int B,
                                 int gamma, int V, float temperature, const spec_verify_options* opt,
                                 int32_t* accepted_len, int32_t* out_tokens, int32_t* req_status, float* stats,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const spec_verify_options o = opt ? *opt : spec_verify_options{};
  if (!sizes_ok(B, gamma, V) || !temperature_ok(temperature) || !stop_ok(o.stop_tokens, o.n_stop))
    return SPEC_EINVAL;
  if (o.q_index && !(o.q_k >= 1 && o.q_k <= SPEC_MAX_SPARSE_K)) return SPEC_EINVAL;
  if (o.lazy_rows < 0) return SPEC_EINVAL;
  if (!dtype_ok(logit_dtype) || !dtype_ok(q_dtype)) return SPEC_EDTYPE;
  if (o.q_index && q_dtype != SPEC_F32) return SPEC_EDTYPE;
  if (!sv::grid_fits(sv::chain_blocks(B, gamma, V))) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!target_logits || !uniforms || !accepted_len || !out_tokens || !req_status) return SPEC_EINVAL;
  if (gamma > 0 && (!draft_probs || !draft_tokens)) return SPEC_EINVAL;
  const sv::ChainLayout L = sv::chain_layout(B, gamma, V);
  if (!workspace || workspace_bytes < L.total || !aligned256(workspace)) return SPEC_EWORKSPACE;

  char* ws = static_cast<char*>(workspace);
  sv::ChainParams p;
  p.logits = target_logits;
  p.q = draft_probs;
  p.tokens = draft_tokens;
  p.u = uniforms;
  p.accepted_len = accepted_len;
  p.out_tokens = out_tokens;
  p.req_status = req_status;
  p.stats = stats;
  p.st = stop_spec(o.stop_tokens, o.n_stop, o.budget, o.finish);
  const bool truncate = o.top_k || o.top_p;
  p.pr = proc_spec(o, V, truncate ? reinterpret_cast<float*>(ws + L.thresh) : nullptr);
  p.thresh_ws = truncate ? reinterpret_cast<float*>(ws + L.thresh) : nullptr;
  p.summ_ws = truncate ? reinterpret_cast<float2*>(ws + L.summ) : nullptr;
  p.q_index = gamma > 0 ? o.q_index : nullptr;
  p.q_k = o.q_k;
  p.part = reinterpret_cast<float2*>(ws + L.part);
  p.gath = reinterpret_cast<unsigned long long*>(ws + L.gath);
  p.tmass = reinterpret_cast<double*>(ws + L.tmass);
  p.xmass = reinterpret_cast<double*>(ws + L.xmass);
  p.B = B;
  p.G = gamma;
  p.R = gamma + 1;
  p.V = V;
  // lazy row groups keep the bf16 slicing for fp32 logits too: every item of a later group
  // first takes a gate decision, and twice the items cost more than they save (fp32, groups
  // of 3 at config 3: 48.6 us against 46.9 us)
  const bool lazy = o.lazy_rows >= 1 && o.lazy_rows < gamma + 1;
  const sv::Slicing sl = sv::chain_slicing((long)B * (gamma + 1), V, logit_dtype == SPEC_F32 && !lazy ? 4 : 2);
  p.P = sl.P;
  p.CPW = sl.CPW;
  p.SL = sl.SL;
  p.S2 = chunks(V, sv::kTermChunk);
  p.LK = lazy ? o.lazy_rows : gamma + 1;
  p.J = (gamma + 1 + p.LK - 1) / p.LK;
  p.LAG = 0;
  p.q_dtype = q_dtype;
  const double c2 = kLog2e / static_cast<double>(temperature);
  p.c2 = static_cast<float>(c2);
  p.inv_t = 1.0 / static_cast<double>(temperature);
  p.c2d = kLog2e / static_cast<double>(temperature);
  const bool vec = (V % 8 == 0) && aligned16(target_logits) &&
                   (gamma == 0 || p.q_index || aligned16(draft_probs)) && (!o.bias || aligned16(o.bias));
  if (truncate) {
    sv::ThreshParams t{};
    t.logits = target_logits;
    t.bias = o.bias;
    t.allowed = o.allowed;
    t.top_k = o.top_k;
    t.top_p = o.top_p;
    t.thresh = p.thresh_ws;
    t.summ = p.summ_ws;
    t.rows = B * (gamma + 1);
    t.R = gamma + 1;
    t.V = V;
    t.W = p.pr.W;
    t.c2 = p.c2;
    SPEC_TRACE_FILL(t);
    if (sv::launch_thresholds(t, logit_dtype, vec, stream) != hipSuccess) return SPEC_EHIP;
  }
  SPEC_TRACE_FILL(p);
  return sv::launch_chain(p, logit_dtype, vec, stream) == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

spec_status spec_verify_greedy(const void* target_logits, int logit_dtype, const int32_t* draft_tokens,
                               int B, int gamma, int V, int32_t* accepted_len, int32_t* out_tokens,
                               int32_t* req_status, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return spec_verify_greedy_ex(target_logits, logit_dtype, draft_tokens, B, gamma, V, nullptr, accepted_len,
                               out_tokens, req_status, workspace, workspace_bytes, stream);
}

spec_status spec_verify_greedy_stop(const void* target_logits, int logit_dtype, const int32_t* draft_tokens,
                                    int B, int gamma, int V, const int32_t* stop_tokens, int n_stop,
                                    const int32_t* budget, int32_t* accepted_len, int32_t* out_tokens,
                                    int32_t* req_status, int32_t* finish, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  spec_verify_options o = {};
  o.stop_tokens = stop_tokens;
  o.n_stop = n_stop;
  o.budget = budget;
  o.finish = finish;
  return spec_verify_greedy_ex(target_logits, logit_dtype, draft_tokens, B, gamma, V, &o, accepted_len,
                               out_tokens, req_status, workspace, workspace_bytes, stream);
}

spec_status spec_verify_greedy_ex(const void* target_logits, int logit_dtype, const int32_t* draft_tokens,
                                  int B, int gamma, int V, const spec_verify_options* opt, int32_t* accepted_len,
                                  int32_t* out_tokens, int32_t* req_status, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  const spec_verify_options o = opt ? *opt : spec_verify_options{};
  if (!sizes_ok(B, gamma, V) || !stop_ok(o.stop_tokens, o.n_stop) || o.lazy_rows < 0) return SPEC_EINVAL;
  if (!dtype_ok(logit_dtype)) return SPEC_EDTYPE;
  if (!sv::grid_fits(sv::greedy_blocks(B, gamma, V))) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!target_logits || !accepted_len || !out_tokens || !req_status) return SPEC_EINVAL;
  if (gamma > 0 && !draft_tokens) return SPEC_EINVAL;
  const sv::GreedyLayout L = sv::greedy_layout(B, gamma, V);
  if (!workspace || workspace_bytes < L.total || !aligned256(workspace)) return SPEC_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  sv::GreedyParams p;
  p.logits = target_logits;
  p.tokens = draft_tokens;
  p.accepted_len = accepted_len;
  p.out_tokens = out_tokens;
  p.req_status = req_status;
  p.st = stop_spec(o.stop_tokens, o.n_stop, o.budget, o.finish);
  p.pr = proc_spec(o, V, nullptr);   // top-k and top-p keep the maximum: no effect on an argmax
  p.part = reinterpret_cast<unsigned long long*>(ws + L.part);
  p.B = B;
  p.G = gamma;
  p.R = gamma + 1;
  p.V = V;
  const sv::Slicing sl = sv::slicing((long)B * (gamma + 1), V, sv::kGreedyTargetBlocks);
  p.P = sl.P;
  p.CPW = sl.CPW;
  p.SL = sl.SL;
  p.LK = (o.lazy_rows >= 1 && o.lazy_rows < gamma + 1) ? o.lazy_rows : gamma + 1;
  p.J = (gamma + 1 + p.LK - 1) / p.LK;
  const bool vec = (V % 8 == 0) && aligned16(target_logits) && (!o.bias || aligned16(o.bias));
  return sv::launch_greedy(p, logit_dtype, vec, stream) == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

spec_status spec_verify_tree(const void* node_logits, int logit_dtype, const int32_t* node_tokens,
                             const int32_t* parents, const float* uniforms, int B, int N, int V,
                             float temperature, int32_t* accepted_len, int32_t* out_tokens,
                             int32_t* out_nodes, int32_t* req_status, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (!(B >= 0 && B <= SPEC_MAX_BATCH && N >= 1 && N <= SPEC_MAX_NODES && V >= 1 && V <= SPEC_MAX_VOCAB))
    return SPEC_EINVAL;
  if (!temperature_ok(temperature)) return SPEC_EINVAL;
  if (!dtype_ok(logit_dtype)) return SPEC_EDTYPE;
  if (!sv::grid_fits(sv::tree_blocks(B, V))) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!node_logits || !node_tokens || !parents || !uniforms || !accepted_len || !out_tokens ||
      !out_nodes || !req_status)
    return SPEC_EINVAL;
  const sv::TreeLayout L = sv::tree_layout(B, N, V);
  if (!workspace || workspace_bytes < L.total || !aligned256(workspace)) return SPEC_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  sv::TreeParams p{};
  p.logits = node_logits;
  p.node_tokens = node_tokens;
  p.parents = parents;
  p.u = uniforms;
  p.accepted_len = accepted_len;
  p.out_tokens = out_tokens;
  p.out_nodes = out_nodes;
  p.req_status = req_status;
  p.part = reinterpret_cast<float2*>(ws + L.part);
  p.deep = reinterpret_cast<float2*>(ws + L.deep);
  p.order = reinterpret_cast<unsigned long long*>(ws + L.order);
  p.counters = sv::request_counters(workspace);
  p.B = B;
  p.N = N;
  p.V = V;
  p.P = chunks(V, sv::kWaveChunk);
  p.WG1 = chunks(p.P, sv::kWavesPerBlock);
  p.WH = (int)sv::tree_helpers(p.P, false);
  p.c2 = static_cast<float>(kLog2e / static_cast<double>(temperature));
  const bool vec = (V % 8 == 0) && aligned16(node_logits);
  SPEC_TRACE_FILL(p);
  return sv::launch_tree(p, logit_dtype, vec, stream) == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

spec_status spec_verify_tree_greedy(const void* node_logits, int logit_dtype, const int32_t* node_tokens,
                                    const int32_t* parents, int B, int N, int V, int32_t* accepted_len,
                                    int32_t* out_tokens, int32_t* out_nodes, int32_t* req_status,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!(B >= 0 && B <= SPEC_MAX_BATCH && N >= 1 && N <= SPEC_MAX_NODES && V >= 1 && V <= SPEC_MAX_VOCAB))
    return SPEC_EINVAL;
  if (!dtype_ok(logit_dtype)) return SPEC_EDTYPE;
  if (!sv::grid_fits(sv::tree_blocks(B, V))) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!node_logits || !node_tokens || !parents || !accepted_len || !out_tokens || !out_nodes || !req_status)
    return SPEC_EINVAL;
  const sv::TreeLayout L = sv::tree_layout(B, N, V);
  if (!workspace || workspace_bytes < L.total || !aligned256(workspace)) return SPEC_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  sv::TreeParams p{};
  p.logits = node_logits;
  p.node_tokens = node_tokens;
  p.parents = parents;
  p.accepted_len = accepted_len;
  p.out_tokens = out_tokens;
  p.out_nodes = out_nodes;
  p.req_status = req_status;
  p.part = reinterpret_cast<float2*>(ws + L.part);
  p.deep = reinterpret_cast<float2*>(ws + L.deep);
  p.order = reinterpret_cast<unsigned long long*>(ws + L.order);
  p.spec = reinterpret_cast<float2*>(ws + L.spec);
  p.stag = reinterpret_cast<unsigned*>(ws + L.stag);
  p.counters = sv::request_counters(workspace);
  p.B = B;
  p.N = N;
  p.V = V;
  p.P = chunks(V, sv::kWaveChunk);
  p.WG1 = chunks(p.P, sv::kWavesPerBlock);
  p.WH = (int)sv::tree_helpers(p.P, false);
  const bool vec = (V % 8 == 0) && aligned16(node_logits);
  SPEC_TRACE_FILL(p);
  return sv::launch_tree_greedy(p, logit_dtype, vec, stream) == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

spec_status spec_verify_tree_residual(const void* node_logits, int logit_dtype, const void* draft_probs,
                                      int q_dtype, const int32_t* node_tokens, const int32_t* parents,
                                      const float* accept_uniforms, const float* draw_uniforms, int B, int N,
                                      int V, float temperature, int32_t* accepted_len, int32_t* out_tokens,
                                      int32_t* out_nodes, int32_t* req_status, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (!residual_sizes_ok(B, N, V)) return SPEC_EINVAL;
  if (!temperature_ok(temperature)) return SPEC_EINVAL;
  if (!dtype_ok(logit_dtype) || !dtype_ok(q_dtype)) return SPEC_EDTYPE;
  if (!sv::grid_fits(sv::tree_blocks(B, V, true))) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!node_logits || !draft_probs || !node_tokens || !parents || !accept_uniforms || !draw_uniforms ||
      !accepted_len || !out_tokens || !out_nodes || !req_status)
    return SPEC_EINVAL;
  const sv::TreeLayout L = sv::tree_layout(B, N, V, true);
  if (!workspace || workspace_bytes < L.total || !aligned256(workspace)) return SPEC_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  sv::TreeParams p{};
  p.logits = node_logits;
  p.node_tokens = node_tokens;
  p.parents = parents;
  p.u = accept_uniforms;
  p.u_draw = draw_uniforms;
  p.q = draft_probs;
  p.q_dtype = q_dtype;
  p.accepted_len = accepted_len;
  p.out_tokens = out_tokens;
  p.out_nodes = out_nodes;
  p.req_status = req_status;
  p.part = reinterpret_cast<float2*>(ws + L.part);
  p.deep = reinterpret_cast<float2*>(ws + L.deep);
  p.order = reinterpret_cast<unsigned long long*>(ws + L.order);
  p.desc = reinterpret_cast<unsigned long long*>(ws + L.desc);
  p.spec = reinterpret_cast<float2*>(ws + L.spec);
  p.stag = reinterpret_cast<unsigned*>(ws + L.stag);
  p.desc_words = 3 + 2 * N;
  p.counters = sv::request_counters(workspace);
  p.B = B;
  p.N = N;
  p.V = V;
  p.P = chunks(V, sv::kWaveChunk);
  p.WG1 = chunks(p.P, sv::kWavesPerBlock);
  p.WH = (int)sv::tree_helpers(p.P, true);
  p.c2 = static_cast<float>(kLog2e / static_cast<double>(temperature));
  const bool vec = (V % 8 == 0) && aligned16(node_logits) && aligned16(draft_probs);
  SPEC_TRACE_FILL(p);
  return sv::launch_tree_residual(p, logit_dtype, vec, stream) == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

spec_status spec_verify_chain_static(const void* target_logits, int logit_dtype, const void* draft_probs,
                                     int q_dtype, const int32_t* draft_tokens, const float* uniforms, int B,
                                     int gamma, int V, float temperature, int32_t* accepted_len,
                                     int32_t* out_tokens, int32_t* req_status, float* stats, hipStream_t stream) {
  const size_t need = spec_chain_workspace_bytes(B, gamma, V);
  if (need == 0) return SPEC_EINVAL;
  if (need > kStaticScratchBytes) return SPEC_ESCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPEC_EHIP;
  void* ptr = device_scratch(dev);
  if (!ptr) return SPEC_EHIP;
  if (B > 0) {
    // every call leaves its words zeroed, but a call that failed (or one that raced on the
    // same GPU) may not have: clear what this call uses
    const size_t words = need / 8, blocks = (words + 255) / 256;
    zero_words<<<dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, stream>>>(
        static_cast<unsigned long long*>(ptr), words);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
  }
  return spec_verify_chain(target_logits, logit_dtype, draft_probs, q_dtype, draft_tokens, uniforms, B, gamma, V,
                           temperature, accepted_len, out_tokens, req_status, stats, ptr, need, stream);
}

}  // extern "C"
