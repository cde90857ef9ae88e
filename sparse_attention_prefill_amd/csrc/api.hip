// Host entry points of libdsa: argument checks, sizes and kernel dispatch. See include/dsa.h.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "dsa_internal.h"

// Scratch of dsa_indexer_topk_noalloc (see static_scratch below): 64 MiB per GPU.
static constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace dsa {

static thread_local std::string g_last_error;

// The events of the calling thread's dsa_indexer_topk_timed call, if one is running.
struct LaunchTap {
  void* const* events;
  int cap;                 // events available
  int n;                   // events recorded
  const char** names;      // optional: names[k] = kernel launched after events[k]
  hipError_t err;          // first failed record
};
static thread_local LaunchTap* g_tap = nullptr;

void tap_launch(const char* kernel, hipStream_t stream) {
  LaunchTap* t = g_tap;
  if (!t || t->n >= t->cap - 1) return;  // the last event is kept for the end of the call
  const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(t->events[t->n]), stream);
  if (e != hipSuccess && t->err == hipSuccess) t->err = e;
  if (t->names) t->names[t->n] = kernel;
  ++t->n;
}

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }
dsa_status fail(dsa_status code, const std::string& msg) {
  g_last_error = msg;
  return code;
}
dsa_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DSA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return DSA_OK;
}

dsa_status launch_cp_metadata(const int32_t*, const int32_t*, int, int, int, int, int, int32_t*, int32_t*, int32_t*,
                              int32_t*, int32_t*, int32_t*, hipStream_t);
dsa_status launch_rerange(const void*, void*, int, int64_t, int, int, int, int, int, hipStream_t);
dsa_status launch_indexer_scores(const dsa_indexer_topk_args*, float*, int64_t, int, int, const CandidateMode*,
                                 hipStream_t);
dsa_status launch_topk(const dsa_indexer_topk_args*, const float*, int64_t, int, hipStream_t);
dsa_status launch_topk_theta(const dsa_indexer_topk_args*, int, const CandidateMode&, hipStream_t);
dsa_status launch_topk_candidates(const dsa_indexer_topk_args*, const float*, int64_t, int, const CandidateMode&,
                                  float*, int64_t, int, hipStream_t);
dsa_status launch_sparse_attn(const dsa_sparse_attn_args*, hipStream_t);

namespace {

bool valid_mode(int32_t m) { return m == DSA_SPLIT_IN_SEQ || m == DSA_SPLIT_ROUND_ROBIN; }

// visible keys of the longest row, and the float32 score-row stride
int max_visible(const dsa_indexer_topk_args* a) {
  return a->compress_ratio > 1 ? a->max_seqlen_kv / a->compress_ratio : a->max_seqlen_kv;
}
int64_t score_ld(const dsa_indexer_topk_args* a) {
  const int64_t mv = max_visible(a) > 0 ? max_visible(a) : 1;
  return (mv + 63) / 64 * 64;
}

// Candidate mode (rows longer than max(kFuseMin, topk) are selected from lists of their best
// scores, see topk.hip): only with the 64 x 128 matrix-core indexer, and only when some row is
// longer than kFuseLaunch keys.
bool candidate_mode(const dsa_indexer_topk_args* a) {
  const bool mfma = a->n_heads == 64 && a->head_dim == 128 && (a->dtype == DSA_BF16 || a->dtype == DSA_FP8_E4M3);
  return mfma && max_visible(a) > std::max(kFuseLaunch, a->topk);
}
// Workspace of candidate mode: per row a 128 KB slot (a score row of kFuseMin floats, or a list
// of kFuseCap entries), thresholds and list lengths, and the refill scratch rows.
struct CandLayout {
  size_t slots, theta, n_cand, status, scratch, total;
  int n_scratch, segs;
  int64_t sld;
};
CandLayout cand_layout(const dsa_indexer_topk_args* a) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  CandLayout L;
  const size_t nq = size_t(a->nq > 0 ? a->nq : 1);
  int chunk_keys = 0;
  L.segs = indexer_key_chunks(a, max_visible(a), &chunk_keys);
  L.slots = 0;
  L.theta = up(nq * size_t(kFuseCap) * sizeof(uint2));
  L.n_cand = L.theta + up(nq * sizeof(uint32_t));
  L.status = L.n_cand + up(nq * size_t(L.segs) * sizeof(int32_t));
  L.scratch = L.status + up(nq * sizeof(int32_t));
  L.n_scratch = std::min(int(nq), kRefillBlocks);
  L.sld = score_ld(a);
  L.total = L.scratch + size_t(L.n_scratch) * size_t(L.sld) * sizeof(float);
  return L;
}

// One wave reads the shader-clock counter (s_memtime) and the 100 MHz real-time counter, spins
// until `ticks` real-time ticks have passed, and reads both again: out = {c0, c1, r0, r1}.
__global__ void clock_probe_kernel(uint64_t* __restrict__ out, uint64_t ticks) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r = r0;
  while (r - r0 < ticks) r = __builtin_amdgcn_s_memrealtime();
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c0;
    out[1] = c1;
    out[2] = r0;
    out[3] = r;
  }
}

dsa_status check_indexer_args(const dsa_indexer_topk_args* a, bool need_out) {
  if (!a) return fail(DSA_ERR_INVALID_ARG, "indexer: args is NULL");
  if (a->nq < 0 || a->nk < 0 || a->batch < 0 || a->n_heads < 1 || a->head_dim < 1)
    return fail(DSA_ERR_INVALID_ARG, "indexer: negative or zero size");
  if (a->topk < 1) return fail(DSA_ERR_INVALID_ARG, "indexer: topk must be >= 1");
  if (a->window < 0) return fail(DSA_ERR_INVALID_ARG, "indexer: window must be >= 0");
  if (a->q_stride < 1) return fail(DSA_ERR_INVALID_ARG, "indexer: q_stride must be >= 1");
  if (a->compress_ratio < 1) return fail(DSA_ERR_INVALID_ARG, "indexer: compress_ratio must be >= 1");
  if (a->max_seqlen_kv < 0) return fail(DSA_ERR_INVALID_ARG, "indexer: max_seqlen_kv must be >= 0");
  if (a->dtype != DSA_F32 && a->dtype != DSA_BF16 && a->dtype != DSA_FP8_E4M3)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: unknown dtype");
  if (a->nq == 0) return DSA_OK;
  if (a->batch < 1) return fail(DSA_ERR_INVALID_ARG, "indexer: batch must be >= 1 when nq > 0");
  if (!a->q_idx || !a->weights || !a->cu_seqlens_q || !a->seqused_kv || !a->cu_seqlens_kv)
    return fail(DSA_ERR_INVALID_ARG, "indexer: NULL input pointer");
  if (a->nk > 0 && !a->k_idx) return fail(DSA_ERR_INVALID_ARG, "indexer: NULL k_idx");
  if (a->dtype == DSA_FP8_E4M3 && (!a->q_scale || !a->k_scale))
    return fail(DSA_ERR_INVALID_ARG, "indexer: fp8 needs q_scale and k_scale");
  if (need_out && !a->topk_idx) return fail(DSA_ERR_INVALID_ARG, "indexer: NULL topk_idx");
  if (a->window > 0 && !a->window_kv_start) return fail(DSA_ERR_INVALID_ARG, "indexer: window needs window_kv_start");
  if (!aligned16(a->q_idx) || (a->k_idx && !aligned16(a->k_idx)))
    return fail(DSA_ERR_INVALID_ARG, "indexer: q_idx / k_idx must be 16-byte aligned");
  if (max_visible(a) > 131072) return fail(DSA_ERR_UNSUPPORTED, "indexer: more than 131072 visible keys per row");
  const bool mfma = a->n_heads == 64 && a->head_dim == 128;
  if (a->dtype == DSA_FP8_E4M3 && !mfma) return fail(DSA_ERR_UNSUPPORTED, "indexer: fp8 needs 64 heads x 128");
  return DSA_OK;
}

// ---------------------------------------------------------------------------------------------
// Scratch of dsa_indexer_topk_noalloc, for callers that cannot allocate: a file-scope device array,
// one copy per GPU the library runs on, held until the process ends. Host code never uses the
// array's name as an address: the device's copy is found once per device with
// hipGetSymbolAddress, with that device current, and that address is what the kernels receive.
// ---------------------------------------------------------------------------------------------
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

dsa_status static_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, std::string("indexer_topk_noalloc: hipGetDevice: ") + hipGetErrorString(e));
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess)
      return fail(DSA_ERR_HIP, std::string("indexer_topk_noalloc: hipStreamGetDevice: ") + hipGetErrorString(e));
    if (int(sdev) != dev) return fail(DSA_ERR_INVALID_ARG, "indexer_topk_noalloc: the stream is not on the current device");
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(DSA_ERR_UNSUPPORTED, "indexer_topk_noalloc: device id too large");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DSA_ERR_HIP, std::string("indexer_topk_noalloc: hipGetSymbolAddress: ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

size_t workspace_need(const dsa_indexer_topk_args* a) {
  return candidate_mode(a) ? cand_layout(a).total : size_t(a->nq) * size_t(score_ld(a)) * sizeof(float);
}

// Indexer + top-k of checked arguments with a large enough workspace, on stream s.
dsa_status run_indexer_topk(const dsa_indexer_topk_args* a, hipStream_t s) {
  dsa_status st;
  if (!candidate_mode(a)) {
    float* scores = static_cast<float*>(a->workspace);
    // rows with at most topk visible keys are taken whole by the top-k: the indexer skips them
    st = launch_indexer_scores(a, scores, score_ld(a), max_visible(a), a->topk, nullptr, s);
    if (st != DSA_OK) return st;
    return launch_topk(a, scores, score_ld(a), max_visible(a), s);
  }
  const CandLayout L = cand_layout(a);
  char* ws = static_cast<char*>(a->workspace);
  CandidateMode cm;
  cm.fuse_above = std::max(kFuseMin, a->topk);
  cm.theta = reinterpret_cast<uint32_t*>(ws + L.theta);
  cm.n_cand = reinterpret_cast<int32_t*>(ws + L.n_cand);
  cm.status = reinterpret_cast<int32_t*>(ws + L.status);
  cm.cand = reinterpret_cast<uint2*>(ws + L.slots);
  cm.cap = kFuseCap;
  cm.segs = L.segs;
  float* score_rows = reinterpret_cast<float*>(ws + L.slots);  // short rows: kFuseMin floats per slot
  st = launch_topk_theta(a, max_visible(a), cm, s);
  if (st != DSA_OK) return st;
  st = launch_indexer_scores(a, score_rows, kFuseMin, max_visible(a), a->topk, &cm, s);
  if (st != DSA_OK) return st;
  return launch_topk_candidates(a, score_rows, kFuseMin, max_visible(a), cm, reinterpret_cast<float*>(ws + L.scratch),
                                L.sld, L.n_scratch, s);
}

}  // namespace
}  // namespace dsa

using namespace dsa;

extern "C" {

const char* dsa_last_error(void) { return g_last_error.c_str(); }

const char* dsa_version(void) { return "dsa-mi355x 0.1 (gfx950)"; }

dsa_status dsa_cp_sizes(int32_t num_tokens, int32_t cp_size, int32_t cp_rank, int32_t mode, int32_t pad_to_cp,
                        int32_t* tokens_per_rank, int32_t* n_local_real, int32_t* num_rows_concat) {
  clear_error();
  if (num_tokens < 0 || cp_size < 1 || cp_rank < 0 || cp_rank >= cp_size)
    return fail(DSA_ERR_INVALID_ARG, "cp_sizes: need num_tokens >= 0 and 0 <= cp_rank < cp_size");
  if (!valid_mode(mode)) return fail(DSA_ERR_INVALID_ARG, "cp_sizes: unknown split mode");
  const int64_t tpr = (int64_t(num_tokens) + cp_size - 1) / cp_size;
  int64_t real;
  if (mode == DSA_SPLIT_ROUND_ROBIN) real = num_tokens > cp_rank ? (num_tokens - cp_rank + cp_size - 1) / cp_size : 0;
  else real = std::max<int64_t>(0, std::min<int64_t>((cp_rank + 1) * tpr, num_tokens) - std::min<int64_t>(cp_rank * tpr, num_tokens));
  if (tokens_per_rank) *tokens_per_rank = int32_t(tpr);
  if (n_local_real) *n_local_real = int32_t(real);
  if (num_rows_concat) *num_rows_concat = pad_to_cp ? int32_t(tpr * cp_size) : num_tokens;
  return DSA_OK;
}

dsa_status dsa_build_cp_metadata(const int32_t* query_start_loc, const int32_t* seq_lens, int32_t batch,
                                 int32_t num_tokens, int32_t cp_size, int32_t cp_rank, int32_t mode, int32_t pad_to_cp,
                                 int32_t* local_query_start_loc, int32_t* local_seq_lens, int32_t* local_kv_start_loc,
                                 int32_t* scalars, int32_t* token_map, int32_t* err_flag, void* stream) {
  clear_error();
  (void)pad_to_cp;
  if (batch < 0 || num_tokens < 0) return fail(DSA_ERR_INVALID_ARG, "cp_metadata: negative batch or num_tokens");
  if (cp_size < 1 || cp_rank < 0 || cp_rank >= cp_size)
    return fail(DSA_ERR_INVALID_ARG, "cp_metadata: need 0 <= cp_rank < cp_size");
  if (!valid_mode(mode)) return fail(DSA_ERR_INVALID_ARG, "cp_metadata: unknown split mode");
  if (!query_start_loc || !local_query_start_loc || !local_kv_start_loc || !scalars ||
      (batch > 0 && (!seq_lens || !local_seq_lens)))
    return fail(DSA_ERR_INVALID_ARG, "cp_metadata: NULL pointer");
  return launch_cp_metadata(query_start_loc, seq_lens, batch, num_tokens, cp_size, cp_rank, mode,
                            local_query_start_loc, local_seq_lens, local_kv_start_loc, scalars, token_map, err_flag,
                            as_stream(stream));
}

size_t dsa_indexer_topk_workspace(const dsa_indexer_topk_args* a) {
  clear_error();
  if (check_indexer_args(a, false) != DSA_OK) return 0;
  if (candidate_mode(a)) return cand_layout(a).total;
  return size_t(a->nq > 0 ? a->nq : 1) * size_t(score_ld(a)) * sizeof(float);
}

dsa_status dsa_indexer_scores(const dsa_indexer_topk_args* a, float* scores, int64_t ld, void* stream) {
  clear_error();
  dsa_status st = check_indexer_args(a, false);
  if (st != DSA_OK) return st;
  if (a->nq == 0) return DSA_OK;
  if (!scores || !aligned16(scores)) return fail(DSA_ERR_INVALID_ARG, "indexer_scores: scores NULL or misaligned");
  if (ld < max_visible(a) || ld % 4 != 0) return fail(DSA_ERR_INVALID_ARG, "indexer_scores: ld too small or not % 4");
  return launch_indexer_scores(a, scores, ld, max_visible(a), 0, nullptr, as_stream(stream));
}

dsa_status dsa_topk_from_scores(const dsa_indexer_topk_args* a, const float* scores, int64_t ld, void* stream) {
  clear_error();
  dsa_status st = check_indexer_args(a, true);
  if (st != DSA_OK) return st;
  if (a->nq == 0) return DSA_OK;
  if (!scores || !aligned16(scores)) return fail(DSA_ERR_INVALID_ARG, "topk: scores NULL or misaligned");
  if (ld < max_visible(a) || ld % 4 != 0) return fail(DSA_ERR_INVALID_ARG, "topk: ld too small or not % 4");
  return launch_topk(a, scores, ld, max_visible(a), as_stream(stream));
}

dsa_status dsa_indexer_topk(const dsa_indexer_topk_args* a, void* stream) {
  clear_error();
  dsa_status st = check_indexer_args(a, true);
  if (st != DSA_OK) return st;
  if (a->nq == 0) return DSA_OK;
  if (!a->workspace || a->workspace_bytes < workspace_need(a) || (reinterpret_cast<uintptr_t>(a->workspace) & 255u))
    return fail(DSA_ERR_WORKSPACE, "indexer_topk: workspace missing, not 256-byte aligned or smaller than "
                                       "dsa_indexer_topk_workspace()");
  return run_indexer_topk(a, as_stream(stream));
}

dsa_status dsa_indexer_topk_noalloc(const dsa_indexer_topk_args* a, void* stream) {
  clear_error();
  dsa_status st = check_indexer_args(a, true);
  if (st != DSA_OK) return st;
  if (a->nq == 0) return DSA_OK;
  const size_t need = workspace_need(a);
  if (need > kStaticScratchBytes)
    return fail(DSA_ERR_WORKSPACE, "indexer_topk_noalloc: the call needs " + std::to_string(need) +
                                       " bytes of scratch; the static scratch holds " +
                                       std::to_string(kStaticScratchBytes) + " (use dsa_indexer_topk with a workspace)");
  void* ptr = nullptr;
  st = static_scratch(as_stream(stream), &ptr);
  if (st != DSA_OK) return st;
  dsa_indexer_topk_args b = *a;
  b.workspace = ptr;
  b.workspace_bytes = kStaticScratchBytes;
  return run_indexer_topk(&b, as_stream(stream));
}

dsa_status dsa_indexer_topk_timed(const dsa_indexer_topk_args* a, void* stream, void* const* events,
                                  int32_t n_events, int32_t* n_kernels, const char** kernel_names) {
  clear_error();
  if (!events || n_events < 2) return fail(DSA_ERR_INVALID_ARG, "indexer_topk_timed: need at least 2 events");
  for (int k = 0; k < n_events; ++k)
    if (!events[k]) return fail(DSA_ERR_INVALID_ARG, "indexer_topk_timed: NULL event");
  LaunchTap tap{events, n_events, 0, kernel_names, hipSuccess};
  g_tap = &tap;
  dsa_status st = dsa_indexer_topk(a, stream);
  g_tap = nullptr;
  if (st != DSA_OK) return st;
  if (tap.n > 0) {
    const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[tap.n]), as_stream(stream));
    if (e != hipSuccess && tap.err == hipSuccess) tap.err = e;
  }
  if (tap.err != hipSuccess) return fail(DSA_ERR_HIP, std::string("indexer_topk_timed: hipEventRecord: ") +
                                                          hipGetErrorString(tap.err));
  if (n_kernels) *n_kernels = tap.n;
  return DSA_OK;
}

dsa_status dsa_clock_probe(uint64_t* out, int64_t ticks, void* stream) {
  clear_error();
  if (!out || ticks < 1 || ticks > 10000000) return fail(DSA_ERR_INVALID_ARG, "clock_probe: need out and 1 <= ticks <= 1e7");
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, as_stream(stream), out, uint64_t(ticks));
  return check_launch("clock_probe_kernel");
}

dsa_status dsa_sparse_attn(const dsa_sparse_attn_args* a, void* stream) {
  clear_error();
  if (!a) return fail(DSA_ERR_INVALID_ARG, "sparse_attn: args is NULL");
  if (a->nq < 0 || a->n_rows < 0 || a->k_tot < 0 || a->n_heads < 1 || a->d_qk < 1 || a->d_v < 1 ||
      a->d_v > a->d_qk)
    return fail(DSA_ERR_INVALID_ARG, "sparse_attn: bad sizes (need d_v <= d_qk)");
  if (a->dtype != DSA_F32 && a->dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "sparse_attn: dtype");
  if (a->nq == 0) return DSA_OK;
  if (!a->q || !a->out || (a->k_tot > 0 && (!a->idx || !a->kv)))
    return fail(DSA_ERR_INVALID_ARG, "sparse_attn: NULL pointer");
  if (a->k_tot > 0 && a->n_rows < 1) return fail(DSA_ERR_INVALID_ARG, "sparse_attn: n_rows must be >= 1");
  if (!aligned16(a->q) || !aligned16(a->out) || (a->kv && !aligned16(a->kv)))
    return fail(DSA_ERR_INVALID_ARG, "sparse_attn: q / kv / out must be 16-byte aligned");
  return launch_sparse_attn(a, as_stream(stream));
}

dsa_status dsa_rerange(const void* in, void* out, int32_t num_tokens, int64_t row_bytes, int32_t cp_size, int32_t mode,
                       int32_t pad_to_cp, int32_t inverse, void* stream) {
  clear_error();
  if (num_tokens < 0 || cp_size < 1 || row_bytes < 16 || row_bytes % 16 != 0 || row_bytes / 16 > INT32_MAX)
    return fail(DSA_ERR_INVALID_ARG, "rerange: need num_tokens >= 0, cp_size >= 1, row_bytes % 16 == 0");
  if (!valid_mode(mode)) return fail(DSA_ERR_INVALID_ARG, "rerange: unknown split mode");
  int32_t rows_concat = 0;
  dsa_cp_sizes(num_tokens, cp_size, 0, mode, pad_to_cp, nullptr, nullptr, &rows_concat);
  const int n_out = inverse ? rows_concat : num_tokens;
  if (n_out == 0) return DSA_OK;
  if (!in || !out) return fail(DSA_ERR_INVALID_ARG, "rerange: NULL pointer");
  if (!aligned16(in) || !aligned16(out)) return fail(DSA_ERR_INVALID_ARG, "rerange: pointers must be 16-byte aligned");
  const int n_in = inverse ? num_tokens : rows_concat;
  const char* ib = static_cast<const char*>(in);
  const char* ob = static_cast<const char*>(out);
  if (ib < ob + int64_t(n_out) * row_bytes && ob < ib + int64_t(n_in) * row_bytes)
    return fail(DSA_ERR_INVALID_ARG, "rerange: in and out overlap");
  return launch_rerange(in, out, num_tokens, row_bytes, cp_size, mode, pad_to_cp, inverse, n_out, as_stream(stream));
}

}  // extern "C"
