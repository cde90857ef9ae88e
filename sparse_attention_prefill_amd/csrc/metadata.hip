// (1) CP-local metadata for one rank's share of a prefill batch, on the GPU.
//
// [xLLM-CP] "feat: DeepSeek-V4 DSA context-parallel on NPU", Implementation §2 (CP-local
// metadata: padded token count, tokens per rank, the rank's interval, intersection with the
// global cu-seqlens, local_kv_start_loc as the right-aligned cumsum of local_seq_lens) and
// Design key points (right-aligned extents; the last rank sees the whole stream).
// [CP-blog] "[DeepSeek v3.2] context parallel explained", §2B (round-robin split by
// token % cp_size and recomputed per-rank cu-seqlens).
//
// Chunked prefill: request b may carry P_b = seq_lens[b] - n_b cached tokens ahead of its
// n_b queries; its KV segment (seq_lens[b] rows, prefix first) follows the previous request's,
// and every extent counts the prefix.
//
// Every per-request value comes from closed forms (no loop over tokens) and prefix scans: one
// wave with wave scans for batches of up to 64 requests (no workgroup barrier on the critical
// path), else one workgroup of 1024 threads with block scans; all workgroups fill the token map.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// inclusive scan over a 64-lane wavefront
__device__ inline int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// exclusive block scan of one value per thread (blockDim == kThreads); returns the block total
__device__ inline int block_excl_scan(int v, int* smem_waves, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = wave_incl_scan(v);
  if (lane == 63) smem_waves[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kWaves ? smem_waves[lane] : 0;
    int wi = wave_incl_scan(w);
    if (lane < kWaves) smem_waves[lane] = wi - w;
    if (lane == kWaves - 1) smem_waves[kWaves] = wi;
  }
  __syncthreads();
  int res = smem_waves[wave] + incl - v;
  *total = smem_waves[kWaves];
  __syncthreads();
  return res;
}

// number of tokens t < x with t % cp == r
__device__ inline int rr_count_below(int x, int cp, int r) { return x > r ? (x - r + cp - 1) / cp : 0; }

// Request b: its local queries nb, its local KV extent ext (cached prefix included) and its KV
// segment length seg; bad collects DSA_DEVERR_* bits of inconsistent input.
struct RequestView {
  int nb, ext, seg, bad;
};
__device__ inline RequestView request_view(const int32_t* __restrict__ qsl, const int32_t* __restrict__ seq_lens,
                                           int b, int batch, int T, int cp, int rank, bool rr, int local_start,
                                           int local_end) {
  RequestView v{0, 0, 0, 0};
  const int qs = qsl[b];
  const int qe = qsl[b + 1];
  if (b == 0 && qs != 0) v.bad |= DSA_DEVERR_QSL_START;
  if (qe < qs) v.bad |= DSA_DEVERR_QSL_ORDER;
  if (b == batch - 1 && qe != T) v.bad |= DSA_DEVERR_QSL_TOTAL;
  const int len = max(qe - qs, 0);
  int prefix = seq_lens[b] - len;
  if (prefix < 0) {
    v.bad |= DSA_DEVERR_SEQ_LENS;
    prefix = 0;
  }
  v.seg = prefix + len;
  if (rr) {
    v.nb = max(rr_count_below(qe, cp, rank) - rr_count_below(qs, cp, rank), 0);
    v.ext = prefix;
    if (v.nb > 0) {
      const int t_last = rank + (rr_count_below(qe, cp, rank) - 1) * cp;
      v.ext += t_last - qs + 1;
    }
  } else {
    v.nb = max(min(qe, local_end) - max(qs, local_start), 0);
    v.ext = prefix + min(max(local_end - qs, 0), len);
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void cp_metadata_kernel(
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ seq_lens, int batch, int T, int cp,
    int rank, int mode, int32_t* __restrict__ lqsl, int32_t* __restrict__ lsl, int32_t* __restrict__ lkv,
    int32_t* __restrict__ scalars, int32_t* __restrict__ token_map, int32_t* __restrict__ err_flag) {
  const int tpr = (T + cp - 1) / cp;
  const bool rr = mode == DSA_SPLIT_ROUND_ROBIN;
  int local_start, local_end;
  if (rr) {
    local_start = min(rank, T);
    const int n = rr_count_below(T, cp, rank);
    local_end = n > 0 ? rank + (n - 1) * cp + 1 : local_start;
  } else {
    local_start = min(rank * tpr, T);
    local_end = min((rank + 1) * tpr, T);
  }

  // token map: every workgroup, grid-stride
  if (token_map) {
    for (int j = blockIdx.x * kThreads + threadIdx.x; j < tpr; j += gridDim.x * kThreads) {
      const int t = rr ? rank + j * cp : rank * tpr + j;
      token_map[j] = t < T ? t : -1;
    }
  }
  if (blockIdx.x != 0) return;

  if (batch <= 64) {  // one wave (uniform branch)
    if (threadIdx.x >= 64) return;
    const int b = threadIdx.x;
    RequestView v{0, 0, 0, 0};
    if (b < batch) {
      v = request_view(qsl, seq_lens, b, batch, T, cp, rank, rr, local_start, local_end);
      lsl[b] = v.ext;
      if (v.bad) raise_flag(err_flag, v.bad);
    }
    const int iq = wave_incl_scan(v.nb), ikv = wave_incl_scan(v.ext), iseg = wave_incl_scan(v.seg);
    if (b < batch) {
      lqsl[b] = iq - v.nb;
      lkv[b] = rr ? iseg - v.seg : ikv - v.ext;
    }
    int mx = v.nb;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) mx = max(mx, __shfl_xor(mx, d, 64));
    const int nreq = __popcll(__builtin_amdgcn_ballot_w64(v.nb > 0));
    const int tot_q = __shfl(iq, 63, 64), tot_kv = __shfl(ikv, 63, 64), tot_seg = __shfl(iseg, 63, 64);
    if (b == 0) {
      lqsl[batch] = tot_q;
      lkv[batch] = rr ? tot_seg : tot_kv;
      scalars[0] = tpr * cp;
      scalars[1] = tpr;
      scalars[2] = local_start;
      scalars[3] = local_end;
      scalars[4] = rr ? cp : 1;
      scalars[5] = rr ? rr_count_below(T, cp, rank) : local_end - local_start;
      scalars[6] = mx;
      scalars[7] = nreq;
    }
    return;
  }

  __shared__ int smem[kWaves + 1];
  __shared__ int s_max, s_nreq;
  if (threadIdx.x == 0) {
    s_max = 0;
    s_nreq = 0;
  }
  __syncthreads();

  int carry_q = 0, carry_kv = 0, carry_seg = 0;
  int bad = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + threadIdx.x;
    int nb = 0, ext = 0, seg = 0;
    if (b < batch) {
      const RequestView v = request_view(qsl, seq_lens, b, batch, T, cp, rank, rr, local_start, local_end);
      nb = v.nb;
      ext = v.ext;
      seg = v.seg;
      bad |= v.bad;
      lsl[b] = ext;
      atomicMax(&s_max, nb);
      if (nb > 0) atomicAdd(&s_nreq, 1);
    }
    int tot_q, tot_kv, tot_seg;
    const int ex_q = block_excl_scan(nb, smem, &tot_q);
    const int ex_kv = block_excl_scan(ext, smem, &tot_kv);
    const int ex_seg = block_excl_scan(seg, smem, &tot_seg);
    if (b < batch) {
      lqsl[b] = carry_q + ex_q;
      lkv[b] = rr ? carry_seg + ex_seg : carry_kv + ex_kv;
    }
    carry_q += tot_q;
    carry_kv += tot_kv;
    carry_seg += tot_seg;
  }
  if (bad) raise_flag(err_flag, bad);
  __syncthreads();
  if (threadIdx.x == 0) {
    lqsl[batch] = carry_q;
    lkv[batch] = rr ? carry_seg : carry_kv;
    scalars[0] = tpr * cp;
    scalars[1] = tpr;
    scalars[2] = local_start;
    scalars[3] = local_end;
    scalars[4] = rr ? cp : 1;
    scalars[5] = rr ? rr_count_below(T, cp, rank) : local_end - local_start;
    scalars[6] = s_max;
    scalars[7] = s_nreq;
  }
}

}  // namespace

dsa_status launch_cp_metadata(const int32_t* qsl, const int32_t* seq_lens, int batch, int T, int cp, int rank,
                              int mode, int32_t* lqsl, int32_t* lsl, int32_t* lkv, int32_t* scalars,
                              int32_t* token_map, int32_t* err_flag, hipStream_t stream) {
  const int tpr = (T + cp - 1) / cp;
  int blocks = token_map ? (tpr + kThreads - 1) / kThreads : 1;
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  hipLaunchKernelGGL(cp_metadata_kernel, dim3(blocks), dim3(kThreads), 0, stream, qsl, seq_lens, batch, T, cp,
                     rank, mode, lqsl, lsl, lkv, scalars, token_map, err_flag);
  return check_launch("cp_metadata_kernel");
}

}  // namespace dsa
