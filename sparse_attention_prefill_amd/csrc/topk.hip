// (3) Per-query causal top-k over indexer scores (+ sliding-window rows), on gfx950.
//
// [xLLM-CP] "feat: DeepSeek-V4 DSA context-parallel on NPU", Design, data-flow step (3) (top-k
// of the local queries over their causal keys) and Implementation §5 (a top-k fed unlocalised
// metadata collapses to position 0, i.e. the selection is per query over its own extent).
//
// One workgroup (1024 threads) per query row:
//  1. Scores become order-preserving 32-bit keys (-0.0 folded into +0.0).
//  2. Radix select, 4 passes of 8 bits from the top, finds the K-th largest key tau and how
//     many keys lie strictly above it; the histograms are LDS atomics.
//  3. Two LDS bitmaps mark the keys above tau and the keys equal to tau; a block scan over the
//     bitmap words turns them into positions in ascending order, taking the ties with the lowest
//     positions (the tie rule: higher score first, then lower key index). The output is thus
//     deterministic and sorted, with no sort.
// Rows of up to 1024*EPT keys are held in registers (EPT keys per thread, coalesced 16-byte
// loads); longer rows are re-read from memory (L2 / MALL) on each pass.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBitmapWords = 131072 / 32;  // rows up to 131072 keys

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;                       // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // larger float -> larger key
}

__device__ inline int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// exclusive scan of one int per thread over the block; *total = block sum
__device__ inline int block_excl_scan(int v, int* smem, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) smem[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int x = lane < kWaves ? smem[lane] : 0;
    const int xi = wave_incl_scan(x);
    if (lane < kWaves) smem[lane] = xi - x;
    if (lane == kWaves - 1) smem[kWaves] = xi;
  }
  __syncthreads();
  const int r = smem[wave] + incl - v;
  *total = smem[kWaves];
  __syncthreads();
  return r;
}

struct TopkShared {
  uint32_t hist[256];
  uint32_t gt[kMaxBitmapWords];  // keys above tau
  uint32_t eq[kMaxBitmapWords];  // keys equal to tau
  int scan[kWaves + 1];
  uint32_t prefix;
  int remaining;
  int tie_count;
};

// EPT > 0: keys in registers (positions 4*(j*1024 + tid) + c); EPT == 0: streamed per pass.
template <int EPT>
__global__ __launch_bounds__(kThreads, 1) void topk_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ used_kv,
    const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ win_kv, int batch, int stride, int ratio, int nq,
    int max_vis, int K, int window, int kv_row_base, int32_t* __restrict__ out, int32_t* __restrict__ err_flag) {
  __shared__ TopkShared sh;
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int k_tot = K + window;
  int32_t* orow = out + int64_t(i) * k_tot;

  QueryView v;
  const bool have = query_view(cu_q, used_kv, cu_kv, batch, stride, i, &v);
  const int ev = have ? (ratio > 1 ? v.E / ratio : v.E) : 0;
  const bool ok = have && v.E >= 1 && ev <= max_vis;
  if (!ok) {
    if (tid == 0) raise_flag(err_flag, DSA_DEVERR_EXTENT);
    for (int j = tid; j < k_tot; j += kThreads) orow[j] = -1;
    return;
  }
  // window rows (original tokens): positions max(0, p-window+1) .. p, p = E-1
  if (window > 0) {
    const int p = v.E - 1;
    const int w0 = max(0, p - window + 1);
    for (int j = tid; j < window; j += kThreads) orow[K + j] = (w0 + j <= p) ? win_kv[v.b] + w0 + j : -1;
  }
  const int base = kv_row_base + v.kv0;
  if (ev <= K) {  // every visible key
    for (int j = tid; j < K; j += kThreads) orow[j] = j < ev ? base + j : -1;
    return;
  }

  const float* srow = scores + int64_t(i) * ld;
  constexpr int kVec = EPT > 0 ? EPT / 4 : 1;
  uint32_t keys[EPT > 0 ? EPT : 1];
  if constexpr (EPT > 0) {
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int p0 = 4 * (j * kThreads + tid);
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
      if (p0 + 3 < ev) x = *reinterpret_cast<const f32x4*>(srow + p0);
      else {
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = p0 + c < ev ? srow[p0 + c] : 0.f;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) keys[4 * j + c] = p0 + c < ev ? order_key(x[c]) : 0u;  // 0: not a key
    }
  }
  // visit every valid key: fn(key, position)
  auto for_each = [&](auto&& fn) {
    if constexpr (EPT > 0) {
#pragma unroll
      for (int j = 0; j < kVec; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int p = 4 * (j * kThreads + tid) + c;
          if (p < ev) fn(keys[4 * j + c], p);
        }
    } else {
      for (int p0 = 4 * tid; p0 < ev; p0 += 4 * kThreads) {
        f32x4 x;
        if (p0 + 3 < ev) x = *reinterpret_cast<const f32x4*>(srow + p0);
        else {
#pragma unroll
          for (int c = 0; c < 4; ++c) x[c] = p0 + c < ev ? srow[p0 + c] : 0.f;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (p0 + c < ev) fn(order_key(x[c]), p0 + c);
      }
    }
  };

  if (tid == 0) {
    sh.prefix = 0;
    sh.remaining = K;
  }
  // ---- radix select: the K-th largest key ----
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int b = tid; b < 256; b += kThreads) sh.hist[b] = 0;
    __syncthreads();
    const uint32_t prefix = sh.prefix;
    const uint32_t hmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for_each([&](uint32_t key, int) {
      if ((key & hmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    if (tid < 64) {
      // bins 4*lane .. 4*lane+3; suffix sums from the top bin down
      uint32_t c[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) c[k] = sh.hist[4 * tid + k];
      const int own = int(c[0] + c[1] + c[2] + c[3]);
      // suffix (inclusive) over lanes: sum of lanes >= tid
      int suf = own;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_down(suf, d, 64);
        if (tid + d < 64) suf += t;
      }
      const int above_lane = suf - own;  // keys in bins above this lane's 4 bins
      const int rem = sh.remaining;
      int above = above_lane;
      // the chosen bin b has above(b) < rem <= above(b) + count(b)
#pragma unroll
      for (int k = 3; k >= 0; --k) {
        const int cnt = int(c[k]);
        if (above < rem && rem <= above + cnt) {
          sh.prefix = prefix | (uint32_t(4 * tid + k) << shift);
          sh.remaining = rem - above;
          sh.tie_count = cnt;
        }
        above += cnt;
      }
    }
    __syncthreads();
  }
  const uint32_t tau = sh.prefix;
  const int need = sh.remaining;  // ties at tau to take (>= 1)
  const int n_words = (ev + 31) >> 5;

  // ---- bitmaps of keys above / equal to tau ----
  for (int wd = tid; wd < n_words; wd += kThreads) {
    sh.gt[wd] = 0;
    sh.eq[wd] = 0;
  }
  __syncthreads();
  for_each([&](uint32_t key, int p) {
    if (key > tau) atomicOr(&sh.gt[p >> 5], 1u << (p & 31));
    else if (key == tau) atomicOr(&sh.eq[p >> 5], 1u << (p & 31));
  });
  __syncthreads();

  // ---- ascending positions: each thread owns a contiguous run of words ----
  const int per = (n_words + kThreads - 1) / kThreads;
  const int w_begin = min(tid * per, n_words), w_end = min(w_begin + per, n_words);
  int my_eq = 0;
  for (int wd = w_begin; wd < w_end; ++wd) my_eq += __popc(sh.eq[wd]);
  int tot;
  int eq_rank = block_excl_scan(my_eq, sh.scan, &tot);
  int my_sel = 0;
  for (int wd = w_begin; wd < w_end; ++wd) {
    uint32_t e = sh.eq[wd];
    // keep only ties with rank < need
    uint32_t keep = 0;
    while (e) {
      const uint32_t bit = e & (~e + 1u);
      if (eq_rank < need) keep |= bit;
      ++eq_rank;
      e ^= bit;
    }
    sh.eq[wd] = keep | sh.gt[wd];  // final selection bitmap
    my_sel += __popc(keep | sh.gt[wd]);
  }
  int pos = block_excl_scan(my_sel, sh.scan, &tot);
  for (int wd = w_begin; wd < w_end; ++wd) {
    uint32_t s = sh.eq[wd];
    while (s) {
      const int b = __ffs(s) - 1;
      if (pos < K) orow[pos] = base + (wd << 5) + b;
      ++pos;
      s &= s - 1;
    }
  }
  for (int j = tot + tid; j < K; j += kThreads) orow[j] = -1;  // only if ties were short (cannot happen)
}

}  // namespace

dsa_status launch_topk(const dsa_indexer_topk_args* a, const float* scores, int64_t ld, int max_vis,
                       hipStream_t stream) {
  if (a->nq == 0) return DSA_OK;
  if (max_vis > 131072) return fail(DSA_ERR_UNSUPPORTED, "topk: rows longer than 131072 keys");
  const dim3 grid(a->nq), block(kThreads);
#define DSA_TOPK_LAUNCH(E)                                                                                       \
  hipLaunchKernelGGL(topk_kernel<E>, grid, block, 0, stream, scores, ld, a->cu_seqlens_q, a->seqused_kv,       \
                     a->cu_seqlens_kv, a->window_kv_start, a->batch, a->q_stride, a->compress_ratio, a->nq, max_vis, \
                     a->topk, a->window, a->kv_row_base, a->topk_idx, a->err_flag)
  if (max_vis <= 4 * kThreads) DSA_TOPK_LAUNCH(4);
  else if (max_vis <= 8 * kThreads) DSA_TOPK_LAUNCH(8);
  else if (max_vis <= 16 * kThreads) DSA_TOPK_LAUNCH(16);
  else if (max_vis <= 32 * kThreads) DSA_TOPK_LAUNCH(32);
  else DSA_TOPK_LAUNCH(0);
#undef DSA_TOPK_LAUNCH
  return check_launch("topk_kernel");
}

}  // namespace dsa
