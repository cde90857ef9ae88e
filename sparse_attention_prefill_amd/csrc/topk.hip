// (3) Per-query causal top-k over indexer scores (+ sliding-window rows), on gfx950.
//
// [xLLM-CP] "feat: DeepSeek-V4 DSA context-parallel on NPU", Design, data-flow step (3) (top-k
// of the local queries over their causal keys) and Implementation §5 (a top-k fed unlocalised
// metadata collapses to position 0, i.e. the selection is per query over its own extent).
//
// One workgroup per query row. Scores become order-preserving 32-bit keys (-0.0 and +0.0 share
// one key) and a radix select finds the K-th largest key tau in three digits, 12 + 10 + 10 bits.
// The tie rule (higher score first, then lower key index) is applied exactly: all keys above tau
// are taken, then the `need` keys equal to tau with the lowest positions. Output ids ascend.
//
// Rows of up to NT*EPT keys (topk_reg_kernel) are loaded once into registers, key j of thread t
// at row position j*NT + t, so one wave instruction covers 64 consecutive positions:
//   1. a 4096-bin LDS histogram of the top 12 bits; one wave finds the bin b* of the K-th key;
//   2. the keys inside b* are appended to an LDS list (wave-aggregated) and one wave resolves
//      the two low digits over that short list (over the registers when b* is too full);
//   3. per 64-key chunk, ballots count keys above / equal to tau; a block scan over the chunks
//      gives each chunk's output offset, and a last pass over the registers writes every
//      selected id at offset + (selected lanes below it): contiguous stores, no sort.
// Longer rows (topk_stream_kernel) are read from memory once in the common case: a stratified
// sample of 8192 keys (16 blocks of 512 spread over the row) gives a threshold theta that about
// 1.6*K keys of the row exceed; one pass appends every key >= theta to the LDS list, the list
// is selected exactly, and the ids are emitted from LDS bitmaps. When the list ends up with
// fewer than K keys or overflows, the row falls back to an exact histogram over the whole row
// (then keys above b* go straight to the bitmaps and only b*'s keys are listed).
// Launches of more than 1024 rows of 4097 .. 32768 keys take topk_sample_kernel: the same
// sample / list / exact-select scheme in 256 threads and about 32 KB of LDS per row, so five
// rows share a CU (its section below).
#include "index_score.h"

namespace dsa {
namespace {

constexpr int kMaxRow = 131072;   // longest row (keys)
constexpr int kBins0 = 4096;      // first digit: key bits 31..20
constexpr int kBinsR = 1024;      // refinement digits: bits 19..10, then 9..0
constexpr int kStreamNT = 1024;   // threads of the streamed path (16 waves)
constexpr int kStreamCand = 5120; // list of the streamed path (two workgroups per CU)
constexpr int kSampleBlock = 512; // sample keys per wave on the streamed path
constexpr int kStreamVec = 4;     // float4 loads in flight per thread on the single pass

// A wave-uniform value the compiler must treat as new: bounds of fully unrolled loops are
// re-derived per pass, so their per-iteration conditions are not kept alive across passes.
__device__ inline int opaque(int v) {
  asm volatile("" : "+s"(v));
  return v;
}
// LDS accesses of this wave issued so far have completed; the compiler moves no access across.
__device__ inline void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Inclusive scan over the 64 lanes on DPP: shifts by 1, 2, 4, 8 inside each row of 16 lanes,
// then the last lane of row 0 / row 2 is added to rows 1 / 3 and the last lane of row 1 to rows
// 2 and 3 (row broadcasts). No LDS round trips.
__device__ inline int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Max / min over the 64 lanes of a wave on DPP, in the order of wave_incl_scan (lane 63 ends with
// the result, returned uniform). Shifted-in lanes contribute 0 to the max and the lane's own
// value to the min.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x111, 0xf, 0xf, true)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x112, 0xf, 0xf, true)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x114, 0xf, 0xf, true)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x118, 0xf, 0xf, true)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x142, 0xa, 0xf, false)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x143, 0xc, 0xf, false)));
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}
__device__ inline uint32_t wave_min_u32(uint32_t v) {
  v = min(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x111, 0xf, 0xf, false)));
  v = min(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x112, 0xf, 0xf, false)));
  v = min(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x114, 0xf, 0xf, false)));
  v = min(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x118, 0xf, 0xf, false)));
  v = min(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x142, 0xa, 0xf, false)));
  v = min(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x143, 0xc, 0xf, false)));
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}

// Exclusive block scan of one int per thread (NW waves); *total = block sum.
template <int NW>
__device__ inline int block_excl_scan(int v, int* smem, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) smem[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int x = lane < NW ? smem[lane] : 0;
    const int xi = wave_incl_scan(x);
    if (lane < NW) smem[lane] = xi - x;
    if (lane == NW - 1) smem[NW] = xi;
  }
  __syncthreads();
  const int r = smem[wave] + incl - v;
  *total = smem[NW];
  __syncthreads();
  return r;
}

// Two exclusive block scans at once (a and b); smem holds 2*(NW+1) ints.
template <int NW>
__device__ inline void block_excl_scan2(int a, int b, int* smem, int* ea, int* eb, int* ta, int* tb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  if (lane == 63) {
    smem[wave] = ia;
    smem[NW + 1 + wave] = ib;
  }
  __syncthreads();
  if (wave == 0) {
    const int x = lane < NW ? smem[lane] : 0, y = lane < NW ? smem[NW + 1 + lane] : 0;
    const int xi = wave_incl_scan(x), yi = wave_incl_scan(y);
    if (lane < NW) {
      smem[lane] = xi - x;
      smem[NW + 1 + lane] = yi - y;
    }
    if (lane == NW - 1) {
      smem[NW] = xi;
      smem[2 * NW + 1] = yi;
    }
  }
  __syncthreads();
  *ea = smem[wave] + ia - a;
  *eb = smem[NW + 1 + wave] + ib - b;
  *ta = smem[NW];
  *tb = smem[2 * NW + 1];
  __syncthreads();
}

// One wave: in a complete NBINS-bin histogram, the bin holding the rem-th largest key (counting
// from the top bin). Lane l first owns bins [NBINS - per*(l+1), NBINS - per*l); the lane whose
// range holds the target then spreads its bins over the wave. Requires rem <= total.
template <int NBINS>
__device__ inline void wave_select(const uint32_t* hist, int rem, int* bin, int* rem_out, int* cnt_out) {
  constexpr int per = NBINS / 64;
  static_assert(per % 4 == 0 && per <= 64, "bins per lane");
  const int lane = threadIdx.x & 63;
  const int lo = NBINS - per * (lane + 1);
  int own = 0;
#pragma unroll
  for (int k = 0; k < per; k += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(hist + lo + k);
    own += int(v.x + v.y + v.z + v.w);
  }
  const int incl = wave_incl_scan(own);
  const int above = incl - own;
  const uint64_t m = ballot(above < rem && rem <= incl);
  const int L = m ? int(__builtin_ctzll(m)) : 63;
  const int above_L = __builtin_amdgcn_readlane(above, L);
  const int lo_L = NBINS - per * (L + 1);
  const int c = lane < per ? int(hist[lo_L + per - 1 - lane]) : 0;  // lane 0: top bin of L
  const int incl2 = wave_incl_scan(c);
  const int above2 = above_L + incl2 - c;
  const uint64_t m2 = ballot(lane < per && above2 < rem && rem <= above2 + c);
  const int l2 = m2 ? int(__builtin_ctzll(m2)) : 0;
  *bin = lo_L + per - 1 - l2;
  *rem_out = rem - __builtin_amdgcn_readlane(above2, l2);
  *cnt_out = __builtin_amdgcn_readlane(c, l2);
}

// Zero p[0, n), n a multiple of 4, with NT threads.
template <int NT>
__device__ inline void zero_words(uint32_t* p, int n) {
  for (int b = 4 * threadIdx.x; b < n; b += 4 * NT) *reinterpret_cast<uint4*>(p + b) = uint4{0, 0, 0, 0};
}

// One wave: resolve the two 10-bit digits below `prefix` (bits 31..20 fixed) over a list of n
// keys through a 1024-bin LDS histogram; updates prefix and the count still to take.
__device__ inline void wave_refine_list(const uint32_t* keys, int n, uint32_t* hist, uint32_t* prefix, int* rem) {
  const int lane = threadIdx.x & 63;
#pragma unroll 1
  for (int r = 0; r < 2; ++r) {
    const int shift = 10 - 10 * r;
#pragma unroll
    for (int b = 4 * lane; b < kBinsR; b += 256) *reinterpret_cast<uint4*>(hist + b) = uint4{0, 0, 0, 0};
    lds_wait();
    const uint32_t pfx = *prefix >> (shift + 10);
    for (int c = lane; c < n; c += 64) {
      const uint32_t key = keys[c];
      if ((key >> (shift + 10)) == pfx) atomicAdd(&hist[(key >> shift) & (kBinsR - 1)], 1u);
    }
    lds_wait();
    int bin, rem_out, cnt;
    wave_select<kBinsR>(hist, *rem, &bin, &rem_out, &cnt);
    *prefix |= uint32_t(bin) << shift;
    *rem = rem_out;
    lds_wait();
  }
}

// ---------------------------------------------------------------------------------------------
// Shared row set-up: window rows, short rows, bad rows. Returns false when the row is done.
// ---------------------------------------------------------------------------------------------
struct RowInfo {
  int ev;    // visible keys
  int base;  // id of position 0
};

template <int NT>
__device__ inline bool row_setup(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ used_kv,
                                 const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ win_kv, int batch,
                                 int stride, int ratio, int nk, int max_vis, int row_cap, int K, int window,
                                 int kv_row_base, int32_t* orow, int32_t* err_flag, RowInfo* ri,
                                 int skip_above = INT32_MAX) {
  const int i = blockIdx.x, tid = threadIdx.x;
  const int k_tot = K + window;
  QueryView v;
  const bool have = query_view(cu_q, used_kv, cu_kv, batch, stride, i, &v);
  const int ev = have ? (ratio > 1 ? v.E / ratio : v.E) : 0;
  // the indexer's test of a usable row: a causal extent inside the key buffer
  const bool ok = have && v.E >= 1 && ev <= max_vis && v.kv0 >= 0 && int64_t(v.kv0) + ev <= nk;
  if (ok && ev > skip_above) return false;  // selected from a candidate list
  if (!ok) {
    if (tid == 0) raise_flag(err_flag, DSA_DEVERR_EXTENT);
    for (int j = tid; j < k_tot; j += NT) orow[j] = -1;
    return false;
  }
  // window rows (original tokens): positions max(0, p-window+1) .. p, p = E-1
  if (window > 0) {
    const int p = v.E - 1;
    const int w0 = max(0, p - window + 1);
    for (int j = tid; j < window; j += NT) orow[K + j] = (w0 + j <= p) ? win_kv[v.b] + w0 + j : -1;
  }
  ri->ev = ev;
  ri->base = kv_row_base + v.kv0;
  if (ev <= K) {  // every visible key
    for (int j = tid; j < K; j += NT) orow[j] = j < ev ? ri->base + j : -1;
    return false;
  }
  if (ev > row_cap) {  // no kernel of this launch holds such a row
    if (tid == 0) raise_flag(err_flag, DSA_DEVERR_EXTENT);
    for (int j = tid; j < K; j += NT) orow[j] = -1;
    return false;
  }
  return true;
}

// ---------------------------------------------------------------------------------------------
// Rows held in registers
// ---------------------------------------------------------------------------------------------
template <int NT, int EPT>
struct RegShared {
  static constexpr int kWaves = NT / 64;
  static constexpr int kList = kWaves >= 16 ? 8192 : 4096;
  static constexpr int kPerWave = kList / kWaves;  // list segment of one wave
  union {
    alignas(16) uint32_t hist[kBins0];  // digit 1
    uint32_t list[kList];               // then: keys of bin b*, (low 20 bits << 12) | chunk
  } u;
  alignas(16) uint32_t hist_r[kBinsR];  // digits 2 and 3
  uint32_t chunk[NT * EPT / 64];        // per 64-key chunk: (#above tau) | (#equal to tau) << 16, then prefix
  int wave_n[kWaves];                   // keys each wave listed
  int scan[kWaves + 1];
  uint32_t prefix;
  int remaining;
  bool take_all;
};

// 1024-thread rows run two workgroups per CU (8 waves per SIMD, at most 64 VGPRs), so one row's
// loads overlap another row's passes.
template <int NT, int EPT>
__global__ __launch_bounds__(NT, NT == 1024 ? 8 : 1) void topk_reg_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ used_kv,
    const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ win_kv, int batch, int stride, int ratio, int nk,
    int max_vis, int K, int window, int kv_row_base, int32_t* __restrict__ out, int32_t* __restrict__ err_flag,
    int skip_above) {
  static_assert(EPT % 4 == 0 && EPT <= 64, "chunks come in groups of 4; one chunk per lane / thread");
  using Sh = RegShared<NT, EPT>;
  __shared__ Sh sh;
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sel_wave = 0;  // runs the single-wave selects
  int32_t* orow = out + int64_t(blockIdx.x) * (K + window);
  RowInfo ri;
  if (!row_setup<NT>(cu_q, used_kv, cu_kv, win_kv, batch, stride, ratio, nk, max_vis, NT * EPT, K, window,
                     kv_row_base, orow, err_flag, &ri, skip_above))
    return;
  const int ev = ri.ev;
  const float* srow = scores + int64_t(blockIdx.x) * ld;

  // Keys. Positions past the row get (lane & 7) << 20: bins 0..7, which hold no finite score,
  // so they never reach the selection and their histogram atomics spread over 8 addresses.
  uint32_t keys[EPT];
  {
    const int g_load = opaque((ev + 4 * NT - 1) / (4 * NT));
    float x[EPT];
#pragma unroll
    for (int g = 0; g < EPT / 4; ++g)
#pragma unroll
      for (int k = 0; k < 4; ++k) x[4 * g + k] = g < g_load ? srow[min((4 * g + k) * NT + tid, ev - 1)] : 0.f;
    const uint32_t pad = uint32_t(lane & 7) << 20;
#pragma unroll
    for (int j = 0; j < EPT; ++j) keys[j] = j * NT + tid < ev ? order_key(x[j]) : pad;
  }
  // This wave's chunk j covers positions j*NT + wave*64 .. +63. Passes visit the groups of four
  // chunks whose first chunk starts inside the row; each pass is fully unrolled and tests the
  // group index against a fresh copy of the scalar bound.
  const int n_grp = __builtin_amdgcn_readfirstlane(min(EPT / 4, max(0, (ev - wave * 64 + 4 * NT - 1) / (4 * NT))));
  auto for_chunks = [&](auto&& fn) {
    const int ng = opaque(n_grp);
#pragma unroll
    for (int g = 0; g < EPT / 4; ++g)
      if (g < ng) {
#pragma unroll
        for (int k = 0; k < 4; ++k) fn(4 * g + k);
      }
  };

  // ---- digit 1 over the whole row ----
  zero_words<NT>(sh.u.hist, kBins0);
  __syncthreads();
  for_chunks([&](int j) { atomicAdd(&sh.u.hist[keys[j] >> 20], 1u); });
  __syncthreads();
  if (wave == sel_wave) {
    int bin, rem, cnt;
    wave_select<kBins0>(sh.u.hist, K, &bin, &rem, &cnt);
    if (lane == 0) {
      sh.prefix = uint32_t(bin) << 20;
      sh.remaining = rem;
      sh.take_all = rem == cnt;  // every key of b* is taken: no lower digits needed
    }
  }
  zero_words<NT>(sh.hist_r, kBinsR);
  __syncthreads();
  const uint32_t bstar = sh.prefix >> 20;

  // ---- one pass: count keys above b* per chunk (lane j of cnt holds chunk j) and list the
  // keys inside b* in this wave's own segment ----
  uint32_t* seg = sh.u.list + wave * Sh::kPerWave;
  {
    int cnt = 0, n_mine = 0;
    for_chunks([&](int j) {
      const uint32_t bin = keys[j] >> 20;
      const int above = __popcll(ballot(bin > bstar));  // whole-wave vote, outside the select
      cnt = lane == j ? above : cnt;
      const bool in_bin = bin == bstar;
      const uint64_t m = ballot(in_bin);
      const int slot = n_mine + lanes_below(m);
      if (in_bin && slot < Sh::kPerWave) seg[slot] = ((keys[j] & 0xFFFFFu) << 12) | uint32_t(j * NW + wave);
      n_mine += __popcll(m);
    });
    if (lane < 4 * n_grp) sh.chunk[lane * NW + wave] = uint32_t(cnt);
    if (lane == 0) sh.wave_n[wave] = n_mine;
  }
  __syncthreads();
  bool listed = true;
#pragma unroll
  for (int w = 0; w < NW; ++w) listed = listed && sh.wave_n[w] <= Sh::kPerWave;
  const int n_mine = sh.wave_n[wave];

  // ---- digits 2 and 3 (stop as soon as the chosen bin is taken whole) ----
#pragma unroll 1
  for (int r = 0; r < 2 && !sh.take_all; ++r) {
    const int shift = 10 - 10 * r;
    if (r == 1) {
      zero_words<NT>(sh.hist_r, kBinsR);
      __syncthreads();
    }
    const uint32_t pfx = sh.prefix >> (shift + 10);
    if (listed) {  // the list entries share bits 31..20
      const uint32_t pfx20 = pfx & ((1u << (10 - shift)) - 1u);
      for (int c = lane; c < n_mine; c += 64) {
        const uint32_t k20 = seg[c] >> 12;
        if ((k20 >> (shift + 10)) == pfx20) atomicAdd(&sh.hist_r[(k20 >> shift) & (kBinsR - 1)], 1u);
      }
    } else {
      for_chunks([&](int j) {
        if ((keys[j] >> (shift + 10)) == pfx) atomicAdd(&sh.hist_r[(keys[j] >> shift) & (kBinsR - 1)], 1u);
      });
    }
    __syncthreads();
    if (wave == sel_wave) {
      int bin, rem, cnt;
      wave_select<kBinsR>(sh.hist_r, sh.remaining, &bin, &rem, &cnt);
      if (lane == 0) {
        sh.prefix |= uint32_t(bin) << shift;
        sh.remaining = rem;
        sh.take_all = rem == cnt;
      }
    }
    __syncthreads();
  }
  // The selection is every key above tau plus `need` keys equal to it, or, when the last
  // chosen bin is taken whole, every key >= tau (tau = that bin's lower edge).
  const uint32_t tau = sh.prefix;
  const bool take_all = sh.take_all;
  const int need = sh.remaining;

  // ---- final per-chunk counts ----
  if (listed) {  // chunks already hold the keys above b*; add b*'s keys above / at tau
    const uint32_t tau20 = tau & 0xFFFFFu;
    for (int c = lane; c < n_mine; c += 64) {
      const uint32_t e = seg[c], k20 = e >> 12;
      if (k20 > tau20) atomicAdd(&sh.chunk[e & 0xFFFu], 1u);
      else if (k20 == tau20) atomicAdd(&sh.chunk[e & 0xFFFu], 1u << 16);
    }
  } else {
    int cnt = 0;
    for_chunks([&](int j) {
      const int c = __popcll(ballot(keys[j] > tau)) | (__popcll(ballot(keys[j] == tau)) << 16);
      cnt = lane == j ? c : cnt;
    });
    if (lane < 4 * n_grp) sh.chunk[lane * NW + wave] = uint32_t(cnt);
  }
  __syncthreads();
  const int n_chunks = (ev + 63) >> 6;
  // one scan carries both counts: the low halves sum to at most 32768, so never carry
  int tot_i;
  const int v = tid < n_chunks ? int(sh.chunk[tid]) : 0;
  const int excl = block_excl_scan<NW>(v, sh.scan, &tot_i);
  if (tid < n_chunks) sh.chunk[tid] = uint32_t(excl);
  const uint32_t tot = uint32_t(tot_i);
  __syncthreads();

  // ---- ordered write: id of each selected key at its chunk's offset + selected lanes below ----
  const uint32_t pref = lane < 4 * n_grp ? sh.chunk[lane * NW + wave] : 0u;  // lane j: chunk j
  if (take_all || int(tot >> 16) == need) {  // every key equal to tau is taken
    for_chunks([&](int j) {
      const uint32_t pj = __builtin_amdgcn_readlane(pref, j);
      const bool sel = keys[j] >= tau;
      const uint64_t s = ballot(sel);
      if (sel && DSA_CHECK(int(pj & 0xFFFFu) + int(pj >> 16) + lanes_below(s) < K, err_flag))
        orow[int(pj & 0xFFFFu) + int(pj >> 16) + lanes_below(s)] = ri.base + j * NT + tid;
    });
  } else {  // ties at tau beyond the quota: the lowest positions win
    for_chunks([&](int j) {
      const uint32_t pj = __builtin_amdgcn_readlane(pref, j);
      const int gt_before = int(pj & 0xFFFFu), eq_before = int(pj >> 16);
      const bool is_eq = keys[j] == tau;
      const uint64_t e = ballot(is_eq);
      const bool sel = keys[j] > tau || (is_eq && eq_before + lanes_below(e) < need);
      const uint64_t s = ballot(sel);
      if (sel && DSA_CHECK(gt_before + min(eq_before, need) + lanes_below(s) < K, err_flag))
        orow[gt_before + min(eq_before, need) + lanes_below(s)] = ri.base + j * NT + tid;
    });
  }
  const int n_sel = int(tot & 0xFFFFu) + (take_all ? int(tot >> 16) : min(int(tot >> 16), need));
  for (int j = n_sel + tid; j < K; j += NT) orow[j] = -1;  // only if ties were short (cannot happen)
}

// ---------------------------------------------------------------------------------------------
// Rows streamed from memory
// ---------------------------------------------------------------------------------------------
struct StreamShared {
  union {
    alignas(16) uint32_t hist[kBins0];  // 16 KB, dead once the bitmaps are in use
    uint64_t bits[2][kMaxRow / 64];     // 32 KB: keys above tau / equal to tau, one bit per position
  } u;
  alignas(16) uint32_t hist_r[kBinsR];  // refinement digits
  uint32_t cand_key[kStreamCand];       // list: keys (raw score bits until the exact select)
  int32_t cand_pos[kStreamCand];
  int scan[2 * (kStreamNT / 64 + 1)];
  uint32_t prefix;
  int remaining;
  int n_cand;
};

// Ascending ids base + position of the selected keys, from the bitmaps of the keys above tau
// and equal to tau (the first `need` of those in position order): each thread owns a run of
// 64-position chunks, and a block scan gives each run its output offset.
template <int NT>
__device__ __attribute__((always_inline)) inline void emit_from_bitmaps(const uint64_t* gt, const uint64_t* eq, int n_chunks, int need, int K,
                                         int base, int32_t* __restrict__ orow, int* scan) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int per = (n_chunks + NT - 1) / NT;
  const int c_begin = min(tid * per, n_chunks), c_end = min(c_begin + per, n_chunks);
  int my_gt = 0, my_eq = 0;
  for (int c = c_begin; c < c_end; ++c) {
    my_gt += __popcll(gt[c]);
    my_eq += __popcll(eq[c]);
  }
  int gt_before, eq_before, gt_tot, eq_tot;
  block_excl_scan2<NW>(my_gt, my_eq, scan, &gt_before, &eq_before, &gt_tot, &eq_tot);
  int pos = gt_before + min(eq_before, need);
  int eq_rank = eq_before;
  for (int c = c_begin; c < c_end; ++c) {
    uint64_t e = eq[c], keep = 0;
    while (e) {  // ties in position order, while the quota lasts
      const uint64_t bit = e & (~e + 1ull);
      if (eq_rank < need) keep |= bit;
      ++eq_rank;
      e ^= bit;
    }
    uint64_t s = gt[c] | keep;
    while (s) {
      const int b = __builtin_ctzll(s);
      if (pos < K) orow[pos] = base + (c << 6) + b;
      ++pos;
      s &= s - 1;
    }
  }
  const int n_sel = gt_tot + min(eq_tot, need);
  for (int j = n_sel + tid; j < K; j += NT) orow[j] = -1;  // only if ties were short (cannot happen)
}

// Top-K of one score row srow[0, ev) (ev > K), streamed from memory by kStreamNT threads; row
// storage is ld floats (loads stay below it). Writes orow[0, K) = base + position, ascending.
__device__ __attribute__((always_inline)) inline void stream_select(const float* __restrict__ srow, int64_t ld, int ev, int K, int base,
                                     int32_t* __restrict__ orow, StreamShared& sh) {
  constexpr int NT = kStreamNT, NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_chunks = (ev + 63) >> 6;
  uint64_t* gt = sh.u.bits[0];
  uint64_t* eq = sh.u.bits[1];

  bool listed = false;
  if (ev >= NW * 2048) {
    // ---- sample: wave w reads 512 consecutive keys starting near w*ev/16 ----
    // (ev >= 16*2048, so the 16 blocks are disjoint and inside the row)
    uint32_t skey[kSampleBlock / 64];
    {
      const int blk = int((int64_t(wave) * ev / NW) & ~int64_t(63));
#pragma unroll
      for (int k = 0; k < kSampleBlock / 64; ++k) skey[k] = order_key(srow[blk + 64 * k + lane]);
    }
    zero_words<NT>(sh.u.hist, kBins0);
    zero_words<NT>(sh.hist_r, kBinsR);
    if (tid == 0) sh.n_cand = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kSampleBlock / 64; ++k) atomicAdd(&sh.u.hist[skey[k] >> 20], 1u);
    __syncthreads();
    // the sample rank whose key about 1.6*K keys of the row exceed
    const int n_sample = NW * kSampleBlock;
    const int r_s = min(n_sample, int(int64_t(13) * K * n_sample / (int64_t(8) * ev)) + 16);
    if (wave == 0) {
      int bin, rem, cnt;
      wave_select<kBins0>(sh.u.hist, r_s, &bin, &rem, &cnt);
      if (lane == 0) {
        sh.prefix = uint32_t(bin) << 20;
        sh.remaining = rem;
      }
    }
    __syncthreads();
    {
      const uint32_t bs = sh.prefix >> 20;
#pragma unroll
      for (int k = 0; k < kSampleBlock / 64; ++k)
        if ((skey[k] >> 20) == bs) atomicAdd(&sh.hist_r[(skey[k] >> 10) & (kBinsR - 1)], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      int bin, rem, cnt;
      wave_select<kBinsR>(sh.hist_r, sh.remaining, &bin, &rem, &cnt);
      if (lane == 0) sh.prefix |= uint32_t(bin) << 10;
    }
    __syncthreads();
    const float theta = key_to_float(sh.prefix);  // key(x) >= prefix  <=>  x >= theta
    // The single pass compares floats; with theta a normal float that matches the key order
    // whatever the denormal mode. Otherwise (theta zero or denormal) take the exact path.
    if (fabsf(theta) >= 1.17549435e-38f) {
    // ---- single pass: list every key >= theta (raw bits and position) ----
    const int n_vec = ev >> 2;  // float4s wholly inside the row
    const int last4 = int(ld >> 2) - 1;
    const float4* s4 = reinterpret_cast<const float4*>(srow);
    for (int v0 = 0; v0 * 4 < ev; v0 += NT * kStreamVec) {
      float4 x[kStreamVec];
#pragma unroll
      for (int u = 0; u < kStreamVec; ++u) x[u] = s4[min(v0 + u * NT + tid, last4)];
      // keys >= theta in this wave's chunks: count, claim their slots with one atomic, place
      auto listed_key = [&](int u, int c) {
        const int q = v0 + u * NT + tid;
        const float xc = c == 0 ? x[u].x : c == 1 ? x[u].y : c == 2 ? x[u].z : x[u].w;
        return xc >= theta && (q < n_vec || 4 * q + c < ev);
      };
      const int n_live = __builtin_amdgcn_readfirstlane(
          min(kStreamVec, max(0, (((ev + 3) >> 2) - v0 - wave * 64 + NT - 1) / NT)));
      int total = 0;
#pragma unroll
      for (int u = 0; u < kStreamVec; ++u)
        if (u < n_live)
#pragma unroll
          for (int c = 0; c < 4; ++c) total += __popcll(ballot(listed_key(u, c)));
      if (total == 0) continue;
      int slot = 0;
      if (lane == 0) slot = atomicAdd(&sh.n_cand, total);
      slot = __builtin_amdgcn_readfirstlane(slot);
      const int nl = opaque(n_live);
#pragma unroll
      for (int u = 0; u < kStreamVec; ++u) {
        if (u >= nl) continue;
        const int q = v0 + u * NT + tid;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bool in = listed_key(u, c);
          const uint64_t m = ballot(in);
          const int sl = slot + lanes_below(m);
          if (in && sl < kStreamCand) {
            sh.cand_key[sl] = __float_as_uint(c == 0 ? x[u].x : c == 1 ? x[u].y : c == 2 ? x[u].z : x[u].w);
            sh.cand_pos[sl] = 4 * q + c;
          }
          slot += __popcll(m);
        }
      }
    }
    __syncthreads();
    const int n_cand = sh.n_cand;
    listed = n_cand >= K && n_cand <= kStreamCand;
    if (listed) {
      // ---- exact select over the list: three digits ----
      for (int c = tid; c < n_cand; c += NT) sh.cand_key[c] = order_key_bits(sh.cand_key[c]);
      zero_words<NT>(sh.u.hist, kBins0);
      __syncthreads();
      for (int c = tid; c < n_cand; c += NT) atomicAdd(&sh.u.hist[sh.cand_key[c] >> 20], 1u);
      __syncthreads();
      if (wave == 0) {
        int bin, rem, cnt;
        wave_select<kBins0>(sh.u.hist, K, &bin, &rem, &cnt);
        uint32_t prefix = uint32_t(bin) << 20;
        wave_refine_list(sh.cand_key, n_cand, sh.hist_r, &prefix, &rem);
        if (lane == 0) {
          sh.prefix = prefix;
          sh.remaining = rem;
        }
      }
      __syncthreads();
      const uint32_t tau = sh.prefix;
      for (int c = tid; c < n_chunks; c += NT) gt[c] = eq[c] = 0;
      __syncthreads();
      for (int c = tid; c < n_cand; c += NT) {
        const uint32_t key = sh.cand_key[c];
        const int p = sh.cand_pos[c];
        if (key > tau) atomicOr(&gt[p >> 6], 1ull << (p & 63));
        else if (key == tau) atomicOr(&eq[p >> 6], 1ull << (p & 63));
      }
    }
    }
  }

  if (!listed) {
    // ---- exact: digit 1 over the whole row, then b*'s keys ----
    // visit 64-key chunks of the row in order: fn(key, position, valid), all lanes of a wave
    auto visit = [&](auto&& fn) {
      constexpr int U = 8;
      for (int j0 = 0; j0 * NT < ev; j0 += U) {
        float x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = srow[min((j0 + u) * NT + tid, ev - 1)];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int p = (j0 + u) * NT + tid;
          if ((j0 + u) * NT + wave * 64 < ev) fn(order_key(x[u]), p, p < ev);
        }
      }
    };
    __syncthreads();  // the sampled attempt's LDS reads are done
    zero_words<NT>(sh.u.hist, kBins0);
    zero_words<NT>(sh.hist_r, kBinsR);
    if (tid == 0) sh.n_cand = 0;
    __syncthreads();
    visit([&](uint32_t key, int, bool valid) { atomicAdd(&sh.u.hist[valid ? key >> 20 : 0u], 1u); });
    __syncthreads();
    if (wave == 0) {
      int bin, rem, cnt;
      wave_select<kBins0>(sh.u.hist, K, &bin, &rem, &cnt);
      if (lane == 0) {
        sh.prefix = uint32_t(bin) << 20;
        sh.remaining = rem;
      }
    }
    __syncthreads();
    const uint32_t bstar = sh.prefix >> 20;
    for (int c = tid; c < n_chunks; c += NT) eq[c] = 0;
    visit([&](uint32_t key, int p, bool valid) {
      const uint32_t bin = key >> 20;
      const uint64_t g = ballot(valid && bin > bstar);
      if (lane == 0) gt[p >> 6] = g;
      const bool in_bin = valid && bin == bstar;
      const uint64_t cm = ballot(in_bin);
      if (cm) {
        int slot = 0;
        if (lane == 0) slot = atomicAdd(&sh.n_cand, __popcll(cm));
        slot = __builtin_amdgcn_readfirstlane(slot) + lanes_below(cm);
        if (in_bin && slot < kStreamCand) {
          sh.cand_key[slot] = key;
          sh.cand_pos[slot] = p;
        }
      }
    });
    __syncthreads();
    const int n_cand = sh.n_cand;
    if (n_cand <= kStreamCand) {
      if (wave == 0) {
        uint32_t prefix = sh.prefix;
        int rem = sh.remaining;
        wave_refine_list(sh.cand_key, n_cand, sh.hist_r, &prefix, &rem);
        if (lane == 0) {
          sh.prefix = prefix;
          sh.remaining = rem;
        }
      }
      __syncthreads();
      const uint32_t tau = sh.prefix;
      for (int c = tid; c < n_cand; c += NT) {
        const uint32_t key = sh.cand_key[c];
        const int p = sh.cand_pos[c];
        if (key > tau) atomicOr(&gt[p >> 6], 1ull << (p & 63));
        else if (key == tau) atomicOr(&eq[p >> 6], 1ull << (p & 63));
      }
    } else {  // b* holds more keys than the list: refine and mark over the row itself
#pragma unroll 1
      for (int r = 0; r < 2; ++r) {
        const int shift = 10 - 10 * r;
        zero_words<NT>(sh.hist_r, kBinsR);
        __syncthreads();
        const uint32_t pfx = sh.prefix >> (shift + 10);
        visit([&](uint32_t key, int, bool valid) {
          if (valid && (key >> (shift + 10)) == pfx) atomicAdd(&sh.hist_r[(key >> shift) & (kBinsR - 1)], 1u);
        });
        __syncthreads();
        if (wave == 0) {
          int bin, rem, cnt;
          wave_select<kBinsR>(sh.hist_r, sh.remaining, &bin, &rem, &cnt);
          if (lane == 0) {
            sh.prefix |= uint32_t(bin) << shift;
            sh.remaining = rem;
          }
        }
        __syncthreads();
      }
      const uint32_t tau = sh.prefix;
      visit([&](uint32_t key, int p, bool valid) {
        const uint64_t g = ballot(valid && key > tau), e = ballot(valid && key == tau);
        if (lane == 0) {
          gt[p >> 6] = g;
          eq[p >> 6] = e;
        }
      });
    }
  }
  __syncthreads();
  const int need = sh.remaining;  // keys equal to tau to take (>= 1)
  emit_from_bitmaps<NT>(gt, eq, n_chunks, need, K, base, orow, sh.scan);
}

__global__ __launch_bounds__(kStreamNT, 8) void topk_stream_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ used_kv,
    const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ win_kv, int batch, int stride, int ratio, int nk,
    int max_vis, int K, int window, int kv_row_base, int32_t* __restrict__ out, int32_t* __restrict__ err_flag,
    int skip_above) {
  __shared__ StreamShared sh;
  int32_t* orow = out + int64_t(blockIdx.x) * (K + window);
  RowInfo ri;
  if (!row_setup<kStreamNT>(cu_q, used_kv, cu_kv, win_kv, batch, stride, ratio, nk, max_vis, kMaxRow, K, window,
                            kv_row_base, orow, err_flag, &ri, skip_above))
    return;
  stream_select(scores + int64_t(blockIdx.x) * ld, ld, ri.ev, K, ri.base, orow, sh);
}

// ---------------------------------------------------------------------------------------------
// Rows of up to kSmpMaxRow keys: 256 threads per row and about 32 KB of LDS, so five rows are in
// flight on each CU and one row's passes overlap the others' loads.
//   * A row of at most kSmpList keys is its own list.
//   * A longer row is sampled first: 16 tiles of 256 consecutive keys spread evenly over it give
//     a threshold theta that about K + 4 spreads of the row's keys reach (the r-th largest of the
//     m = 4096 sample keys, r the smallest rank whose expected count r*ev/m stays 4 binomial
//     spreads sqrt(r)*ev/m above K). One float4 pass over the row then appends every key >= theta
//     (its order key and 16-bit position) to the LDS list, one LDS atomic per wave per step.
//   * The list is selected exactly, keys taken relative to the list's base key (theta, or the
//     row's smallest key) so that the 11-bit digits spread over the list's own span; ids are
//     emitted ascending from position bitmaps.
//   * A list that overflowed or holds fewer than K keys (ties, adversarial rows) sends the row to
//     an exact radix select over the row in memory (11 + 11 + 10 bits).
// ---------------------------------------------------------------------------------------------
constexpr int kSmpMaxRow = 32768;
constexpr int kSmpList = 3584;                 // list entries: 21 KB with 16-bit positions
constexpr int kSmpTiles = 16, kSmpTile = 256;  // sample: 16 tiles of 256 consecutive keys
constexpr int kSmpSample = kSmpTiles * kSmpTile;
constexpr int kSmpBins = 2048;                 // 11-bit digits
constexpr int kSmpInFlight = 2048;             // float4 loads in flight per workgroup on the pass (32 KB)

template <int NT>
struct SampleShared {
  uint32_t key[kSmpList];  // order keys of the list
  uint16_t pos[kSmpList];  // their positions in the row
  union {
    alignas(16) uint32_t hist[kSmpBins];
    uint64_t bits[2][kSmpMaxRow / 64];  // keys above tau / equal to tau, one bit per position
  } u;
  int scan[2 * (NT / 64 + 1)];
  uint32_t red[2][NT / 64];
  uint32_t prefix;   // selected digits so far (relative keys >> lo)
  int remaining;     // keys still to take inside the prefix's bin
  int lo;            // lowest bit the prefix covers
  int take_all;      // every key of the prefix's bin is taken
  int count;         // keys in the prefix's bin
  int n_small;       // keys of that bin gathered for the single-wave finish
  int n_list;
};

// Workgroup-wide min and max of one value per thread, returned in every thread (one barrier;
// `red` is free again after the caller's next barrier).
template <int NT>
__device__ inline void smp_minmax(uint32_t mn, uint32_t mx, uint32_t (*red)[NT / 64], uint32_t* omn,
                                  uint32_t* omx) {
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wave] = mn;
    red[1][wave] = mx;
  }
  __syncthreads();
  mn = red[0][0];
  mx = red[1][0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) {
    mn = min(mn, red[0][w]);
    mx = max(mx, red[1][w]);
  }
  *omn = mn;
  *omx = mx;
}

// One wave selects in sh.u.hist the bin of the rem-th largest key and records the digit.
template <int NT>
__device__ inline void smp_select_digit(SampleShared<NT>& sh, uint32_t pfx, int wb, int lo, int rem) {
  if ((threadIdx.x >> 6) == 0) {
    int bin, r, cnt;
    wave_select<kSmpBins>(sh.u.hist, rem, &bin, &r, &cnt);
    if ((threadIdx.x & 63) == 0) {
      sh.prefix = wb >= 32 ? uint32_t(bin) : (pfx << wb) | uint32_t(bin);
      sh.remaining = r;
      sh.take_all = r == cnt;
      sh.count = cnt;
      sh.n_small = 0;
      sh.lo = lo;
    }
  }
}

// Exact K-th largest over the n list keys, relative to `base` (every listed key >= base): the
// first digit is the 11 bits below the highest set bit of the largest relative key, the lower
// bits follow in digits of at most 11 bits, stopping once the chosen bin is taken whole.
template <int NT>
__device__ inline void smp_list_select(SampleShared<NT>& sh, int n, int K, uint32_t base) {
  const int tid = threadIdx.x;
  uint32_t mx = 0, mn;
  for (int c = tid; c < n; c += NT) mx = max(mx, sh.key[c] - base);
  smp_minmax<NT>(0u, mx, sh.red, &mn, &mx);
  const int s1 = max(0, 32 - int(__builtin_clz(mx | 1u)) - 11);  // (d >> s1) < 2048
  zero_words<NT>(sh.u.hist, kSmpBins);
  __syncthreads();
  for (int c = tid; c < n; c += NT) atomicAdd(&sh.u.hist[(sh.key[c] - base) >> s1], 1u);
  __syncthreads();
  smp_select_digit(sh, 0u, 32, s1, K);
  __syncthreads();
  if (!sh.take_all && s1 > 0 && sh.count <= 64) {  // uniform
    // The chosen bin holds at most 64 keys: gather them (relative key, position) and let one wave
    // find the rem-th largest exactly; the ties at it are then resolved by position on emission.
    const uint32_t b = sh.prefix;
    uint32_t* small_d = sh.u.hist;
    for (int c = tid; c < n; c += NT) {
      const uint32_t d = sh.key[c] - base;
      if ((d >> s1) == b) small_d[atomicAdd(&sh.n_small, 1)] = d;
    }
    __syncthreads();
    if ((tid >> 6) == 0) {
      const int lane = tid & 63, m = sh.n_small, rem = sh.remaining;
      const uint32_t d = lane < m ? small_d[lane] : 0u;
      int gt = 0, ge = 0;
      for (int j = 0; j < m; ++j) {
        const uint32_t dj = __builtin_amdgcn_readlane(d, j);
        gt += dj > d;
        ge += dj >= d;
      }
      const uint64_t hit = ballot(lane < m && gt < rem && rem <= ge);
      const int l = int(__builtin_ctzll(hit | (1ull << 63)));
      if (lane == l) {
        sh.prefix = d;  // the whole relative key
        sh.remaining = rem - gt;
        sh.lo = 0;
      }
    }
    __syncthreads();
    return;
  }
  int lo = s1;
#pragma unroll 1
  while (!sh.take_all && lo > 0) {  // uniform: read after a barrier
    const int wb = min(11, lo);
    lo -= wb;
    const uint32_t pfx = sh.prefix;
    const int rem = sh.remaining;
    zero_words<NT>(sh.u.hist, kSmpBins);
    __syncthreads();
    for (int c = tid; c < n; c += NT) {
      const uint32_t d = sh.key[c] - base;
      if ((d >> (lo + wb)) == pfx) atomicAdd(&sh.u.hist[(d >> lo) & ((1u << wb) - 1u)], 1u);
    }
    __syncthreads();
    smp_select_digit(sh, pfx, wb, lo, rem);
    __syncthreads();
  }
}

// The selection of the list (after smp_list_select) as ascending ids, through position bitmaps.
template <int NT>
__device__ inline void smp_list_emit(SampleShared<NT>& sh, int n, int ev, int K, uint32_t base, int id_base,
                                     int32_t* __restrict__ orow) {
  const int tid = threadIdx.x;
  const uint32_t pfx = sh.prefix;
  const int lo = sh.lo, need = sh.remaining;
  const int n_chunks = (ev + 63) >> 6;
  uint64_t* gt = sh.u.bits[0];
  uint64_t* eq = sh.u.bits[1];
  for (int c = tid; c < n_chunks; c += NT) gt[c] = eq[c] = 0;  // the select's reads are done
  __syncthreads();
  for (int c = tid; c < n; c += NT) {
    const uint32_t d = (sh.key[c] - base) >> lo;
    const int p = sh.pos[c];
    if (d > pfx) atomicOr(&gt[p >> 6], 1ull << (p & 63));
    else if (d == pfx) atomicOr(&eq[p >> 6], 1ull << (p & 63));
  }
  __syncthreads();
  emit_from_bitmaps<NT>(gt, eq, n_chunks, need, K, id_base, orow, sh.scan);
}

// Exact select over the row in memory (a list that overflowed or fell short): three digits of
// the order keys (11 + 11 + 10 bits), then the bitmaps from one more pass.
template <int NT>
__device__ inline void smp_row_select(const float* __restrict__ srow, int ev, int K, int id_base,
                                      int32_t* __restrict__ orow, SampleShared<NT>& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t pfx = 0;
  int rem = K, lo = 32;
#pragma unroll 1
  for (int dg = 0; dg < 3; ++dg) {
    const int wb = dg < 2 ? 11 : 10;
    lo -= wb;
    zero_words<NT>(sh.u.hist, kSmpBins);
    __syncthreads();
    for (int p = tid; p < ev; p += NT) {
      const uint32_t key = order_key(srow[p]);
      if (dg == 0 || (key >> (lo + wb)) == pfx) atomicAdd(&sh.u.hist[(key >> lo) & ((1u << wb) - 1u)], 1u);
    }
    __syncthreads();
    smp_select_digit(sh, pfx, dg == 0 ? 32 : wb, lo, rem);
    __syncthreads();
    pfx = sh.prefix;
    rem = sh.remaining;
    if (sh.take_all) break;  // uniform
  }
  const int n_chunks = (ev + 63) >> 6;
  uint64_t* gt = sh.u.bits[0];
  uint64_t* eq = sh.u.bits[1];
  for (int c = wave; c < n_chunks; c += NT / 64) {
    const int p = c * 64 + lane;
    const bool valid = p < ev;
    const uint32_t d = valid ? order_key(srow[p]) >> lo : 0u;
    const uint64_t g = ballot(valid && d > pfx), e = ballot(valid && d == pfx);
    if (lane == 0) {
      gt[c] = g;
      eq[c] = e;
    }
  }
  __syncthreads();
  emit_from_bitmaps<NT>(gt, eq, n_chunks, rem, K, id_base, orow, sh.scan);
}

// NT threads per row (256: five rows per CU).
template <int NT>
__global__ __launch_bounds__(NT, NT == 256 ? 5 : 8) void topk_sample_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ used_kv,
    const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ win_kv, int batch, int stride, int ratio, int nk,
    int max_vis, int K, int window, int kv_row_base, int32_t* __restrict__ out, int32_t* __restrict__ err_flag,
    int skip_above) {
  __shared__ SampleShared<NT> sh;
  const int tid = threadIdx.x, lane = tid & 63;
  int32_t* orow = out + int64_t(blockIdx.x) * (K + window);
  RowInfo ri;
  if (!row_setup<NT>(cu_q, used_kv, cu_kv, win_kv, batch, stride, ratio, nk, max_vis, kSmpMaxRow, K, window,
                         kv_row_base, orow, err_flag, &ri, skip_above))
    return;
  const int ev = ri.ev;  // K < ev <= kSmpMaxRow
  const float* srow = scores + int64_t(blockIdx.x) * ld;
  const float4* s4 = reinterpret_cast<const float4*>(srow);  // rows are 16-byte aligned, ld % 4 == 0
  int n;
  uint32_t base;
  if (ev <= kSmpList) {
    // ---- the whole row is the list (position p at slot p) ----
    uint32_t mn = 0xFFFFFFFFu, mx;
    for (int q = tid; 4 * q < ev; q += NT) {
      const float4 x = s4[q];
      const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int p = 4 * q + c;
        if (p < ev) {
          const uint32_t k = order_key(xs[c]);
          sh.key[p] = k;
          sh.pos[p] = uint16_t(p);
          mn = min(mn, k);
        }
      }
    }
    smp_minmax<NT>(mn, 0u, sh.red, &mn, &mx);
    n = ev;
    base = mn;
  } else {
    // ---- sample: kSU float4s per thread; a wave's load covers one 256-key tile ----
    constexpr int kSU = kSmpSample / 4 / NT;
    uint32_t sk[4 * kSU];
#pragma unroll
    for (int u = 0; u < kSU; ++u) {
      const int f = u * NT + tid, t = f >> 6;
      const int start = int(int64_t(t) * (ev - kSmpTile) / (kSmpTiles - 1)) & ~3;
      const float4 x = s4[(start >> 2) + (f & 63)];
      sk[4 * u] = order_key(x.x);
      sk[4 * u + 1] = order_key(x.y);
      sk[4 * u + 2] = order_key(x.z);
      sk[4 * u + 3] = order_key(x.w);
    }
    // theta = the 22-bit order-key prefix of the sample's r-th largest key: digit 1 is bits 31..21
    // (in sh.u.hist), digit 2 bits 20..10 among the sample keys of digit 1's bin (in the list's
    // memory, free until the pass)
    uint32_t* hist2 = sh.key;
    zero_words<NT>(sh.u.hist, kSmpBins);
    zero_words<NT>(hist2, kSmpBins);
    if (tid == 0) sh.n_list = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4 * kSU; ++k) atomicAdd(&sh.u.hist[sk[k] >> 21], 1u);
    __syncthreads();
    // r: smallest rank with r * ev / m - 4 sqrt(r) * ev / m >= K
    const float y = 2.f + sqrtf(4.f + float(K) * float(kSmpSample) / float(ev));
    const int r = min(kSmpSample, int(ceilf(y * y)));
    if ((tid >> 6) == 0) {
      int bin, rem, cnt;
      wave_select<kSmpBins>(sh.u.hist, r, &bin, &rem, &cnt);
      if (lane == 0) {
        sh.prefix = uint32_t(bin);
        sh.remaining = rem;
      }
    }
    __syncthreads();
    const uint32_t b1 = sh.prefix;
    const int r2 = sh.remaining;
#pragma unroll
    for (int k = 0; k < 4 * kSU; ++k)
      if ((sk[k] >> 21) == b1) atomicAdd(&hist2[(sk[k] >> 10) & (kSmpBins - 1)], 1u);
    __syncthreads();
    if ((tid >> 6) == 0) {
      int bin, rem, cnt;
      wave_select<kSmpBins>(hist2, r2, &bin, &rem, &cnt);
      if (lane == 0) sh.prefix = (b1 << 21) | (uint32_t(bin) << 10);
    }
    __syncthreads();
    base = sh.prefix;  // theta as an order key
    // ---- one pass: list every key >= theta (raw float bits and position). The kernels keep f32
    // denormals (the compiler's default for this library), so the IEEE compare x >= theta orders
    // every finite score exactly as the order keys do (-0 == +0 in both). ----
    const float theta = key_to_float(base);
    const int n4 = (ev + 3) >> 2;
    constexpr int kSmpU = kSmpInFlight / NT;  // float4 loads in flight per thread (a multiple of 4)
    static_assert(kSmpU % 4 == 0, "groups of 4 float4s");
    // one step of NT * kSmpU float4s from v0; FULL: every position of the step is inside the row
    auto step = [&](auto full_tag, int v0) {
      constexpr bool FULL = decltype(full_tag)::value;
      float4 x[kSmpU];
#pragma unroll
      for (int u = 0; u < kSmpU; ++u) {
        const int q = v0 + u * NT + tid;
        x[u] = (FULL || q < n4) ? s4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      // hits are placed in groups of 4 float4s (16 ballots, one LDS slot reservation per group)
#pragma unroll
      for (int g = 0; g < kSmpU; g += 4) {
        uint64_t m[4][4];
        int total = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float xc = c == 0 ? x[g + u].x : c == 1 ? x[g + u].y : c == 2 ? x[g + u].z : x[g + u].w;
            const bool in = FULL || 4 * (v0 + (g + u) * NT + tid) + c < ev;
            m[u][c] = ballot(in && xc >= theta);
            total += __popcll(m[u][c]);
          }
        if (total == 0) continue;  // uniform per wave
        int slot = 0;
        if (lane == 0) slot = atomicAdd(&sh.n_list, total);
        slot = __builtin_amdgcn_readfirstlane(slot);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int sl = slot + lanes_below(m[u][c]);
            if (((m[u][c] >> lane) & 1ull) && sl < kSmpList) {
              const float xc = c == 0 ? x[g + u].x : c == 1 ? x[g + u].y : c == 2 ? x[g + u].z : x[g + u].w;
              sh.key[sl] = __float_as_uint(xc);
              sh.pos[sl] = uint16_t(4 * (v0 + (g + u) * NT + tid) + c);
            }
            slot += __popcll(m[u][c]);
          }
      }
    };
    int v0 = 0;
#pragma unroll 1
    for (; 4 * (v0 + NT * kSmpU) <= ev; v0 += NT * kSmpU) step(std::true_type{}, v0);
    if (v0 < n4) step(std::false_type{}, v0);
    __syncthreads();
    // raw bits -> order keys, once per listed key
    const int nl = min(sh.n_list, kSmpList);
    for (int c = tid; c < nl; c += NT) sh.key[c] = order_key_bits(sh.key[c]);
    __syncthreads();
    n = sh.n_list;
  }
  if (n >= K && n <= kSmpList) {  // uniform
    smp_list_select(sh, n, K, base);
    smp_list_emit(sh, n, ev, K, base, ri.base, orow);
  } else {
    __syncthreads();
    smp_row_select(srow, ev, K, ri.base, orow, sh);
  }
}

// ---------------------------------------------------------------------------------------------
// Rows selected from candidate lists (no score row in memory)
// ---------------------------------------------------------------------------------------------
constexpr int kThetaBins = 2048;                       // 11-bit digits of the sample select
constexpr int kSampleTiles = 16;                       // sampled 128-key tiles per row
constexpr int kSampleKeys = kSampleTiles * 128;        // 2048 sample scores per row
constexpr int kCandNT = 1024;
constexpr int kCandEPT = kFuseCap / kCandNT;           // 16 list entries per thread

// Threshold of each candidate row (one wave per row, 8 rows per workgroup): the scores of 16
// tiles of 128 consecutive keys spread evenly over the row, and theta = the 22-bit key prefix of
// the sample's r-th largest score. With m = 2048 sampled of ev keys, the keys reaching the r-th
// sample number about r * ev / m with a spread of about sqrt(r) * ev / m; r is the smallest
// rank whose count stays 5.5 spreads above K, so a list falls short of K very rarely (those rows
// are recomputed) while holding about K + 5.5 sqrt(K ev / m) ev / m entries. When the 8 rows of
// the workgroup are candidate rows of one request they share the sample positions (those of the
// shortest row) and each tile is staged once in LDS; otherwise each wave reads its own keys.
// Shared fp8 samples are scored with the indexer's arithmetic (|x| head sums, the linear part on
// the matrix cores for the 8 rows at once), so they are the indexer's floats; the per-wave path
// keeps the ReLU form. Also zeroes every row's list-segment counts.
template <bool FP8>
__global__ __launch_bounds__(512, FP8 ? 4 : 1) void topk_theta_kernel(
    const unsigned char* __restrict__ qi, const float* __restrict__ q_scale, const float* __restrict__ w,
    const unsigned char* __restrict__ ki, const float* __restrict__ k_scale, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ used_kv, const int32_t* __restrict__ cu_kv, int batch, int stride, int ratio, int nq,
    int nk, int max_vis, int K, int fuse_above, uint32_t* __restrict__ theta, int32_t* __restrict__ n_cand,
    int segs) {
  constexpr int kBytes = IdxOps<FP8>::kKeyBytes, kChunks = kBytes / 16;
  constexpr int kTileBytes = 128 * kBytes;                           // 16 KB (fp8) or 32 KB (bf16)
  constexpr int kBufs = int(sizeof(uint32_t)) * 8 * kThetaBins / kTileBytes;  // 4 or 2
  constexpr int kLoads = kTileBytes / (512 * 16);                   // direct loads per thread per tile
  constexpr int kInFlight = kLoads + (FP8 ? 1 : 0);                  // per wave per tile (+ the scales)
  static_assert(kBufs >= 2 && kBufs - 2 <= 2, "one to three tiles ahead");
  // The sample tiles of the shared path live in the histogram's memory: the histograms are used
  // only after the last tile.
  __shared__ union {
    alignas(16) uint32_t hist[8][kThetaBins];
    alignas(16) unsigned char tiles[kBufs][kTileBytes];
  } u;
  __shared__ alignas(16) float ks_tiles[kBufs][FP8 ? 128 : 4];
  // fp8 shared path: the group's split c rows (row 8j + 4h + p: part p of row 2j + h) and each
  // tile's linear parts c . k times k_scale, [row][key of the tile] (pitch: the two lane halves
  // write rows 2j and 2j + 1 at once, 32 banks apart)
  constexpr int kLinPitch = 128 + 32;
  __shared__ alignas(16) unsigned char lin_rows[FP8 ? 32 * kIdxDim : 16];
  __shared__ alignas(16) float lin_v[FP8 ? 8 * kLinPitch : 4];
  __shared__ int s_kv0[8], s_ev[8], s_e0[8];
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = blockIdx.x * 8 + wave;
  bool cand = false;
  int kv0 = 0, ev = 0;
  if (i < nq) {
    for (int y = lane; y < segs; y += 64) n_cand[int64_t(i) * segs + y] = 0;
    QueryView v;
    if (query_view(cu_q, used_kv, cu_kv, batch, stride, i, &v)) {
      ev = ratio > 1 ? v.E / ratio : v.E;
      kv0 = v.kv0;
      cand = v.E >= 1 && ev > fuse_above && ev <= max_vis && v.kv0 >= 0 && int64_t(v.kv0) + ev <= nk;
    }
  }
  if (lane == 0) {
    s_kv0[wave] = cand ? kv0 : -1;
    s_ev[wave] = cand ? ev : 0;
  }
  __syncthreads();
  bool shared = true;
  int ev_s = INT32_MAX;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    shared = shared && s_kv0[k] >= 0 && s_kv0[k] == s_kv0[0];
    ev_s = min(ev_s, s_ev[k]);
  }
  if (!shared) {
    if (!cand) return;  // no workgroup barrier on this path
    ev_s = ev;
  }

  typename IdxOps<FP8>::AOp qa[2][IdxOps<FP8>::kKsteps];
  float wv[2][16];
  load_query_operands<FP8>(qi, w, q_scale, i, qa, wv);
  // fp8 shared path: the indexer's arithmetic (score = sum_h w'' |x_h| + c . k, w'' = w q_scale / 2,
  // the linear part on the matrix cores for the group's 8 rows), so the sample scores are the
  // indexer's own floats; the per-wave path keeps the ReLU form (it only places theta)
  if (FP8 && shared) {  // uniform
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) wv[m][r] *= 0.5f;
    uint32_t part[kLinParts];
    const int e0 = lin_split(qi, wv, i, part);
    if (half == 0) {
#pragma unroll
      for (int p = 0; p < kLinParts; ++p)
        lin_row_store(lin_rows, 8 * (wave >> 1) + 4 * (wave & 1) + p, l32, part[p]);
    }
    if (lane == 0) s_e0[wave] = e0;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // visible to the group after the first tile barrier
  }
  // Wait here, visibly to the compiler, for the query operands (and the segment-count stores):
  // the tiles below arrive by direct loads the compiler does not see, and a wait it placed at
  // the first use of the operands would also drain them. vmcnt(0), other counters untouched.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  auto tile_start = [&](int tl) { return int(int64_t(tl) * (ev_s - 128) / (kSampleTiles - 1)); };
  // Shared path: tile tl goes to buffer tl % kBufs by direct global->LDS loads (the swizzled
  // layout of key_operand_lds: slot (n, c) holds chunk kswz(n, c)), its key scales beside it
  // (16 per wave).
  // Addresses are a wave-uniform base plus a 32-bit lane offset recomputed from an opaque copy of
  // the lane id, so that no per-lane address stays live across the tile loop (a spilled one,
  // reloaded after tiles were issued, would wait for those tiles too: the wait counts loads in
  // issue order).
  auto issue_tile = [&](int tl) {
    const int b = tl % kBufs, start = tile_start(tl);
    const unsigned char* gbase = ki + int64_t(kv0 + start) * kBytes;
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int f0 = 64 * (kLoads * wave + j);  // this wave's 64 consecutive 16-byte slots
      const int f = f0 + ln;
      const int n = f / kChunks, c = kswz<kChunks>(n, f - n * kChunks);
      lds_dma16_s(uniform_ptr(gbase), uint32_t(n * kBytes + c * 16), lds_offset(u.tiles[b] + f0 * 16));
    }
    if constexpr (FP8) {
      if (ln < 16) lds_dma4_s(k_scale + kv0 + start + 16 * wave, uint32_t(4 * ln), lds_offset(ks_tiles[b] + 16 * wave));
    }
  };
  if (shared) {
#pragma unroll
    for (int tl = 0; tl < kBufs - 1; ++tl) issue_tile(tl);
  }
  // block b = 4 * tile + sub covers positions start(tile) + 32 sub + [0, 32); lanes of half h keep
  // the keys of block 2p + h
  uint32_t sk[kSampleKeys / 64];
#pragma unroll 1
  for (int tl = 0; tl < kSampleTiles; ++tl) {
    const int start = tile_start(tl);
    const int b = tl % kBufs;
    if (shared) {
      // tile tl has landed for every wave (the tiles issued after it may stay in flight) and
      // every wave is done with tile tl - 1, whose buffer takes tile tl + kBufs - 1
      const int ahead = min(kSampleTiles - 1, tl + kBufs - 2) - tl;  // uniform, 0 .. kBufs - 2
      static_assert(FP8 ? (kInFlight == 3 && kBufs == 4) : kBufs == 2, "the wait counts below are literals");
      if (ahead >= 2) DSA_TILE_BARRIER_VMCNT(6);
      else if (ahead == 1) DSA_TILE_BARRIER_VMCNT(3);
      else DSA_TILE_BARRIER_VMCNT(0);
      if (tl + kBufs - 1 < kSampleTiles) issue_tile(tl + kBufs - 1);
    }
    if constexpr (FP8) {
      if (shared) {
        // lane-derived LDS addresses come from an opaque copy of the lane id, recomputed every
        // tile: kept live they are spilled, and a reload would wait for the tiles in flight too
        int ol = lane;
        asm volatile("" : "+v"(ol));
        const int o32 = ol & 31, ohalf = ol >> 5;
        // waves 0..3: c . k of block `wave` of the tile for the group's 8 rows (lane half h: rows
        // 2j + h in output rows 8j + 4h + p), times k_scale, published for every wave
        if (wave < 4) {
          const int n = 32 * wave + o32;
          f32x16 L = f32x16{};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            L = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(lin_a_operand(lin_rows, o32, ks, ohalf),
                                                                key_operand_lds<true>(u.tiles[b], n, ks, ohalf), L, 0,
                                                                0, 0, 127, 0, 127);
          const float ksn = ks_tiles[b][n];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int q = 2 * j + ohalf;
            lin_v[q * kLinPitch + n] = lin_combine(L, 4 * j, s_e0[q], ksn);
          }
        }
        DSA_TILE_BARRIER_LDS();
        // blocks 2pp and 2pp + 1: pair_sum leaves block 2pp's head sum in half 0 and block
        // 2pp + 1's in half 1, each lane with the key it keeps
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          float part[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int n = 32 * (2 * pp + h) + o32;
            f32x16 a0, a1;
            block_mfma_chains<true>(qa, [&](int ks) { return key_operand_lds<true>(u.tiles[b], n, ks, ohalf); }, a0,
                                    a1);
            part[h] = block_abs_part(wv, a0, a1);
          }
          const int n = 32 * (2 * pp + ohalf) + o32;
          const float x = fmaf(pair_sum(part[0], part[1]), ks_tiles[b][n], lin_v[wave * kLinPitch + n]);
          sk[2 * tl + pp] = order_key(x + 0.f);
        }
        continue;
      }
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      float sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = 32 * (2 * pp + h) + l32;  // row in the tile
        const int row = kv0 + start + n;
        f32x16 a0, a1;
        float x;
        if (shared) {
          block_mfma_chains<FP8>(qa, [&](int ks) { return key_operand_lds<FP8>(u.tiles[b], n, ks); }, a0, a1);
          x = block_head_sum(wv, a0, a1);
          if constexpr (FP8) x *= ks_tiles[b][n];
        } else {
          block_mfma_chains<FP8>(qa, [&](int ks) { return key_operand_global<FP8>(ki, row, ks); }, a0, a1);
          x = block_head_sum(wv, a0, a1);
          if constexpr (FP8) x *= k_scale[row];
        }
        sc[h] = x + 0.f;
      }
      sk[2 * tl + pp] = order_key(half ? sc[1] : sc[0]);
    }
  }
  if (shared) __syncthreads();  // every wave is done with the tiles before the histograms take their memory
  if (!cand) return;  // shared path: every wave is a candidate row; kept for clarity

  // r: smallest rank with r * ev / m - 5.5 sqrt(r) * ev / m >= K
  const double km = double(K) * kSampleKeys / ev;
  const double sr = 2.75 + sqrt(2.75 * 2.75 + km);
  const int r_s = int(min(double(kSampleKeys), ceil(sr * sr)));
  uint32_t* h = u.hist[wave];
  int bin1, bin2, rem, cnt;
  for (int b = 4 * lane; b < kThetaBins; b += 256) *reinterpret_cast<uint4*>(h + b) = uint4{0, 0, 0, 0};
  lds_wait();
#pragma unroll
  for (int p = 0; p < kSampleKeys / 64; ++p) atomicAdd(&h[sk[p] >> 21], 1u);
  lds_wait();
  wave_select<kThetaBins>(h, r_s, &bin1, &rem, &cnt);
  lds_wait();
  for (int b = 4 * lane; b < kThetaBins; b += 256) *reinterpret_cast<uint4*>(h + b) = uint4{0, 0, 0, 0};
  lds_wait();
#pragma unroll
  for (int p = 0; p < kSampleKeys / 64; ++p)
    if (int(sk[p] >> 21) == bin1) atomicAdd(&h[(sk[p] >> 10) & (kThetaBins - 1)], 1u);
  lds_wait();
  wave_select<kThetaBins>(h, rem, &bin2, &rem, &cnt);
  if (lane == 0) theta[i] = (uint32_t(bin1) << 21) | (uint32_t(bin2) << 10);
}

struct CandShared {
  union {
    alignas(16) uint32_t hist[kBins0];
    uint64_t bits[2][kMaxRow / 64];  // keys above tau / equal to tau, one bit per position
  } u;
  alignas(16) uint32_t hist_r[kBinsR];
  int scan[2 * (kCandNT / 64 + 1)];
  int seg_n[64];  // list-segment counts
  uint32_t prefix;
  int remaining, count, n_small;
};

// Exact top-K of a candidate row from its list (every key >= theta, with its position). The
// list keys are taken relative to theta, d = key - theta: the first digit is the 12 bits of d
// below its highest set bit across the list, so even a list packed into a few float exponents
// spreads over the 4096-bin histogram; the lower bits follow in digits of at most 10 bits. The
// ids are then emitted from position bitmaps. A row whose list holds fewer than K entries or
// overflowed is left to topk_refill_kernel.
__global__ __launch_bounds__(kCandNT, 2) void topk_cand_kernel(
    const uint2* __restrict__ cand, const int32_t* __restrict__ n_cand, int32_t* __restrict__ status,
    const uint32_t* __restrict__ theta, int cap, int segs, int fuse_above, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ used_kv,
    const int32_t* __restrict__ cu_kv, const int32_t* __restrict__ win_kv, int batch, int stride, int ratio, int nk,
    int max_vis, int K, int window, int kv_row_base, int32_t* __restrict__ out, int32_t* __restrict__ err_flag) {
  constexpr int NT = kCandNT, NW = NT / 64;
  __shared__ CandShared sh;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  QueryView v;
  const bool have = query_view(cu_q, used_kv, cu_kv, batch, stride, row, &v);
  const int ev = have ? (ratio > 1 ? v.E / ratio : v.E) : 0;
  // not a candidate row (rows outside the key buffer are flagged and cleared by topk_reg_kernel)
  if (!have || v.E < 1 || ev <= fuse_above || ev > max_vis || v.kv0 < 0 || int64_t(v.kv0) + ev > nk) return;
  int32_t* orow = out + int64_t(row) * (K + window);
  RowInfo ri;
  if (!row_setup<NT>(cu_q, used_kv, cu_kv, win_kv, batch, stride, ratio, nk, max_vis, kMaxRow, K, window,
                     kv_row_base, orow, err_flag, &ri))
    return;
  // the list: segment y holds its first min(count_y, seg_cap) slots; a segment that overflowed
  // or a list shorter than K sends the row to the recompute
  const int seg_cap = cap / segs;
  if (tid < segs) sh.seg_n[tid] = n_cand[int64_t(row) * segs + tid];
  __syncthreads();
  int n = 0;
  bool usable = true;
  for (int y = 0; y < segs; ++y) {
    n += sh.seg_n[y];
    usable = usable && sh.seg_n[y] <= seg_cap;
  }
  usable = usable && n >= K;
  if (tid == 0) status[row] = usable ? 1 : 0;
  if (!usable) return;

  const uint2* crow = cand + int64_t(row) * cap;
  const uint32_t th = theta[row];
  uint32_t d[kCandEPT];
  int pos[kCandEPT];
  uint32_t mx = 0;
#pragma unroll
  for (int j = 0; j < kCandEPT; ++j) {
    const int c = j * NT + tid, y = c / seg_cap;
    const bool valid = y < segs && c - y * seg_cap < sh.seg_n[min(y, segs - 1)];
    const uint2 e = valid ? crow[c] : uint2{0u, 0u};
    pos[j] = valid && DSA_CHECK(e.y < uint32_t(ev), err_flag) ? int(e.y) : -1;  // list positions index the bitmaps
    d[j] = valid ? order_key_bits(e.x) - th : 0u;
    mx = max(mx, d[j]);
  }
  // highest set bit of d over the list -> shift of the first digit
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = max(mx, uint32_t(__shfl_xor(int(mx), o, 64)));
  if (lane == 0) sh.scan[wave] = int(mx);
  zero_words<NT>(sh.u.hist, kBins0);
  __syncthreads();
  uint32_t mall = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) mall = max(mall, uint32_t(sh.scan[k]));
  const int s1 = max(0, 32 - int(__builtin_clz(mall | 1u)) - 12);  // d >> s1 < 4096
#pragma unroll
  for (int j = 0; j < kCandEPT; ++j)
    if (pos[j] >= 0) atomicAdd(&sh.u.hist[d[j] >> s1], 1u);
  __syncthreads();
  if (wave == 0) {
    int bin, rem, cnt;
    wave_select<kBins0>(sh.u.hist, K, &bin, &rem, &cnt);
    if (lane == 0) {
      sh.prefix = uint32_t(bin);
      sh.remaining = rem;
      sh.count = cnt;
      sh.n_small = 0;
    }
  }
  __syncthreads();
  // lower digits: bits [lo, lo + wb) among the keys whose bits above match the prefix
  int lo = s1;
  if (s1 > 0 && sh.count <= 64) {  // uniform
    // The chosen bin holds at most 64 keys: gather their relative keys and let one wave find the
    // rem-th largest exactly (its ties are then taken by position on emission).
    const uint32_t pfx = sh.prefix;
    uint32_t* small_d = sh.hist_r;
#pragma unroll
    for (int j = 0; j < kCandEPT; ++j)
      if (pos[j] >= 0 && (d[j] >> s1) == pfx) small_d[atomicAdd(&sh.n_small, 1)] = d[j];
    __syncthreads();
    if (wave == 0) {
      const int m = sh.n_small, rem = sh.remaining;
      const uint32_t dl = lane < m ? small_d[lane] : 0u;
      int n_gt = 0, n_ge = 0;
      for (int j = 0; j < m; ++j) {
        const uint32_t dj = __builtin_amdgcn_readlane(dl, j);
        n_gt += dj > dl;
        n_ge += dj >= dl;
      }
      const uint64_t hit = ballot(lane < m && n_gt < rem && rem <= n_ge);
      const int l = int(__builtin_ctzll(hit | (1ull << 63)));
      if (lane == l) {
        sh.prefix = dl;  // the whole relative key
        sh.remaining = rem - n_gt;
      }
    }
    lo = 0;
  }
#pragma unroll 1
  while (lo > 0) {
    const int wb = min(10, lo);
    lo -= wb;
    zero_words<NT>(sh.hist_r, kBinsR);
    __syncthreads();
    const uint32_t pfx = sh.prefix;
#pragma unroll
    for (int j = 0; j < kCandEPT; ++j)
      if (pos[j] >= 0 && (d[j] >> (lo + wb)) == pfx) atomicAdd(&sh.hist_r[(d[j] >> lo) & ((1u << wb) - 1u)], 1u);
    __syncthreads();
    if (wave == 0) {
      int bin, rem, cnt;
      wave_select<kBinsR>(sh.hist_r, sh.remaining, &bin, &rem, &cnt);
      if (lane == 0) {
        sh.prefix = (pfx << wb) | uint32_t(bin);
        sh.remaining = rem;
      }
    }
    __syncthreads();  // the select has read hist_r before the next digit clears it
  }
  __syncthreads();
  const uint32_t tau = sh.prefix;  // relative to theta
  const int need = sh.remaining;
  const int n_chunks = (ev + 63) >> 6;
  uint64_t* gt = sh.u.bits[0];
  uint64_t* eq = sh.u.bits[1];
  for (int c = tid; c < n_chunks; c += NT) gt[c] = eq[c] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kCandEPT; ++j) {
    if (pos[j] < 0) continue;
    if (d[j] > tau) atomicOr(&gt[pos[j] >> 6], 1ull << (pos[j] & 63));
    else if (d[j] == tau) atomicOr(&eq[pos[j] >> 6], 1ull << (pos[j] & 63));
  }
  __syncthreads();
  emit_from_bitmaps<NT>(gt, eq, n_chunks, need, K, ri.base, orow, sh.scan);
}

// Candidate rows whose list was unusable (status 0): a persistent workgroup recomputes
// each such row's scores (the same arithmetic as the indexer) into its own scratch row and
// selects from it like topk_stream_kernel. Rows whose list was usable are skipped.
template <bool FP8>
__global__ __launch_bounds__(kStreamNT, 1) void topk_refill_kernel(
    const unsigned char* __restrict__ qi, const float* __restrict__ q_scale, const float* __restrict__ w,
    const unsigned char* __restrict__ ki, const float* __restrict__ k_scale, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ used_kv, const int32_t* __restrict__ cu_kv, int batch, int stride, int ratio, int nq,
    int nk, int max_vis, int K, int window, int kv_row_base, int fuse_above, const int32_t* __restrict__ status,
    float* __restrict__ scratch, int64_t sld, int32_t* __restrict__ out) {
  __shared__ StreamShared sh;
  // fp8: each wave's copy of the row's split c (kLinParts rows of 128 bytes)
  __shared__ __attribute__((aligned(16))) unsigned char lin_rows[FP8 ? kStreamNT / 64 : 1][FP8 ? kLinParts * kIdxDim : 16];
  // this workgroup's rows (blockIdx.x + k gridDim.x) that need a recompute, found kStreamNT at a
  // time with one status read per thread rather than one dependent read per row
  __shared__ int todo[kStreamNT];
  __shared__ int n_todo;
  const int lane = threadIdx.x & 63, l32 = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float* srow = scratch + int64_t(blockIdx.x) * sld;
  auto candidate = [&](int row, QueryView* v) {
    if (!query_view(cu_q, used_kv, cu_kv, batch, stride, row, v)) return false;
    const int ev = ratio > 1 ? v->E / ratio : v->E;
    return v->E >= 1 && ev > fuse_above && ev <= max_vis && v->kv0 >= 0 && int64_t(v->kv0) + ev <= nk;
  };
#pragma unroll 1
  for (int64_t base = blockIdx.x; base < nq; base += int64_t(gridDim.x) * kStreamNT) {
    if (threadIdx.x == 0) n_todo = 0;
    __syncthreads();
    const int64_t mine = base + int64_t(threadIdx.x) * gridDim.x;
    QueryView vm;
    if (mine < nq && candidate(int(mine), &vm) && status[mine] == 0) todo[atomicAdd(&n_todo, 1)] = int(mine);
    __syncthreads();
    const int n_rows = n_todo;
#pragma unroll 1
    for (int k = 0; k < n_rows; ++k) {
      const int row = __builtin_amdgcn_readfirstlane(todo[k]);
      QueryView v;
      candidate(row, &v);
      const int ev = ratio > 1 ? v.E / ratio : v.E;
      typename IdxOps<FP8>::AOp qa[2][IdxOps<FP8>::kKsteps];
      float wv[2][16];
      load_query_operands<FP8>(qi, w, q_scale, row, qa, wv);
      int e0 = 0;
      if constexpr (FP8) {
        // the indexer's fp8 arithmetic: halved weights and the row's split c (every wave its own copy)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) wv[m][r] *= 0.5f;
        uint32_t part[kLinParts];
        e0 = lin_split(qi, wv, row, part);
        if (half == 0) {
#pragma unroll
          for (int p = 0; p < kLinParts; ++p) lin_row_store(lin_rows[wave], p, l32, part[p]);
        }
      }
#pragma unroll 1
      for (int b = wave; 32 * b < ev; b += kStreamNT / 64) {
        const int p = 32 * b + l32;
        const float sc =
            key_score_global<FP8>(qa, wv, lin_rows[FP8 ? wave : 0], e0, ki, k_scale, v.kv0 + min(p, ev - 1));
        if (half == 0 && p < ev) srow[p] = sc;
      }
      __syncthreads();  // the row's scores are visible to the workgroup
      stream_select(srow, sld, ev, K, kv_row_base + v.kv0, out + int64_t(row) * (K + window), sh);
      __syncthreads();  // before the next row overwrites the scratch row and the shared state
    }
    __syncthreads();  // every thread has read n_todo and todo before the next batch resets them
  }
}

}  // namespace

dsa_status launch_topk(const dsa_indexer_topk_args* a, const float* scores, int64_t ld, int max_vis,
                       hipStream_t stream) {
  if (a->nq == 0) return DSA_OK;
  if (max_vis > kMaxRow) return fail(DSA_ERR_UNSUPPORTED, "topk: rows longer than 131072 keys");
  const dim3 grid(a->nq);
#define DSA_TOPK_ARGS                                                                                          \
  scores, ld, a->cu_seqlens_q, a->seqused_kv, a->cu_seqlens_kv, a->window_kv_start, a->batch, a->q_stride,     \
      a->compress_ratio, a->nk, max_vis, a->topk, a->window, a->kv_row_base, a->topk_idx, a->err_flag, INT32_MAX
#define DSA_TOPK_REG(NT, E) hipLaunchKernelGGL((topk_reg_kernel<NT, E>), grid, dim3(NT), 0, stream, DSA_TOPK_ARGS)
  // Rows of up to 4096 keys stay in registers (256 threads, many rows per CU). Launches that fill
  // the GPU about once (at most four rows per CU) are bound by one row's latency: rows of up to
  // 32768 keys stay in registers too, 512 or 1024 threads each. More rows of up to 32768 keys take
  // the sampled kernel, five per CU; longer rows are streamed.
  const bool few = a->nq <= 1024 || max_vis <= 256 * 16;
  tap_launch(max_vis > kSmpMaxRow ? "topk_stream_kernel" : few ? "topk_reg_kernel" : "topk_sample_kernel", stream);
  if (max_vis > kSmpMaxRow) hipLaunchKernelGGL(topk_stream_kernel, grid, dim3(kStreamNT), 0, stream, DSA_TOPK_ARGS);
  else if (!few) hipLaunchKernelGGL(topk_sample_kernel<256>, grid, dim3(256), 0, stream, DSA_TOPK_ARGS);
  else if (max_vis <= 256 * 16) DSA_TOPK_REG(256, 16);
  else if (max_vis <= 512 * 16) DSA_TOPK_REG(512, 16);
  else if (max_vis <= 1024 * 16) DSA_TOPK_REG(1024, 16);
  else DSA_TOPK_REG(1024, 32);
#undef DSA_TOPK_REG
#undef DSA_TOPK_ARGS
  return check_launch("topk_kernel");
}

// Candidate-list selection: thresholds (before the indexer), then, after it, the score rows of
// short rows, the lists of candidate rows and the refill of rows whose list was unusable.
dsa_status launch_topk_theta(const dsa_indexer_topk_args* a, int max_vis, const CandidateMode& cm,
                             hipStream_t stream) {
  if (a->nq == 0) return DSA_OK;
  const dim3 grid((a->nq + 7) / 8);
#define DSA_THETA_ARGS                                                                                        \
  static_cast<const unsigned char*>(a->q_idx), a->q_scale, a->weights, static_cast<const unsigned char*>(a->k_idx), \
      a->k_scale, a->cu_seqlens_q, a->seqused_kv, a->cu_seqlens_kv, a->batch, a->q_stride, a->compress_ratio, a->nq, \
      a->nk, max_vis, a->topk, cm.fuse_above, cm.theta, cm.n_cand, cm.segs
  tap_launch("topk_theta_kernel", stream);
  if (a->dtype == DSA_FP8_E4M3) hipLaunchKernelGGL(topk_theta_kernel<true>, grid, dim3(512), 0, stream, DSA_THETA_ARGS);
  else hipLaunchKernelGGL(topk_theta_kernel<false>, grid, dim3(512), 0, stream, DSA_THETA_ARGS);
#undef DSA_THETA_ARGS
  return check_launch("topk_theta_kernel");
}

dsa_status launch_topk_candidates(const dsa_indexer_topk_args* a, const float* score_rows, int64_t ld, int max_vis,
                                  const CandidateMode& cm, float* scratch, int64_t sld, int n_scratch,
                                  hipStream_t stream) {
  if (a->nq == 0) return DSA_OK;
  if (max_vis > kMaxRow) return fail(DSA_ERR_UNSUPPORTED, "topk: rows longer than 131072 keys");
  const dim3 grid(a->nq);
  tap_launch("topk_reg_kernel", stream);
  hipLaunchKernelGGL((topk_reg_kernel<1024, 32>), grid, dim3(1024), 0, stream, score_rows, ld, a->cu_seqlens_q,
                     a->seqused_kv, a->cu_seqlens_kv, a->window_kv_start, a->batch, a->q_stride, a->compress_ratio,
                     a->nk, max_vis, a->topk, a->window, a->kv_row_base, a->topk_idx, a->err_flag, cm.fuse_above);
  dsa_status st = check_launch("topk_reg_kernel");
  if (st != DSA_OK) return st;
  tap_launch("topk_cand_kernel", stream);
  hipLaunchKernelGGL(topk_cand_kernel, grid, dim3(kCandNT), 0, stream, cm.cand, cm.n_cand, cm.status, cm.theta,
                     cm.cap, cm.segs, cm.fuse_above,
                     a->cu_seqlens_q, a->seqused_kv, a->cu_seqlens_kv, a->window_kv_start, a->batch, a->q_stride,
                     a->compress_ratio, a->nk, max_vis, a->topk, a->window, a->kv_row_base, a->topk_idx, a->err_flag);
  st = check_launch("topk_cand_kernel");
  if (st != DSA_OK) return st;
#define DSA_REFILL_ARGS                                                                                       \
  static_cast<const unsigned char*>(a->q_idx), a->q_scale, a->weights, static_cast<const unsigned char*>(a->k_idx), \
      a->k_scale, a->cu_seqlens_q, a->seqused_kv, a->cu_seqlens_kv, a->batch, a->q_stride, a->compress_ratio, a->nq, \
      a->nk, max_vis, a->topk, a->window, a->kv_row_base, cm.fuse_above, cm.status, scratch, sld, a->topk_idx
  const dim3 rgrid(n_scratch);
  tap_launch("topk_refill_kernel", stream);
  if (a->dtype == DSA_FP8_E4M3) hipLaunchKernelGGL(topk_refill_kernel<true>, rgrid, dim3(kStreamNT), 0, stream, DSA_REFILL_ARGS);
  else hipLaunchKernelGGL(topk_refill_kernel<false>, rgrid, dim3(kStreamNT), 0, stream, DSA_REFILL_ARGS);
#undef DSA_REFILL_ARGS
  return check_launch("topk_refill_kernel");
}

}  // namespace dsa
