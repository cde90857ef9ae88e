// (2) Lightning-indexer scores on gfx950.
//
// [xLLM-CP] "feat: DeepSeek-V4 DSA context-parallel on NPU", Design, data-flow step (3) and
// Implementation §4: the indexer's query, weights and top-k use the rank's local rows and
// local cu-seqlens, while the index keys cover the full token stream.
//
//   score(i, s) = sum_h w[i,h] * max(0, q_hat[i,h,:] . k_hat[kv0(i) + s, :]),   s < Ev(i)
//
// Kernels:
//  * indexer_mfma<bf16|fp8>: 64 heads x 128. A workgroup of 8 waves owns 8 consecutive local
//    queries (one per wave, whose 64 x 128 query block stays in VGPRs as the MFMA A operand)
//    and sweeps 256-key tiles of key chunks (grid.y; at least 4096 keys, longer for long
//    batches) of the union of their causal key ranges, so even short query batches fill the GPU;
//    tiles are staged in LDS with direct global->LDS loads (double buffered) and shared by the 8
//    waves. Each wave computes the logits of 32-key blocks on 32x32 MFMAs (bf16 32x32x16, or fp8
//    32x32x64), then applies ReLU, the head weight and the head sum in fp32: the 32x32
//    accumulator layout puts one key per lane and 16 heads per lane, so a lane's half of the head
//    sum is 32 in-lane FMAs, and one lane swap between the halves finishes two blocks at once.
//    Tiles outside a wave's range are skipped by that wave.
//    fp8: q_scale folds into the head weight and k_scale multiplies the head sum (both > 0);
//    the tile's k_scale values are staged into LDS by the same direct loads as the keys, and the
//    ReLU goes through (x + |x|) / 2 with the linear part on the matrix cores (index_score.h).
//    Candidate mode (rows longer than the fused-selection bound): instead of writing a score
//    row, a wave keeps only the scores at or above its row's threshold theta (a 32-bit order
//    key, see topk.hip) and appends them, with their positions, to its own segment of the row's
//    candidate list (one segment per grid.y slice, so no two workgroups share one and no atomics
//    are needed). The top-k then selects from the segments: no full score row is written.
//  * indexer_generic: float32 / bf16, small shapes (VALU, one thread per (query, key)).
#include <algorithm>

#include "index_score.h"

namespace dsa {
namespace {

// ---------------------------------------------------------------------------------------------
// Generic VALU kernel
// ---------------------------------------------------------------------------------------------
constexpr int kGenThreads = 256;

template <typename T> __device__ inline float ld_elt(const T* p, int64_t i);
template <> __device__ inline float ld_elt<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ inline float ld_elt<uint16_t>(const uint16_t* p, int64_t i) { return bf16_bits_to_float(p[i]); }
// elements i .. i + 3 (i a multiple of 4, the buffer 16-byte aligned) in one load
template <typename T> __device__ inline float4 ld_elt4(const T* p, int64_t i);
template <> __device__ inline float4 ld_elt4<float>(const float* p, int64_t i) {
  return *reinterpret_cast<const float4*>(p + i);
}
template <> __device__ inline float4 ld_elt4<uint16_t>(const uint16_t* p, int64_t i) {
  const uint2 u = *reinterpret_cast<const uint2*>(p + i);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xFFFF0000u));
}

// KD > 0: key rows of D <= KD elements (D a multiple of 4) are read once into registers; otherwise
// every head reads the row from memory again. Same arithmetic, in the same order, either way.
template <typename T, int KD>
__global__ __launch_bounds__(kGenThreads) void indexer_generic(
    const T* __restrict__ qi, const float* __restrict__ w, const T* __restrict__ ki, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ used_kv, const int32_t* __restrict__ cu_kv, int batch, int stride, int ratio,
    int nq, int nk, int H, int D, int max_vis, int skip_le, float* __restrict__ scores, int64_t ld,
    int32_t* __restrict__ err_flag) {
  extern __shared__ float sq[];  // [H*D] query block, then [H] weights
  const int i = blockIdx.y;
  QueryView v;
  if (!query_view(cu_q, used_kv, cu_kv, batch, stride, i, &v)) return;
  const int ev = ratio > 1 ? v.E / ratio : v.E;
  if (v.E < 1 || ev > max_vis || v.kv0 < 0 || int64_t(v.kv0) + ev > nk) {
    if (threadIdx.x == 0 && blockIdx.x == 0) raise_flag(err_flag, DSA_DEVERR_EXTENT);
    return;
  }
  if (ev <= skip_le) return;  // the top-k keeps every visible key of this row without its scores
  for (int e = threadIdx.x; e < H * D; e += kGenThreads) sq[e] = ld_elt(qi, int64_t(i) * H * D + e);
  for (int e = threadIdx.x; e < H; e += kGenThreads) sq[H * D + e] = w[int64_t(i) * H + e];
  __syncthreads();
  const int s = blockIdx.x * kGenThreads + threadIdx.x;
  if (s >= ev || !DSA_CHECK(s < ld, err_flag)) return;
  const int64_t krow = int64_t(v.kv0 + s) * D;
  float acc = 0.f;
  if constexpr (KD > 0) {
    float kr[KD];
#pragma unroll
    for (int d = 0; d < KD; d += 4) {
      const float4 x = d < D ? ld_elt4(ki, krow + d) : make_float4(0.f, 0.f, 0.f, 0.f);
      kr[d] = x.x;
      kr[d + 1] = x.y;
      kr[d + 2] = x.z;
      kr[d + 3] = x.w;
    }
    for (int h = 0; h < H; ++h) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < KD; ++d)
        if (d < D) dot = fmaf(sq[h * D + d], kr[d], dot);
      acc = fmaf(sq[H * D + h], fmaxf(dot, 0.f), acc);
    }
  } else {
    for (int h = 0; h < H; ++h) {
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(sq[h * D + d], ld_elt(ki, krow + d), dot);
      acc = fmaf(sq[H * D + h], fmaxf(dot, 0.f), acc);
    }
  }
  scores[int64_t(i) * ld + s] = acc + 0.f;  // -0.0 -> +0.0
}

// ---------------------------------------------------------------------------------------------
// MFMA kernel: 64 heads x 128
// ---------------------------------------------------------------------------------------------
constexpr int kHi = kIdxHeads, kDi = kIdxDim;
constexpr int kWaves = 8, kThreads = kWaves * 64;

constexpr int kKeyTile = 256;     // keys per LDS tile (one barrier per tile)
constexpr int kChunkKeys = 4096;  // smallest key chunk per workgroup (grid.y splits longer ranges)
constexpr int kTargetWorkgroups = 4096;    // chunks grow until the grid is about this large
// fp8: row pitch (floats) of the per-query linear parts of a tile; the two lane halves write rows
// q and q + 1 at once, 32 banks apart
constexpr int kLinPitch = kKeyTile + 32;

template <bool FP8>
struct IdxCfg {
  static constexpr int kKeyBytes = FP8 ? kDi : kDi * 2;          // 128 or 256
  static constexpr int kChunks = kKeyBytes / 16;                  // 8 or 16
  static constexpr int kTileBytes = kKeyTile * kKeyBytes;         // 32 or 64 KiB
  static constexpr int kLoads = kKeyTile * kChunks / kThreads;    // direct loads per lane per tile: 4 or 8
};

// bf16: one workgroup per CU (its 64 x 128 query operand takes 64 VGPRs per lane), with the
// epilogue software-pipelined against the next block's MFMAs. fp8: two workgroups per CU
// (4 waves per SIMD, at most 128 VGPRs), which hides more than the pipelining does.
// Candidate mode (CAND): rows with more than fuse_above visible keys append their scores at or
// above theta[i] to segment blockIdx.y of cand[i * cand_cap ...] (cand_cap / gridDim.y entries;
// count in n_cand[i * gridDim.y + blockIdx.y], which the caller zeroes); shorter rows write score
// rows.
template <bool FP8, bool CAND>
__global__ __launch_bounds__(kThreads, FP8 ? 4 : 1) void indexer_mfma(
    const unsigned char* __restrict__ qi, const float* __restrict__ q_scale, const float* __restrict__ w,
    const unsigned char* __restrict__ ki, const float* __restrict__ k_scale, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ used_kv, const int32_t* __restrict__ cu_kv, int batch, int stride, int ratio, int nq,
    int nk, int max_vis, int chunk_keys, int skip_le, float* __restrict__ scores, int64_t ld,
    int32_t* __restrict__ err_flag, int fuse_above, const uint32_t* __restrict__ theta, int32_t* __restrict__ n_cand,
    uint2* __restrict__ cand, int cand_cap) {
  using C = IdxCfg<FP8>;
  __shared__ __attribute__((aligned(16))) unsigned char tiles[2 * C::kTileBytes];
  __shared__ __attribute__((aligned(16))) float ks_tile[2][FP8 ? kKeyTile : 4];
  // fp8: the group's split c rows (row 8j + 4h + p: part p of query 2j + h) and each tile's linear
  // parts c . k times k_scale, [query][key of the tile]
  __shared__ __attribute__((aligned(16))) unsigned char lin_rows[FP8 ? 32 * kDi : 16];
  __shared__ __attribute__((aligned(16))) float lin_v[FP8 ? kWaves * kLinPitch : 4];
  __shared__ int s_lo[kWaves], s_hi[kWaves], s_e0[kWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave (known to the compiler)
  const int half = lane >> 5, l32 = lane & 31;
  const int i = blockIdx.x * kWaves + wave;

  // this wave's query: absolute key range [lo, hi)
  int lo = 0, hi = 0, ev = 0;
  QueryView v{0, 0, 0};
  bool ok = false;
  if (i < nq && query_view(cu_q, used_kv, cu_kv, batch, stride, i, &v)) {
    ev = ratio > 1 ? v.E / ratio : v.E;
    ok = v.E >= 1 && ev <= max_vis && v.kv0 >= 0 && int64_t(v.kv0) + ev <= nk;
    if (!ok && lane == 0) raise_flag(err_flag, DSA_DEVERR_EXTENT);
    // rows the top-k keeps whole (ev <= skip_le) need no scores: they join no key range
    if (ok && ev > skip_le) {
      lo = v.kv0;
      hi = v.kv0 + ev;
    }
  }
  if (!ok) lo = hi = 0;
  const int q_origin = lo;  // score column 0 of this query
  if (lane == 0) {
    s_lo[wave] = ok && hi > lo ? lo : INT32_MAX;
    s_hi[wave] = ok && hi > lo ? hi : INT32_MIN;
  }
  __syncthreads();
  int ulo = INT32_MAX, uhi = INT32_MIN;  // union of the 8 queries' key ranges
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    ulo = min(ulo, s_lo[k]);
    uhi = max(uhi, s_hi[k]);
  }
  // the same in every lane; scalar, so that the tile addresses derived from them are too
  ulo = __builtin_amdgcn_readfirstlane(ulo);
  uhi = __builtin_amdgcn_readfirstlane(uhi);
  // The union is cut into chunks of chunk_keys keys; workgroup y takes chunks y, y + gridDim.y,
  // ... A union can be longer than the longest single range (queries of two requests), so the
  // grid-stride loop, not the grid size, guarantees that every chunk is covered.
  if (uhi <= ulo || int64_t(blockIdx.y) * chunk_keys >= int64_t(uhi) - ulo) return;  // uniform

  // ---- A operand: this wave's query block, heads 32m + l32, d-slices per k-step ----
  constexpr int kKsteps = IdxOps<FP8>::kKsteps;  // 2 or 8
  typename IdxOps<FP8>::AOp qa[2][kKsteps];
  float wv[2][16];  // weights of the 16 heads this lane holds per head block, in output layout
  if (ok) load_query_operands<FP8>(qi, w, q_scale, i, qa, wv);
  if constexpr (FP8) {
    // score = sum_h w'' |x_h| + c . k with w'' = w q_scale / 2 (exact halving); this wave splits
    // its query's c and stores the parts as rows of the group's c-row operand
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) wv[m][r] *= 0.5f;
    uint32_t part[kLinParts] = {0u, 0u, 0u, 0u};
    const int e0 = ok && hi > lo ? lin_split(qi, wv, i, part) : 0;
    if (half == 0) {
#pragma unroll
      for (int p = 0; p < kLinParts; ++p)
        lin_row_store(lin_rows, 8 * (wave >> 1) + 4 * (wave & 1) + p, l32, part[p]);
    }
    if (lane == 0) s_e0[wave] = e0;
  }

  // Candidate mode: this wave's row keeps the scores whose order key is >= theta_k, appended to
  // its own segment of the row's list (segment blockIdx.y of gridDim.y, seg_cap entries) with a
  // register count; no atomics. The count is stored once at the end, overflow included.
  const bool cand_row = CAND && ok && hi - lo > fuse_above;  // wave-uniform
  const uint32_t theta_k = cand_row ? theta[i] : 0u;
  // The same test on floats: theta_k is the 22-bit key prefix of a finite sample score, i.e. the
  // key of a finite float (or of -inf), and keys grow with the float order (+0 and -0 share one),
  // so for a finite score x, order_key(x) >= theta_k exactly when x >= theta_f.
  const float theta_f = key_to_float(theta_k);
  const int seg_cap = cand_cap / int(gridDim.y);
  uint2* seg = CAND ? cand + int64_t(i) * cand_cap + int64_t(blockIdx.y) * seg_cap : nullptr;
  float* srow = scores + int64_t(i) * ld;  // this query's score row (score-row mode)
  int st_n = 0;  // entries this wave found for its row (wave-uniform)
  // The key sweep, compiled once per epilogue (candidate list or score row) so that the per-key
  // code holds no test of the wave-uniform choice between them.
  auto sweep = [&](auto list_tag) {
    constexpr bool LIST = decltype(list_tag)::value;
#pragma unroll 1
    for (int64_t cs = int64_t(blockIdx.y) * chunk_keys; cs < int64_t(uhi) - ulo;
         cs += int64_t(gridDim.y) * chunk_keys) {
      const int glo = ulo + int(cs);
      const int ghi = int(min(int64_t(uhi), int64_t(glo) + chunk_keys));
      const int lo_c = max(lo, glo), hi_c = min(hi, ghi);
      const uint32_t n_in = uint32_t(max(hi_c - lo_c, 0));  // key - lo_c < n_in (unsigned): key in [lo_c, hi_c)
      const int n_tiles = (ghi - glo + kKeyTile - 1) / kKeyTile;
      // ---- staging: tile t holds keys glo + 256t + [0, 256); lane loads 16-byte chunks ----
      // Addresses are a wave-uniform base (scalar registers) plus a 32-bit lane offset, which keeps
      // the per-lane part to one register per load. Rows past the key buffer read its last row (the
      // tile may run past the chunk's end).
      auto issue_tile = [&](int t, int buf) {
        unsigned char* dst = tiles + buf * C::kTileBytes;
        const int row0 = glo + t * kKeyTile;  // < nk: every range ends inside the key buffer
        const int last = nk - 1 - row0;
        const unsigned char* gbase = ki + int64_t(row0) * C::kKeyBytes;
        if constexpr (FP8) {
          if (last >= kKeyTile - 1) {  // wave-uniform: every row of the tile is inside the key buffer
            // load j of this wave covers row n0 + 8j, chunk lane % 8, with n0 = 32 wave + lane / 8;
            // the swizzle reads row bits 0..3, so only bit 3 (j odd) changes it
            const int n0 = 32 * wave + (lane >> 3);
            const uint32_t b0 = uint32_t(n0 * C::kKeyBytes + kswz<C::kChunks>(n0, lane & 7) * 16);
            const uint32_t b1 = uint32_t(n0 * C::kKeyBytes + kswz<C::kChunks>(n0 + 8, lane & 7) * 16);
            if (DSA_CHECK(row0 >= 0, err_flag)) {
#pragma unroll
              for (int j = 0; j < C::kLoads; ++j)
                lds_dma16_s(uniform_ptr(gbase), ((j & 1) ? b1 : b0) + 8u * C::kKeyBytes * j,
                            lds_offset(dst + 64 * (C::kLoads * wave + j) * 16));
            }
            return;
          }
        }
        // recomputed from an opaque copy of the lane id: the kernels have no registers to keep
        // these offsets in across the tile loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int j = 0; j < C::kLoads; ++j) {
          const int f0 = 64 * (C::kLoads * wave + j);
          const int f = f0 + ln;
          const int n = f / C::kChunks;
          const int cp = f - n * C::kChunks;
          const int c = kswz<C::kChunks>(n, cp);
          const int nr = min(n, last);
          if (DSA_CHECK(row0 + nr >= 0, err_flag))
            lds_dma16_s(uniform_ptr(gbase), uint32_t(nr * C::kKeyBytes + c * 16), lds_offset(dst + f0 * 16));
        }
      };

      // fp8: the tile's per-key scales are staged next to it in LDS: wave w copies keys
      // [32w, 32w + 32) with one more direct load (32 active lanes of 4 bytes)
      auto issue_kscale = [&](int t, int buf) {
        if constexpr (FP8) {
          constexpr int kPerWave = kKeyTile / kWaves;  // scales each wave stages
          const int row0 = glo + t * kKeyTile;
          if (lane < kPerWave) {
            const int nr = min(kPerWave * wave + lane, nk - 1 - row0);
            if (DSA_CHECK(row0 + nr >= 0, err_flag))
              lds_dma4_s(k_scale + row0, uint32_t(4 * nr), lds_offset(ks_tile[buf] + kPerWave * wave));
          }
        }
      };
      issue_kscale(0, 0);
      issue_tile(0, 0);
      for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        // One barrier per tile: after it, tile t has landed for every wave and every wave is done
        // with tile t - 1, whose buffer then takes tile t + 1 (loaded while tile t is computed).
        DSA_TILE_BARRIER_ALL();
        if (t + 1 < n_tiles) {
          issue_kscale(t + 1, buf ^ 1);
          issue_tile(t + 1, buf ^ 1);
        }
        const int key0 = glo + t * kKeyTile;
        // fp8: lane-derived LDS addresses come from an opaque copy of the lane id, recomputed every
        // tile rather than kept live across the loop. Kept live they are spilled, and a spill reload
        // after this tile's direct loads were issued would wait for those loads as well (the wait
        // counts loads in issue order).
        int tl = lane;
        if constexpr (FP8) asm volatile("" : "+v"(tl));
        const int t32 = tl & 31, thalf = tl >> 5;
        // fp8: this lane's B-operand chunk addresses for key row t32 of the tile ([k-step][chunk]);
        // row 32 nb + t32 is 4096 nb bytes further (the swizzle reads row bits 0..3 only)
        const unsigned char* kp[2][2];
        if constexpr (FP8) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int x = 0; x < 2; ++x)
              kp[ks][x] = tiles + buf * C::kTileBytes + t32 * C::kKeyBytes +
                          kswz<C::kChunks>(t32, 4 * ks + 2 * thalf + x) * 16;
        }
        auto fp8_key_op = [&](int nb, int ks) {
          const i32x4 x0 = *reinterpret_cast<const i32x4*>(kp[ks][0] + 32 * C::kKeyBytes * nb);
          const i32x4 x1 = *reinterpret_cast<const i32x4*>(kp[ks][1] + 32 * C::kKeyBytes * nb);
          return i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        };
        if constexpr (FP8) {
          // c . k of block `wave` of this tile for the group's 8 queries (lane half h: queries
          // 2j + h in output rows 8j + 4h + p), times k_scale, published for every wave
          const int n = 32 * wave + t32;
          f32x16 L = f32x16{};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            L = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(lin_a_operand(lin_rows, t32, ks, thalf),
                                                                fp8_key_op(wave, ks), L, 0, 0, 0, 127, 0, 127);
          const float ksn = ks_tile[buf][n];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int q = 2 * j + thalf;
            lin_v[q * kLinPitch + n] = lin_combine(L, 4 * j, s_e0[q], ksn);
          }
          DSA_TILE_BARRIER_LDS();
        }
        if (ok && key0 < hi_c && key0 + kKeyTile > lo_c) {  // wave-uniform
          const unsigned char* tb = tiles + buf * C::kTileBytes;
          // 32-key blocks; bf16 issues block nb+1's MFMAs before block nb's ReLU * w head sum, so
          // the VALU work runs under the matrix-core work
          auto block_mfma = [&](int nb, f32x16& a0, f32x16& a1) {
            const int n = 32 * nb + t32;
            if constexpr (FP8) block_mfma_chains<FP8>(qa, [&](int ks) { return fp8_key_op(nb, ks); }, a0, a1);
            else block_mfma_chains<FP8>(qa, [&](int ks) { return key_operand_lds<FP8>(tb, n, ks, thalf); }, a0, a1);
          };
          // fp8: this lane's key scale and linear part for key tl of the tile (block pair nb, nb + 1
          // at 32 nb floats further)
          const float* ksp = ks_tile[buf] + tl;
          const float* lvp = lin_v + wave * kLinPitch + tl;
          // The MFMAs leave lane l with key 32nb + (l & 31) and heads 32m + 8(r/4) + 4(l/32) + r%4;
          // the scores are emitted two blocks at a time: pair_sum puts block nb's score in half 0
          // and block nb + 1's in half 1, so every lane emits a key of its own.
          auto emit = [&](int nb, float hsum) {
            // lane tl holds key 32 nb + tl of the tile (n = 32 (nb + thalf) + t32)
            float sacc = hsum;
            if constexpr (FP8) sacc = fmaf(hsum, ksp[32 * nb], lvp[32 * nb]);
            const int key = key0 + 32 * nb + tl;
            const bool in = uint32_t(key0 + 32 * nb - lo_c) + uint32_t(tl) < n_in;
            if constexpr (LIST) {
              sacc += 0.f;  // -0.0 -> +0.0
              const bool hit = in && sacc >= theta_f;
              // two compares straight into lane masks (the ballot of their conjunction would go
              // through a 0/1 register and a third compare)
              const uint64_t m = ballot(in) & ballot(sacc >= theta_f);
              if (m) {
                const int slot = st_n + lanes_below(m);
                if (hit && slot < seg_cap && DSA_CHECK(key >= q_origin, err_flag))  // 32-bit offset, scalar base
                  *reinterpret_cast<uint2*>(reinterpret_cast<unsigned char*>(seg) + uint32_t(slot) * 8u) =
                      make_uint2(__float_as_uint(sacc), uint32_t(key0 + 32 * nb - q_origin) + uint32_t(tl));
                st_n += __popcll(m);
              }
            } else if (in && DSA_CHECK(key >= q_origin && key - q_origin < ld, err_flag)) {
              srow[uint32_t(key - q_origin)] = sacc + 0.f;  // -0.0 -> +0.0
            }
          };
          if constexpr (!FP8) {
            f32x16 acc[2][2];
            float part = 0.f;  // the previous block's half sum
            block_mfma(0, acc[0][0], acc[0][1]);
#pragma unroll
            for (int nb = 0; nb < kKeyTile / 32; ++nb) {
              if (nb + 1 < kKeyTile / 32) block_mfma(nb + 1, acc[(nb + 1) & 1][0], acc[(nb + 1) & 1][1]);
              const float p = block_head_part(wv, acc[nb & 1][0], acc[nb & 1][1]);
              if (nb & 1) emit(nb - 1, pair_sum(part, p));
              else part = p;
            }
          } else {
            float part = 0.f;  // the previous block's half sum
#pragma unroll
            for (int nb = 0; nb < kKeyTile / 32; ++nb) {
              f32x16 acc0, acc1;
              block_mfma(nb, acc0, acc1);
              const float p = block_abs_part(wv, acc0, acc1);
              if (nb & 1) emit(nb - 1, pair_sum(part, p));
              else part = p;
            }
          }
        }
      }
      DSA_TILE_BARRIER_LDS();  // every wave is done with this chunk's buffers before the next chunk's first tile
    }
  };
  if (cand_row) sweep(std::true_type{});
  else sweep(std::false_type{});
  if (CAND && cand_row && lane == 0) n_cand[int64_t(i) * gridDim.y + blockIdx.y] = st_n;
}

}  // namespace

// Chunks of at least 4096 keys (1024 queries over an 8192-key causal range: 256 workgroups, one round of the
// GPU, 2.2% faster than 2048-key chunks and 6% faster than 1024); long batches take larger chunks
// (fewer reloads of each group's query block, fewer workgroup start-ups) until the grid is about
// kTargetWorkgroups (4096 rather than 2048 or 1024: ~1% faster on 5377 round-robin queries over up
// to 32K keys and on 16 384 queries over up to 131K keys).
int indexer_key_chunks(const dsa_indexer_topk_args* a, int max_vis, int* chunk_keys) {
  const int64_t groups = (a->nq + kWaves - 1) / kWaves, base_chunks = (max_vis + kChunkKeys - 1) / kChunkKeys;
  const int64_t merge = std::max<int64_t>(1, groups * base_chunks / kTargetWorkgroups);
  *chunk_keys = int(std::min<int64_t>(merge, base_chunks) * kChunkKeys);
  return std::max(1, (max_vis + *chunk_keys - 1) / *chunk_keys);
}

dsa_status launch_indexer_scores(const dsa_indexer_topk_args* a, float* scores, int64_t ld, int max_vis,
                                 int skip_le, const CandidateMode* cm, hipStream_t stream) {
  if (a->nq == 0 || max_vis <= skip_le) return DSA_OK;
  const int stride = a->q_stride, ratio = a->compress_ratio;
  if (a->n_heads == kHi && a->head_dim == kDi && (a->dtype == DSA_BF16 || a->dtype == DSA_FP8_E4M3)) {
    int chunk_keys = 0;
    const int gy = indexer_key_chunks(a, max_vis, &chunk_keys);
    const dim3 grid(unsigned((a->nq + kWaves - 1) / kWaves), unsigned(gy));
    if (cm && cm->segs != gy) return fail(DSA_ERR_INVALID_ARG, "indexer: candidate segments do not match the grid");
    const CandidateMode none{INT32_MAX, nullptr, nullptr, nullptr, 0};
    const CandidateMode& c = cm ? *cm : none;
#define DSA_IDX_ARGS                                                                                           \
  static_cast<const unsigned char*>(a->q_idx), a->q_scale, a->weights, static_cast<const unsigned char*>(a->k_idx), \
      a->k_scale, a->cu_seqlens_q, a->seqused_kv, a->cu_seqlens_kv, a->batch, stride, ratio, a->nq, a->nk, max_vis,  \
      chunk_keys, skip_le, scores, ld, a->err_flag, c.fuse_above, c.theta, c.n_cand, c.cand, c.cap
    if (a->dtype == DSA_BF16) {
      tap_launch(cm ? "indexer_mfma<bf16,candidates>" : "indexer_mfma<bf16>", stream);
      if (cm) hipLaunchKernelGGL((indexer_mfma<false, true>), grid, dim3(kThreads), 0, stream, DSA_IDX_ARGS);
      else hipLaunchKernelGGL((indexer_mfma<false, false>), grid, dim3(kThreads), 0, stream, DSA_IDX_ARGS);
    } else {
      tap_launch(cm ? "indexer_mfma<fp8,candidates>" : "indexer_mfma<fp8>", stream);
      if (cm) hipLaunchKernelGGL((indexer_mfma<true, true>), grid, dim3(kThreads), 0, stream, DSA_IDX_ARGS);
      else hipLaunchKernelGGL((indexer_mfma<true, false>), grid, dim3(kThreads), 0, stream, DSA_IDX_ARGS);
    }
#undef DSA_IDX_ARGS
    return check_launch("indexer_mfma");
  }
  if (cm) return fail(DSA_ERR_UNSUPPORTED, "indexer: candidate lists need the 64 x 128 matrix-core kernel");
  if (a->dtype == DSA_FP8_E4M3) return fail(DSA_ERR_UNSUPPORTED, "indexer: fp8 needs 64 heads x 128");
  if (a->n_heads * a->head_dim > 8192 || a->n_heads > 256)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: shape not supported by the generic kernel");
  const dim3 grid((max_vis + kGenThreads - 1) / kGenThreads, a->nq);
  const size_t lds = sizeof(float) * (size_t(a->n_heads) * a->head_dim + a->n_heads);
  const int D = a->head_dim;
  const int kd = D % 4 != 0 ? 0 : D <= 32 ? 32 : D <= 64 ? 64 : 0;  // key-row register cache
#define DSA_GEN_IDX(T, KD)                                                                                    \
  hipLaunchKernelGGL((indexer_generic<T, KD>), grid, dim3(kGenThreads), lds, stream,                         \
                     static_cast<const T*>(a->q_idx), a->weights, static_cast<const T*>(a->k_idx), a->cu_seqlens_q, \
                     a->seqused_kv, a->cu_seqlens_kv, a->batch, stride, ratio, a->nq, a->nk, a->n_heads, D, max_vis, \
                     skip_le, scores, ld, a->err_flag)
  if (a->dtype == DSA_F32 || a->dtype == DSA_BF16) tap_launch("indexer_generic", stream);
  if (a->dtype == DSA_F32) {
    if (kd == 32) DSA_GEN_IDX(float, 32);
    else if (kd == 64) DSA_GEN_IDX(float, 64);
    else DSA_GEN_IDX(float, 0);
  } else if (a->dtype == DSA_BF16) {
    if (kd == 32) DSA_GEN_IDX(uint16_t, 32);
    else if (kd == 64) DSA_GEN_IDX(uint16_t, 64);
    else DSA_GEN_IDX(uint16_t, 0);
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "indexer: unknown dtype");
  }
#undef DSA_GEN_IDX
  return check_launch("indexer_generic");
}

}  // namespace dsa
