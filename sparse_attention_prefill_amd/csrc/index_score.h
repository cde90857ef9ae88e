// Lightning-indexer score arithmetic on gfx950 matrix cores, shared by every kernel that emits a
// score (the indexer, the recomputation of unusable candidate rows and the threshold sample of
// candidate rows), so that a (query, key) score is the same float whichever of them produced it.
// The one exception: fp8 threshold samples of a group of rows that do not share their sample keys
// keep the ReLU form below (they only place a threshold).
//
// [xLLM-CP] "feat: DeepSeek-V4 DSA context-parallel on NPU", Design, data-flow step (3):
//   score(i, s) = sum_h w[i,h] * max(0, q_idx[i,h,:] . k_idx[s,:])   (64 heads x 128)
// fp8 (E4M3): q_scale[i,h] is folded into the weight and k_scale[s] multiplies the head sum, which
// fp8 computes through ReLU(x) = (x + |x|) / 2 (see "fp8: the score through ..." below).
//
// Layout: one wave owns one query. A 32-key block takes two 32x32 MFMA chains (heads 0..31 and
// 32..63) over the 128 dimensions; lane l holds key 32*nb + (l & 31) and, in each chain, heads
// 8(r/4) + 4(l/32) + r%4 for r < 16. The head sum of both halves is combined across the halves,
// so every lane ends with the full score of its key.
#pragma once
#include <type_traits>

#include "dsa_internal.h"

namespace dsa {

constexpr int kIdxHeads = 64, kIdxDim = 128;

// max(x, 0) on the float's bits: non-negative floats are non-negative ints, and negative floats
// (-0.0 included) are negative ints, so an integer max with 0 is an exact ReLU in one VALU op
// (a float max on MFMA results would first canonicalize its input).
__device__ inline float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

template <bool FP8>
struct IdxOps {
  static constexpr int kKsteps = FP8 ? kIdxDim / 64 : kIdxDim / 16;  // 2 or 8 MFMAs per chain
  static constexpr int kKeyBytes = FP8 ? kIdxDim : kIdxDim * 2;      // 128 or 256
  using AOp = typename std::conditional<FP8, i32x8, bf16x8>::type;
};

// Head weight the lane uses at output slot (m, r): head 32m + 8(r/4) + 4(lane/32) + r%4 of row i
template <bool FP8>
__device__ inline float head_weight(const float* __restrict__ w, const float* __restrict__ q_scale, int i, int m,
                                    int r, int half) {
  const int hh = 32 * m + 8 * (r >> 2) + 4 * half + (r & 3);
  float wt = w[int64_t(i) * kIdxHeads + hh];
  if constexpr (FP8) wt *= q_scale[int64_t(i) * kIdxHeads + hh];
  return wt;
}

// Query operands of row i for this lane: qa[m][ks] (heads 32m + (lane & 31)) and the weights of
// the 16 heads the lane holds per chain, in output layout (times q_scale for fp8).
template <bool FP8>
__device__ inline void load_query_operands(const unsigned char* __restrict__ qi, const float* __restrict__ w,
                                           const float* __restrict__ q_scale, int i,
                                           typename IdxOps<FP8>::AOp (&qa)[2][IdxOps<FP8>::kKsteps],
                                           float (&wv)[2][16]) {
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const unsigned char* qrow = qi + (int64_t(i) * kIdxHeads + 32 * m + l32) * IdxOps<FP8>::kKeyBytes;
#pragma unroll
    for (int ks = 0; ks < IdxOps<FP8>::kKsteps; ++ks) {
      if constexpr (FP8) {
        const i32x4* p = reinterpret_cast<const i32x4*>(qrow + 64 * ks + 32 * half);
        const i32x4 x0 = p[0], x1 = p[1];
        qa[m][ks] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      } else {
        qa[m][ks] = *reinterpret_cast<const bf16x8*>(qrow + 2 * (16 * ks + 8 * half));
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) wv[m][r] = head_weight<FP8>(w, q_scale, i, m, r, half);
  }
}

// The two MFMA chains of one 32-key block; kb(ks) gives this lane's B operand of k-step ks
// (bf16: dimensions 16ks + 8(lane/32) .. +8 of the lane's key; fp8: 64ks + 32(lane/32) .. +32).
template <bool FP8, typename KB>
__device__ inline void block_mfma_chains(const typename IdxOps<FP8>::AOp (&qa)[2][IdxOps<FP8>::kKsteps], KB&& kb,
                                         f32x16& a0, f32x16& a1) {
  a0 = f32x16{};
  a1 = f32x16{};
#pragma unroll
  for (int ks = 0; ks < IdxOps<FP8>::kKsteps; ++ks) {
    const typename IdxOps<FP8>::AOp b = kb(ks);
    if constexpr (FP8) {
      a0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[0][ks], b, a0, 0, 0, 0, 127, 0, 127);
      a1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[1][ks], b, a1, 0, 0, 0, 127, 0, 127);
    } else {
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][ks], b, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][ks], b, a1, 0, 0, 0);
    }
  }
}

// this lane's half of the sum over the 64 heads of w * relu(q . k) (the 32 heads it holds)
__device__ inline float block_head_part(const float (&wv)[2][16], const f32x16& a0, const f32x16& a1) {
  float sacc = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sacc = fmaf(wv[0][r], relu_bits(a0[r]), sacc);
    sacc = fmaf(wv[1][r], relu_bits(a1[r]), sacc);
  }
  return sacc;
}
// sum over the 64 heads of w * relu(q . k) for the lane's key (both halves hold the result);
// fp8 scores still need the key's scale
__device__ inline float block_head_sum(const float (&wv)[2][16], const f32x16& a0, const f32x16& a1) {
  return xor32_sum(block_head_part(wv, a0, a1));
}

// ---- fp8: the score through ReLU(x) = (x + |x|) / 2 ----
// With w''_h = w_h q_scale_h / 2 and x_h = q_h . k (the fp8 dot product of the matrix cores),
//   sum_h w_h q_scale_h ReLU(x_h) = sum_h w''_h |x_h| + c . k,   c_d = sum_h w''_h q_hd,
// an identity, not an approximation. The first sum costs one FMA per head (|x| is a free source
// modifier of the FMA) where the ReLU form costs a max and an FMA; the second is one dot product
// per key, computed on the matrix cores from c split into kLinParts fp8 parts:
//   c_d = 2^e0 * sum_p 16^-p P_pd + r_d,   2^(e0 + 7) <= max_d |c_d| < 2^(e0 + 8),
//   |r_d| <= 2^(e0 - 9) <= 2^-16 max_d |c_d|.
// Every split step is exact: P_pd is the running remainder (in units of 2^e0 16^-p, below 256 in
// magnitude) rounded to E4M3 (round to nearest even, so within 8 units), remainder - P_pd is exact
// in fp32 (Sterbenz: the two are within a factor of two, or P_pd is 0), and the scaling by 16 that
// gives the next remainder (below 128) is exact. The indexer, the recomputation and the shared
// threshold sample all go through lin_split, lin_combine and the |x| half sums (block_abs_part, the
// two halves then added), so an fp8 score is the same float whichever of them computed it.
constexpr int kLinParts = 4;

// The four dimensions 4 (lane & 31) .. +3 of c for query i, in both halves of the wave, split into
// fp8 parts: part[p] holds P_p of those dimensions (byte k = dimension 4 (lane & 31) + k). wv are
// the halved weights w'' in output layout (load_query_operands, then * 0.5). Returns e0.
__device__ inline int lin_split(const unsigned char* __restrict__ qi, const float (&wv)[2][16], int i,
                                uint32_t (&part)[kLinParts]) {
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const unsigned char* qrow = qi + int64_t(i) * kIdxHeads * kIdxDim + 4 * l32;
  float c[4] = {0.f, 0.f, 0.f, 0.f};
  // half h sums the 32 heads it holds in output layout (head bit 2 == h); the halves then add
#pragma unroll
  for (int r = 0; r < 16; ++r) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int hh = 32 * m + 8 * (r >> 2) + 4 * half + (r & 3);
      const int x = *reinterpret_cast<const int*>(qrow + hh * kIdxDim);
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(x, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(x, true);
      c[0] = fmaf(wv[m][r], lo[0], c[0]);
      c[1] = fmaf(wv[m][r], lo[1], c[1]);
      c[2] = fmaf(wv[m][r], hi[0], c[2]);
      c[3] = fmaf(wv[m][r], hi[1], c[3]);
    }
  }
  float mx = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    c[k] = xor32_sum(c[k]);
    mx = fmaxf(mx, fabsf(c[k]));
  }
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  // 2^(e0 + 7) <= max |c| < 2^(e0 + 8): the leading part spans [128, 256) at most; the clamp keeps
  // every part scale a normal float (an all-zero c takes e0 = 0)
  const int e_max = int((__float_as_uint(mx) >> 23) & 255u) - 127;
  const int e0 = mx > 0.f ? min(max(e_max - 7, -110), 120) : 0;
  float r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = ldexpf(c[k], -e0);
#pragma unroll
  for (int p = 0; p < kLinParts; ++p) {
    int wd = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
    wd = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], wd, true);
    part[p] = uint32_t(wd);
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd, true);
    r[0] = (r[0] - lo[0]) * 16.f;
    r[1] = (r[1] - lo[1]) * 16.f;
    r[2] = (r[2] - hi[0]) * 16.f;
    r[3] = (r[3] - hi[1]) * 16.f;
  }
  return e0;
}

// A operand of k-step ks for output row `row` from part rows of 128 fp8 bytes in LDS, stored with
// the key tiles' chunk swizzle (lin_row_store), so that the 32 rows read together hit distinct
// banks: the row's dimensions 64ks + 32(lane/32) .. +32
__device__ inline i32x8 lin_a_operand(const unsigned char* rows, int row, int ks,
                                       int half = (threadIdx.x & 63) >> 5);

// c . k of one query from its parts' products L[b + p] (the matrix cores' P_p . k), times k's
// scale. The result is pinned where it is computed: a value used only under a lane condition could
// otherwise have its MFMAs moved into that branch, where the inactive lanes' operand halves drop
// out of the products.
__device__ inline float lin_combine(const f32x16& L, int b, int e0, float k_scale) {
  float s = fmaf(L[b + 3], 0.0625f, L[b + 2]);
  s = fmaf(s, 0.0625f, L[b + 1]);
  s = fmaf(s, 0.0625f, L[b]);
  float r = ldexpf(s, e0) * k_scale;
  asm volatile("" : "+v"(r));
  return r;
}

// this lane's half of the sum over the 64 heads of w'' * |q . k| (the 32 heads it holds)
__device__ inline float block_abs_part(const float (&wv)[2][16], const f32x16& a0, const f32x16& a1) {
  float sacc = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sacc = fmaf(wv[0][r], fabsf(a0[r]), sacc);
    sacc = fmaf(wv[1][r], fabsf(a1[r]), sacc);
  }
  return sacc;
}
// sum over the 64 heads of w'' * |q . k| for the lane's key (both halves hold the result)
__device__ inline float block_abs_sum(const float (&wv)[2][16], const f32x16& a0, const f32x16& a1) {
  return xor32_sum(block_abs_part(wv, a0, a1));
}
// Two blocks' head sums from their half sums pa and pb: lanes 0..31 get block a's (pa[l] +
// pa[l + 32]), lanes 32..63 block b's (pb[l - 32] + pb[l]); one lane swap between the halves.
// Each is the same float block_abs_sum gives (the same two halves added).
__device__ inline float pair_sum(float pa, float pb) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa), __float_as_uint(pb), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// B operand of k-step ks read straight from key row `row` in global memory
template <bool FP8>
__device__ inline typename IdxOps<FP8>::AOp key_operand_global(const unsigned char* __restrict__ ki, int row, int ks) {
  const int half = (threadIdx.x & 63) >> 5;
  const unsigned char* p = ki + int64_t(row) * IdxOps<FP8>::kKeyBytes;
  if constexpr (FP8) {
    const i32x4* q = reinterpret_cast<const i32x4*>(p + 64 * ks + 32 * half);
    const i32x4 x0 = q[0], x1 = q[1];
    return i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  } else {
    return *reinterpret_cast<const bf16x8*>(p + 2 * (16 * ks + 8 * half));
  }
}

// A wave-uniform pointer, in scalar registers whatever the compiler could prove about it.
__device__ inline const void* uniform_ptr(const void* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(u >> 32));
  return reinterpret_cast<const void*>((uint64_t(hi) << 32) | lo);
}
// Direct global->LDS 4-byte loads from a uniform base and a per-lane byte offset: lane l's word
// lands at lds_base + 4*l (M0 is written only here and in the other direct-load helpers).
__device__ inline void lds_dma4_s(const void* gbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(uniform_ptr(gbase)),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

// Physical 16-byte chunk of logical chunk c of key row n in an LDS key tile. 256-byte rows
// (bf16): XOR with n & 15, so the 16 rows read together by one MFMA operand load hit 16
// distinct bank groups. 128-byte rows (fp8): a 3-bit XOR chosen so that rows n and n + 8 (which
// share banks) also differ.
template <int CHUNKS>
__device__ inline int kswz(int n, int c) {
  if constexpr (CHUNKS == 16) return c ^ (n & 15);
  else return c ^ (((n >> 1) & 3) | (((n ^ (n >> 3)) & 1) << 2));
}

// B operand of k-step ks for key row n of an LDS tile laid out with kswz
template <bool FP8>
__device__ inline typename IdxOps<FP8>::AOp key_operand_lds(const unsigned char* tb, int n, int ks,
                                                            int half = (threadIdx.x & 63) >> 5) {
  constexpr int kBytes = IdxOps<FP8>::kKeyBytes, kChunks = kBytes / 16;
  if constexpr (FP8) {
    const int c0 = 4 * ks + 2 * half;  // two 16-byte chunks: d in [64ks + 32half, +32)
    const i32x4 x0 = *reinterpret_cast<const i32x4*>(tb + n * kBytes + kswz<kChunks>(n, c0) * 16);
    const i32x4 x1 = *reinterpret_cast<const i32x4*>(tb + n * kBytes + kswz<kChunks>(n, c0 + 1) * 16);
    return i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  } else {
    return *reinterpret_cast<const bf16x8*>(tb + n * kBytes + kswz<kChunks>(n, 2 * ks + half) * 16);
  }
}

// Store dword `word` (dimensions 4c .. 4c + 3) of part row `row` in the swizzled layout
__device__ inline void lin_row_store(unsigned char* rows, int row, int c, uint32_t word) {
  *reinterpret_cast<uint32_t*>(rows + row * kIdxDim + kswz<kIdxDim / 16>(row, c >> 2) * 16 + 4 * (c & 3)) = word;
}
__device__ inline i32x8 lin_a_operand(const unsigned char* rows, int row, int ks, int half) {
  const int c0 = 4 * ks + 2 * half;
  const i32x4 x0 = *reinterpret_cast<const i32x4*>(rows + row * kIdxDim + kswz<kIdxDim / 16>(row, c0) * 16);
  const i32x4 x1 = *reinterpret_cast<const i32x4*>(rows + row * kIdxDim + kswz<kIdxDim / 16>(row, c0 + 1) * 16);
  return i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
}

// Full score of key row `row` for the lane (every lane of the wave computes its own key; the
// 32 lanes of each half must name the same 32 keys, lanes l and l + 32 the same key). fp8: wv are
// the halved weights, lin_rows this query's kLinParts part rows (128 bytes each, in LDS) and e0
// its scale exponent (lin_split).
template <bool FP8>
__device__ inline float key_score_global(const typename IdxOps<FP8>::AOp (&qa)[2][IdxOps<FP8>::kKsteps],
                                         const float (&wv)[2][16], const unsigned char* lin_rows, int e0,
                                         const unsigned char* __restrict__ ki, const float* __restrict__ k_scale,
                                         int row) {
  f32x16 a0, a1;
  if constexpr (FP8) {
    // the linear part first (its accumulators are dead before the head chains start); output
    // rows 8j + 4h + p all read part p, so L[p] is P_p . k in both halves
    f32x16 L = f32x16{};
    // read here for every key block (an opaque lane index keeps the compiler from holding this
    // 16-register operand across the caller's loop)
    int l32 = threadIdx.x & 31;
    asm volatile("" : "+v"(l32));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      L = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(lin_a_operand(lin_rows, l32 & (kLinParts - 1), ks),
                                                          key_operand_global<true>(ki, row, ks), L, 0, 0, 0, 127, 0, 127);
    const float ks_row = k_scale[row];
    const float lin = lin_combine(L, 0, e0, ks_row);
    block_mfma_chains<FP8>(qa, [&](int ks) { return key_operand_global<FP8>(ki, row, ks); }, a0, a1);
    return fmaf(block_abs_sum(wv, a0, a1), ks_row, lin) + 0.f;  // -0.0 -> +0.0
  } else {
    block_mfma_chains<FP8>(qa, [&](int ks) { return key_operand_global<FP8>(ki, row, ks); }, a0, a1);
    return block_head_sum(wv, a0, a1) + 0.f;
  }
}

}  // namespace dsa
