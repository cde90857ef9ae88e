// (4) Sparse shared-KV (MLA) attention with a per-head sink, on gfx950.
//
// [xLLM-CP] "feat: DeepSeek-V4 DSA context-parallel on NPU", Design, data-flow step (4): the
// local queries of ALL heads attend over the KV rows of the full stream that the indexer
// selected, output [T_local, num_heads, head_dim]; Design key points: the attention sink is
// held for all heads on every rank.
//
// For query row i, head h, over the selected rows S (idx != -1):
//   l_s = scale * q[i,h,:] . kv[s,:];  out = sum_s e^(l_s) kv[s,:d_v] / (e^(sink_h) + sum_s e^(l_s))
//
// Two kernels:
//  * sparse_attn_mla_bf16: 128 heads x 576 (value = first 512 columns), bf16 in, fp32 accumulate.
//    One workgroup per query, 4 waves x 32 heads. The selected rows are gathered once per query
//    into LDS, 64 rows (73 KiB) per tile, double-buffered with direct global->LDS loads that are
//    issued between the first half-tile's logit MFMAs (one load per two MFMAs); every
//    wave then runs S^T = K Q^T (32 rows x 32 heads, Q^T held in VGPRs) and O += P V on
//    32x32x16 bf16 MFMAs. S^T puts one head per lane, so the softmax reductions are in-lane,
//    and its accumulator layout is directly the A operand of P V (the contraction order over
//    rows is permuted identically on both operands). The softmax reference max m of each head is
//    fixed from the first 32 selected rows (and the sink), so O is never rescaled. A pass is kept
//    when every head's denominator stays <= 2^64 (which bounds every probability by 2^64, far
//    inside fp32 / bf16 range); otherwise the workgroup sweeps the query's logits for their exact
//    max and reruns it with that max.
//  * sparse_attn_generic: float32 or bf16, small head counts (n_heads * d_v <= 4096); VALU.
#include <atomic>

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------------------------
// Generic kernel (VALU), any small shape
// ---------------------------------------------------------------------------------------------
constexpr int kGenThreads = 256;
constexpr int kGenTile = 32;

template <typename T> __device__ inline float load_elt(const T* p, int64_t i);
template <> __device__ inline float load_elt<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ inline float load_elt<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_float(p[i]);
}
// elements i .. i + 3 in one load (i a multiple of 4 of a 16-byte aligned buffer)
template <typename T> __device__ inline float4 load_elt4(const T* p, int64_t i);
template <> __device__ inline float4 load_elt4<float>(const float* p, int64_t i) {
  return *reinterpret_cast<const float4*>(p + i);
}
template <> __device__ inline float4 load_elt4<uint16_t>(const uint16_t* p, int64_t i) {
  const uint2 u = *reinterpret_cast<const uint2*>(p + i);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xFFFF0000u));
}
template <typename T> __device__ inline void store_elt(T* p, int64_t i, float v);
template <> __device__ inline void store_elt<float>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ inline void store_elt<uint16_t>(uint16_t* p, int64_t i, float v) {
  p[i] = float_to_bf16_bits(v);
}

// LDS row pitch (floats) of the generic kernel's Q and KV rows: a whole number of 16-byte chunks,
// and an odd one, so the 16-byte reads of 16 consecutive rows fall on 16 distinct bank groups.
// The pad columns hold zeros.
__host__ __device__ constexpr int gen_pitch(int d) {
  const int p = (d + 3) / 4 * 4;
  return (p / 4) % 2 == 0 ? p + 4 : p;
}
static_assert(kGenThreads % kGenTile == 0 && kGenTile == 32, "a head's logits of a tile are 32 lanes of one wave");

template <typename T>
__global__ __launch_bounds__(kGenThreads) void sparse_attn_generic(
    const T* __restrict__ q, const T* __restrict__ kv, const int32_t* __restrict__ idx,
    const float* __restrict__ sink, T* __restrict__ out, float* __restrict__ lse, int32_t* __restrict__ err_flag,
    float scale_log2, int n_rows, int H, int Dqk, int Dv, int k_tot) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int P = gen_pitch(Dqk), n4 = P / 4;
  float* sq = smem;                          // [H, P]
  float* skv = sq + H * P;                   // [kGenTile, P]
  float* sl = skv + kGenTile * P;            // [H, kGenTile] probabilities of the tile
  float* sm = sl + H * kGenTile;             // [H] running max (log2 units)
  float* ssum = sm + H;                      // [H] running denominator
  float* salpha = ssum + H;                  // [H] rescale factor of this tile
  int* srow = reinterpret_cast<int*>(salpha + H);  // [kGenTile]

  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  if (Dqk % 4 == 0) {  // 4 elements per load; the pad chunk (if any) is zeroed
    const int c4 = P / 4, n = H * c4;
#pragma unroll 4
    for (int e = tid; e < n; e += kGenThreads) {
      const int h = e / c4, c = e - h * c4;
      *reinterpret_cast<float4*>(sq + h * P + 4 * c) =
          4 * c < Dqk ? load_elt4(q, (int64_t(i) * H + h) * Dqk + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  } else {
    for (int e = tid; e < H * P; e += kGenThreads) {
      const int h = e / P, d = e - h * P;
      sq[e] = d < Dqk ? load_elt(q, (int64_t(i) * H + h) * Dqk + d) : 0.f;
    }
  }
  for (int h = tid; h < H; h += kGenThreads) {
    sm[h] = sink ? sink[h] * kLog2e : -INFINITY;
    ssum[h] = sink ? 1.f : 0.f;
  }
  for (int e = tid; e < kGenTile * (P - Dqk); e += kGenThreads) {
    const int rr = e / (P - Dqk);
    skv[rr * P + Dqk + (e - rr * (P - Dqk))] = 0.f;
  }
  constexpr int kMaxPer = 4096 / kGenThreads;  // H*Dv <= 4096
  float acc[kMaxPer];
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) acc[k] = 0.f;
  __syncthreads();

  for (int t0 = 0; t0 < k_tot; t0 += kGenTile) {
    if (tid < kGenTile) {
      int r = t0 + tid < k_tot ? idx[int64_t(i) * k_tot + t0 + tid] : -1;
      if (r < -1 || r >= n_rows) {
        raise_flag(err_flag, DSA_DEVERR_INDEX);
        r = -1;
      }
      srow[tid] = r;
    }
    __syncthreads();
    if (Dqk % 4 == 0) {
      // 4 elements per load, all of a thread's loads issued before any is stored (the pad
      // columns, zeroed before the first tile, are never written)
      constexpr int kIt = kGenTile * (512 / 4) / kGenThreads;  // Dqk <= 512
      const int c4 = Dqk / 4, n = kGenTile * c4;
      float4 x[kIt];
#pragma unroll
      for (int k = 0; k < kIt; ++k) {
        const int e = tid + k * kGenThreads;
        x[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e < n) {
          const int rr = e / c4, c = e - rr * c4;
          const int r = srow[rr];
          if (r >= 0 && DSA_CHECK(r < n_rows, err_flag)) x[k] = load_elt4(kv, int64_t(r) * Dqk + 4 * c);
        }
      }
#pragma unroll
      for (int k = 0; k < kIt; ++k) {
        const int e = tid + k * kGenThreads;
        if (e < n) {
          const int rr = e / c4, c = e - rr * c4;
          *reinterpret_cast<float4*>(skv + rr * P + 4 * c) = x[k];
        }
      }
    } else {
      for (int e = tid; e < kGenTile * P; e += kGenThreads) {
        const int rr = e / P, d = e - rr * P;
        const int r = srow[rr];
        skv[e] = r >= 0 && d < Dqk && DSA_CHECK(r < n_rows, err_flag) ? load_elt(kv, int64_t(r) * Dqk + d) : 0.f;
      }
    }
    __syncthreads();
    // Logits and the online softmax. Lane e holds (head e / 32, tile row e % 32): the 32 rows of a
    // head are 32 lanes of one wave, so its max and sum are lane reductions; the lane of row 0
    // updates the head's running max, denominator and rescale factor.
    for (int e = tid; e < H * kGenTile; e += kGenThreads) {
      const int h = e / kGenTile, rr = e - h * kGenTile;
      float s = -INFINITY;
      if (srow[rr] >= 0) {
        const float4* a = reinterpret_cast<const float4*>(sq + h * P);
        const float4* b = reinterpret_cast<const float4*>(skv + rr * P);
        float dot = 0.f;
#pragma unroll 4
        for (int d4 = 0; d4 < n4; ++d4) {
          const float4 x = a[d4], y = b[d4];
          dot = fmaf(x.x, y.x, dot);
          dot = fmaf(x.y, y.y, dot);
          dot = fmaf(x.z, y.z, dot);
          dot = fmaf(x.w, y.w, dot);
        }
        s = dot * scale_log2;
      }
      float mx = s;
#pragma unroll
      for (int o = kGenTile / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kGenTile));
      const float m_old = sm[h];
      const float m_new = fmaxf(m_old, mx);
      const float pr = m_new == -INFINITY ? 0.f : exp2f(s - m_new);
      float sum = pr;
#pragma unroll
      for (int o = kGenTile / 2; o > 0; o >>= 1) sum += __shfl_xor(sum, o, kGenTile);
      sl[e] = pr;
      if (rr == 0) {
        const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_old - m_new);
        sm[h] = m_new;
        ssum[h] = ssum[h] * alpha + sum;
        salpha[h] = alpha;
      }
    }
    __syncthreads();
    for (int k = 0; k < kMaxPer; ++k) {
      const int e = tid + k * kGenThreads;
      if (e < H * Dv) {
        const int h = e / Dv, d = e - h * Dv;
        float a = acc[k] * salpha[h];
        for (int rr = 0; rr < kGenTile; ++rr) a = fmaf(sl[h * kGenTile + rr], skv[rr * P + d], a);
        acc[k] = a;
      }
    }
    __syncthreads();
  }
  for (int k = 0; k < kMaxPer; ++k) {
    const int e = tid + k * kGenThreads;
    if (e < H * Dv) {
      const int h = e / Dv;
      const float z = ssum[h];
      store_elt(out, int64_t(i) * H * Dv + e, z > 0.f ? acc[k] / z : 0.f);
    }
  }
  if (lse) {
    for (int h = tid; h < H; h += kGenThreads) {
      const float z = ssum[h];
      lse[int64_t(i) * H + h] = z > 0.f ? (sm[h] + log2f(z)) / kLog2e : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// MLA kernel: 128 heads, 576-wide rows (512 latent + 64 rope), value = first 512 columns, bf16
// ---------------------------------------------------------------------------------------------
constexpr int kH = 128, kDqk = 576, kDv = 512;
constexpr int kWaves = 4, kThreads = kWaves * 64;
constexpr int kTile = 64;                          // KV rows per LDS tile
constexpr int kRowBytes = kDqk * 2;                // 1152 bytes per KV row in HBM
constexpr int kLatBytes = kDv * 2;                 // 1024: latent columns of a row
constexpr int kLatPitch = kLatBytes + 16;          // 1040: latent row pitch in LDS (16-byte skew per row)
constexpr int kRopeBytes = kRowBytes - kLatBytes;  // 128: rope columns
constexpr int kLatTile = kTile * kLatPitch;        // 65 KiB
constexpr int kTileBytes = kLatTile + kTile * kRopeBytes;  // 73 KiB
constexpr int kMaxKtot = 2304;                     // selected rows per query held in LDS (9 KiB)
constexpr int kLoadsPerWave = 18;                  // 16 latent rows + 2 rope instructions
// Q staging: 32 head rows per wave at a pitch of 1168 bytes (73 chunks of 16: the row, then one
// pad chunk), so the 16 lanes of one 16-byte operand read fall on 16 distinct bank groups
constexpr int kQPitch = kRowBytes + 16, kQChunks = kQPitch / 16;
constexpr int kQLoads = (32 * kQChunks + 63) / 64;  // 1 KiB direct loads per wave (37)
static_assert(kWaves * 32 * kQPitch <= 2 * kTileBytes, "Q staging fits in the tile buffers");
static_assert(kDqk / 32 == kLoadsPerWave, "one gather load per four logit MFMAs of a tile");
#ifndef DSA_LOOKK
#define DSA_LOOKK 3
#endif
#ifndef DSA_LOOKV
#define DSA_LOOKV 2
#endif
constexpr int kLookK = DSA_LOOKK, kLookV = DSA_LOOKV;  // LDS operand reads issued ahead of their MFMA
constexpr float kMaxDenominator = 0x1p64f;         // a pass is kept while every head's sum of e^(l - m) <= 2^64

// LDS tile layout: latent region [64 rows][1040 bytes] (the 1024 latent bytes of a row, then 16
// unused), then rope region [64 rows][8 chunks of 16 B] with chunk c of row n at physical chunk
// c ^ rope_swz(n). The 16-byte skew of the latent rows puts row n on banks shifted by 16n bytes,
// so (a) the 16 rows of one K operand read (same column) hit 16 distinct 16-byte bank groups, and
// (b) a transposed V read, whose 4 rows per 16 lanes are 4 rows apart (see row_of_mfma_row),
// covers 256 contiguous bytes modulo the bank width. No address XOR is needed, so every latent
// operand read is a per-lane base plus an immediate offset. rope_swz does (a) for 128-byte rows.
//
// MFMA row m of a 32-row half-tile reads tile row row_of_mfma_row(m): writing m = 8a + 4b + c
// (a < 4, b < 2, c < 4), the row is 16(a/2) + 4c + 2(a%2) + b. The S^T accumulator gives lane
// (half b) rows m = 8(v/4) + 4b + v%4, so the four rows v%4 = 0..3 that one transposed V read
// gathers per 16 lanes are 4 tile rows apart.
__device__ inline int row_of_mfma_row(int m) {
  const int a = m >> 3, b = (m >> 2) & 1, c = m & 3;
  return 16 * (a >> 1) + 4 * c + 2 * (a & 1) + b;
}
__device__ inline int rope_swz(int n) { return ((n >> 1) & 3) | (((n ^ (n >> 3)) & 1) << 2); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Logit MFMAs with the accumulator in VGPRs. Every MFMA the compiler emits in this kernel takes
// the AGPR form (the kernel needs AGPRs for O), and with O filling all 256 AGPRs the compiler
// would move one O block out and back around every logit chain. Hazards are handled here: the
// chain accumulates back to back into the same registers (as compiler-emitted chains do), the
// first MFMA's result never shares registers with its operands (early clobber), the
// memory clobber keeps the LDS operand reads where the source puts them (the compiler still
// waits for each read before the asm that uses it), and logit_chain_done() pads the 8-pass
// MFMA's result latency before any VALU may read the logits (it takes them as an operand).
__device__ inline void logit_mfma_first(f32x16& s, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "v"(b) : "memory");
}
__device__ inline void logit_mfma(f32x16& s, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b) : "memory");
}
__device__ inline void logit_chain_done(f32x16& s) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2" : "+v"(s)::"memory");  // 19 wait states
}

// ds_read_b64_tr_b16: inside each 16-lane group, lane o receives element o%4 of the 4-element
// runs addressed by lanes 4j + o/4 (j = 0..3) -- a 16x4 -> 4x16 transpose.
__device__ inline s16x4 lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

constexpr int kSelPer = kMaxKtot / kThreads;  // selection entries per thread (9)

// This thread's share of query i's selected row ids: entries kSelPer*tid .. +kSelPer (-1 past k_tot)
__device__ inline void load_selection(const int32_t* __restrict__ idx, int i, int k_tot, int (&vals)[kSelPer]) {
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) {
    const int e = threadIdx.x * kSelPer + k;
    vals[k] = e < k_tot ? idx[int64_t(i) * k_tot + e] : -1;
  }
}

// Selected row ids (from load_selection) -> rows[], validated (-1 skipped, out-of-range flagged
// and skipped) and compacted in order; the tail up to a multiple of `tile` is padded with row 0
// (a valid row whose logits are masked). Returns the number of selected rows. All threads call it.
__device__ inline int compact_rows(int (&vals)[kSelPer], int n_rows, int tile, int* rows, int* scan,
                                   int32_t* err_flag) {
  constexpr int kPer = kSelPer;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int cnt = 0;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    int r = vals[k];
    if (r < -1 || r >= n_rows) {
      bad = true;
      r = -1;
    }
    vals[k] = r;
    cnt += r >= 0;
  }
  if (bad) raise_flag(err_flag, DSA_DEVERR_INDEX);
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d, 64);
    if (lane >= d) incl += t;
  }
  if (lane == 63) scan[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += scan[w];
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < kWaves; ++w) tot += scan[w];
    scan[kWaves] = tot;
  }
  int pos = base + incl - cnt;
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    if (vals[k] >= 0 && DSA_CHECK(pos < kMaxKtot, err_flag)) rows[pos++] = vals[k];
  __syncthreads();
  const int n_sel = scan[kWaves];
  const int padded = (n_sel + tile - 1) / tile * tile;
  for (int e = n_sel + tid; e < padded; e += kThreads)
    if (DSA_CHECK(e < kMaxKtot, err_flag)) rows[e] = 0;
  __syncthreads();
  return n_sel;
}

__global__ __launch_bounds__(kThreads, 1) void sparse_attn_mla_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const float* __restrict__ sink, uint16_t* __restrict__ out, float* __restrict__ lse,
    int32_t* __restrict__ err_flag, float scale_log2, int n_rows, int k_tot) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* tiles = lds;                                        // 2 x kTileBytes
  int* rows = reinterpret_cast<int*>(lds + 2 * kTileBytes);          // [kMaxKtot] compacted row ids
  int* scan = rows + kMaxKtot;                                       // [kWaves + 1], then the rerun flag
  int* redo_flag = scan + kWaves + 1;

  const int i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave (known to the compiler)
  const int half = lane >> 5, l32 = lane & 31;
  const int h = wave * 32 + l32;  // this lane's head in S^T / softmax

  // ---- Q^T operand for S^T = K Q^T: lane holds q[h, 16ks + 8half .. +8) ----
  // Staged through the (still unused) tile buffers: wave w copies its 32 head rows, contiguous in
  // HBM, with 1 KiB direct loads into rows of kQPitch bytes, and each lane then reads its operand
  // 16 bytes at a time. (Loading the operand straight into registers fetches every 128-byte line
  // in four 32-byte pieces, 32 lines per instruction.) The selection loads are issued behind the
  // copy; the compaction's wait for them is a full vmcnt wait (the compiler does not count the
  // direct loads), so it also covers the copy.
  unsigned char* qstage = tiles + wave * 32 * kQPitch;
  {
    const unsigned char* qrows = reinterpret_cast<const unsigned char*>(q + (int64_t(i) * kH + wave * 32) * kDqk);
    const uint32_t dst = lds_offset(qstage);
#pragma unroll
    for (int j = 0; j < kQLoads; ++j) {
      const int c = 64 * j + lane;  // 16-byte chunk of the staging rows: row c / 73, chunk c % 73
      const int r = c / kQChunks, col = c % kQChunks;
      const uint32_t src = uint32_t(r * kRowBytes + 16 * (col < kQChunks - 1 ? col : 0));  // pad: any chunk
      if (c < 32 * kQChunks) lds_dma16_s(qrows, src, dst + 1024 * j);
    }
  }
  int sel[kSelPer];
  load_selection(idx, i, k_tot, sel);
  const int n_sel = compact_rows(sel, n_rows, kTile, rows, scan, err_flag);
  const int n_tiles = (n_sel + kTile - 1) / kTile;
  bf16x8 qreg[kDqk / 16];
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's staging rows have landed
#pragma unroll
  for (int ks = 0; ks < kDqk / 16; ++ks)
    qreg[ks] = *reinterpret_cast<const bf16x8*>(qstage + l32 * kQPitch + 32 * ks + 16 * half);
  DSA_TILE_BARRIER_LDS();  // every wave holds its operand before the first gather reuses the space

  // ---- gather of one tile into LDS with direct global->LDS loads ----
  //  latent: instruction j of this wave moves row n = 16*wave + j (one uniform row id, 64 lanes x
  //          16 B = 1024 B; lane l lands in chunk l of the row);
  //  rope:   2 instructions of 8 rows x 8 chunks (lane l: row 8r + l/8, physical chunk l%8).
  const unsigned char* kvb = reinterpret_cast<const unsigned char*>(kv);
  // The row ids a wave needs for tile t: lane l holds latent row 16*wave + (l & 15) and, for
  // the two rope loads, rows 16*wave + 8j + l/8.
  struct GatherRows {
    int lat, rope0, rope1;
  };
  auto gather_rows = [&](int t) {
    if (!DSA_CHECK((t + 1) * kTile <= kMaxKtot, err_flag)) return GatherRows{0, 0, 0};
    return GatherRows{rows[t * kTile + 16 * wave + (lane & 15)], rows[t * kTile + 16 * wave + (lane >> 3)],
                      rows[t * kTile + 16 * wave + 8 + (lane >> 3)]};
  };
  // load j (0..kLoadsPerWave-1) of this wave's share of the gather of a tile into buffer buf
  const uint32_t lane16 = uint32_t(lane) << 4;  // every latent load's per-lane offset
  auto gather_one = [&](const GatherRows& gr, int buf, int j) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_offset(tiles + buf * kTileBytes));
    if (j < 16) {
      const int r = __builtin_amdgcn_readlane(gr.lat, j);
      if (DSA_CHECK(r >= 0 && r < n_rows, err_flag))
        lds_dma16_s(kvb + int64_t(r) * kRowBytes, lane16, dst + uint32_t((16 * wave + j) * kLatPitch));
    } else {
      const int n0 = 16 * wave + 8 * (j - 16);  // rows n0 + lane/8
      const int c = (lane & 7) ^ rope_swz(n0 + (lane >> 3));
      const int r = j == 16 ? gr.rope0 : gr.rope1;
      if (DSA_CHECK(r >= 0 && r < n_rows, err_flag))
        lds_dma16_v(kvb + int64_t(r) * kRowBytes + kLatBytes + (c << 4), dst + uint32_t(kLatTile + n0 * kRopeBytes));
    }
  };
  auto issue_tile = [&](int t, int buf) {
    const GatherRows gr = gather_rows(t);
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) gather_one(gr, buf, j);
  };

  // per-lane LDS byte offsets (tile-relative); the rest of each address is an immediate offset:
  //  K operand of half-tile hb, k-step ks < 32 (tile row 32hb + row_of_mfma_row(l32), latent
  //      chunk 2ks + half): k_base + 32hb*1040 + 32ks
  //  rope operand (chunk 2(ks-32) + half): r_base + 32hb*128 + ((32 (ks-32)) ^ r_x)
  //  transposed V reads (see lds_read_tr16) of P.V step kk: lane L supplies tile row
  //      32hb + 16kk + 2hl + 4((L%16)/4) + L/32 (hl = 0: k-slots 0..3 of its half, hl = 1: 4..7)
  //      and columns 32db + 16((L/16)&1) + 4(L%4) .. +3: v_base + (32hb + 16kk + 2hl)*1040 + 64db
  const int k_row = row_of_mfma_row(l32);
  const int k_base = k_row * kLatPitch + 16 * half;
  const int r_base = kLatTile + k_row * kRopeBytes, r_x0 = (half ^ rope_swz(k_row)) << 4;
  const int v_base = (4 * ((lane & 15) >> 2) + half) * kLatPitch + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

  f32x16 oacc[kDv / 32];
  float m_used = -INFINITY, l_run = 0.f, m_seen = -INFINITY;
  if (tid == 0) *redo_flag = 0;
  if (n_tiles > 0) issue_tile(0, 0);  // the first pass's first tile
  const float sink_l2 = sink ? sink[h] * kLog2e : -INFINITY;
  // Wait here, visibly to the compiler, for the sink load (and the first tile). The tile
  // barriers are inline asm the compiler does not see through; without this it would place
  // graded vmcnt waits before the first MFMAs of every tile, which also drain the next tile's
  // gather loads. Encoding: vmcnt(0), expcnt and lgkmcnt left at their maximum.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // Logits-only sweep over the selection (the rare rerun): the exact max of this lane's head's
  // logits, in log2 units. Same gather and logit MFMAs as the main pass, without the pipelining.
  auto max_sweep = [&]() {
    float mx = -INFINITY;
    if (n_tiles > 0) issue_tile(0, 0);
#pragma unroll 1
    for (int t = 0; t < n_tiles; ++t) {
      DSA_TILE_BARRIER_VMCNT(0);  // tile t landed; every wave is done with tile t - 1's buffer
      if (t + 1 < n_tiles) issue_tile(t + 1, (t + 1) & 1);
      const unsigned char* tb = tiles + (t & 1) * kTileBytes;
      const int valid = n_sel - t * kTile;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        f32x16 s = f32x16{};
#pragma unroll
        for (int ks = 0; ks < kDqk / 16; ++ks) {
          const bf16x8 a = ks < kDv / 16
                               ? *reinterpret_cast<const bf16x8*>(tb + k_base + 32 * hb * kLatPitch + 32 * ks)
                               : *reinterpret_cast<const bf16x8*>(tb + r_base + 32 * hb * kRopeBytes +
                                                                  ((32 * (ks - kDv / 16)) ^ r_x0));
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], s, 0, 0, 0);
        }
        const int lim = valid - 32 * hb - half;
        float tmax = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (16 * (v >> 3) + 4 * (v & 3) + 2 * ((v >> 2) & 1) < lim) tmax = fmaxf(tmax, s[v]);
        mx = fmaxf(mx, xor32_max(tmax) * scale_log2);
      }
    }
    DSA_TILE_BARRIER_LDS();  // every wave is done reading before the next pass refills the buffers
    return mx;
  };

#pragma unroll 1
  for (int attempt = 0; attempt < 2; ++attempt) {
    // attempt 0: m from the first 32 selected rows (and the sink); attempt 1 runs only when a
    // head's denominator overflowed the bound, with m = the exact max from a logits-only sweep
    // (an empty selection keeps m = sink, l = 1: out = 0, lse = sink)
    if (attempt == 1) m_seen = max_sweep();
    m_used = attempt == 0 ? sink_l2 : fmaxf(sink_l2, m_seen);
    l_run = sink ? exp2f(sink_l2 - m_used) : 0.f;
#pragma unroll
    for (int db = 0; db < kDv / 32; ++db) oacc[db] = f32x16{};

    if (attempt == 1 && n_tiles > 0) issue_tile(0, 0);
    for (int t = 0; t < n_tiles; ++t) {
      const int buf = t & 1;
      // One barrier per tile: after it, this tile has landed for every wave AND every wave has
      // finished the previous tile, so the other buffer can take the next tile while this one is
      // computed.
      DSA_TILE_BARRIER_VMCNT(0);
      // the next tile's gather is issued inside both half-tiles' logit MFMAs (one load per four
      // MFMAs), so in-order issue does not hold the matrix core while the loads queue up (one load
      // per two MFMAs of the first half-tile only was 1.5% slower)
      const bool gather_next = t + 1 < n_tiles;
      const GatherRows gr = gather_next ? gather_rows(t + 1) : GatherRows{0, 0, 0};
      const unsigned char* tb = tiles + buf * kTileBytes;
      const int valid = n_sel - t * kTile;  // real rows in this tile (>= 1)

#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {  // 32-row halves of the tile
        // S^T[n][h] = K[n,:] . Q[h,:] for rows n = 32hb + 0..31
        f32x16 s;
        if (gather_next) {
          // explicit software pipeline: kLookK operand reads ahead; after every fourth MFMA one
          // gather load (its memory clobber keeps the operand reads in this order)
          int r_x = r_x0;
          asm volatile("" : "+v"(r_x));
          auto k_read = [&](int ks) {
            return ks < kDv / 16
                       ? *reinterpret_cast<const bf16x8*>(tb + k_base + 32 * hb * kLatPitch + 32 * ks)
                       : *reinterpret_cast<const bf16x8*>(tb + r_base + ((32 * (ks - kDv / 16)) ^ r_x) +
                                                          32 * hb * kRopeBytes);
          };
          bf16x8 a[kDqk / 16];
#pragma unroll
          for (int ks = 0; ks < kLookK; ++ks) a[ks] = k_read(ks);
#pragma unroll
          for (int c = 0; c < kDqk / 32; ++c) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int ks = 2 * c + u;
              if (ks + kLookK < kDqk / 16) a[ks + kLookK] = k_read(ks + kLookK);
              if (ks == 0) logit_mfma_first(s, a[ks], qreg[ks]);
              else logit_mfma(s, a[ks], qreg[ks]);
            }
            if ((c & 1) == 0) gather_one(gr, buf ^ 1, (kLoadsPerWave / 2) * hb + c / 2);
          }
        } else {
          int r_x = r_x0;
          asm volatile("" : "+v"(r_x));  // recomputed per half-tile: no hoisting of the rope offsets
          bf16x8 a[kDqk / 16];
          auto k_read = [&](int ks) {
            return ks < kDv / 16
                       ? *reinterpret_cast<const bf16x8*>(tb + k_base + 32 * hb * kLatPitch + 32 * ks)
                       : *reinterpret_cast<const bf16x8*>(tb + r_base + ((32 * (ks - kDv / 16)) ^ r_x) +
                                                          32 * hb * kRopeBytes);
          };
          // issue order: kLookK operand reads ahead, then one MFMA per read
#pragma unroll
          for (int ks = 0; ks < kLookK; ++ks) a[ks] = k_read(ks);
#pragma unroll
          for (int ks = 0; ks < kDqk / 16; ++ks) {
            if (ks + kLookK < kDqk / 16) a[ks + kLookK] = k_read(ks + kLookK);
            if (ks == 0) logit_mfma_first(s, a[ks], qreg[ks]);
            else logit_mfma(s, a[ks], qreg[ks]);
          }
        }
        logit_chain_done(s);

        // register v of the lane holds tile row 32hb + row_of_mfma_row(8(v/4) + 4half + v%4) =
        // 32hb + 16(v/8) + 4(v%4) + 2((v/4)%2) + half of head h; mask rows past the selection (only
        // the last tile can be partial: wave-uniform branch)
        // (raw logits; the positive scale is applied inside the exponent below)
        if (__builtin_expect(valid < kTile, 0)) {  // kept a branch: selects on every tile cost VALU
          const int lim = valid - 32 * hb - half;
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (16 * (v >> 3) + 4 * (v & 3) + 2 * ((v >> 2) & 1) >= lim) s[v] = -INFINITY;
        }
        if (attempt == 0 && t == 0 && hb == 0) {  // uniform
          // O is still zero: fix the reference max here, no rescale needed
          float tmax = -INFINITY;
#pragma unroll
          for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, s[v]);
          m_used = fmaxf(sink_l2, xor32_max(tmax) * scale_log2);
          l_run = sink ? exp2f(sink_l2 - m_used) : 0.f;
        }

        // probabilities (bf16) in the P.V A-operand layout; row sums
        float psum = 0.f;
        bf16x8 pa[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[8 * kk + jj], scale_log2, -m_used));  // v_exp_f32; tiny -> 0
            psum += p;
            pa[kk][jj] = (__bf16)p;
          }
        }
        psum = xor32_sum(psum);
        l_run += psum;

        // O^T[d][h] += V^T[d][n] P^T[n][h] (V as the A operand, P as B: the same registers as
        // for O = P V, which would leave a lane one column of 16 heads; O^T leaves it 16 columns
        // of its own head); k-slot 8half + jj of step kk is the S^T row of register 8kk + jj:
        // tile row 32hb + 16kk + 4(jj%4) + 2(jj/4) + half
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const unsigned char* vb = tb + v_base + (32 * hb + 16 * kk) * kLatPitch;
          s16x4 lo[kDv / 32], hi[kDv / 32];
#pragma unroll
          for (int db = 0; db < kDv / 32; ++db) {
            lo[db] = lds_read_tr16(vb + 64 * db);
            hi[db] = lds_read_tr16(vb + 2 * kLatPitch + 64 * db);
          }
#pragma unroll
          for (int db = 0; db < kDv / 32; ++db) {
            const s16x8 vv = s16x8{lo[db][0], lo[db][1], lo[db][2], lo[db][3], hi[db][0], hi[db][1], hi[db][2], hi[db][3]};
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pa[kk], oacc[db],
                                                                0, 0, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * kLookV, 0);
#pragma unroll
          for (int db = 0; db < kDv / 32 - kLookV; ++db) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, kLookV, 0);
        }
      }
    }
    if (attempt == 0) {
      // every probability is at most its head's denominator, so l_run <= 2^64 bounds them all
      // (and the O sums) far inside the fp32 / bf16 range; inf or NaN also fail the test
      const bool overflow = !(l_run <= kMaxDenominator);
      if (__any(overflow) && lane == 0) atomicOr(redo_flag, 1);
      __syncthreads();
      if (*redo_flag == 0) break;  // uniform
    }
  }

  // ---- normalise and store: oacc[db][4g + c] = O[h][32db + 8g + 4half + c] ----
  // Each wave stages its 32 x 512 block in LDS (row pitch 1040: the lanes of one 8-byte write hit
  // every bank once per 32 lanes) and writes whole 1 KiB output rows with 16-byte stores.
  __syncthreads();  // every wave is done with the tile buffers
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  constexpr int kOutPitch = kDv * 2 + 16;
  static_assert(kWaves * 32 * kOutPitch <= 2 * kTileBytes, "output staging fits in the tile buffers");
  unsigned char* stage = tiles + wave * 32 * kOutPitch;
#pragma unroll
  for (int db = 0; db < kDv / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 o;  // round to nearest even (the hardware conversion)
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = (__bf16)(oacc[db][4 * g + c] * inv);
      *reinterpret_cast<bf16x4*>(stage + l32 * kOutPitch + 2 * (32 * db + 8 * g + 4 * half)) = o;
    }
  }
  asm volatile("" ::: "memory");  // the wave reads back what its own lanes wrote (LDS keeps order)
  uint16_t* op = out + (int64_t(i) * kH + wave * 32) * kDv;
#pragma unroll
  for (int r = 0; r < 32; ++r)
    *reinterpret_cast<bf16x8*>(op + r * kDv + 8 * lane) = *reinterpret_cast<const bf16x8*>(stage + r * kOutPitch + 16 * lane);
  if (lse && half == 0) lse[int64_t(i) * kH + h] = l_run > 0.f ? (m_used + log2f(l_run)) / kLog2e : -INFINITY;
}


}  // namespace

size_t mla_attn_lds_bytes() { return 2 * kTileBytes + (kMaxKtot + kWaves + 2) * sizeof(int); }

namespace {
// Dynamic LDS above the default limit has to be allowed per kernel and per device: done once
// per device (bit d of `done`; devices past 63 set it on every call). Safe from several threads.
dsa_status allow_lds(const void* fn, int bytes, std::atomic<uint64_t>& done, const char* what) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return check_launch(what);
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return DSA_OK;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
    return check_launch(what);
  done.fetch_or(bit, std::memory_order_release);
  return DSA_OK;
}
std::atomic<uint64_t> g_mla_lds{0};
}  // namespace

dsa_status launch_sparse_attn(const dsa_sparse_attn_args* a, hipStream_t stream) {
  if (a->nq == 0) return DSA_OK;
  const float scale_log2 = a->softmax_scale * kLog2e;
  if (a->dtype == DSA_BF16 && a->n_heads == kH && a->d_qk == kDqk && a->d_v == kDv) {
    if (a->k_tot > kMaxKtot) return fail(DSA_ERR_UNSUPPORTED, "sparse_attn: k_tot > 2304 for the MLA kernel");
    const dsa_status st = allow_lds(reinterpret_cast<const void*>(sparse_attn_mla_bf16), int(mla_attn_lds_bytes()),
                                    g_mla_lds, "hipFuncSetAttribute(sparse_attn_mla_bf16)");
    if (st != DSA_OK) return st;
    hipLaunchKernelGGL(sparse_attn_mla_bf16, dim3(a->nq), dim3(kThreads), mla_attn_lds_bytes(), stream,
                       static_cast<const uint16_t*>(a->q), static_cast<const uint16_t*>(a->kv), a->idx, a->sink,
                       static_cast<uint16_t*>(a->out), a->lse, a->err_flag, scale_log2, a->n_rows, a->k_tot);
    return check_launch("sparse_attn_mla_bf16");
  }
  // generic kernel
  if (a->n_heads * a->d_v > 4096 || a->d_qk > 512 || a->n_heads * a->d_qk > 16384)
    return fail(DSA_ERR_UNSUPPORTED, "sparse_attn: shape not supported by the generic kernel");
  const size_t pitch = size_t(gen_pitch(a->d_qk));
  const size_t lds = sizeof(float) * (size_t(a->n_heads) * pitch + size_t(kGenTile) * pitch +
                                      size_t(a->n_heads) * kGenTile + 3 * size_t(a->n_heads)) +
                     sizeof(int) * kGenTile;
  // the LDS size depends on the shape: allowed on every call
  if (a->dtype == DSA_F32) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_attn_generic<float>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
      return check_launch("hipFuncSetAttribute(sparse_attn_generic)");
    hipLaunchKernelGGL(sparse_attn_generic<float>, dim3(a->nq), dim3(kGenThreads), lds, stream,
                       static_cast<const float*>(a->q), static_cast<const float*>(a->kv), a->idx, a->sink,
                       static_cast<float*>(a->out), a->lse, a->err_flag, scale_log2, a->n_rows, a->n_heads,
                       a->d_qk, a->d_v, a->k_tot);
  } else if (a->dtype == DSA_BF16) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_attn_generic<uint16_t>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
      return check_launch("hipFuncSetAttribute(sparse_attn_generic)");
    hipLaunchKernelGGL(sparse_attn_generic<uint16_t>, dim3(a->nq), dim3(kGenThreads), lds, stream,
                       static_cast<const uint16_t*>(a->q), static_cast<const uint16_t*>(a->kv), a->idx, a->sink,
                       static_cast<uint16_t*>(a->out), a->lse, a->err_flag, scale_log2, a->n_rows, a->n_heads,
                       a->d_qk, a->d_v, a->k_tot);
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "sparse_attn: dtype must be f32 or bf16");
  }
  return check_launch("sparse_attn_generic");
}

}  // namespace dsa
