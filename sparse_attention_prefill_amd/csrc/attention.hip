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
//    into LDS, 64 rows (72 KiB) per tile, double-buffered with direct global->LDS loads; every
//    wave then runs S^T = K Q^T (32 rows x 32 heads, Q^T held in VGPRs) and O += P V on
//    32x32x16 bf16 MFMAs. S^T puts one head per lane, so the softmax reductions are in-lane,
//    and its accumulator layout is directly the A operand of P V (the contraction order over
//    rows is permuted identically on both operands). Online softmax starts from the sink
//    (m = sink, l = 1) and rescales O only when a head's running max grows by more than 2^8.
//  * sparse_attn_generic: float32 or bf16, small head counts (n_heads * d_v <= 4096); VALU.
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
template <typename T> __device__ inline void store_elt(T* p, int64_t i, float v);
template <> __device__ inline void store_elt<float>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ inline void store_elt<uint16_t>(uint16_t* p, int64_t i, float v) {
  p[i] = float_to_bf16_bits(v);
}

template <typename T>
__global__ __launch_bounds__(kGenThreads) void sparse_attn_generic(
    const T* __restrict__ q, const T* __restrict__ kv, const int32_t* __restrict__ idx,
    const float* __restrict__ sink, T* __restrict__ out, float* __restrict__ lse, int32_t* __restrict__ err_flag,
    float scale_log2, int n_rows, int H, int Dqk, int Dv, int k_tot) {
  extern __shared__ float smem[];
  float* sq = smem;                          // [H, Dqk]
  float* skv = sq + H * Dqk;                 // [kGenTile, Dqk]
  float* sl = skv + kGenTile * Dqk;          // [H, kGenTile] logits -> probabilities
  float* sm = sl + H * kGenTile;             // [H] running max (log2 units)
  float* ssum = sm + H;                      // [H] running denominator
  float* salpha = ssum + H;                  // [H] rescale factor of this tile
  int* srow = reinterpret_cast<int*>(salpha + H);  // [kGenTile]

  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  for (int e = tid; e < H * Dqk; e += kGenThreads) sq[e] = load_elt(q, int64_t(i) * H * Dqk + e);
  for (int h = tid; h < H; h += kGenThreads) {
    sm[h] = sink ? sink[h] * kLog2e : -INFINITY;
    ssum[h] = sink ? 1.f : 0.f;
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
    for (int e = tid; e < kGenTile * Dqk; e += kGenThreads) {
      const int rr = e / Dqk, d = e - rr * Dqk;
      const int r = srow[rr];
      skv[e] = r >= 0 ? load_elt(kv, int64_t(r) * Dqk + d) : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < H * kGenTile; e += kGenThreads) {
      const int h = e / kGenTile, rr = e - h * kGenTile;
      float s = -INFINITY;
      if (srow[rr] >= 0) {
        float dot = 0.f;
        for (int d = 0; d < Dqk; ++d) dot = fmaf(sq[h * Dqk + d], skv[rr * Dqk + d], dot);
        s = dot * scale_log2;
      }
      sl[e] = s;
    }
    __syncthreads();
    for (int h = tid; h < H; h += kGenThreads) {
      float mx = sm[h];
      for (int rr = 0; rr < kGenTile; ++rr) mx = fmaxf(mx, sl[h * kGenTile + rr]);
      const float alpha = mx == -INFINITY ? 1.f : exp2f(sm[h] - mx);
      float sum = ssum[h] * alpha;
      for (int rr = 0; rr < kGenTile; ++rr) {
        const float p = mx == -INFINITY ? 0.f : exp2f(sl[h * kGenTile + rr] - mx);
        sl[h * kGenTile + rr] = p;
        sum += p;
      }
      sm[h] = mx;
      ssum[h] = sum;
      salpha[h] = alpha;
    }
    __syncthreads();
    for (int k = 0; k < kMaxPer; ++k) {
      const int e = tid + k * kGenThreads;
      if (e < H * Dv) {
        const int h = e / Dv, d = e - h * Dv;
        float a = acc[k] * salpha[h];
        for (int rr = 0; rr < kGenTile; ++rr) a = fmaf(sl[h * kGenTile + rr], skv[rr * Dqk + d], a);
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
constexpr int kTile = 64;                       // KV rows per LDS tile
constexpr int kRowBytes = kDqk * 2;             // 1152
constexpr int kChunks = kRowBytes / 16;         // 72 x 16-byte chunks per row
constexpr int kTileBytes = kTile * kRowBytes;   // 73728
constexpr int kMaxKtot = 2304;                  // selected rows per query held in LDS (<= 9 KiB)
constexpr int kLoadsPerWave = kTile * kChunks / (kWaves * 64);  // 18
constexpr float kRescaleThresh = 8.f;           // log2 units

static_assert(kTile * kChunks % (kWaves * 64) == 0, "tile must split evenly into wave loads");

// physical 16-byte chunk of logical chunk c in tile row n (XOR swizzle inside groups of 8)
__device__ inline int swz(int n, int c) { return c ^ (n & 7); }

__global__ __launch_bounds__(kThreads, 1) void sparse_attn_mla_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const float* __restrict__ sink, uint16_t* __restrict__ out, float* __restrict__ lse,
    int32_t* __restrict__ err_flag, float scale_log2, int n_rows, int k_tot) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* tiles = lds;                                        // 2 x kTileBytes
  int* rows = reinterpret_cast<int*>(lds + 2 * kTileBytes);          // [kMaxKtot] compacted row ids
  int* scan = rows + kMaxKtot;                                       // [kWaves + 1]

  const int i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int h = wave * 32 + l32;  // this lane's head in S^T / softmax

  // ---- selected row ids -> LDS, validated and compacted (order kept) ----
  {
    constexpr int kPer = kMaxKtot / kThreads;  // 16 entries per thread
    int vals[kPer];
    int cnt = 0;
    bool bad = false;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = tid * kPer + k;
      int r = e < k_tot ? idx[int64_t(i) * k_tot + e] : -1;
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
      if (vals[k] >= 0) rows[pos++] = vals[k];
    __syncthreads();
  }
  const int n_sel = scan[kWaves];
  const int n_tiles = (n_sel + kTile - 1) / kTile;

  // ---- Q^T operand for S^T = K Q^T: lane holds q[h, 16ks + 8half .. +8) ----
  bf16x8 qreg[kDqk / 16];
  {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(q + (int64_t(i) * kH + h) * kDqk) + half;
#pragma unroll
    for (int ks = 0; ks < kDqk / 16; ++ks) qreg[ks] = qp[2 * ks];
  }

  // ---- gather of one tile: lane takes 16-byte chunks f = 64*(18*wave + j) + lane ----
  auto issue_tile = [&](int t, int buf) {
    unsigned char* dst = tiles + buf * kTileBytes;
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
      const int f0 = 64 * (kLoadsPerWave * wave + j);
      const int f = f0 + lane;
      const int n = f / kChunks;
      const int cp = f - n * kChunks;  // physical chunk in the LDS row
      const int c = swz(n, cp);        // logical chunk it holds
      const int e = t * kTile + n;
      const int r = e < n_sel ? rows[e] : 0;
      const unsigned char* src = reinterpret_cast<const unsigned char*>(kv) + int64_t(r) * kRowBytes + c * 16;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst + f0 * 16), 16, 0, 0);
    }
  };

  // ---- running softmax state (one head per lane; both halves agree) ----
  float m_run = sink ? sink[h] * kLog2e : -INFINITY;
  float l_run = sink ? 1.f : 0.f;
  f32x16 oacc[kDv / 32];
#pragma unroll
  for (int db = 0; db < kDv / 32; ++db) oacc[db] = f32x16{};

  if (n_tiles > 0) issue_tile(0, 0);

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) {
      issue_tile(t + 1, buf ^ 1);
      asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    const unsigned char* tb = tiles + buf * kTileBytes;

    // S^T[n][h] for n in [0,64): two 32-row blocks
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kDqk / 16; ++ks) {
      const int c = 2 * ks + half;
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(tb + l32 * kRowBytes + swz(l32, c) * 16);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(tb + (32 + l32) * kRowBytes + swz(32 + l32, c) * 16);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ks], s1, 0, 0, 0);
    }

    // mask rows past n_sel; lane holds rows n = 32nb + 8(v/4) + 4half + v%4
    const int valid = n_sel - t * kTile;  // rows of this tile that are real (>= 1)
    float tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int n0 = 8 * (v >> 2) + 4 * half + (v & 3);
      s0[v] = n0 < valid ? s0[v] * scale_log2 : -INFINITY;
      s1[v] = n0 + 32 < valid ? s1[v] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, fmaxf(s0[v], s1[v]));
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));

    // lazy rescale: only when some head's max grew by more than 2^8 (or was -inf)
    const bool grow = tmax > m_run + kRescaleThresh || (m_run == -INFINITY && tmax > -INFINITY);
    if (__any(grow)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float av = __shfl(alpha, 8 * (v >> 2) + 4 * half + (v & 3), 64);
#pragma unroll
        for (int db = 0; db < kDv / 32; ++db) oacc[db][v] *= av;
      }
    }

    // probabilities (bf16) in the PV A-operand layout; row sums
    float psum = 0.f;
    bf16x8 pa[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int v = 8 * (kk & 1) + j;
        const float sv = (kk < 2) ? s0[v] : s1[v];
        const float p = m_run == -INFINITY ? 0.f : exp2f(sv - m_run);
        psum += p;
        pa[kk][j] = (__bf16)p;
      }
    }
    psum += __shfl_xor(psum, 32, 64);
    l_run += psum;

    // O[h][d] += P[h][n] V[n][d]; row of k-slot j in step kk: n = 16kk + 8(j/4) + 4half + j%4
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int db = 0; db < kDv / 32; ++db) {
        const int d = 32 * db + l32;
        bf16x8 vb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int n = 16 * kk + 8 * (j >> 2) + 4 * half + (j & 3);
          const uint16_t bits =
              *reinterpret_cast<const uint16_t*>(tb + n * kRowBytes + swz(n, d >> 3) * 16 + (d & 7) * 2);
          vb[j] = __builtin_bit_cast(__bf16, bits);
        }
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[kk], vb, oacc[db], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave is done with this buffer before it is refilled
  }

  // ---- normalise and store: lane holds d = 32db + l32 for heads 8(v/4) + 4half + v%4 ----
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  uint16_t* op = out + (int64_t(i) * kH + wave * 32) * kDv;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int hl = 8 * (v >> 2) + 4 * half + (v & 3);
    const float iv = __shfl(inv, hl, 64);
#pragma unroll
    for (int db = 0; db < kDv / 32; ++db) op[hl * kDv + 32 * db + l32] = float_to_bf16_bits(oacc[db][v] * iv);
  }
  if (lse && half == 0) lse[int64_t(i) * kH + h] = l_run > 0.f ? (m_run + log2f(l_run)) / kLog2e : -INFINITY;
}

}  // namespace

size_t mla_attn_lds_bytes() { return 2 * kTileBytes + (kMaxKtot + kWaves + 1) * sizeof(int); }

dsa_status launch_sparse_attn(const dsa_sparse_attn_args* a, hipStream_t stream) {
  if (a->nq == 0) return DSA_OK;
  const float scale_log2 = a->softmax_scale * kLog2e;
  if (a->dtype == DSA_BF16 && a->n_heads == kH && a->d_qk == kDqk && a->d_v == kDv) {
    if (a->k_tot > kMaxKtot) return fail(DSA_ERR_UNSUPPORTED, "sparse_attn: k_tot > 2304 for the MLA kernel");
    static bool attr_set = false;
    if (!attr_set) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_attn_mla_bf16),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(mla_attn_lds_bytes())) != hipSuccess)
        return check_launch("hipFuncSetAttribute(sparse_attn_mla_bf16)");
      attr_set = true;
    }
    hipLaunchKernelGGL(sparse_attn_mla_bf16, dim3(a->nq), dim3(kThreads), mla_attn_lds_bytes(), stream,
                       static_cast<const uint16_t*>(a->q), static_cast<const uint16_t*>(a->kv), a->idx, a->sink,
                       static_cast<uint16_t*>(a->out), a->lse, a->err_flag, scale_log2, a->n_rows, a->k_tot);
    return check_launch("sparse_attn_mla_bf16");
  }
  // generic kernel
  if (a->n_heads * a->d_v > 4096 || a->d_qk > 512 || a->n_heads * a->d_qk > 16384)
    return fail(DSA_ERR_UNSUPPORTED, "sparse_attn: shape not supported by the generic kernel");
  const size_t lds = sizeof(float) * (size_t(a->n_heads) * a->d_qk + size_t(kGenTile) * a->d_qk +
                                      size_t(a->n_heads) * kGenTile + 3 * size_t(a->n_heads)) +
                     sizeof(int) * kGenTile;
  if (a->dtype == DSA_F32) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_attn_generic<float>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    hipLaunchKernelGGL(sparse_attn_generic<float>, dim3(a->nq), dim3(kGenThreads), lds, stream,
                       static_cast<const float*>(a->q), static_cast<const float*>(a->kv), a->idx, a->sink,
                       static_cast<float*>(a->out), a->lse, a->err_flag, scale_log2, a->n_rows, a->n_heads,
                       a->d_qk, a->d_v, a->k_tot);
  } else if (a->dtype == DSA_BF16) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_attn_generic<uint16_t>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
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
