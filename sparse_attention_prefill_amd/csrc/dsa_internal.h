// Internal helpers shared by the gfx950 kernels and the host entry points of libdsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "dsa.h"

namespace dsa {

// ---------------------------------------------------------------------------------------------
// Host-side error reporting: a per-thread message behind dsa_last_error().
// ---------------------------------------------------------------------------------------------
void set_error(const std::string& msg);
void clear_error();
dsa_status fail(dsa_status code, const std::string& msg);
dsa_status check_launch(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Kernel-boundary events of one library call (dsa_indexer_topk_timed): while a tap is set on the
// calling thread, every launch site records the tap's next event on its stream right before it
// launches, and the entry point records one more after the last launch. No tap: a no-op.
void tap_launch(const char* kernel, hipStream_t stream);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Workgroup barriers for double-buffered direct global->LDS tile loads, as inline asm so the
// compiler adds no waits of its own (it cannot see the direct loads). VMCNT(n): this wave's
// vector-memory operations except the newest n have completed (loads return in order, so a
// prefetch issued just before may stay in flight); LDS: its LDS reads have returned; ALL: both.
// The memory clobber keeps the compiler from moving accesses across.
#define DSA_TILE_BARRIER_VMCNT(n) asm volatile("s_waitcnt vmcnt(" #n ")\n\ts_barrier" ::: "memory")
#define DSA_TILE_BARRIER_LDS() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")
#define DSA_TILE_BARRIER_ALL() asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory")

// Direct global->LDS 16-byte loads: lane l's 16 bytes land at lds_base + 16*l (lds_base is
// wave-uniform, passed in M0). Issued as inline asm so the compiler does not add its own
// conservative vmcnt waits before later LDS reads; the caller owns the bookkeeping through
// DSA_TILE_BARRIER_VMCNT. M0 is written only here.
__device__ inline uint32_t lds_offset(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}
// uniform 64-bit global base + per-lane 32-bit byte offset
__device__ inline void lds_dma16_s(const void* gbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
// per-lane 64-bit global address
__device__ inline void lds_dma16_v(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

// per-lane 64-bit global address, 4 bytes: lane l's word lands at lds_base + 4*l
__device__ inline void lds_dma4_v(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gaddr),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

__device__ inline void raise_flag(int32_t* err_flag, int32_t bits) {
  if (err_flag) atomicOr(err_flag, bits);
}

// Checked build (DSA_CHECKED): DSA_CHECK(cond, err_flag) is false, after OR-ing
// DSA_DEVERR_BOUNDS into *err_flag, when cond fails; the caller then skips the access. In the
// product build it is the constant true and the condition is not evaluated.
#ifdef DSA_CHECKED
#define DSA_CHECK(cond, err_flag) \
  (__builtin_expect(!!(cond), 1) ? true : (raise_flag((err_flag), DSA_DEVERR_BOUNDS), false))
#else
#define DSA_CHECK(cond, err_flag) true
#endif

// Causal view of local query row i: request b, extent E (keys seen), key offset kv0.
// Returns false (and flags) when the row is not covered by the local cu-seqlens.
struct QueryView {
  int b;
  int E;
  int kv0;
};

__device__ inline bool query_view(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ used_kv,
                                  const int32_t* __restrict__ cu_kv, int batch, int stride, int i,
                                  QueryView* v) {
  // largest b with cu_q[b] <= i, among requests that actually own rows
  int lo = 0, hi = batch;  // invariant: cu_q[lo] <= i < cu_q[hi]
  if (i < cu_q[0] || i >= cu_q[batch]) return false;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu_q[mid] <= i) lo = mid; else hi = mid;
  }
  const int nb = cu_q[lo + 1] - cu_q[lo];
  const int j = i - cu_q[lo];
  v->b = lo;
  v->E = used_kv[lo] - (nb - 1 - j) * stride;
  v->kv0 = cu_kv[lo];
  return true;
}

// ---------------------------------------------------------------------------------------------
// Indexer + top-k without score rows for long rows. A launch whose longest row has more than
// kFuseLaunch visible keys runs in candidate mode: there a row with more than fuse_above visible
// keys (fuse_above = max(kFuseMin, K)) is a candidate row, a sample of its scores sets a
// threshold, the indexer appends only the scores at or above it to the row's list, and the top-k
// selects from the list. Shorter rows keep score rows of kFuseMin floats in the same per-row
// slot. (The sample, the list select and the list appends cost about as much per row as reading
// a 100K-key score row once, so shorter launches keep the score rows.)
// ---------------------------------------------------------------------------------------------
constexpr int kFuseLaunch = 98304;  // candidate mode when some row has more visible keys
constexpr int kFuseMin = 32768;   // longest score row (keys) outside candidate mode
constexpr int kFuseCap = 16384;   // list entries per row: 8 bytes each, the size of that score row
constexpr int kRefillBlocks = 256;  // workgroups (and scratch rows) recomputing unusable lists

struct CandidateMode {
  int fuse_above;     // rows with more visible keys are candidate rows
  uint32_t* theta;    // [nq] thresholds as order keys
  int32_t* n_cand;    // [nq, segs] entries found per list segment (past the segment's end: counted only)
  int32_t* status;    // [nq] 1 when the row was selected from its list, 0 when it must be recomputed
  uint2* cand;        // [nq, cap] (score bits, position): segs segments of cap / segs entries
  int cap;
  int segs;           // list segments per row = grid.y of the indexer launch
};

// grid.y (key chunks per query group) of the 64 x 128 indexer launch, and its chunk length
int indexer_key_chunks(const dsa_indexer_topk_args* a, int max_vis, int* chunk_keys);

// Order-preserving 32-bit keys of float scores: -0.0 and +0.0 -> 0x80000000; a larger float
// gives a larger key; finite floats stay above 2^23.
__device__ inline uint32_t order_key_bits(uint32_t u) {
  const uint32_t m = u & 0x7FFFFFFFu;
  return (u >> 31) ? 0x80000000u - m : 0x80000000u + m;
}
__device__ inline uint32_t order_key(float f) { return order_key_bits(__float_as_uint(f)); }
// the float whose key is k (k >= 2^23, i.e. not a NaN pattern)
__device__ inline float key_to_float(uint32_t k) {
  return k >= 0x80000000u ? __uint_as_float(k - 0x80000000u) : __uint_as_float((0x80000000u - k) | 0x80000000u);
}

// x[l] + x[l ^ 32] (and the max) in every lane of a wave: one VALU lane swap between the two
// 32-lane halves instead of an LDS permute round trip. The two swap outputs hold x[l] and
// x[l ^ 32] in every lane, so the sum is the same float as x[l] + x[l ^ 32] by commutativity.
__device__ inline float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }
// lanes below this one whose bit is set in m
__device__ inline int lanes_below(uint64_t m) {
  return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
}

__device__ inline float bf16_bits_to_float(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bfloat16 bits, round to nearest even (finite inputs)
__device__ inline uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

}  // namespace dsa
