// Measurement hook: how busy one CU can keep its matrix cores when every 32x32x16 bf16 MFMA takes
// its A operand from LDS, in the two read forms the MLA attention kernel uses.
//
//  operand 0 (K form): one 16-byte read per lane per MFMA (ds_read_b128), 32 rows of a tile whose
//            rows are 1040 bytes apart, as the logit MFMAs read K.
//  operand 1 (V form): two 8-byte transposed reads per lane per MFMA (ds_read_b64_tr_b16) at the
//            same row pitch, as the P.V MFMAs read V.
//  operand 2: no LDS operand (the MFMA chain alone).
//
// Every wave runs `iters` x 32 MFMAs into one accumulator, its operand reads issued three MFMAs
// ahead, and reports the shader-clock cycles this took. With one wave per SIMD (256 threads) this
// is the issue pattern of the attention kernel; two waves per SIMD (512 threads) show what a
// second wave would add. The LDS contents are arbitrary (the MFMA results are not used) and every
// address is masked into the 64 KiB array.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kPrbLds = 65536;
constexpr int kPrbSteps = 32;
constexpr int kPrbLook = 3;
constexpr int kPrbBlocks = 256;
constexpr int kPrbPitch = 1040;
constexpr int kPrbSlots = 8;  // cycle counts per workgroup (waves)

typedef short s16x4p __attribute__((ext_vector_type(4)));

template <int kOperand>
__device__ inline bf16x8 probe_read(const unsigned char* lds, int base, int j, int o) {
  if constexpr (kOperand == 0) {
    return *reinterpret_cast<const bf16x8*>(lds + ((base + 32 * j + o) & (kPrbLds - 16)));
  } else {
    const int a0 = (base + 64 * (j & 15) + 4 * kPrbPitch * (j >> 4) + o) & (kPrbLds - 8);
    const int a1 = (a0 + 2 * kPrbPitch) & (kPrbLds - 8);
    const s16x4p lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4p*)(lds + a0));
    const s16x4p hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4p*)(lds + a1));
    return __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  }
}

template <int kOperand>
__global__ __launch_bounds__(512) void lds_mfma_probe_kernel(uint64_t* __restrict__ cycles, float* __restrict__ sink,
                                                              int iters) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kPrbLds];
  for (int e = threadIdx.x; e < kPrbLds / 4; e += blockDim.x)
    reinterpret_cast<uint32_t*>(lds)[e] = 0x3F803F80u ^ (uint32_t(e) << 3);  // finite bf16 pairs
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  // K form: lane reads row l32, 16-byte column chunk `half` (+ 2 per step); V form: the transposed
  // read pattern of 16-lane groups (4 rows, 4 lanes per row), rows spread by the 16-byte skew
  const int base = kOperand == 0
                       ? l32 * kPrbPitch + 16 * half + wave * 4096
                       : (4 * ((lane & 15) >> 2) + half) * kPrbPitch + 32 * ((lane >> 4) & 1) + 8 * (lane & 3) + wave * 4096;
  bf16x8 b;
#pragma unroll
  for (int k = 0; k < 8; ++k) b[k] = (__bf16)(0.001f * float(lane + k));
  f32x16 c = {};
  bf16x8 a[kPrbLook];
  if constexpr (kOperand == 2) {
#pragma unroll
    for (int d = 0; d < kPrbLook; ++d) a[d] = b;
  } else {
#pragma unroll
    for (int d = 0; d < kPrbLook; ++d) a[d] = probe_read<kOperand>(lds, base, d, 0);
  }
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the clock read has returned before the loop
  int o = 0;
  for (int it = 0; it < iters; ++it) {
    const int on = ((it + 1) * 16) & 0x3F0;
#pragma unroll
    for (int j = 0; j < kPrbSteps; ++j) {
      const bf16x8 cur = a[j % kPrbLook];
      if constexpr (kOperand != 2) {
        a[j % kPrbLook] = j + kPrbLook < kPrbSteps ? probe_read<kOperand>(lds, base, j + kPrbLook, o)
                                                   : probe_read<kOperand>(lds, base, j + kPrbLook - kPrbSteps, on);
      }
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, b, c, 0, 0, 0);
      if constexpr (kOperand == 1) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      if constexpr (kOperand == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    o = on;
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += c[k];
#pragma unroll
  for (int d = 0; d < kPrbLook; ++d) s += float(a[d][0]);
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the chain live
  if (lane == 0) cycles[blockIdx.x * kPrbSlots + wave] = t1 - t0;
}

}  // namespace
}  // namespace dsa

extern "C" dsa_status dsa_lds_mfma_probe(int32_t operand, int32_t waves_per_simd, int32_t iters, uint64_t* cycles,
                                         int64_t n_cycles, float* sink, int64_t n_sink, void* stream) {
  using namespace dsa;
  clear_error();
  if (operand < 0 || operand > 2 || waves_per_simd < 1 || waves_per_simd > 2 || iters < 1 || iters > 100000)
    return fail(DSA_ERR_INVALID_ARG, "lds_mfma_probe: need operand 0..2, waves_per_simd 1..2, 1 <= iters <= 1e5");
  const int threads = 256 * waves_per_simd;
  if (!cycles || !sink || n_cycles < int64_t(kPrbBlocks) * kPrbSlots || n_sink < int64_t(kPrbBlocks) * threads)
    return fail(DSA_ERR_INVALID_ARG, "lds_mfma_probe: cycles needs 2048 entries and sink 256 x threads");
  hipStream_t s = as_stream(stream);
  if (operand == 0)
    hipLaunchKernelGGL(lds_mfma_probe_kernel<0>, dim3(kPrbBlocks), dim3(threads), 0, s, cycles, sink, iters);
  else if (operand == 1)
    hipLaunchKernelGGL(lds_mfma_probe_kernel<1>, dim3(kPrbBlocks), dim3(threads), 0, s, cycles, sink, iters);
  else
    hipLaunchKernelGGL(lds_mfma_probe_kernel<2>, dim3(kPrbBlocks), dim3(threads), 0, s, cycles, sink, iters);
  return check_launch("lds_mfma_probe_kernel");
}
