// (5) Rerange: rank-concatenated rows <-> logical token order.
//
// [CP-blog] "[DeepSeek v3.2] context parallel explained", Part 3 step B: after the all-gather
// the rows sit concatenated by rank (T0,T4, T1,T5, ... for cp 4) and are permuted back to
// T0,T1,T2,...; §2B: the split keeps rows rank, rank+cp, ...
// [CP-gathers] "The role of the two all-gathers in NSA prefill CP", Gather #1: the same helper
// restores logical order after either split mode.
//
// A pure permutation of 16-byte chunks: each thread moves whole chunks, consecutive threads
// take consecutive chunks of a row, so both the gather side and the scatter side are
// contiguous per row and HBM-friendly. Row sources are closed forms (no index tensor).
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;

struct RerangeGeom {
  int T, cp, tpr, pad, rr, q, rem;  // q, rem: T = q*cp + rem (unpadded round-robin counts)
  __device__ inline int off(int r) const {  // first concatenated row of rank r
    if (pad) return r * tpr;
    return rr ? r * q + min(r, rem) : min(r * tpr, T);
  }
};

__global__ __launch_bounds__(kThreads) void rerange_kernel(const int4* __restrict__ in, int4* __restrict__ out,
                                                           RerangeGeom g, int n_out_rows, int chunks_per_row,
                                                           int inverse) {
  const int64_t total = int64_t(n_out_rows) * chunks_per_row;
  for (int64_t f = int64_t(blockIdx.x) * kThreads + threadIdx.x; f < total; f += int64_t(gridDim.x) * kThreads) {
    const int row = int(f / chunks_per_row);
    const int c = int(f - int64_t(row) * chunks_per_row);
    int src;
    if (!inverse) {
      // logical token row -> its place in the rank-concatenated buffer
      if (g.rr) src = g.off(row % g.cp) + row / g.cp;
      else src = row;  // in-seq: ranks hold consecutive blocks, concatenation is the identity
    } else {
      // concatenated row -> logical token (or a pad row)
      int r, k;
      if (g.pad) {
        r = row / g.tpr;
        k = row - r * g.tpr;
      } else if (g.rr) {
        // ranks < rem hold q+1 rows, the others q
        const int big = g.rem * (g.q + 1);
        if (row < big) {
          r = row / (g.q + 1);
          k = row - r * (g.q + 1);
        } else {
          r = g.rem + (row - big) / g.q;
          k = row - big - (r - g.rem) * g.q;
        }
      } else {
        r = row / g.tpr;
        k = row - r * g.tpr;
      }
      const int t = g.rr ? r + k * g.cp : r * g.tpr + k;
      src = t < g.T ? t : -1;
    }
    int4 v = make_int4(0, 0, 0, 0);
    if (src >= 0) v = in[int64_t(src) * chunks_per_row + c];
    out[f] = v;
  }
}

}  // namespace

dsa_status launch_rerange(const void* in, void* out, int T, int64_t row_bytes, int cp, int mode, int pad,
                          int inverse, int n_out_rows, hipStream_t stream) {
  RerangeGeom g;
  g.T = T;
  g.cp = cp;
  g.tpr = (T + cp - 1) / cp;
  g.pad = pad;
  g.rr = mode == DSA_SPLIT_ROUND_ROBIN;
  g.q = T / cp;
  g.rem = T % cp;
  const int chunks = int(row_bytes / 16);
  const int64_t total = int64_t(n_out_rows) * chunks;
  if (total == 0) return DSA_OK;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(rerange_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                     static_cast<const int4*>(in), static_cast<int4*>(out), g, n_out_rows, chunks, inverse);
  return check_launch("rerange_kernel");
}

}  // namespace dsa
