// Merge of split-KV partial outputs on gfx950.
//
// "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
// (summary of arXiv 2205.14135), Method, incremental softmax tracking: statistics of
// a vector split into parts combine as m = max_p m_p, l = sum_p e^{m_p - m} l_p, and
// the outputs are rescaled by the same factors. With normalised partial outputs O_p and
// their LSE_p = m_p + ln l_p, folding that rule over the splits gives
//   LSE = m + ln sum_p e^{LSE_p - m},   O = sum_p e^{LSE_p - LSE} O_p,   m = max_p LSE_p.
// A split whose LSE_p is -inf (no visible key) weighs 0; a row with every LSE_p = -inf
// gets O = 0, LSE = -inf.
//
// The merge is bandwidth-bound (it reads n_splits*(d+1) floats per row and writes d+1):
// each thread owns 4 consecutive columns of one row, so the reads of every split are
// 16-byte, fully coalesced loads; the per-row weights are computed redundantly by the
// row's d/4 threads from the (cached) LSE values instead of being exchanged.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    float* __restrict__ o, float* __restrict__ lse, int n_splits, size_t rows) {
  constexpr int kTPR = D / 4;  // threads per row
  const size_t idx = (size_t)blockIdx.x * kMergeThreads + threadIdx.x;
  const size_t row = idx / kTPR;
  const int col = (int)(idx % kTPR) * 4;
  if (row >= rows) return;
  float m = -INFINITY;
  for (int p = 0; p < n_splits; ++p) m = fmaxf(m, lse_part[(size_t)p * rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float out_lse = -INFINITY;
  if (m > -INFINITY) {
    float wsum = 0.f;
    for (int p = 0; p < n_splits; ++p) {
      const float lp = lse_part[(size_t)p * rows + row];
      const float w = exp2_fast((lp - m) * kLog2e);  // 0 for lp = -inf
      wsum += w;
      if (w > 0.f) {
        const f32x4 op = *reinterpret_cast<const f32x4*>(o_part + ((size_t)p * rows + row) * D + col);
        acc[0] = fmaf(w, op[0], acc[0]);
        acc[1] = fmaf(w, op[1], acc[1]);
        acc[2] = fmaf(w, op[2], acc[2]);
        acc[3] = fmaf(w, op[3], acc[3]);
      }
    }
    const float inv = 1.0f / wsum;  // wsum >= 1: the maximum split weighs 1
    acc[0] *= inv;
    acc[1] *= inv;
    acc[2] *= inv;
    acc[3] *= inv;
    out_lse = m + log2_fast(wsum) * kLn2;
  }
  *reinterpret_cast<f32x4*>(o + row * D + col) = acc;
  if (col == 0) lse[row] = out_lse;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const size_t rows = (size_t)a.B * a.H * a.N;
  const size_t threads = rows * (a.d / 4);
  const unsigned blocks = (unsigned)((threads + kMergeThreads - 1) / kMergeThreads);
  if (a.d == 64)
    hipLaunchKernelGGL((merge_kernel<64>), dim3(blocks), dim3(kMergeThreads), 0, stream,
                       a.o_part, a.lse_part, a.o, a.lse, a.n_splits, rows);
  else
    hipLaunchKernelGGL((merge_kernel<128>), dim3(blocks), dim3(kMergeThreads), 0, stream,
                       a.o_part, a.lse_part, a.o, a.lse, a.n_splits, rows);
  return hipGetLastError();
}

}  // namespace fa
