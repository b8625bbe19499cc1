// Host-side interface between the C ABI layer (fa_api.cpp) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fa_index.h"

namespace fa {

// block-sparse mask geometry shared by the kernels: 128 x 128 blocks, at most 2048 per
// row or column (N <= 2^18; the LDS lists of enabled blocks are sized for it)
constexpr int kSparseBlock = 128;
constexpr int kSparseMaxBlocks = 2048;

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;
constexpr int kDtypeF16 = 2;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  int B, H, N, d;
  float scale;
  int causal;
  int dtype;
  const int* kv_len;
  // split-KV: keys per split (a multiple of 64), 0 for none. With a split, o and lse
  // point at [n_splits, B, H, N, d] and [n_splits, B, H, N] partial outputs.
  int split_len = 0;
  // block-sparse: ceil(N/128) x ceil(N/128) bytes, nonzero = (query block, key block)
  // evaluated; nullptr for dense attention
  const uint8_t* block_mask = nullptr;
  // dropout: byte threshold t in [0, 255] (keep iff byte >= t), -1 for none; the mask
  // generator is keyed by seed, its counters carry offset
  int drop_t = -1;
  uint64_t seed = 0;
  uint32_t offset = 0;
};

struct FwdGrid {
  int n_mblk;
  int heads_per_xcd;
  int blocks;
};

// Waves per workgroup of the 16-bit forward (32 query rows each) on a device with `cus`
// compute units: 8 when the 8-wave grid gives every compute unit a workgroup, else 4
// (twice the workgroups). At head_dim 128 the LDS leaves room for one workgroup per
// compute unit, so 4 waves pay only while all of them fit at once (8-wave grid at most
// half the compute units: B=1 H=4 N=8192 187 -> 169 us, causal 183 -> 163 us, B=1 H=8
// N=4096 causal 97 -> 86 us); the split-KV and block-sparse modes there keep 8.
inline int fwd_waves(int B, int H, int N, int d, int dtype, int cus) {
  if (dtype == kDtypeF32) return 4;
  const long long blocks8 = (long long)B * H * ((N + 255) / 256);
  if (d == 128) return 2 * blocks8 <= cus ? 4 : 8;
  return blocks8 >= cus ? 8 : 4;
}

// Key length per split that fa_fwd_partial + fa_merge should use instead of the unsplit
// forward, or 0 to run it unsplit. Splitting pays when the unsplit grid of query-block
// workgroups leaves compute units idle: without a causal mask from half a workgroup per
// compute unit down (two splits), under it from one per compute unit down (four
// splits: the longest blocks of a causal grid are split too), keeping at least 1024
// keys per split under the mask and 2048 without it (where the unsplit forward of a
// small grid runs 4-wave workgroups: 1x16x2048 d=128, two 1024-key splits 53 us against
// 50 us unsplit). Measured on the MI355X (unsplit against split totals, partials plus
// merge): 1x4x8192 d=128 188 -> 143 us (2 splits), causal 184 -> 94 us (4); 1x2x16384
// d=128 365 -> 264 us, causal 358 -> 154 us; 1x8x4096 d=128 100 -> 82 us, causal
// 98 -> 64 us; 1x4x16384 d=64 causal 274 -> 215 us; at 256 non-causal workgroups
// (1x8x8192 d=128: 249 against 275 us) or 384 and more causal ones the unsplit
// kernel is as fast or faster.
inline int fwd_split_hint(int B, int H, int N, int d, int causal, int dtype, int cus) {
  if (dtype == kDtypeF32 || N < 2048 || B <= 0 || H <= 0 || cus <= 0) return 0;
  // (query-block workgroups counted as the split-KV kernel runs them: 8 waves at d = 128)
  const long long rows = d == 128 ? 256 : 32LL * fwd_waves(B, H, N, d, dtype, cus);
  const long long wgs = (long long)B * H * ((N + rows - 1) / rows);
  int P = 1;
  if (causal) {
    if (wgs <= cus) P = 4;
  } else if (2 * wgs <= cus) {
    P = 2;
  }
  const int min_keys = causal ? 1024 : 2048;
  while (P > 1 && N / P < min_keys) P /= 2;
  if (P == 1) return 0;
  const int per = (N + P - 1) / P;
  return (per + 63) / 64 * 64;
}

FwdGrid fwd_grid(int B, int H, int N, int waves);
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// compute units of the current device (read once per process; 256 if the query fails)
int device_cu_count();
// forward with the P V product deferred to the end of each query block's key row
// (bf16/f16, d in {64, 128}, N <= kDeferredMaxN); split, block mask and dropout unused
constexpr int kDeferredMaxN = 512;
hipError_t launch_fwd_deferred(const FwdArgs& a, hipStream_t stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* o;
  const void* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  int B, H, N, d;
  float scale;
  int causal;
  int dtype;
  const int* kv_len;
  float* delta;  // workspace: D_i = rowsum(dO * O), [B,H,N]
  // workspace, after D: the largest |dO| of every group of 32 query rows, [B,H,ceil(N/32)]
  // (each (batch, head) starts a new group); the dK/dV kernel derives its dO scale from it
  float* dmax = nullptr;
  const uint8_t* block_mask = nullptr;  // block-sparse mask as in FwdArgs, or nullptr
  int drop_t = -1;                      // dropout as in FwdArgs
  uint64_t seed = 0;
  uint32_t offset = 0;
};

// the workspace: D ([B,H,N] floats) then the dO maxima ([B,H,ceil(N/32)] floats), each
// region starting on a 256-byte boundary
constexpr int kDmaxRows = 32;
size_t bwd_delta_bytes(int B, int H, int N);
size_t bwd_workspace_bytes(int B, int H, int N, int d);

struct MergeArgs {
  const float* o_part;    // [n_splits, B, H, N, d]
  const float* lse_part;  // [n_splits, B, H, N]
  float* o;               // [B, H, N, d]
  float* lse;             // [B, H, N]
  int n_splits, B, H, N, d;
};
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
// stages: bit 0 = D (bwd_pre), bit 2 = dQ (which forms D for its own rows), bit 3 = the
// dQ kernel also writes D to the workspace, bit 1 = dK/dV (reads D); launched in that
// order. The whole backward pass is bits 2, 3 and 1: dQ and D in one kernel, then dK/dV.
constexpr int kBwdAll = 2 | 4 | 8;
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream, int stages = kBwdAll);
// the dK/dV kernel alone (fa_bwd_dkdv.hip; reads the D that bwd_pre wrote)
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
// head_dim 128, bf16/f16: the dK/dV kernel with two waves per SIMD
// (fa_bwd_dkdv_pair.hip); launch_bwd_dkdv dispatches those cases to it
hipError_t launch_bwd_dkdv_pair(const BwdArgs& a, hipStream_t stream);
// fp32 inputs (fa_bwd_f32.hip): the same stages on the fp32 matrix cores
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t stream, int stages);

// records msg as the thread's last error (fa_last_error) and returns status
int api_fail(int status, const char* msg);
// the backward entry points' checks of sizes, dtype and scale (no pointer is looked at)
int bwd_check_sizes(int B, int H, int N, int d, float scale, int dtype);

}  // namespace fa
