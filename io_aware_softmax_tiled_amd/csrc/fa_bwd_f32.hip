// Backward pass of exact attention for fp32 inputs on gfx950, on the 32x32x2 fp32
// matrix cores (fp32 operands, fp32 accumulation, no 16-bit rounding anywhere).
//
// The same method as the 16-bit backward pass ("FlashAttention: Fast and
// Memory-Efficient Exact Attention with IO-Awareness", Key ideas: recomputation): P is
// rebuilt tile by tile from Q, K and the saved LSE, and the gradients follow the chain
// rule of L = sum(dO * O): dP = dO V^T, D_i = sum_k dO_ik O_ik, dS = P * (dP - D),
// dV = P^T dO, dK = scale * dS^T Q, dQ = scale * dS K.
//
// Two kernels, each one wave per workgroup with every operand tile staged in LDS as
// fp32 rows (padded by one element so that the 32 rows a matrix instruction reads lie in
// distinct banks); P and dS pass through LDS to reach the operand layout of the products
// that contract over queries or keys:
//   bwd_f32_dq: 32 queries per workgroup (forms D for its rows, writes it when asked),
//               loops over 32-key tiles, accumulates dQ in registers.
//   bwd_f32_dkdv: 32 keys per workgroup, loops over 32-query tiles (causal: from the
//               diagonal on), reads D from the workspace, accumulates dK and dV.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kT = 32;  // rows of every tile (queries or keys)

// C[32 x 32] += A[32 x K] B[K x 32] on 32x32x2 fp32 matrix instructions; a(m, k) and
// b(k, n) return the operand elements (lane l supplies A[l%32][k0 + l/32] and
// B[k0 + l/32][l%32]). Accumulator register r of lane l is C[8(r/4) + 4(l/32) + r%4][l%32].
template <int K, typename FA, typename FB>
__device__ inline void mm(f32x16& c, FA a, FB b) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, hk = lane >> 5;
#pragma unroll 8
  for (int i = 0; i < K / 2; ++i) {
    const int kk = 2 * i + hk;
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a(col, kk), b(kk, col), c, 0, 0, 0);
  }
}

__device__ inline int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// rows [r0, r0 + 32) of a [rows][D] fp32 array into an LDS tile with row stride D + 1
// (rows past n read as zeros)
template <int D>
__device__ inline void stage_rows(float* t, const float* __restrict__ src, int r0, int n) {
  for (int e = threadIdx.x; e < kT * D; e += 64) {
    const int row = e / D, c = e % D;
    t[row * (D + 1) + c] = r0 + row < n ? src[(size_t)(r0 + row) * D + c] : 0.f;
  }
}

template <int D>
__global__ __launch_bounds__(64) void bwd_f32_dq_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ delta, int write_delta, float* __restrict__ dQ, int BH, int H, int N,
    float scale, int causal, const int* __restrict__ kv_len, int n_qblk) {
  constexpr int kLd = D + 1;
  constexpr int kDB = D / 32;
  __shared__ float Qs[kT * kLd], dOs[kT * kLd], Ks[kT * kLd], Vs[kT * kLd];
  __shared__ float dSs[kT * (kT + 1)];
  __shared__ float Ls[kT], Ds[kT];
  const int bh = blockIdx.x / n_qblk, q0 = (blockIdx.x % n_qblk) * kT;
  const int b = bh / H;
  const size_t head = (size_t)bh * N * D;
  const int lane = threadIdx.x;
  int kv_lim = N;
  if (kv_len != nullptr) kv_lim = min(N, max(1, kv_len[b]));
  const int kend = causal ? min(kv_lim, q0 + kT) : kv_lim;

  stage_rows<D>(Qs, Q + head, q0, N);
  stage_rows<D>(dOs, dO + head, q0, N);
  // D_i = sum_k dO_ik O_ik for the 32 rows, in element order
  if (lane < kT) {
    float s = 0.f;
    if (q0 + lane < N) {
      const float* o = O + head + (size_t)(q0 + lane) * D;
      const float* g = dO + head + (size_t)(q0 + lane) * D;
      for (int c = 0; c < D; ++c) s = fmaf(g[c], o[c], s);
      if (write_delta) delta[(size_t)bh * N + q0 + lane] = s;
    }
    Ds[lane] = s;
    Ls[lane] = q0 + lane < N ? LSE[(size_t)bh * N + q0 + lane] : 0.f;
  }
  f32x16 dq[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[i][r] = 0.f;
  const int key = lane & 31;

  for (int k0 = 0; k0 < kend; k0 += kT) {
    __syncthreads();  // the previous tile's K, V and dS are no longer read
    stage_rows<D>(Ks, K + head, k0, N);
    stage_rows<D>(Vs, V + head, k0, N);
    __syncthreads();
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
    // S[q][key] = Q K^T and dP[q][key] = dO V^T (lane: key, registers: queries)
    mm<D>(s, [&](int m, int k) { return Qs[m * kLd + k]; }, [&](int k, int n) { return Ks[n * kLd + k]; });
    mm<D>(dp, [&](int m, int k) { return dOs[m * kLd + k]; }, [&](int k, int n) { return Vs[n * kLd + k]; });
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = acc_row(r, lane), qg = q0 + qr, kg = k0 + key;
      const bool ok = qg < N && kg < kv_lim && (!causal || kg <= qg);
      const float p = ok ? expf(fmaf(s[r], scale, -Ls[qr])) : 0.f;
      dSs[qr * (kT + 1) + key] = p * (dp[r] - Ds[qr]);
    }
    __syncthreads();
    // dQ[q][d] += dS[q][key] K[key][d]
#pragma unroll
    for (int db = 0; db < kDB; ++db)
      mm<kT>(dq[db], [&](int m, int k) { return dSs[m * (kT + 1) + k]; },
             [&](int k, int n) { return Ks[k * kLd + 32 * db + n]; });
  }
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qg = q0 + acc_row(r, lane);
      if (qg < N) dQ[head + (size_t)qg * D + 32 * db + key] = scale * dq[db][r];
    }
}

template <int D>
__global__ __launch_bounds__(64) void bwd_f32_dkdv_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE,
    const float* __restrict__ delta, float* __restrict__ dK, float* __restrict__ dV, int BH,
    int H, int N, float scale, int causal, const int* __restrict__ kv_len, int n_kblk) {
  constexpr int kLd = D + 1;
  constexpr int kDB = D / 32;
  __shared__ float Ks[kT * kLd], Vs[kT * kLd], Qs[kT * kLd], dOs[kT * kLd];
  __shared__ float Ps[kT * (kT + 1)], dSs[kT * (kT + 1)];
  __shared__ float Ls[kT], Ds[kT];
  const int bh = blockIdx.x / n_kblk, k0 = (blockIdx.x % n_kblk) * kT;
  const int b = bh / H;
  const size_t head = (size_t)bh * N * D;
  const int lane = threadIdx.x;
  int kv_lim = N;
  if (kv_len != nullptr) kv_lim = min(N, max(1, kv_len[b]));

  stage_rows<D>(Ks, K + head, k0, N);
  stage_rows<D>(Vs, V + head, k0, N);
  f32x16 dk[kDB], dv[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[i][r] = dv[i][r] = 0.f;
  const int key = lane & 31;
  // a block of padded keys sees nothing: its gradients stay zero
  const int qbeg = causal ? k0 : 0;
  const int qend = k0 < kv_lim ? N : 0;

  for (int q0 = qbeg - qbeg % kT; q0 < qend; q0 += kT) {
    __syncthreads();
    stage_rows<D>(Qs, Q + head, q0, N);
    stage_rows<D>(dOs, dO + head, q0, N);
    if (lane < kT) {
      const bool in = q0 + lane < N;
      Ls[lane] = in ? LSE[(size_t)bh * N + q0 + lane] : 0.f;
      Ds[lane] = in ? delta[(size_t)bh * N + q0 + lane] : 0.f;
    }
    __syncthreads();
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
    mm<D>(s, [&](int m, int k) { return Qs[m * kLd + k]; }, [&](int k, int n) { return Ks[n * kLd + k]; });
    mm<D>(dp, [&](int m, int k) { return dOs[m * kLd + k]; }, [&](int k, int n) { return Vs[n * kLd + k]; });
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = acc_row(r, lane), qg = q0 + qr, kg = k0 + key;
      const bool ok = qg < N && kg < kv_lim && (!causal || kg <= qg);
      const float p = ok ? expf(fmaf(s[r], scale, -Ls[qr])) : 0.f;
      Ps[qr * (kT + 1) + key] = p;
      dSs[qr * (kT + 1) + key] = p * (dp[r] - Ds[qr]);
    }
    __syncthreads();
    // dV[key][d] += P[q][key] dO[q][d], dK[key][d] += dS[q][key] Q[q][d]
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      mm<kT>(dv[db], [&](int m, int k) { return Ps[k * (kT + 1) + m]; },
             [&](int k, int n) { return dOs[k * kLd + 32 * db + n]; });
      mm<kT>(dk[db], [&](int m, int k) { return dSs[k * (kT + 1) + m]; },
             [&](int k, int n) { return Qs[k * kLd + 32 * db + n]; });
    }
  }
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kg = k0 + acc_row(r, lane);
      if (kg < N) {
        dK[head + (size_t)kg * D + 32 * db + key] = scale * dk[db][r];
        dV[head + (size_t)kg * D + 32 * db + key] = dv[db][r];
      }
    }
}

// D = rowsum(dO * O) for fp32 inputs, one row per thread, in element order (the dq
// kernel sums in the same order, so both routes give the same bits)
template <int D>
__global__ __launch_bounds__(256) void bwd_f32_pre_kernel(const float* __restrict__ dO,
                                                          const float* __restrict__ O,
                                                          float* __restrict__ delta, size_t rows) {
  const size_t r = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  float s = 0.f;
  for (int c = 0; c < D; ++c) s = fmaf(dO[r * D + c], O[r * D + c], s);
  delta[r] = s;
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t stream, int stages) {
  const int BH = a.B * a.H;
  const int nb = (a.N + kT - 1) / kT;
  const auto* q = static_cast<const float*>(a.q);
  const auto* k = static_cast<const float*>(a.k);
  const auto* v = static_cast<const float*>(a.v);
  const auto* g = static_cast<const float*>(a.dout);
  const size_t rows = (size_t)BH * a.N;
#define FA_F32_BWD(DIM)                                                                          \
  do {                                                                                           \
    if (stages & 1)                                                                              \
      hipLaunchKernelGGL((bwd_f32_pre_kernel<DIM>), dim3((unsigned)((rows + 255) / 256)),       \
                         dim3(256), 0, stream, g, a.o, a.delta, rows);                           \
    if (stages & 4)                                                                              \
      hipLaunchKernelGGL((bwd_f32_dq_kernel<DIM>), dim3(BH * nb), dim3(64), 0, stream, q, k, v, \
                         g, a.o, a.lse, a.delta, (stages & 8) ? 1 : 0, a.dq, BH, a.H, a.N,     \
                         a.scale, a.causal, a.kv_len, nb);                                       \
    if (stages & 2)                                                                              \
      hipLaunchKernelGGL((bwd_f32_dkdv_kernel<DIM>), dim3(BH * nb), dim3(64), 0, stream, q, k, \
                         v, g, a.lse, a.delta, a.dk, a.dv, BH, a.H, a.N, a.scale, a.causal,     \
                         a.kv_len, nb);                                                          \
  } while (0)
  if (a.d == 64) FA_F32_BWD(64); else FA_F32_BWD(128);
#undef FA_F32_BWD
  return hipGetLastError();
}

}  // namespace fa
