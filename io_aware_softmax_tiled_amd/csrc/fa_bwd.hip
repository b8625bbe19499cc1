// Backward pass of exact attention on gfx950.
//
// "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness", Key
// ideas (recomputation in the backward pass): only O and the softmax statistics are
// kept from the forward pass; S and P are rebuilt block by block on chip. Here the
// statistics are the per-row LSE, so P = exp(scale*q.k - LSE) is already normalised.
// The gradient formulas are the chain rule of L = sum(dO * O) (the pages do not print
// them): dV = P^T dO, dP = dO V^T, D_i = sum_k dO_ik O_ik, dS = P * (dP - D),
// dQ = scale * dS K, dK = scale * dS^T Q.
//
// Kernels:
// 1. bwd_pre: D_i = rowsum(dO * O) into the workspace, and dq := 0.
// 2. bwd_main: one workgroup per 128 keys of one (batch, head), 32 keys per wave. The
//    loop runs over 32-query tiles (for causal attention, from the first tile that
//    reaches the block's keys). Per tile each wave recomputes S = Q K^T and
//    dP = dO V^T with keys on lanes, forms P and dS in registers, accumulates
//    dV^T += dO^T P and dK^T += Q^T dS in registers, publishes dS^T through LDS, and
//    then contributes dQ = dS K for the tile, added to dq with fp32 atomics.
//
// Precision: every matrix-core product runs in fp16 with fp32 accumulation. bf16
// inputs are converted to fp16 when staged (exact for magnitudes in the fp16 normal
// range); P and dS are rounded to fp16, whose 11-bit significand keeps dK and dQ well
// inside the bf16 tolerance where bf16 rounding of dS would not.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 128;  // keys per workgroup
constexpr int kBQ = 32;   // queries per iteration

__device__ inline int kappa(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// 8 input elements (16 bytes of bf16 or f16) -> 8 fp16 (16 bytes)
template <typename T> __device__ inline u32x4 to_f16x8(u32x4 x);
template <> __device__ inline u32x4 to_f16x8<F16>(u32x4 x) { return x; }
template <> __device__ inline u32x4 to_f16x8<BF16>(u32x4 x) {
  return {bf16x2_to_f16x2(x[0]), bf16x2_to_f16x2(x[1]), bf16x2_to_f16x2(x[2]),
          bf16x2_to_f16x2(x[3])};
}

template <typename T> __device__ inline float to_f32(uint16_t x);
template <> __device__ inline float to_f32<BF16>(uint16_t x) {
  return __uint_as_float((uint32_t)x << 16);
}
template <> __device__ inline float to_f32<F16>(uint16_t x) {
  return (float)__builtin_bit_cast(_Float16, x);
}

// byte offset in the dS^T tile [128 keys][32 queries] fp16 (64-byte rows): the
// 16-byte chunk index is XORed with bits 2..3 of the row.
__device__ inline int dst_off(int row, int byte) {
  return row * 64 + (byte ^ (((row >> 2) & 3) << 4));
}

// ---------------------------------------------------------------------------------
// 1. D = rowsum(dO * O), dq = 0. One thread per 8 elements; D/8 threads per row.
// ---------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(
    const uint16_t* __restrict__ dO, const float* __restrict__ O, float* __restrict__ delta,
    float* __restrict__ dQ, size_t rows) {
  constexpr int kTPR = D / 8;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t row = idx / kTPR;
  float s = 0.f;
  if (row < rows) {
    const u32x4 g = *reinterpret_cast<const u32x4*>(dO + idx * 8);
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(O + idx * 8);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(O + idx * 8 + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = to_f32<T>((uint16_t)(g[j] & 0xffff));
      const float hi = to_f32<T>((uint16_t)(g[j] >> 16));
      const float olo = j < 2 ? o0[2 * j] : o1[2 * j - 4];
      const float ohi = j < 2 ? o0[2 * j + 1] : o1[2 * j - 3];
      s = fmaf(lo, olo, s);
      s = fmaf(hi, ohi, s);
    }
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(dQ + idx * 8) = z;
    *reinterpret_cast<f32x4*>(dQ + idx * 8 + 4) = z;
  }
#pragma unroll
  for (int off = kTPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kTPR);
  if (row < rows && (threadIdx.x % kTPR) == 0) delta[row] = s;
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel_f32(
    const float* __restrict__ dO, const float* __restrict__ O, float* __restrict__ delta,
    float* __restrict__ dQ, size_t rows) {
  constexpr int kTPR = D / 8;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t row = idx / kTPR;
  float s = 0.f;
  if (row < rows) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x4 g = *reinterpret_cast<const f32x4*>(dO + idx * 8 + 4 * j);
      const f32x4 o = *reinterpret_cast<const f32x4*>(O + idx * 8 + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fmaf(g[e], o[e], s);
    }
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(dQ + idx * 8) = z;
    *reinterpret_cast<f32x4*>(dQ + idx * 8 + 4) = z;
  }
#pragma unroll
  for (int off = kTPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kTPR);
  if (row < rows && (threadIdx.x % kTPR) == 0) delta[row] = s;
}

// ---------------------------------------------------------------------------------
// 2. main backward kernel, 16-bit inputs
// ---------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_main_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ delta, float* __restrict__ dQ,
    float* __restrict__ dK, float* __restrict__ dV, int BH, int H, int N, float scale,
    float sl2, int causal, const int* __restrict__ kv_len, int n_kblk, int heads_per_xcd) {
  constexpr int kKC = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kCPR = D / 8;  // 16-byte chunks per row
  __shared__ __attribute__((aligned(1024))) uint8_t Ks[kBK * D * 2];
  __shared__ __attribute__((aligned(1024))) uint8_t Qs[kBQ * D * 2];
  __shared__ __attribute__((aligned(1024))) uint8_t dOs[kBQ * D * 2];
  __shared__ __attribute__((aligned(1024))) uint8_t dSt[kBK * kBQ * 2];
  __shared__ __attribute__((aligned(16))) float lse_s[kBQ];
  __shared__ __attribute__((aligned(16))) float dlt_s[kBQ];

  // workgroup -> (head, key block): XCD-major; key block 0 (the most query tiles
  // under a causal mask) first
  const int w = blockIdx.x;
  const int xcd = w & 7, slot = w >> 3;
  const int bh = (slot % heads_per_xcd) * 8 + xcd;
  const int kblk = slot / heads_per_xcd;
  if (bh >= BH || kblk >= n_kblk) return;
  const int b = bh / H;
  const size_t head = (size_t)bh * N * D;
  int kv_lim = N;
  if (kv_len != nullptr) kv_lim = min(N, max(1, kv_len[b]));
  const int k0 = kblk * kBK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int li = lane & 31, hh = lane >> 5;
  const int g = lane >> 4, gi = lane & 15;
  const int kw0 = k0 + 32 * wave;   // first key of this wave
  const int key = kw0 + li;         // this lane's key in accumulator layouts

  if (k0 >= kv_lim) {
    // every key of the block is padded: zero gradients
    for (int e = tid; e < kBK * D / 4; e += kThreads) {
      const int row = e / (D / 4), c4 = e % (D / 4);
      if (k0 + row < N) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(dK + head + (size_t)(k0 + row) * D + 4 * c4) = z;
        *reinterpret_cast<f32x4*>(dV + head + (size_t)(k0 + row) * D + 4 * c4) = z;
      }
    }
    return;
  }

  // K block -> LDS (fp16, swizzled rows): B operand source of dQ = dS K
  for (int ci = tid; ci < kBK * kCPR; ci += kThreads) {
    const int row = ci / kCPR, ch = ci % kCPR;
    const size_t goff = head + (size_t)min(k0 + row, N - 1) * D + ch * 8;
    lds_write16((FA_LDS uint8_t*)Ks + tile_off<D>(row, ch),
                to_f16x8<T>(*reinterpret_cast<const u32x4*>(K + goff)));
  }
  // this lane's key row of K and V as B operands (fp16): [key][16c + 8hh + 0..7]
  u32x4 kf[kKC], vf[kKC];
  {
    const size_t roff = head + (size_t)min(key, N - 1) * D;
#pragma unroll
    for (int c = 0; c < kKC; ++c) {
      kf[c] = to_f16x8<T>(*reinterpret_cast<const u32x4*>(K + roff + 16 * c + 8 * hh));
      vf[c] = to_f16x8<T>(*reinterpret_cast<const u32x4*>(V + roff + 16 * c + 8 * hh));
    }
  }

  f32x16 dkacc[kDB], dvacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkacc[i][r] = 0.f;
      dvacc[i][r] = 0.f;
    }

  const bool wave_dead = kw0 >= kv_lim;
  const int nq = (N + kBQ - 1) / kBQ;
  const int i0 = causal ? k0 / kBQ : 0;
  const int arow = kappa(li);  // A-operand row (query) read by this lane
  const FA_LDS uint8_t* Qsl = (const FA_LDS uint8_t*)Qs;
  const FA_LDS uint8_t* dOsl = (const FA_LDS uint8_t*)dOs;
  const FA_LDS uint8_t* Ksl = (const FA_LDS uint8_t*)Ks;
  FA_LDS uint8_t* dStl = (FA_LDS uint8_t*)dSt;

  for (int it = i0; it < nq; ++it) {
    const int q0 = it * kBQ;
    // stage Q and dO tiles (fp16), the LSE (log2 units) and D of the tile
    for (int ci = tid; ci < kBQ * kCPR; ci += kThreads) {
      const int row = ci / kCPR, ch = ci % kCPR;
      const size_t goff = head + (size_t)min(q0 + row, N - 1) * D + ch * 8;
      lds_write16((FA_LDS uint8_t*)Qs + tile_off<D>(row, ch),
                  to_f16x8<T>(*reinterpret_cast<const u32x4*>(Q + goff)));
      lds_write16((FA_LDS uint8_t*)dOs + tile_off<D>(row, ch),
                  to_f16x8<T>(*reinterpret_cast<const u32x4*>(dO + goff)));
    }
    if (tid < kBQ) {
      const size_t r = (size_t)bh * N + min(q0 + tid, N - 1);
      lse_s[tid] = LSE[r] * kLog2e;
      dlt_s[tid] = delta[r];
    }
    __syncthreads();

    const bool active = !wave_dead && !(causal && kw0 > q0 + kBQ - 1);
    if (active) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < kKC; ++c) {
        const int off = tile_off<D>(arow, 2 * c + hh);
        s = Mfma<F16>::run(lds_read16(Qsl + off), kf[c], s);
        dp = Mfma<F16>::run(lds_read16(dOsl + off), vf[c], dp);
      }
      // lane (key, hh), register r <-> query q0 + 16*(r/8) + 8*hh + r%8
      const bool need_mask = (causal && kw0 + 31 > q0) || (q0 + kBQ > N) || (kw0 + 32 > kv_lim);
      uint32_t pp[8], dsp[8];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int qb = 16 * c + 8 * hh;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(&lse_s[qb]);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(&lse_s[qb + 4]);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&dlt_s[qb]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&dlt_s[qb + 4]);
        float p[8], ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * c + j;
          const float lq = j < 4 ? l0[j] : l1[j - 4];
          const float dq = j < 4 ? d0[j] : d1[j - 4];
          float pj = exp2_fast(fmaf(s[r], sl2, -lq));
          if (need_mask) {
            const int qq = q0 + qb + j;
            const bool hide = qq >= N || key >= kv_lim || (causal && key > qq);
            pj = hide ? 0.f : pj;
          }
          p[j] = pj;
          ds[j] = pj * (dp[r] - dq);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pp[4 * c + j] = Mfma<F16>::pack(p[2 * j], p[2 * j + 1]);
          dsp[4 * c + j] = Mfma<F16>::pack(ds[2 * j], ds[2 * j + 1]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS; A operands through the transposing read
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x4 bp = {pp[4 * c], pp[4 * c + 1], pp[4 * c + 2], pp[4 * c + 3]};
        const u32x4 bs = {dsp[4 * c], dsp[4 * c + 1], dsp[4 * c + 2], dsp[4 * c + 3]};
        const int trow = 16 * c + 8 * hh + (gi >> 2);
        const int inner = 8 * (gi & 1);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const int ch = db * 4 + 2 * (g & 1) + ((gi & 3) >> 1);
          const u32x2 a0 = lds_read_tr16(dOsl + tile_off<D>(trow, ch) + inner);
          const u32x2 a1 = lds_read_tr16(dOsl + tile_off<D>(trow + 4, ch) + inner);
          dvacc[db] = Mfma<F16>::run(u32x4{a0[0], a0[1], a1[0], a1[1]}, bp, dvacc[db]);
          const u32x2 b0 = lds_read_tr16(Qsl + tile_off<D>(trow, ch) + inner);
          const u32x2 b1 = lds_read_tr16(Qsl + tile_off<D>(trow + 4, ch) + inner);
          dkacc[db] = Mfma<F16>::run(u32x4{b0[0], b0[1], b1[0], b1[1]}, bs, dkacc[db]);
        }
      }
      // publish dS^T: row = key (block-local), queries 16c + 8hh + 0..7
#pragma unroll
      for (int c = 0; c < 2; ++c)
        lds_write16(dStl + dst_off(32 * wave + li, 32 * c + 16 * hh),
                    u32x4{dsp[4 * c], dsp[4 * c + 1], dsp[4 * c + 2], dsp[4 * c + 3]});
    } else {
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int c = 0; c < 2; ++c) lds_write16(dStl + dst_off(32 * wave + li, 32 * c + 16 * hh), z);
    }
    __syncthreads();

    // dQ[q0 .. q0+31][d-block] += scale * dS K over this block's keys
    {
      const int db = wave % kDB;
      const int nparts = 4 / kDB;              // waves sharing one d-block
      const int part = wave / kDB;
      const int kpp = kBK / nparts;            // keys per part
      const bool any_live = !(causal && k0 + part * kpp > q0 + kBQ - 1) && (k0 + part * kpp < kv_lim);
      if (any_live) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        const int dch = db * 4 + 2 * (g & 1) + ((gi & 3) >> 1);
        const int sbyte = 32 * (g & 1) + 8 * (gi & 3);
        const int kinner = 8 * (gi & 1);
#pragma unroll
        for (int c = 0; c < kpp / 16; ++c) {
          const int krow = part * kpp + 16 * c + 8 * hh + (gi >> 2);
          const u32x2 a0 = lds_read_tr16(dStl + dst_off(krow, sbyte));
          const u32x2 a1 = lds_read_tr16(dStl + dst_off(krow + 4, sbyte));
          const u32x2 b0 = lds_read_tr16(Ksl + tile_off<D>(krow, dch) + kinner);
          const u32x2 b1 = lds_read_tr16(Ksl + tile_off<D>(krow + 4, dch) + kinner);
          acc = Mfma<F16>::run(u32x4{a0[0], a0[1], a1[0], a1[1]}, u32x4{b0[0], b0[1], b1[0], b1[1]},
                               acc);
        }
        // lane (d = 32db + li, hh), register r <-> query q0 + 8*(r/4) + 4*hh + r%4
        float* dqb = dQ + head + 32 * db + li;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qq = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (qq < N) unsafeAtomicAdd(dqb + (size_t)qq * D, scale * acc[r]);
        }
      }
    }
    __syncthreads();
  }

  // dK = scale * dK_acc, dV = dV_acc: lane (key, hh), register r <-> d = 32db + 8(r/4) + 4hh + r%4
  if (key < N) {
    float* dkr = dK + head + (size_t)key * D;
    float* dvr = dV + head + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * db + 8 * a4 + 4 * hh;
        const f32x4 kk = {scale * dkacc[db][4 * a4], scale * dkacc[db][4 * a4 + 1],
                          scale * dkacc[db][4 * a4 + 2], scale * dkacc[db][4 * a4 + 3]};
        const f32x4 vv = {dvacc[db][4 * a4], dvacc[db][4 * a4 + 1], dvacc[db][4 * a4 + 2],
                          dvacc[db][4 * a4 + 3]};
        *reinterpret_cast<f32x4*>(dkr + d0) = kk;
        *reinterpret_cast<f32x4*>(dvr + d0) = vv;
      }
  }
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  const size_t bytes = (size_t)B * H * N * sizeof(float);
  return (bytes + 255) / 256 * 256;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  const int BH = a.B * a.H;
  const size_t rows = (size_t)BH * a.N;
  const size_t pre_threads = rows * (a.d / 8);
  const int pre_blocks = (int)((pre_threads + kThreads - 1) / kThreads);
  const float sl2 = a.scale * kLog2e;
  if (a.dtype == kDtypeF32) return hipErrorNotSupported;  // rejected by the API layer
  const auto* dO16 = static_cast<const uint16_t*>(a.dout);
#define FA_PRE(TAG, DIM)                                                                  \
  hipLaunchKernelGGL((bwd_pre_kernel<TAG, DIM>), dim3(pre_blocks), dim3(kThreads), 0, stream, \
                     dO16, a.o, a.delta, a.dq, rows)
  if (a.dtype == kDtypeBF16) {
    if (a.d == 64) FA_PRE(BF16, 64); else FA_PRE(BF16, 128);
  } else {
    if (a.d == 64) FA_PRE(F16, 64); else FA_PRE(F16, 128);
  }
#undef FA_PRE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int n_kblk = (a.N + kBK - 1) / kBK;
  const int hpx = (BH + 7) / 8;
  const int blocks = 8 * hpx * n_kblk;
  const auto* q16 = static_cast<const uint16_t*>(a.q);
  const auto* k16 = static_cast<const uint16_t*>(a.k);
  const auto* v16 = static_cast<const uint16_t*>(a.v);
#define FA_MAIN(TAG, DIM)                                                                   \
  hipLaunchKernelGGL((bwd_main_kernel<TAG, DIM>), dim3(blocks), dim3(kThreads), 0, stream, \
                     q16, k16, v16, dO16, a.lse, a.delta, a.dq, a.dk, a.dv, BH, a.H, a.N,   \
                     a.scale, sl2, a.causal, a.kv_len, n_kblk, hpx)
  if (a.dtype == kDtypeBF16) {
    if (a.d == 64) FA_MAIN(BF16, 64); else FA_MAIN(BF16, 128);
  } else {
    if (a.d == 64) FA_MAIN(F16, 64); else FA_MAIN(F16, 128);
  }
#undef FA_MAIN
  return hipGetLastError();
}

}  // namespace fa
