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
// Kernels (no atomics; every output is written once, so all of them are deterministic):
// 1. bwd_pre: D_i = rowsum(dO * O) into the workspace.
// 2. bwd_dkdv: one workgroup per 128 keys of one (batch, head), 32 keys per wave, keys
//    on lanes. It loops over 64-query tiles (causal: from the block's diagonal on),
//    recomputes S = Q K^T and dP = dO V^T, forms P and dS in registers, and accumulates
//    dV^T += dO^T P and dK^T += Q^T dS in registers (dO^T and Q^T through the
//    transposing LDS read). Q/dO tiles are prefetched one tile ahead through buffer
//    resources and double-buffered: one barrier per tile, waiting for LDS traffic
//    only.
// 3. bwd_dq: one workgroup per 128 queries, 32 per wave, queries on lanes -- the
//    forward kernel's layout. Per 64-key tile it recomputes S^T = K Q^T and
//    dP^T = V dO^T, forms dS^T in registers and accumulates dQ^T += K^T dS^T (K^T
//    through the transposing LDS read). Recomputing S and dP here costs two extra
//    products per score, in exchange for no fp32 atomics on dq and no dS round trip
//    through LDS.
//
// Precision: every matrix-core product runs in fp16 with fp32 accumulation. bf16
// inputs are converted to fp16 when staged (exact for magnitudes in the fp16 normal
// range); P and dS are rounded to fp16, whose 11-bit significand keeps dK and dQ well
// inside the bf16 tolerance where bf16 rounding of dS would not.
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kThreads = 256;

template <typename T> __device__ inline float to_f32(uint16_t x);
template <> __device__ inline float to_f32<BF16>(uint16_t x) {
  return __uint_as_float((uint32_t)x << 16);
}
template <> __device__ inline float to_f32<F16>(uint16_t x) {
  return (float)__builtin_bit_cast(_Float16, x);
}

// ---------------------------------------------------------------------------------
// 1. D = rowsum(dO * O). One thread per 8 elements; D/8 threads per row.
// ---------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(
    const uint16_t* __restrict__ dO, const float* __restrict__ O, float* __restrict__ delta,
    size_t rows) {
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
  }
#pragma unroll
  for (int off = kTPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kTPR);
  if (row < rows && (threadIdx.x % kTPR) == 0) delta[row] = s;
}

// ---------------------------------------------------------------------------------
// 2. dK, dV: keys on lanes
// ---------------------------------------------------------------------------------
constexpr int kBK = 128;  // keys per workgroup
constexpr int kBQ = 64;   // queries per tile (two 32-query halves)

// kSparse: bmask is the n_sb x n_sb byte matrix over 128-query x 128-key blocks (this
// workgroup's 128 keys are one key block); query tiles in disabled blocks are skipped.
constexpr int kSparseBlock = 128;
constexpr int kSparseMaxBlocks = 2048;  // blocks per row/column of the mask (N <= 2^18)

// kDropout: the probabilities carry the forward pass's dropout mask Z, regenerated here
// from the same Philox4x32-10 blocks (element (i, 32 g + u) of head bh: byte
// 8 (u / 16) + u % 8 of the block at counter (i, 2 g + (u / 8) % 2, bh, offset); kept
// iff >= drop_t):
// dV = (P Z / keep)^T dO, dP = (Z / keep) (dO V^T), dS = P (dP - D).
template <typename T, int D, bool kSparse, bool kDropout>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ delta, float* __restrict__ dK,
    float* __restrict__ dV, int BH, int H, int N, float scale, float sl2, int causal,
    const int* __restrict__ kv_len, int n_kblk, int heads_per_xcd,
    const uint8_t* __restrict__ bmask, int n_sb, uint32_t seed_lo, uint32_t seed_hi,
    uint32_t offset, int drop_t, float keep_scale) {
  constexpr int kKC = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kCPR = D / 8;                        // 16-byte chunks per row
  constexpr int kTile = kBQ * D * 2;                 // one Q or dO tile (fp16), bytes
  constexpr int kSC = kTile / 16 / kThreads;         // staged chunks per thread per tensor
  __shared__ __attribute__((aligned(1024))) uint8_t Qb0[kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t Qb1[kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t Ob0[kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t Ob1[kTile];
  __shared__ __attribute__((aligned(16))) float St0[2 * kBQ];  // LSE*log2(e), then D
  __shared__ __attribute__((aligned(16))) float St1[2 * kBQ];
  __shared__ uint16_t tlist[kSparse ? 2 * kSparseMaxBlocks : 1];  // enabled query tiles
  __shared__ int tlist_len;
  // dropout: each wave's random bytes of the current tile, [query][its 32 keys]
  __shared__ __attribute__((aligned(16))) uint8_t zbuf[kDropout ? 4 * kBQ * 32 : 16];

  const WgPos pos = wg_position(heads_per_xcd, blockIdx.x, BH);
  const int kblk = pos.blk;  // key block 0 has the most query tiles under a causal mask
  if (pos.bh >= BH || kblk >= n_kblk) return;
  const int bh = pos.bh;
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

  const int nq = (N + kBQ - 1) / kBQ;
  const int i0 = causal ? k0 / kBQ : 0;
  // the query tiles this workgroup visits: i0 .. nq-1, or (sparse) those of them in
  // query blocks enabled for this key block, listed by wave 0
  int nt = max(nq - i0, 0);
  if constexpr (kSparse) {
    if (wave == 0) {
      int count = 0;
      for (int base = i0; base < nq; base += 64) {
        const int it = base + lane;
        const bool on = it < nq && bmask[(size_t)(it * kBQ / kSparseBlock) * n_sb + kblk] != 0;
        const uint64_t m = __ballot(on);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (on) tlist[count + before] = (uint16_t)it;
        count += __popcll(m);
      }
      if (lane == 0) tlist_len = count;
    }
    __syncthreads();
    nt = tlist_len;
  }
  auto tile_at = [&](int s) {
    if constexpr (kSparse) return __builtin_amdgcn_readfirstlane((int)tlist[s]);
    else return i0 + s;
  };

  // staging of query tile `it` through registers (coalesced 16-byte loads)
  u32x4 qs[kSC], os[kSC];
  float s_lse = 0.f, s_dlt = 0.f;
  // loads go through buffer resources placed at the tile: rows past the end of the
  // sequence read as zeros, and moving to the next tile is scalar arithmetic
  uint32_t ld_off[kSC];
#pragma unroll
  for (int j = 0; j < kSC; ++j) {
    const int ci = tid + kThreads * j;
    ld_off[j] = (uint32_t)((ci / kCPR) * D + (ci % kCPR) * 8) * 2;
  }
  auto load_tile = [&](int it) {
    const int q0 = it * kBQ;
    const uint32_t bytes = (uint32_t)(N - q0) * D * 2;
    const auto rq = buffer_rsrc(Q + head + (size_t)q0 * D, bytes);
    const auto ro = buffer_rsrc(dO + head + (size_t)q0 * D, bytes);
#pragma unroll
    for (int j = 0; j < kSC; ++j) {
      qs[j] = buffer_load16(rq, ld_off[j]);
      os[j] = buffer_load16(ro, ld_off[j]);
    }
    if (tid < kBQ) {
      const size_t r = (size_t)bh * N + min(q0 + tid, N - 1);
      // a row that sees no key (LSE = -inf, block-sparse) must give P = 0: +inf here
      const float l = LSE[r];
      s_lse = l == -INFINITY ? INFINITY : l * kLog2e;
      s_dlt = delta[r];
    }
  };
  auto store_tile = [&](FA_LDS uint8_t* qb, FA_LDS uint8_t* ob, FA_LDS float* st) {
#pragma unroll
    for (int j = 0; j < kSC; ++j) {
      const int ci = tid + kThreads * j;
      const int row = ci / kCPR, ch = ci % kCPR;
      lds_write16(qb + tile_off<D>(row, ch), to_f16x8<T>(qs[j]));
      lds_write16(ob + tile_off<D>(row, ch), to_f16x8<T>(os[j]));
    }
    if (tid < kBQ) {
      st[tid] = s_lse;
      st[kBQ + tid] = s_dlt;
    }
  };

  if (nt > 0) load_tile(tile_at(0));

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

  // Per-lane byte offsets inside a Q or dO tile, fixed for the whole loop (the
  // swizzle depends on the low 4 bits of the row only, so 16- and 32-row steps and
  // the buffer choice are immediate offsets).
  int aoff[kKC];  // A-operand rows (queries, order kappa) for S = Q K^T and dP = dO V^T
#pragma unroll
  for (int c = 0; c < kKC; ++c) aoff[c] = tile_off<D>(kappa(li), 2 * c + hh);
  int toff[2][kDB];  // transposing reads of dO^T and Q^T
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int db = 0; db < kDB; ++db)
      toff[r][db] = tile_off<D>(8 * hh + (gi >> 2) + 4 * r, db * 4 + 2 * (g & 1) + ((gi & 3) >> 1)) +
                    8 * (gi & 1);

  if (nt > 0) store_tile((FA_LDS uint8_t*)Qb0, (FA_LDS uint8_t*)Ob0, (FA_LDS float*)St0);

  // S = Q K^T and dP = dO V^T for the 32 queries of half `hf`:
  // lane (key, hh), register r <-> query q0 + 32*hf + 16*(r/8) + 8*hh + r%8
  auto products = [&](const FA_LDS uint8_t* Qc, const FA_LDS uint8_t* Oc, int hf, f32x16& s,
                      f32x16& dp) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < kKC; ++c) {
      const int off = aoff[c] + hf * 32 * D * 2;
      s = Mfma<F16>::run(lds_read16(Qc + off), kf[c], s);
      dp = Mfma<F16>::run(lds_read16(Oc + off), vf[c], dp);
    }
  };
  // -inf where the query does not see this lane's key (diagonal, padding, sequence end)
  auto mask = [&](f32x16& s, int q0, int hf) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qq = q0 + 32 * hf + 16 * (r >> 3) + 8 * hh + (r & 7);
      const bool hide = qq >= N || key >= kv_lim || (causal && key > qq);
      s[r] = hide ? -INFINITY : s[r];
    }
  };
  FA_LDS uint8_t* zw = (FA_LDS uint8_t*)zbuf + (kDropout ? wave * kBQ * 32 : 0);  // wave bytes
  // P and dS for half `hf` (masked scores are -inf, so P = dS = 0 there), packed fp16
  auto p_ds = [&](const FA_LDS float* Stc, int hf, const f32x16& s, const f32x16& dp,
                  uint32_t (&pp)[8], uint32_t (&dsp)[8]) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int qb = 32 * hf + 16 * c + 8 * hh;
      const f32x4 l0 = *reinterpret_cast<const FA_LDS f32x4*>(&Stc[qb]);
      const f32x4 l1 = *reinterpret_cast<const FA_LDS f32x4*>(&Stc[qb + 4]);
      const f32x4 d0 = *reinterpret_cast<const FA_LDS f32x4*>(&Stc[kBQ + qb]);
      const f32x4 d1 = *reinterpret_cast<const FA_LDS f32x4*>(&Stc[kBQ + qb + 4]);
      float p[8], ds[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * c + j;
        const float lq = j < 4 ? l0[j] : l1[j - 4];
        const float dq = j < 4 ? d0[j] : d1[j - 4];
        const float pj = exp2_fast(fmaf(s[r], sl2, -lq));
        if constexpr (kDropout) {
          // byte of (query qb + j of the tile, this lane's key)
          const bool keep = (int)zw[(qb + j) * 32 + li] >= drop_t;
          p[j] = keep ? pj : 0.f;                      // dV takes P Z (1/keep at the end)
          ds[j] = pj * ((keep ? dp[r] * keep_scale : 0.f) - dq);
        } else {
          p[j] = pj;
          ds[j] = pj * (dp[r] - dq);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pp[4 * c + j] = Mfma<F16>::pack(p[2 * j], p[2 * j + 1]);
        dsp[4 * c + j] = Mfma<F16>::pack(ds[2 * j], ds[2 * j + 1]);
      }
    }
  };
  // dV^T += dO^T P and dK^T += Q^T dS for half `hf`
  auto accumulate = [&](const FA_LDS uint8_t* Qc, const FA_LDS uint8_t* Oc, int hf,
                        const uint32_t (&pp)[8], const uint32_t (&dsp)[8]) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const u32x4 bp = {pp[4 * c], pp[4 * c + 1], pp[4 * c + 2], pp[4 * c + 3]};
      const u32x4 bs = {dsp[4 * c], dsp[4 * c + 1], dsp[4 * c + 2], dsp[4 * c + 3]};
      const int rows = (32 * hf + 16 * c) * D * 2;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const u32x2 a0 = lds_read_tr16(Oc + toff[0][db] + rows);
        const u32x2 a1 = lds_read_tr16(Oc + toff[1][db] + rows);
        dvacc[db] = Mfma<F16>::run(u32x4{a0[0], a0[1], a1[0], a1[1]}, bp, dvacc[db]);
        const u32x2 b0 = lds_read_tr16(Qc + toff[0][db] + rows);
        const u32x2 b1 = lds_read_tr16(Qc + toff[1][db] + rows);
        dkacc[db] = Mfma<F16>::run(u32x4{b0[0], b0[1], b1[0], b1[1]}, bs, dkacc[db]);
      }
    }
  };
  // keeps P and dS in the region that computes them (the compiler would otherwise sink
  // them past the masking branch into the product that uses them, losing the overlap)
  auto pin = [&](const uint32_t (&pp)[8], const uint32_t (&dsp)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(pp[i]), "v"(dsp[i]));
  };
  // each of the region's 4*kDB or 2*kKC MFMAs followed by its share of the ~90 vector
  // instructions of p_ds and of the LDS reads
  auto hint = [&](auto n_mfma, auto n_ds) {
    constexpr int kM = decltype(n_mfma)::value;
    constexpr int kDs = decltype(n_ds)::value;
#pragma unroll
    for (int i = 0; i < kM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, kDs / kM, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, (96 + kM - 1) / kM, 0);
    }
  };

  // One 64-query tile: publish it (barrier), prefetch the next one, then (head_dim 64)
  // three regions that keep the matrix cores busy while the vector units form P and dS:
  //   products of half 0 | products of half 1 with P, dS of half 0 |
  //   dV, dK products of half 0 with P, dS of half 1 | dV, dK products of half 1.
  auto step = [&](int s, const FA_LDS uint8_t* Qc, const FA_LDS uint8_t* Oc,
                  const FA_LDS float* Stc, FA_LDS uint8_t* Qn, FA_LDS uint8_t* On,
                  FA_LDS float* Stn) {
    barrier_lds();  // tile s visible; the other buffers are free
    load_tile(tile_at(min(s + 1, nt - 1)));  // unconditional: same loads on every path
    const int q0 = tile_at(s) * kBQ;
    // a tile entirely above this wave's keys' diagonal (or a wave whose keys are all
    // padded) is skipped; otherwise both halves run, and a half hidden from every key is
    // masked to P = 0 like any other hidden entry (one code path: no accumulator copies)
    const bool active = !wave_dead && !(causal && kw0 > q0 + kBQ - 1);
    const bool need_mask =
        (causal && kw0 + 31 > q0) || (q0 + kBQ > N) || (kw0 + 32 > kv_lim);
    if (kDropout && active) {
      // lane l draws the two blocks of (query q0 + l, this wave's 32 keys) and stores
      // the 32 bytes in key order for the wave (keys 0-7: bytes 0-7 of the first block,
      // 8-15: of the second, 16-23: bytes 8-15 of the first, 24-31: of the second);
      // each lane then reads the bytes of its own key
      const uint32_t qg = (uint32_t)(q0 + lane), kb = (uint32_t)(2 * (kw0 >> 5));
      const Philox4x32 b0 = philox4x32(qg, kb, (uint32_t)bh, offset, seed_lo, seed_hi);
      const Philox4x32 b1 = philox4x32(qg, kb + 1, (uint32_t)bh, offset, seed_lo, seed_hi);
      lds_write16(zw + lane * 32, u32x4{b0.w[0], b0.w[1], b1.w[0], b1.w[1]});
      lds_write16(zw + lane * 32 + 16, u32x4{b0.w[2], b0.w[3], b1.w[2], b1.w[3]});
    }
    if (active) {
      f32x16 s0, dp0, s1, dp1;
      uint32_t pp0[8], ds0[8], pp1[8], ds1[8];
      if constexpr (D == 64) {
        // three overlapped regions (see above)
        products(Qc, Oc, 0, s0, dp0);
        if (need_mask) mask(s0, q0, 0);
        products(Qc, Oc, 1, s1, dp1);
        p_ds(Stc, 0, s0, dp0, pp0, ds0);
        hint(std::integral_constant<int, 2 * kKC>{}, std::integral_constant<int, 2 * kKC + 4>{});
        pin(pp0, ds0);
        if (need_mask) mask(s1, q0, 1);
        accumulate(Qc, Oc, 0, pp0, ds0);
        p_ds(Stc, 1, s1, dp1, pp1, ds1);
        hint(std::integral_constant<int, 4 * kDB>{}, std::integral_constant<int, 8 * kDB + 4>{});
        pin(pp1, ds1);
        accumulate(Qc, Oc, 1, pp1, ds1);
      } else {
        // head_dim 128: both halves' products first, then P/dS and the dV/dK products
        // per half, scheduled by the compiler (the overlapped regions measured slower
        // here: twice the vector work per matrix product and the accumulators in AGPRs)
        products(Qc, Oc, 0, s0, dp0);
        products(Qc, Oc, 1, s1, dp1);
        if (need_mask) {
          mask(s0, q0, 0);
          mask(s1, q0, 1);
        }
        p_ds(Stc, 0, s0, dp0, pp0, ds0);
        accumulate(Qc, Oc, 0, pp0, ds0);
        p_ds(Stc, 1, s1, dp1, pp1, ds1);
        accumulate(Qc, Oc, 1, pp1, ds1);
      }
    }
    store_tile(Qn, On, Stn);  // tile it+1 (clamped) into the free buffers
  };

  for (int s = 0; s < nt; s += 2) {
    step(s, (const FA_LDS uint8_t*)Qb0, (const FA_LDS uint8_t*)Ob0, (const FA_LDS float*)St0,
         (FA_LDS uint8_t*)Qb1, (FA_LDS uint8_t*)Ob1, (FA_LDS float*)St1);
    if (s + 1 < nt)
      step(s + 1, (const FA_LDS uint8_t*)Qb1, (const FA_LDS uint8_t*)Ob1,
           (const FA_LDS float*)St1, (FA_LDS uint8_t*)Qb0, (FA_LDS uint8_t*)Ob0,
           (FA_LDS float*)St0);
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
        const float vs = kDropout ? keep_scale : 1.0f;
        const f32x4 vv = {vs * dvacc[db][4 * a4], vs * dvacc[db][4 * a4 + 1],
                          vs * dvacc[db][4 * a4 + 2], vs * dvacc[db][4 * a4 + 3]};
        *reinterpret_cast<f32x4*>(dkr + d0) = kk;
        *reinterpret_cast<f32x4*>(dvr + d0) = vv;
      }
  }
}

// ---------------------------------------------------------------------------------
// 3. dQ: queries on lanes (the forward kernel's layout)
// ---------------------------------------------------------------------------------
constexpr int kBM = 128;  // queries per workgroup
constexpr int kBN = 64;   // keys per tile

// kSparse: this workgroup's 128 queries are one query block of bmask; key tiles in
// disabled key blocks are skipped. kDropout: as in the dK/dV kernel, dP = (Z / keep) dP~.
template <typename T, int D, bool kSparse, bool kDropout>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ delta, float* __restrict__ dQ,
    int BH, int H, int N, float scale, float sl2, int causal,
    const int* __restrict__ kv_len, int n_mblk, int heads_per_xcd,
    const uint8_t* __restrict__ bmask, int n_sb, uint32_t seed_lo, uint32_t seed_hi,
    uint32_t offset, int drop_t, float keep_scale) {
  constexpr int kKC = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kCPR = D / 8;
  constexpr int kTile = kBN * D * 2;                 // one K or V tile (fp16), bytes
  constexpr int kSC = kTile / 16 / kThreads;         // staged chunks per thread per tensor
  __shared__ __attribute__((aligned(1024))) uint8_t Kb0[kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t Kb1[kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t Vb0[kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t Vb1[kTile];
  __shared__ uint16_t tlist[kSparse ? 2 * kSparseMaxBlocks : 1];  // enabled key tiles
  __shared__ int tlist_len;

  const WgPos pos = wg_position(heads_per_xcd, blockIdx.x, BH);
  if (pos.bh >= BH) return;
  const int mblk = n_mblk - 1 - pos.blk;  // heaviest query block first
  const int bh = pos.bh;
  const int b = bh / H;
  const size_t head = (size_t)bh * N * D;
  int kv_lim = N;
  if (kv_len != nullptr) kv_lim = min(N, max(1, kv_len[b]));
  const int m0 = mblk * kBM;
  const int kend = causal ? min(kv_lim, m0 + kBM) : kv_lim;
  int ntiles = (kend + kBN - 1) / kBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  // the key tiles this workgroup visits: 0 .. ntiles-1, or (sparse) those of them in
  // key blocks enabled for this query block, listed by wave 0
  if constexpr (kSparse) {
    if (wave == 0) {
      int count = 0;
      for (int base = 0; base < ntiles; base += 64) {
        const int t = base + lane;
        const bool on = t < ntiles && bmask[(size_t)mblk * n_sb + t * kBN / kSparseBlock] != 0;
        const uint64_t m = __ballot(on);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (on) tlist[count + before] = (uint16_t)t;
        count += __popcll(m);
      }
      if (lane == 0) tlist_len = count;
    }
    __syncthreads();
    ntiles = tlist_len;
  }
  auto tile_key = [&](int t) {
    if constexpr (kSparse) return __builtin_amdgcn_readfirstlane((int)tlist[t]) * kBN;
    else return t * kBN;
  };
  const int qi = lane & 31, hh = lane >> 5;
  const int g = lane >> 4, gi = lane & 15;
  const int wq0 = m0 + wave * 32;
  const int qrow = wq0 + qi;
  const int qrow_c = min(qrow, N - 1);

  u32x4 ks[kSC], vs[kSC];
  uint32_t ld_off[kSC];
#pragma unroll
  for (int j = 0; j < kSC; ++j) {
    const int ci = tid + kThreads * j;
    ld_off[j] = (uint32_t)((ci / kCPR) * D + (ci % kCPR) * 8) * 2;
  }
  auto load_tile = [&](int t) {
    const int n0 = tile_key(t);
    const uint32_t bytes = (uint32_t)(N - n0) * D * 2;
    const auto rk = buffer_rsrc(K + head + (size_t)n0 * D, bytes);
    const auto rv = buffer_rsrc(V + head + (size_t)n0 * D, bytes);
#pragma unroll
    for (int j = 0; j < kSC; ++j) {
      ks[j] = buffer_load16(rk, ld_off[j]);
      vs[j] = buffer_load16(rv, ld_off[j]);
    }
  };
  auto store_tile = [&](FA_LDS uint8_t* kb, FA_LDS uint8_t* vb) {
#pragma unroll
    for (int j = 0; j < kSC; ++j) {
      const int ci = tid + kThreads * j;
      const int row = ci / kCPR, ch = ci % kCPR;
      lds_write16(kb + tile_off<D>(row, ch), to_f16x8<T>(ks[j]));
      lds_write16(vb + tile_off<D>(row, ch), to_f16x8<T>(vs[j]));
    }
  };

  if (ntiles > 0) load_tile(0);

  // this lane's query row of Q and dO as B operands (fp16): [query][16c + 8hh + 0..7]
  u32x4 qf[kKC], of[kKC];
#pragma unroll
  for (int c = 0; c < kKC; ++c) {
    const size_t off = head + (size_t)qrow_c * D + 16 * c + 8 * hh;
    qf[c] = to_f16x8<T>(*reinterpret_cast<const u32x4*>(Q + off));
    of[c] = to_f16x8<T>(*reinterpret_cast<const u32x4*>(dO + off));
  }
  // a row that sees no key (LSE = -inf, block-sparse) must give P = 0: +inf here
  const float lse_row = LSE[(size_t)bh * N + qrow_c];
  const float lse2 = lse_row == -INFINITY ? INFINITY : lse_row * kLog2e;
  const float dlt = delta[(size_t)bh * N + qrow_c];
  f32x16 dqacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[i][r] = 0.f;
  const int krow_base = kappa(qi);

  if (ntiles > 0) store_tile((FA_LDS uint8_t*)Kb0, (FA_LDS uint8_t*)Vb0);

  auto step = [&](int t, const FA_LDS uint8_t* Ks, const FA_LDS uint8_t* Vs, FA_LDS uint8_t* Kn,
                  FA_LDS uint8_t* Vn) {
    barrier_lds();  // tile t visible; the other buffers are free
    load_tile(min(t + 1, ntiles - 1));  // unconditional: same loads in flight on every path
    const int n0 = tile_key(t);
    const bool need_mask = (n0 + kBN > kv_lim) || (causal && n0 + kBN - 1 > wq0);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const bool vis = (n0 + 32 * sub < kv_lim) && (!causal || n0 + 32 * sub <= wq0 + 31);
      if (!vis) continue;
      // S^T = K Q^T and dP^T = V dO^T for 32 keys; lane (query, hh), register r <->
      // key n0 + 32*sub + 16*(r/8) + 8*hh + r%8
      f32x16 st, dpt;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st[r] = 0.f;
        dpt[r] = 0.f;
      }
      const int krow = sub * 32 + krow_base;
#pragma unroll
      for (int c = 0; c < kKC; ++c) {
        const int off = tile_off<D>(krow, 2 * c + hh);
        st = Mfma<F16>::run(lds_read16(Ks + off), qf[c], st);
        dpt = Mfma<F16>::run(lds_read16(Vs + off), of[c], dpt);
      }
      if (need_mask) {  // -inf where the key is hidden from this lane's query
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = n0 + 32 * sub + 16 * (r >> 3) + 8 * hh + (r & 7);
          const bool hide = kk >= kv_lim || (causal && kk > qrow);
          st[r] = hide ? -INFINITY : st[r];
        }
      }
      uint32_t dsk[8];
      uint32_t rnd[4] = {0, 0, 0, 0};
      if constexpr (kDropout) {
        // register r holds key n0 + 32 sub + 16 (r / 8) + 8 hh + r % 8, whose byte is
        // byte r of the block at counter (query, 2 (sub-block) + hh, head, offset)
        const Philox4x32 ph = philox4x32((uint32_t)qrow,
                                         (uint32_t)(2 * ((n0 + 32 * sub) >> 5) + hh),
                                         (uint32_t)bh, offset, seed_lo, seed_hi);
#pragma unroll
        for (int w = 0; w < 4; ++w) rnd[w] = ph.w[w];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p0 = exp2_fast(fmaf(st[2 * i], sl2, -lse2));
        const float p1 = exp2_fast(fmaf(st[2 * i + 1], sl2, -lse2));
        float dp0 = dpt[2 * i], dp1 = dpt[2 * i + 1];
        if constexpr (kDropout) {
          const uint32_t wv = rnd[i >> 1] >> (16 * (i & 1));
          dp0 = (int)(wv & 0xff) >= drop_t ? dp0 * keep_scale : 0.f;
          dp1 = (int)((wv >> 8) & 0xff) >= drop_t ? dp1 * keep_scale : 0.f;
        }
        dsk[i] = Mfma<F16>::pack(p0 * (dp0 - dlt), p1 * (dp1 - dlt));
      }
      // dQ^T += K^T dS^T: two 16-key steps; K^T through the transposing read
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const u32x4 bs = {dsk[4 * c2], dsk[4 * c2 + 1], dsk[4 * c2 + 2], dsk[4 * c2 + 3]};
        const int trow = 32 * sub + 16 * c2 + 8 * hh + (gi >> 2);
        const int inner = 8 * (gi & 1);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const int ch = db * 4 + 2 * (g & 1) + ((gi & 3) >> 1);
          const u32x2 lo = lds_read_tr16(Ks + tile_off<D>(trow, ch) + inner);
          const u32x2 hi = lds_read_tr16(Ks + tile_off<D>(trow + 4, ch) + inner);
          dqacc[db] = Mfma<F16>::run(u32x4{lo[0], lo[1], hi[0], hi[1]}, bs, dqacc[db]);
        }
      }
    }
    store_tile(Kn, Vn);  // tile t+1 (clamped) into the free buffers
  };

  for (int t = 0; t < ntiles; t += 2) {
    step(t, (const FA_LDS uint8_t*)Kb0, (const FA_LDS uint8_t*)Vb0, (FA_LDS uint8_t*)Kb1,
         (FA_LDS uint8_t*)Vb1);
    if (t + 1 < ntiles)
      step(t + 1, (const FA_LDS uint8_t*)Kb1, (const FA_LDS uint8_t*)Vb1, (FA_LDS uint8_t*)Kb0,
           (FA_LDS uint8_t*)Vb0);
  }

  // dQ = scale * dQ_acc: lane (query, hh), register r <-> d = 32db + 8(r/4) + 4hh + r%4
  if (qrow < N) {
    float* dqr = dQ + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 val = {scale * dqacc[db][4 * a4 + 0], scale * dqacc[db][4 * a4 + 1],
                           scale * dqacc[db][4 * a4 + 2], scale * dqacc[db][4 * a4 + 3]};
        *reinterpret_cast<f32x4*>(dqr + db * 32 + 8 * a4 + 4 * hh) = val;
      }
  }
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  const size_t bytes = (size_t)B * H * N * sizeof(float);
  return (bytes + 255) / 256 * 256;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream, int stages) {
  if (a.dtype == kDtypeF32) return hipErrorNotSupported;  // rejected by the API layer
  const int BH = a.B * a.H;
  const size_t rows = (size_t)BH * a.N;
  const int pre_blocks = (int)((rows * (a.d / 8) + kThreads - 1) / kThreads);
  const float sl2 = a.scale * kLog2e;
  const int hpx = heads_per_xcd(BH);
  const int n_kblk = (a.N + kBK - 1) / kBK;
  const int n_mblk = (a.N + kBM - 1) / kBM;
  const auto* q16 = static_cast<const uint16_t*>(a.q);
  const auto* k16 = static_cast<const uint16_t*>(a.k);
  const auto* v16 = static_cast<const uint16_t*>(a.v);
  const auto* dO16 = static_cast<const uint16_t*>(a.dout);
  const int n_sb = (a.N + kSparseBlock - 1) / kSparseBlock;
  const bool dropout = a.drop_t >= 0;
  const float keep_scale = dropout ? 256.0f / (float)(256 - a.drop_t) : 1.0f;
  const uint32_t seed_lo = (uint32_t)a.seed, seed_hi = (uint32_t)(a.seed >> 32);
#define FA_BWD_LAUNCH2(TAG, DIM, SP, DR)                                                     \
  do {                                                                                       \
    if (stages & 1)                                                                          \
      hipLaunchKernelGGL((bwd_pre_kernel<TAG, DIM>), dim3(pre_blocks), dim3(kThreads), 0,    \
                         stream, dO16, a.o, a.delta, rows);                                  \
    if (stages & 2)                                                                          \
      hipLaunchKernelGGL((bwd_dkdv_kernel<TAG, DIM, SP, DR>), dim3(BH * n_kblk),              \
                         dim3(kThreads), 0, stream, q16, k16, v16, dO16, a.lse, a.delta,     \
                         a.dk, a.dv, BH, a.H, a.N, a.scale, sl2, a.causal, a.kv_len, n_kblk, \
                         hpx, a.block_mask, n_sb, seed_lo, seed_hi, a.offset, a.drop_t,      \
                         keep_scale);                                                        \
    if (stages & 4)                                                                          \
      hipLaunchKernelGGL((bwd_dq_kernel<TAG, DIM, SP, DR>), dim3(BH * n_mblk),                \
                         dim3(kThreads), 0, stream, q16, k16, v16, dO16, a.lse, a.delta,     \
                         a.dq, BH, a.H, a.N, a.scale, sl2, a.causal, a.kv_len, n_mblk, hpx,  \
                         a.block_mask, n_sb, seed_lo, seed_hi, a.offset, a.drop_t, keep_scale); \
  } while (0)
#define FA_BWD_LAUNCH(TAG, DIM)                                          \
  do {                                                                   \
    if (a.block_mask != nullptr) FA_BWD_LAUNCH2(TAG, DIM, true, false);  \
    else if (dropout) FA_BWD_LAUNCH2(TAG, DIM, false, true);             \
    else FA_BWD_LAUNCH2(TAG, DIM, false, false);                         \
  } while (0)
  if (a.dtype == kDtypeBF16) {
    if (a.d == 64) FA_BWD_LAUNCH(BF16, 64); else FA_BWD_LAUNCH(BF16, 128);
  } else {
    if (a.d == 64) FA_BWD_LAUNCH(F16, 64); else FA_BWD_LAUNCH(F16, 128);
  }
#undef FA_BWD_LAUNCH2
#undef FA_BWD_LAUNCH
  return hipGetLastError();
}

}  // namespace fa
