// dK and dV of exact attention on gfx950 (the keys-outer kernel of the backward pass;
// the rest of the backward pass, and the method it follows, is in fa_bwd.hip).
//
// One workgroup per 128 keys of one (batch, head), 32 keys per wave, keys on lanes. It
// loops over 64-query tiles (causal: from the block's diagonal on), recomputes
// S = Q K^T and dP = dO V^T, forms P and dS in registers, and accumulates dV^T += dO^T P
// and dK^T += Q^T dS in registers (dO^T and Q^T through the transposing LDS read). Q/dO
// tiles are prefetched one tile ahead through buffer resources and double-buffered:
// one barrier per tile, waiting for LDS traffic only. Every matrix-core product runs in
// fp16 with fp32 accumulation (Q, dO, K, V converted when staged; P and dS rounded).
// This kernel serves head_dim 64 (about 232 registers, so two workgroups, and two waves
// per SIMD, share a compute unit) when the grid has at least two workgroups per compute
// unit; head_dim 128, and smaller head_dim-64 grids, run the two-wave kernel of
// fa_bwd_dkdv_pair.hip.
//
// This file is compiled on its own so that it can take its own instruction-scheduling
// strategy (see the build script).
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------------
// 2. dK, dV: keys on lanes
// ---------------------------------------------------------------------------------
constexpr int kBK = 128;  // keys per workgroup
constexpr int kBQ = 64;   // queries per tile (two 32-query halves)

// kSparse: bmask is the n_sb x n_sb byte matrix over 128-query x 128-key blocks (this
// workgroup's 128 keys are one key block); query tiles in disabled blocks are skipped.

// kDropout: the probabilities carry the forward pass's dropout mask Z, regenerated here
// from the same Philox4x32-10 blocks (element (i, 32 g + u) of head bh: byte
// 8 (u / 16) + u % 8 of the block at counter (i, 2 g + (u / 8) % 2, bh, offset); kept
// iff >= drop_t):
// dV = (P Z / keep)^T dO, dP = (Z / keep) (dO V^T), dS = P (dP - D).
template <typename T, int D, bool kSparse, bool kDropout>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ delta,
    const float* __restrict__ dmax, float* __restrict__ dK,
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
  // the power-of-two scale of dO (set below, before the first tile is stored)
  float sc = 1.0f;
  bool unscaled = true;
  auto store_tile = [&](FA_LDS uint8_t* qb, FA_LDS uint8_t* ob, FA_LDS float* st) {
#pragma unroll
    for (int j = 0; j < kSC; ++j) {
      const int ci = tid + kThreads * j;
      const int row = ci / kCPR, ch = ci % kCPR;
      lds_write16(qb + tile_off<D>(row, ch), to_f16x8<T>(qs[j]));
    }
    if (unscaled) {  // wave-uniform: dO as it is
#pragma unroll
      for (int j = 0; j < kSC; ++j) {
        const int ci = tid + kThreads * j;
        lds_write16(ob + tile_off<D>(ci / kCPR, ci % kCPR), to_f16x8<T>(os[j]));
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSC; ++j) {
        const int ci = tid + kThreads * j;
        lds_write16(ob + tile_off<D>(ci / kCPR, ci % kCPR), to_f16x8_scaled<T>(os[j], sc));
      }
    }
    if (tid < kBQ) {
      st[tid] = s_lse;
      st[kBQ + tid] = s_dlt * sc;
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

  // dO is taken times the power of two sc = pow2_scale(largest |dO| of the query rows this
  // workgroup visits, from the 32-row maxima the D pass wrote) before it is rounded to
  // fp16; dP, D, dS and both accumulators scale with it, and the epilogue divides by sc
  // (exact). The maxima are read once the first tile's loads are in flight, so the two
  // latencies overlap; every wave forms the same value.
  {
    const int ng = (N + kDmaxRows - 1) / kDmaxRows;
    const float* mp = dmax + (size_t)bh * ng;
    float m = 0.f;
    for (int gi2 = i0 * (kBQ / kDmaxRows) + lane; gi2 < ng; gi2 += 64) m = fmaxf(m, mp[gi2]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    sc = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, pow2_scale(m))));
  }
  unscaled = sc == 1.0f;
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
  // -inf where the query does not see this lane's key (diagonal, padding, sequence end).
  // Register r of half hf holds query base + 16*(r/8) + r%8 with base = q0 + 32*hf +
  // 8*hh; the queries that see the lane's key are one window [lo, hi) of those offsets
  // (empty for a padded key), so each entry costs one unsigned compare against it.
  auto mask = [&](f32x16& s, int q0, int hf) {
    const int base = q0 + 32 * hf + 8 * hh;
    const int lo = (causal ? key : 0) - base;
    const int hi = key < kv_lim ? N - base : lo;
    const uint32_t span = (uint32_t)max(hi - lo, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rel = 16 * (r >> 3) + (r & 7);
      s[r] = (uint32_t)(rel - lo) < span ? s[r] : -INFINITY;
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

  // One 64-query tile: publish it (barrier), prefetch the next one, then
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
        const float ks = scale / sc;
        const f32x4 kk = {ks * dkacc[db][4 * a4], ks * dkacc[db][4 * a4 + 1],
                          ks * dkacc[db][4 * a4 + 2], ks * dkacc[db][4 * a4 + 3]};
        const float vs = (kDropout ? keep_scale : 1.0f) / sc;
        const f32x4 vv = {vs * dvacc[db][4 * a4], vs * dvacc[db][4 * a4 + 1],
                          vs * dvacc[db][4 * a4 + 2], vs * dvacc[db][4 * a4 + 3]};
        *reinterpret_cast<f32x4*>(dkr + d0) = kk;
        *reinterpret_cast<f32x4*>(dvr + d0) = vv;
      }
  }
}

}  // namespace

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  if (a.dtype == kDtypeF32) return hipErrorNotSupported;  // rejected by the API layer
  const int BH = a.B * a.H;
  const float sl2 = a.scale * kLog2e;
  const int hpx = heads_per_xcd(BH);
  const int n_kblk = (a.N + kBK - 1) / kBK;
  const auto* q16 = static_cast<const uint16_t*>(a.q);
  const auto* k16 = static_cast<const uint16_t*>(a.k);
  const auto* v16 = static_cast<const uint16_t*>(a.v);
  const auto* dO16 = static_cast<const uint16_t*>(a.dout);
  const int n_sb = (a.N + kSparseBlock - 1) / kSparseBlock;
  const bool dropout = a.drop_t >= 0;
  const float keep_scale = dropout ? 256.0f / (float)(256 - a.drop_t) : 1.0f;
  const uint32_t seed_lo = (uint32_t)a.seed, seed_hi = (uint32_t)(a.seed >> 32);
#define FA_DKDV_LAUNCH2(TAG, DIM, SP, DR)                                                    \
  hipLaunchKernelGGL((bwd_dkdv_kernel<TAG, DIM, SP, DR>), dim3(BH * n_kblk), dim3(kThreads), \
                     0, stream, q16, k16, v16, dO16, a.lse, a.delta, a.dmax, a.dk, a.dv, BH, \
                     a.H,                                                                     \
                     a.N, a.scale, sl2, a.causal, a.kv_len, n_kblk, hpx, a.block_mask, n_sb, \
                     seed_lo, seed_hi, a.offset, a.drop_t, keep_scale)
#define FA_DKDV_LAUNCH(TAG, DIM)                                              \
  do {                                                                        \
    if (a.block_mask != nullptr) FA_DKDV_LAUNCH2(TAG, DIM, true, false);      \
    else if (dropout) FA_DKDV_LAUNCH2(TAG, DIM, false, true);                 \
    else FA_DKDV_LAUNCH2(TAG, DIM, false, false);                             \
  } while (0)
  // head_dim 128 always runs the two-wave kernel; head_dim 64 runs it when this kernel
  // would not give every compute unit two workgroups (B=4 H=12 N=1024 causal: 29.7
  // against 42.7 us), and this one otherwise (B=8 H=16 N=512: 30.2 against 33.6 us;
  // B=16 H=32 N=1024 causal: 253 against 271 us)
  if (a.d == 128 || (long long)BH * n_kblk < 2LL * device_cu_count())
    return launch_bwd_dkdv_pair(a, stream);
  if (a.dtype == kDtypeBF16) FA_DKDV_LAUNCH(BF16, 64);
  else FA_DKDV_LAUNCH(F16, 64);
#undef FA_DKDV_LAUNCH2
#undef FA_DKDV_LAUNCH
  return hipGetLastError();
}

}  // namespace fa
