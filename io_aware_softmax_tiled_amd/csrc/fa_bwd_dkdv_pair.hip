// dK and dV: the keys-outer kernel of the backward pass with two waves per SIMD, with or
// without a block mask or dropout, for every head_dim-128 backward and for head_dim-64
// ones whose grid is too small to give every compute unit two workgroups of the
// one-wave kernel in fa_bwd_dkdv.hip (fa_bwd.hip has the rest of the backward pass and
// the method it follows).
//
// Kept in a file of its own because it runs faster under the compiler's default
// instruction scheduler, where the one-wave-per-SIMD kernel wants another strategy
// (see the build script).
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBK = 128;  // keys per workgroup
constexpr int kBQ = 64;   // queries per tile (two 32-query halves)

// ---------------------------------------------------------------------------------
// Two waves per SIMD. Eight waves per workgroup share its 128 keys in
// pairs: waves w and w + 4 hold the same 32 keys (w % 4) and take the two 32-query
// halves of every 64-query tile, each accumulating partial dK and dV in its registers;
// the pairs add their partials through LDS at the end. K and V (fp16) stay in LDS for
// the whole loop and each wave reads its operands from there, so a wave needs no
// K/V registers and two of them fit on a SIMD; Q and dO tiles are staged and
// double-buffered as in the kernel above.
// ---------------------------------------------------------------------------------
constexpr int kPairThreads = 512;

//
// kSparse: bmask is the n_sb x n_sb byte matrix over 128-query x 128-key blocks (this
// workgroup's 128 keys are one key block); query tiles in disabled blocks are skipped.
// kDropout: the probabilities carry the forward pass's dropout mask Z, regenerated from
// the same Philox4x32-10 blocks (element (i, 32 g + u) of head bh: byte
// 8 (u / 16) + u % 8 of the block at counter (i, 2 g + (u / 8) % 2, bh, offset); kept
// iff >= drop_t): dV = (P Z / keep)^T dO, dP = (Z / keep) (dO V^T), dS = P (dP - D).
template <typename T, int D, bool kSparse, bool kDropout>
__global__ __launch_bounds__(kPairThreads, 1) void bwd_dkdv_pair_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ delta,
    const float* __restrict__ dmax, float* __restrict__ dK, float* __restrict__ dV, int BH,
    int H, int N, float scale, float sl2, int causal, const int* __restrict__ kv_len,
    int n_kblk, int heads_per_xcd, const uint8_t* __restrict__ bmask, int n_sb,
    uint32_t seed_lo, uint32_t seed_hi, uint32_t offset, int drop_t, float keep_scale) {
  constexpr int kKC = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kCPR = D / 8;                            // 16-byte chunks per row
  constexpr int kTile = kBQ * D * 2;                     // one Q or dO tile (fp16), bytes
  constexpr int kKV = kBK * D * 2;                       // the K or V block (fp16), bytes
  constexpr int kSC = kTile / 16 / kPairThreads;         // staged chunks per thread per tensor
  constexpr int kKVC = kKV / 16 / kPairThreads;          // K/V chunks per thread
  // LDS: K, V blocks, then two Q and two dO tile buffers; after the loop the whole
  // region holds the partial accumulators of waves 4-7 (4 x 8 kDB KiB)
  constexpr int kOffV = kKV, kOffQ0 = 2 * kKV, kOffQ1 = kOffQ0 + kTile;
  constexpr int kOffO0 = kOffQ1 + kTile, kOffO1 = kOffO0 + kTile;
  constexpr int kLds = kOffO1 + kTile;
  constexpr int kRed = 2 * kDB * 4;  // 16-byte chunks of partial dK and dV per lane
  static_assert(kLds >= 4 * 64 * kRed * 16, "reduction area");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
  __shared__ __attribute__((aligned(16))) float St0[2 * kBQ];  // LSE*log2(e), then D
  __shared__ __attribute__((aligned(16))) float St1[2 * kBQ];
  __shared__ uint16_t tlist[kSparse ? 2 * kSparseMaxBlocks : 1];  // enabled query tiles
  __shared__ int tlist_len;
  // dropout: each wave's random bytes of the current tile, [its 32 queries][its 32 keys]
  __shared__ __attribute__((aligned(16))) uint8_t zbuf[kDropout ? 8 * 32 * 32 : 16];

  const WgPos pos = wg_position(heads_per_xcd, blockIdx.x, BH);
  const int kblk = pos.blk;
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
  const int kg = wave & 3, hf = wave >> 2;  // key group, query half
  const int li = lane & 31, hh = lane >> 5;
  const int g = lane >> 4, gi = lane & 15;
  const int kw0 = k0 + 32 * kg;
  const int key = kw0 + li;

  if (k0 >= kv_lim) {
    for (int e = tid; e < kBK * D / 4; e += kPairThreads) {
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

  u32x4 qs[kSC], os[kSC];
  float s_lse = 0.f, s_dlt = 0.f;
  uint32_t ld_off[kSC];
#pragma unroll
  for (int j = 0; j < kSC; ++j) {
    const int ci = tid + kPairThreads * j;
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
      const float l = LSE[r];
      s_lse = l == -INFINITY ? INFINITY : l * kLog2e;
      s_dlt = delta[r];
    }
  };
  float sc = 1.0f;
  bool unscaled = true;
  auto store_tile = [&](FA_LDS uint8_t* qb, FA_LDS uint8_t* ob, FA_LDS float* st) {
#pragma unroll
    for (int j = 0; j < kSC; ++j) {
      const int ci = tid + kPairThreads * j;
      lds_write16(qb + tile_off<D>(ci / kCPR, ci % kCPR), to_f16x8<T>(qs[j]));
    }
    if (unscaled) {
#pragma unroll
      for (int j = 0; j < kSC; ++j) {
        const int ci = tid + kPairThreads * j;
        lds_write16(ob + tile_off<D>(ci / kCPR, ci % kCPR), to_f16x8<T>(os[j]));
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSC; ++j) {
        const int ci = tid + kPairThreads * j;
        lds_write16(ob + tile_off<D>(ci / kCPR, ci % kCPR), to_f16x8_scaled<T>(os[j], sc));
      }
    }
    if (tid < kBQ) {
      st[tid] = s_lse;
      st[kBQ + tid] = s_dlt * sc;
    }
  };

  if (nt > 0) load_tile(tile_at(0));

  // the K and V block -> LDS as fp16 (rows past the end of the sequence as zeros)
  {
    const uint32_t bytes = (uint32_t)(N - k0) * D * 2;
    const auto rk = buffer_rsrc(K + head + (size_t)k0 * D, bytes);
    const auto rv = buffer_rsrc(V + head + (size_t)k0 * D, bytes);
#pragma unroll
    for (int j = 0; j < kKVC; ++j) {
      const int ci = tid + kPairThreads * j;
      const uint32_t off = (uint32_t)((ci / kCPR) * D + (ci % kCPR) * 8) * 2;
      const u32x4 kk = buffer_load16(rk, off), vv = buffer_load16(rv, off);
      lds_write16((FA_LDS uint8_t*)lds + tile_off<D>(ci / kCPR, ci % kCPR), to_f16x8<T>(kk));
      lds_write16((FA_LDS uint8_t*)lds + kOffV + tile_off<D>(ci / kCPR, ci % kCPR), to_f16x8<T>(vv));
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

  int aoff[kKC];  // A-operand rows (queries, order kappa) of this wave's half
#pragma unroll
  for (int c = 0; c < kKC; ++c) aoff[c] = tile_off<D>(32 * hf + kappa(li), 2 * c + hh);
  int boff[kKC];  // B-operand rows of K and V: this lane's key
#pragma unroll
  for (int c = 0; c < kKC; ++c) boff[c] = tile_off<D>(32 * kg + li, 2 * c + hh);
  int toff[2][kDB];  // transposing reads of dO^T and Q^T, this wave's half
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int db = 0; db < kDB; ++db)
      toff[r][db] = tile_off<D>(32 * hf + 8 * hh + (gi >> 2) + 4 * r,
                                db * 4 + 2 * (g & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);

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
  if (nt > 0) store_tile((FA_LDS uint8_t*)lds + kOffQ0, (FA_LDS uint8_t*)lds + kOffO0, (FA_LDS float*)St0);

  const FA_LDS uint8_t* Kl = (const FA_LDS uint8_t*)lds;
  const FA_LDS uint8_t* Vl = (const FA_LDS uint8_t*)lds + kOffV;
  // S = Q K^T and dP = dO V^T for this wave's 32 queries of the tile:
  // lane (key, hh), register r <-> query q0 + 32*hf + 16*(r/8) + 8*hh + r%8
  auto products = [&](const FA_LDS uint8_t* Qc, const FA_LDS uint8_t* Oc, f32x16& s, f32x16& dp) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < kKC; ++c) {
      s = Mfma<F16>::run(lds_read16(Qc + aoff[c]), lds_read16(Kl + boff[c]), s);
      dp = Mfma<F16>::run(lds_read16(Oc + aoff[c]), lds_read16(Vl + boff[c]), dp);
    }
  };
  auto mask = [&](f32x16& s, int q0) {
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
  FA_LDS uint8_t* zw = (FA_LDS uint8_t*)zbuf + (kDropout ? wave * 32 * 32 : 0);  // wave bytes
  auto p_ds = [&](const FA_LDS float* Stc, const f32x16& s, const f32x16& dp, uint32_t (&pp)[8],
                  uint32_t (&dsp)[8]) {
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
          // byte of (query 16 c + 8 hh + j of this wave's half, this lane's key)
          const bool keep = (int)zw[(16 * c + 8 * hh + j) * 32 + li] >= drop_t;
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
  auto accumulate = [&](const FA_LDS uint8_t* Qc, const FA_LDS uint8_t* Oc, const uint32_t (&pp)[8],
                        const uint32_t (&dsp)[8]) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const u32x4 bp = {pp[4 * c], pp[4 * c + 1], pp[4 * c + 2], pp[4 * c + 3]};
      const u32x4 bs = {dsp[4 * c], dsp[4 * c + 1], dsp[4 * c + 2], dsp[4 * c + 3]};
      const int rows = 16 * c * D * 2;
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

  auto step = [&](int s, const FA_LDS uint8_t* Qc, const FA_LDS uint8_t* Oc,
                  const FA_LDS float* Stc, FA_LDS uint8_t* Qn, FA_LDS uint8_t* On,
                  FA_LDS float* Stn) {
    barrier_lds();  // tile s (and, at s = 0, K and V) visible; the other buffers are free
    load_tile(tile_at(min(s + 1, nt - 1)));  // unconditional: same loads on every path
    const int q0 = tile_at(s) * kBQ;
    const int hq0 = q0 + 32 * hf;  // first query of this wave's half
    // a half entirely above this wave's keys' diagonal, or past the sequence end, or a
    // wave whose keys are all padded, is skipped
    const bool active = !wave_dead && hq0 < N && !(causal && kw0 > hq0 + 31);
    const bool need_mask = (causal && kw0 + 31 > hq0) || (hq0 + 32 > N) || (kw0 + 32 > kv_lim);
    if (kDropout && active) {
      // lane (l, c) draws the block of (query hq0 + l % 32, this wave's keys 32 g + u with
      // (u / 8) % 2 = c) and writes its bytes 0-7 (keys 8 c + 0..7) and 8-15 (keys
      // 16 + 8 c + 0..7) to the wave's strip in key order; lanes then read their own key
      const int c = lane >> 5;
      const Philox4x32 blk = philox4x32((uint32_t)(hq0 + li), (uint32_t)(2 * (kw0 >> 5) + c),
                                        (uint32_t)bh, offset, seed_lo, seed_hi);
      *reinterpret_cast<FA_LDS u32x2*>(zw + li * 32 + 8 * c) = u32x2{blk.w[0], blk.w[1]};
      *reinterpret_cast<FA_LDS u32x2*>(zw + li * 32 + 16 + 8 * c) = u32x2{blk.w[2], blk.w[3]};
    }
    if (active) {
      f32x16 s0, dp0;
      uint32_t pp0[8], ds0[8];
      products(Qc, Oc, s0, dp0);
      if (need_mask) mask(s0, q0);
      p_ds(Stc, s0, dp0, pp0, ds0);
      accumulate(Qc, Oc, pp0, ds0);
    }
    store_tile(Qn, On, Stn);
  };

  FA_LDS uint8_t* const Qb0 = (FA_LDS uint8_t*)lds + kOffQ0;
  FA_LDS uint8_t* const Qb1 = (FA_LDS uint8_t*)lds + kOffQ1;
  FA_LDS uint8_t* const Ob0 = (FA_LDS uint8_t*)lds + kOffO0;
  FA_LDS uint8_t* const Ob1 = (FA_LDS uint8_t*)lds + kOffO1;
  for (int s = 0; s < nt; s += 2) {
    step(s, Qb0, Ob0, (const FA_LDS float*)St0, Qb1, Ob1, (FA_LDS float*)St1);
    if (s + 1 < nt) step(s + 1, Qb1, Ob1, (const FA_LDS float*)St1, Qb0, Ob0, (FA_LDS float*)St0);
  }

  // the pairs add their partial accumulators: waves 4-7 write theirs to LDS (chunk j of
  // 4 floats of lane l at ((kg * kRed + j) * 64 + l) * 16), waves 0-3 add them and store
  __syncthreads();
  FA_LDS f32x4* red = (FA_LDS f32x4*)lds + kg * kRed * 64 + lane;
  if (hf == 1) {
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        red[(db * 4 + a4) * 64] = f32x4{dkacc[db][4 * a4], dkacc[db][4 * a4 + 1],
                                        dkacc[db][4 * a4 + 2], dkacc[db][4 * a4 + 3]};
        red[(4 * kDB + db * 4 + a4) * 64] = f32x4{dvacc[db][4 * a4], dvacc[db][4 * a4 + 1],
                                             dvacc[db][4 * a4 + 2], dvacc[db][4 * a4 + 3]};
      }
  }
  __syncthreads();
  if (hf == 0 && key < N) {
    float* dkr = dK + head + (size_t)key * D;
    float* dvr = dV + head + (size_t)key * D;
    const float ks = scale / sc, vs = (kDropout ? keep_scale : 1.0f) / sc;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * db + 8 * a4 + 4 * hh;
        const f32x4 pk = red[(db * 4 + a4) * 64], pv = red[(4 * kDB + db * 4 + a4) * 64];
        const f32x4 kk = {ks * (dkacc[db][4 * a4] + pk[0]), ks * (dkacc[db][4 * a4 + 1] + pk[1]),
                          ks * (dkacc[db][4 * a4 + 2] + pk[2]), ks * (dkacc[db][4 * a4 + 3] + pk[3])};
        const f32x4 vv = {vs * (dvacc[db][4 * a4] + pv[0]), vs * (dvacc[db][4 * a4 + 1] + pv[1]),
                          vs * (dvacc[db][4 * a4 + 2] + pv[2]), vs * (dvacc[db][4 * a4 + 3] + pv[3])};
        *reinterpret_cast<f32x4*>(dkr + d0) = kk;
        *reinterpret_cast<f32x4*>(dvr + d0) = vv;
      }
  }
}

}  // namespace

hipError_t launch_bwd_dkdv_pair(const BwdArgs& a, hipStream_t stream) {
  const int BH = a.B * a.H;
  const float sl2 = a.scale * kLog2e;
  const int n_kblk = (a.N + kBK - 1) / kBK;
  const auto* q16 = static_cast<const uint16_t*>(a.q);
  const auto* k16 = static_cast<const uint16_t*>(a.k);
  const auto* v16 = static_cast<const uint16_t*>(a.v);
  const auto* dO16 = static_cast<const uint16_t*>(a.dout);
  const int n_sb = (a.N + kSparseBlock - 1) / kSparseBlock;
  const bool dropout = a.drop_t >= 0;
  const float keep_scale = dropout ? 256.0f / (float)(256 - a.drop_t) : 1.0f;
  const uint32_t seed_lo = (uint32_t)a.seed, seed_hi = (uint32_t)(a.seed >> 32);
#define FA_DKDV_PAIR2(TAG, DIM, SP, DR)                                                     \
  hipLaunchKernelGGL((bwd_dkdv_pair_kernel<TAG, DIM, SP, DR>), dim3(BH * n_kblk),           \
                     dim3(kPairThreads), 0, stream, q16, k16, v16, dO16, a.lse, a.delta,     \
                     a.dmax, a.dk, a.dv, BH, a.H, a.N, a.scale, sl2, a.causal, a.kv_len,     \
                     n_kblk, heads_per_xcd(BH), a.block_mask, n_sb, seed_lo, seed_hi,        \
                     a.offset, a.drop_t, keep_scale)
#define FA_DKDV_PAIR1(TAG, DIM)                                            \
  do {                                                                     \
    if (a.block_mask != nullptr) FA_DKDV_PAIR2(TAG, DIM, true, false);     \
    else if (dropout) FA_DKDV_PAIR2(TAG, DIM, false, true);                \
    else FA_DKDV_PAIR2(TAG, DIM, false, false);                            \
  } while (0)
#define FA_DKDV_PAIR(TAG)                                \
  do {                                                   \
    if (a.d == 128) FA_DKDV_PAIR1(TAG, 128);             \
    else FA_DKDV_PAIR1(TAG, 64);                         \
  } while (0)
  if (a.d != 128 && a.d != 64) return hipErrorNotSupported;
  if (a.dtype == kDtypeBF16) FA_DKDV_PAIR(BF16);
  else if (a.dtype == kDtypeF16) FA_DKDV_PAIR(F16);
  else return hipErrorNotSupported;
#undef FA_DKDV_PAIR
#undef FA_DKDV_PAIR1
#undef FA_DKDV_PAIR2
  return hipGetLastError();
}

}  // namespace fa
