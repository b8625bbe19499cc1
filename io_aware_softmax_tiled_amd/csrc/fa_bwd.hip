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
// 2. bwd_dkdv (fa_bwd_dkdv.hip, launched from here): one workgroup per 128 keys of one
//    (batch, head), 32 keys per wave, keys
//    on lanes. It loops over 64-query tiles (causal: from the block's diagonal on),
//    recomputes S = Q K^T and dP = dO V^T, forms P and dS in registers, and accumulates
//    dV^T += dO^T P and dK^T += Q^T dS in registers (dO^T and Q^T through the
//    transposing LDS read). Q/dO tiles are prefetched one tile ahead through buffer
//    resources and double-buffered: one barrier per tile, waiting for LDS traffic
//    only.
// 3. bwd_dq: one workgroup per 256 queries at head_dim 128 (128 at 64, and for block-
//    sparse masks), 32 per wave, queries on lanes -- the forward kernel's layout. Per 64-key tile it recomputes S^T = K Q^T and
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
// 1. D = rowsum(dO * O) and the largest |dO| of every 32-row group. One workgroup per
//    group of 32 rows of one head, one thread per 8 elements (D/8 threads per row).
// ---------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(4 * D) void bwd_pre_kernel(
    const uint16_t* __restrict__ dO, const float* __restrict__ O, float* __restrict__ delta,
    float* __restrict__ dmax, int N, int n_groups) {
  constexpr int kTPR = D / 8;
  constexpr int kWaves = 4 * D / 64;
  __shared__ float wmax[kWaves];
  const int bh = blockIdx.x / n_groups, grp = blockIdx.x % n_groups;
  const int r = grp * kDmaxRows + (int)threadIdx.x / kTPR;   // row inside the head
  const size_t idx = ((size_t)bh * N + r) * D + (threadIdx.x % kTPR) * 8;
  float s = 0.f, m = 0.f;
  if (r < N) {
    const u32x4 g = *reinterpret_cast<const u32x4*>(dO + idx);
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(O + idx);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(O + idx + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = to_f32<T>((uint16_t)(g[j] & 0xffff));
      const float hi = to_f32<T>((uint16_t)(g[j] >> 16));
      const float olo = j < 2 ? o0[2 * j] : o1[2 * j - 4];
      const float ohi = j < 2 ? o0[2 * j + 1] : o1[2 * j - 3];
      s = fmaf(lo, olo, s);
      s = fmaf(hi, ohi, s);
    }
    m = absmax8<T>(g);
  }
#pragma unroll
  for (int off = kTPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kTPR);
  if (r < N && (threadIdx.x % kTPR) == 0) delta[(size_t)bh * N + r] = s;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = wmax[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, wmax[w]);
    dmax[(size_t)bh * n_groups + grp] = mm;
  }
}

// ---------------------------------------------------------------------------------
// 3. dQ: queries on lanes (the forward kernel's layout)
// ---------------------------------------------------------------------------------
constexpr int kBN = 64;   // keys per tile

// W waves of 32 queries per workgroup: 8 at head_dim 128 (each K/V tile then serves 256
// queries; 5% faster than 4 there), 4 at 64 and for block-sparse masks.
// kSparse: this workgroup's 128 queries (W = 4) are one query block of bmask; key tiles
// in disabled key blocks are skipped. kDropout: as in the dK/dV kernel,
// dP = (Z / keep) dP~.
template <typename T, int D, int W, bool kSparse, bool kDropout>
__global__ __launch_bounds__(64 * W, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ O, const float* __restrict__ LSE, float* __restrict__ delta,
    float* __restrict__ dmax, int write_delta, float* __restrict__ dQ, int BH, int H, int N,
    float scale, float sl2,
    int causal, const int* __restrict__ kv_len, int n_mblk, int heads_per_xcd,
    const uint8_t* __restrict__ bmask, int n_sb, uint32_t seed_lo, uint32_t seed_hi,
    uint32_t offset, int drop_t, float keep_scale) {
  constexpr int kKC = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kCPR = D / 8;
  constexpr int kTile = kBN * D * 2;                 // one K or V tile (fp16), bytes
  constexpr int kThr = 64 * W;
  constexpr int kBM = 32 * W;                        // queries per workgroup
  constexpr int kSC = kTile / 16 / kThr;             // staged chunks per thread per tensor
  static_assert(!kSparse || kBM == kSparseBlock, "a sparse workgroup is one query block");
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
  // waves w and w + 4 share a SIMD: with 8 waves the second four take the row groups
  // in reverse order, so under the causal mask each SIMD holds a short and a long one
  const int wrow = (W == 8 && wave >= 4) ? 11 - wave : wave;
  const int wq0 = m0 + wrow * 32;
  const int qrow = wq0 + qi;
  const int qrow_c = min(qrow, N - 1);

  u32x4 ks[kSC], vs[kSC];
  uint32_t ld_off[kSC];
#pragma unroll
  for (int j = 0; j < kSC; ++j) {
    const int ci = tid + kThr * j;
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
      const int ci = tid + kThr * j;
      const int row = ci / kCPR, ch = ci % kCPR;
      lds_write16(kb + tile_off<D>(row, ch), to_f16x8<T>(ks[j]));
      lds_write16(vb + tile_off<D>(row, ch), to_f16x8<T>(vs[j]));
    }
  };

  if (ntiles > 0) load_tile(0);

  // this lane's query row of Q and dO as B operands (fp16): [query][16c + 8hh + 0..7],
  // and D = rowsum(dO * O) of the row from the same dO and the row of O, summed in the
  // order of bwd_pre (each 8-element chunk by FMAs in element order, then chunks t and
  // t ^ off pairwise for off = D/16 .. 1; chunk t = 2c + hh lives in this lane for the
  // even offsets and in the other half of the wave for off = 1), so the two agree bit
  // for bit
  u32x4 qf[kKC], of[kKC];
  float dpart[kKC];
  float dmx = 0.f;  // largest |dO| of this lane's half of the row
#pragma unroll
  for (int c = 0; c < kKC; ++c) {
    const size_t off = head + (size_t)qrow_c * D + 16 * c + 8 * hh;
    qf[c] = to_f16x8<T>(*reinterpret_cast<const u32x4*>(Q + off));
    const u32x4 g = *reinterpret_cast<const u32x4*>(dO + off);
    of[c] = g;
    dmx = fmaxf(dmx, absmax8<T>(g));
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(O + off);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(O + off + 4);
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sum = fmaf(to_f32<T>((uint16_t)(g[j] & 0xffff)), j < 2 ? o0[2 * j] : o1[2 * j - 4], sum);
      sum = fmaf(to_f32<T>((uint16_t)(g[j] >> 16)), j < 2 ? o0[2 * j + 1] : o1[2 * j - 3], sum);
    }
    dpart[c] = sum;
  }
#pragma unroll
  for (int m = kKC / 2; m > 0; m >>= 1)
#pragma unroll
    for (int c = 0; c < kKC; ++c)
      if (c < (c ^ m)) {
        const float t2 = dpart[c] + dpart[c ^ m];
        dpart[c] = t2;
        dpart[c ^ m] = t2;
      }
  const float dlt_raw = sum_halves(dpart[0]);
  if (write_delta && hh == 0 && qrow < N) delta[(size_t)bh * N + qrow] = dlt_raw;
  // dO of this row is taken times a power of two r that brings its largest magnitude
  // into [1, 2) before rounding to fp16; dP, D and dS scale with it, and dQ is divided
  // by r at the end (exact)
  const float row_max = max_halves(dmx);
  const float rsc = pow2_scale(row_max);
#pragma unroll
  for (int c = 0; c < kKC; ++c) of[c] = to_f16x8_scaled<T>(of[c], rsc);
  const float dlt = dlt_raw * rsc;
  if (write_delta) {
    // the largest |dO| of the wave's 32 rows, for the dK/dV kernel's scale
    float gm = row_max;
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) gm = fmaxf(gm, __shfl_xor(gm, off, 32));
    if (lane == 0 && wq0 < N) dmax[(size_t)bh * ((N + kDmaxRows - 1) / kDmaxRows) + wq0 / kDmaxRows] = gm;
  }
  // a row that sees no key (LSE = -inf, block-sparse) must give P = 0: +inf here
  const float lse_row = LSE[(size_t)bh * N + qrow_c];
  const float lse2 = lse_row == -INFINITY ? INFINITY : lse_row * kLog2e;
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
      // issue priority high in the two matrix-core phases of the sub-block and low in
      // the vector phase between them, so that the SIMD's other wave, when it is in a
      // different phase, keeps the matrix cores busy (3-4% faster)
      __builtin_amdgcn_s_setprio(1);
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
      __builtin_amdgcn_s_setprio(0);
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
      __builtin_amdgcn_s_setprio(1);
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

  // dQ = scale / r * dQ_acc: lane (query, hh), register r <-> d = 32db + 8(r/4) + 4hh + r%4
  if (qrow < N) {
    float* dqr = dQ + head + (size_t)qrow * D;
    const float sq = scale / rsc;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 val = {sq * dqacc[db][4 * a4 + 0], sq * dqacc[db][4 * a4 + 1],
                           sq * dqacc[db][4 * a4 + 2], sq * dqacc[db][4 * a4 + 3]};
        *reinterpret_cast<f32x4*>(dqr + db * 32 + 8 * a4 + 4 * hh) = val;
      }
  }
}

}  // namespace

size_t bwd_delta_bytes(int B, int H, int N) {
  const size_t bytes = (size_t)B * H * N * sizeof(float);
  return (bytes + 255) / 256 * 256;
}

size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  const size_t groups = (size_t)B * H * ((N + kDmaxRows - 1) / kDmaxRows);
  return bwd_delta_bytes(B, H, N) + (groups * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream, int stages) {
  if (a.dtype == kDtypeF32) return launch_bwd_f32(a, stream, stages);
  const int BH = a.B * a.H;
  const int n_groups = (a.N + kDmaxRows - 1) / kDmaxRows;
  const float sl2 = a.scale * kLog2e;
  const int hpx = heads_per_xcd(BH);
  const auto* q16 = static_cast<const uint16_t*>(a.q);
  const auto* k16 = static_cast<const uint16_t*>(a.k);
  const auto* v16 = static_cast<const uint16_t*>(a.v);
  const auto* dO16 = static_cast<const uint16_t*>(a.dout);
  const int n_sb = (a.N + kSparseBlock - 1) / kSparseBlock;
  const bool dropout = a.drop_t >= 0;
  const float keep_scale = dropout ? 256.0f / (float)(256 - a.drop_t) : 1.0f;
  const uint32_t seed_lo = (uint32_t)a.seed, seed_hi = (uint32_t)(a.seed >> 32);
  // head_dim 128 runs the dQ kernel with 8 waves (256 query rows per workgroup, each K/V
  // tile serving twice the rows) unless that grid leaves compute units idle; head_dim 64
  // and block-sparse patterns (one 128-row query block per workgroup) always run 4
  const bool dq_narrow = (long long)BH * ((a.N + 255) / 256) < device_cu_count();
#define FA_DQ_LAUNCH(TAG, DIM, WV, SP, DR)                                                    \
  do {                                                                                       \
    const int n_mblk = (a.N + 32 * WV - 1) / (32 * WV);                                      \
    hipLaunchKernelGGL((bwd_dq_kernel<TAG, DIM, WV, SP, DR>), dim3(BH * n_mblk),              \
                       dim3(64 * WV), 0, stream, q16, k16, v16, dO16, a.o, a.lse, a.delta,    \
                       a.dmax, (stages & 8) ? 1 : 0, a.dq, BH, a.H, a.N, a.scale, sl2,        \
                       a.causal, a.kv_len, n_mblk, hpx, a.block_mask, n_sb, seed_lo, seed_hi, \
                       a.offset, a.drop_t, keep_scale);                                       \
  } while (0)
#define FA_BWD_LAUNCH2(TAG, DIM, SP, DR)                                                     \
  do {                                                                                       \
    if (stages & 1)                                                                          \
      hipLaunchKernelGGL((bwd_pre_kernel<TAG, DIM>), dim3(BH * n_groups), dim3(4 * DIM), 0,  \
                         stream, dO16, a.o, a.delta, a.dmax, a.N, n_groups);                  \
    if (stages & 4) {                                                                        \
      constexpr int kWide = (DIM == 128 && !SP) ? 8 : 4;                                     \
      if (dq_narrow) FA_DQ_LAUNCH(TAG, DIM, 4, SP, DR);                                      \
      else FA_DQ_LAUNCH(TAG, DIM, kWide, SP, DR);                                            \
    }                                                                                        \
    if (stages & 2) {                                                                        \
      const hipError_t e = launch_bwd_dkdv(a, stream);                                       \
      if (e != hipSuccess) return e;                                                         \
    }                                                                                        \
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
#undef FA_DQ_LAUNCH
  return hipGetLastError();
}

}  // namespace fa
