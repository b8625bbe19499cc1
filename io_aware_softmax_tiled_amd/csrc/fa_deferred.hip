// Forward pass with the P V product deferred to the end of the key row, on gfx950.
//
// Method: "Fewer matrix multiplications, same results, should we consider adopting it?"
// (flash-attention issue thread): per query block every score block of the key row is
// turned into its numerator block f_j while the running maximum and denominator are
// tracked; when the maximum rises, the earlier numerator blocks are rescaled; the
// output is one product (f / l) V at the end, instead of one output update per key
// block. The thread's own argument is that this needs on-chip room for a query block's
// whole numerator row; it fits when N is short.
//
// Layout on CDNA4 (not taken from the thread):
// * Four waves of 32 query rows per workgroup. Scores are computed transposed,
//   S^T = K Q^T, so each lane owns a query row and its half of the keys; the numerator
//   row stays in that lane's registers as packed fp16 pairs (f[sub-block][8], 16 keys a
//   lane per 32-key sub-block), which is the B-operand layout of the final
//   O^T = V^T f^T product: nothing is moved between the two phases. N <= 32 * NSB.
// * Phase 1 streams K tiles (64 keys) through LDS, phase 2 streams V tiles; each tile is
//   read from HBM once per workgroup, as in the single-pass kernel, with the next tile's
//   global load in flight while the current one is used (two LDS buffers, one barrier
//   per tile).
// * The reference maximum in the exponent is raised only when a sub-block's maximum
//   exceeds it by more than 2^15 in the exponent (f stays inside fp16); only then are
//   the earlier numerator blocks and the denominator rescaled, which is the thread's
//   rescale step applied to the reference actually used.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kDefBM = 128;      // query rows per workgroup (4 waves x 32)
constexpr int kDefBN = 64;       // key rows per tile
constexpr int kDefThreads = 256;

template <typename T, int D, int NSB>
__global__ __launch_bounds__(kDefThreads, 1) void fwd_deferred_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
    int BH, int H, int N, float scale, float sl2, int causal,
    const int* __restrict__ kv_len, int n_mblk, int heads_per_xcd) {
  constexpr int kTileBytes = kDefBN * D * 2;
  constexpr int kKC = D / 16;                              // 16-wide k-steps over head_dim
  constexpr int kDB = D / 32;                              // 32-row blocks of O^T
  constexpr int kCPR = D / 8;                              // 16-byte chunks per row
  constexpr int kChunks = kTileBytes / 16 / kDefThreads;   // per thread per tile
  constexpr int kMaxTiles = NSB / 2;
  __shared__ __attribute__((aligned(1024))) uint8_t Tb0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t Tb1[kTileBytes];

  const WgPos pos = wg_position(heads_per_xcd, blockIdx.x, BH);
  if (pos.bh >= BH) return;
  const int mblk = n_mblk - 1 - pos.blk;  // heaviest query block first
  const int b = pos.bh / H;
  const size_t head = (size_t)pos.bh * N * D;
  const uint16_t* q = Q + head;
  const uint16_t* k = K + head;
  const uint16_t* v = V + head;

  int kv_lim = N;
  if (kv_len != nullptr) kv_lim = min(N, max(1, kv_len[b]));
  const int m0 = mblk * kDefBM;
  const int kend = causal ? min(kv_lim, m0 + kDefBM) : kv_lim;
  const int ntiles = (kend + kDefBN - 1) / kDefBN;  // >= 1: key 0 is always visible

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = lane & 31;
  const int hh = lane >> 5;
  const int g = lane >> 4, gi = lane & 15;
  const int wq0 = m0 + wave * 32;
  const int qrow = wq0 + qi;
  const int qrow_c = min(qrow, N - 1);
  // last key any row of this wave sees; sub-blocks past it are skipped by the wave
  const int wave_last = causal ? min(kv_lim - 1, wq0 + 31) : kv_lim - 1;
  // this lane's last visible key, relative to its first key of a sub-block
  const int last_vis = (causal ? min(kv_lim - 1, qrow) : kv_lim - 1) - 8 * hh;

  // tiles u = 0 .. ntiles-1 are K, ntiles .. 2 ntiles-1 are V; u lives in buffer u % 2
  u32x4 st[kChunks];
  uint32_t ld_off[kChunks];
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const int ci = tid + kDefThreads * j;
    ld_off[j] = (uint32_t)((ci / kCPR) * D + (ci % kCPR) * 8) * 2;
  }
  auto load_tile = [&](int u) {
    const bool is_v = u >= ntiles;
    const int n0 = (is_v ? u - ntiles : u) * kDefBN;
    const auto r = buffer_rsrc((is_v ? v : k) + (size_t)n0 * D, (uint32_t)(N - n0) * D * 2);
#pragma unroll
    for (int j = 0; j < kChunks; ++j) st[j] = buffer_load16(r, ld_off[j]);
  };
  auto store_tile = [&](int u) {
    FA_LDS uint8_t* buf = (u & 1) ? (FA_LDS uint8_t*)Tb1 : (FA_LDS uint8_t*)Tb0;
    const bool is_v = u >= ntiles;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int ci = tid + kDefThreads * j;
      lds_write16(buf + tile_off<D>(ci / kCPR, ci % kCPR), is_v ? to_f16x8<T>(st[j]) : st[j]);
    }
  };
  auto tile_buf = [&](int u) {
    return (u & 1) ? (const FA_LDS uint8_t*)Tb1 : (const FA_LDS uint8_t*)Tb0;
  };
  // opens tile u: writes it to LDS, starts the global load of tile u+1, barrier
  auto open_tile = [&](int u) {
    store_tile(u);
    if (u + 1 < 2 * ntiles) load_tile(u + 1);
    barrier_lds();
  };

  // Q fragment: B operand of S^T = K Q^T, lane (qi, hh) holds Q[qrow][16c + 8hh + 0..7]
  u32x4 qf[kKC];
#pragma unroll
  for (int c = 0; c < kKC; ++c)
    qf[c] = *reinterpret_cast<const u32x4*>(q + (size_t)qrow_c * D + 16 * c + 8 * hh);
  int koff[kKC];
#pragma unroll
  for (int c = 0; c < kKC; ++c) koff[c] = tile_off<D>(kappa(qi), 2 * c + hh);

  // ---- phase 1: numerator blocks f (register r of sub-block sb: key
  // 32 sb + 16 (r/8) + 8 hh + r%8), running reference maximum and denominator
  uint32_t f[NSB][8];
  float m_ref = -INFINITY;
  float lsum = 0.f;
  load_tile(0);
#pragma unroll
  for (int t = 0; t < kMaxTiles; ++t) {
    if (t >= ntiles) break;
    open_tile(t);
    const FA_LDS uint8_t* Ks = tile_buf(t);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int sb = 2 * t + sub;
      const int n0 = 32 * sb;
      if (n0 > wave_last) {  // no row of this wave sees these keys
#pragma unroll
        for (int i = 0; i < 8; ++i) f[sb][i] = 0u;
        continue;
      }
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int c = 0; c < kKC; ++c)
        s = Mfma<T>::run(lds_read16(Ks + koff[c] + sub * 32 * D * 2), qf[c], s);
      if (n0 + 31 > wave_last || (causal && n0 + 31 > wq0)) {
        const int lim = last_vis - n0;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = (16 * (r >> 3) + (r & 7) > lim) ? -INFINITY : s[r];
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = max3f(mx, s[r], s[r + 1]);
      mx = max_halves(mx);
      const bool grow = (mx - m_ref) * sl2 > 15.0f;
      if (__any(grow)) {
        const float m_new = grow ? mx : m_ref;
        const float alpha = exp2_fast((m_ref - m_new) * sl2);  // 1 if kept, 0 from -inf
        m_ref = m_new;
        lsum *= alpha;
        // the earlier numerator blocks move to the new reference
#pragma unroll
        for (int j = 0; j < NSB; ++j) {
          if (j >= sb) break;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const f16x2 x = __builtin_bit_cast(f16x2, f[j][i]);
            f[j][i] = Mfma<F16>::pack((float)x[0] * alpha, (float)x[1] * alpha);
          }
        }
      }
      const float nms = -m_ref * sl2;  // m_ref is finite: key 0 is visible to every row
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p0 = exp2_fast(fmaf(s[2 * i], sl2, nms));
        const float p1 = exp2_fast(fmaf(s[2 * i + 1], sl2, nms));
        f[sb][i] = Mfma<F16>::pack(p0, p1);
        lsum = Mfma<F16>::dot_ones(f[sb][i], lsum);
      }
    }
  }

  // ---- phase 2: O^T = V^T f^T, one pass over the V tiles
  f32x16 oacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  int voff[2][kDB];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int db = 0; db < kDB; ++db)
      voff[r][db] = tile_off<D>(8 * hh + (gi >> 2) + 4 * r, db * 4 + 2 * (g & 1) + ((gi & 3) >> 1)) +
                    8 * (gi & 1);
#pragma unroll
  for (int t = 0; t < kMaxTiles; ++t) {
    if (t >= ntiles) break;
    open_tile(ntiles + t);
    const FA_LDS uint8_t* Vs = tile_buf(ntiles + t);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int sb = 2 * t + sub;
      if (32 * sb > wave_last) continue;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const u32x4 bp = {f[sb][4 * c2], f[sb][4 * c2 + 1], f[sb][4 * c2 + 2], f[sb][4 * c2 + 3]};
        const int rows = (32 * sub + 16 * c2) * D * 2;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const u32x2 lo = lds_read_tr16(Vs + voff[0][db] + rows);
          const u32x2 hi = lds_read_tr16(Vs + voff[1][db] + rows);
          oacc[db] = Mfma<F16>::run(u32x4{lo[0], lo[1], hi[0], hi[1]}, bp, oacc[db]);
        }
      }
    }
  }

  // epilogue: O = O_acc / l, LSE = scale*m_ref + ln(l)
  const float ltot = sum_halves(lsum);
  if (qrow < N) {
    const float inv = 1.0f / ltot;
    float* orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 val = {oacc[db][4 * a4 + 0] * inv, oacc[db][4 * a4 + 1] * inv,
                           oacc[db][4 * a4 + 2] * inv, oacc[db][4 * a4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * a4 + 4 * hh) = val;
      }
    if (hh == 0) LSE[(size_t)pos.bh * N + qrow] = m_ref * scale + log2_fast(ltot) * kLn2;
  }
}

}  // namespace

hipError_t launch_fwd_deferred(const FwdArgs& a, hipStream_t stream) {
  if (a.N > kDeferredMaxN || a.dtype == kDtypeF32 || (a.d != 64 && a.d != 128))
    return hipErrorInvalidValue;
  const int BH = a.B * a.H;
  const int n_mblk = (a.N + kDefBM - 1) / kDefBM;
  const int hpx = heads_per_xcd(BH);
  const int blocks = BH * n_mblk;
  const float sl2 = a.scale * kLog2e;
  const auto* q16 = static_cast<const uint16_t*>(a.q);
  const auto* k16 = static_cast<const uint16_t*>(a.k);
  const auto* v16 = static_cast<const uint16_t*>(a.v);
#define FA_DEF_LAUNCH(TAG, DIM, NS)                                                        \
  hipLaunchKernelGGL((fwd_deferred_kernel<TAG, DIM, NS>), dim3(blocks), dim3(kDefThreads), \
                     0, stream, q16, k16, v16, a.o, a.lse, BH, a.H, a.N, a.scale, sl2,     \
                     a.causal, a.kv_len, n_mblk, hpx)
#define FA_DEF_NSB(TAG, DIM)                            \
  do {                                                  \
    if (a.N <= 128) FA_DEF_LAUNCH(TAG, DIM, 4);         \
    else if (a.N <= 256) FA_DEF_LAUNCH(TAG, DIM, 8);    \
    else FA_DEF_LAUNCH(TAG, DIM, 16);                   \
  } while (0)
  if (a.dtype == kDtypeBF16) {
    if (a.d == 64) FA_DEF_NSB(BF16, 64); else FA_DEF_NSB(BF16, 128);
  } else {
    if (a.d == 64) FA_DEF_NSB(F16, 64); else FA_DEF_NSB(F16, 128);
  }
#undef FA_DEF_NSB
#undef FA_DEF_LAUNCH
  return hipGetLastError();
}

}  // namespace fa
