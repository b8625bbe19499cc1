// Forward pass of exact attention on gfx950: one workgroup per block of query rows of
// one (batch, head), 32 rows per wave; key/value tiles of 64 rows stream through LDS
// while the online-softmax state (running maximum, running denominator, unnormalised
// output) stays in registers, so the N x N scores never reach HBM.
//
// Method: "[Review] From Online Softmax to Flash Attention", Algorithm FlashAttention
// (Tiling) -- per key tile: local maximum, new running maximum, denominator rescaled
// by e^{m_old - m_new} plus the tile's sum, output rescaled the same way plus the
// tile's P V. "FlashAttention: Fast and Memory-Efficient Exact Attention with
// IO-Awareness", Method: the same update in Br x Bc block form. Loop order: query
// blocks outer (one per workgroup), key/value tiles inner, as in the review's
// Thoughts section on FlashAttention-2.
//
// Choices made for CDNA4 (not taken from the pages):
// * Scores are computed transposed, S^T = K Q^T, on 32x32x16 matrix cores, so each
//   lane owns one query row: the row maximum and row sum are in-lane reductions plus
//   one swap between the two 32-lane halves, and the output rescale is a per-lane
//   scalar. K rows are read with bits 2 and 3 of the row index swapped, which makes
//   every lane's 8 consecutive accumulator registers hold 8 consecutive keys: the
//   packed P feeds the P V product as its B operand with no data movement.
// * O^T = V^T P^T takes V^T through the transposing LDS read, so V is staged in LDS
//   row-major exactly like K.
// * K and V tiles are staged global -> registers -> LDS (V converted to fp16 on the
//   way) into an XOR-swizzled layout with three buffers per tensor: the tile two ahead
//   is written and the one three ahead is fetched while the current one is used, with
//   one barrier per tile that waits for LDS traffic only. Loads go through buffer
//   resources placed at the tile, so rows past the end of the sequence read as zeros.
// * The key loop is software-pipelined over 32-key sub-blocks: the score product of the
//   next sub-block (matrix cores) runs beside the exponentials of the current one
//   (vector units), and the P V product beside the next row maximum; the LDS fragments
//   of each product are read one region ahead. Scheduling hints interleave the streams.
// * exp2 with scale*log2(e) folded into one FMA; the output is normalised once at the
//   end (the pages normalise every step; the results are equal). The reference
//   maximum used in the exponent is only raised when a sub-block's maximum exceeds it
//   by more than 2^15 in the exponent (P stays inside fp16), so the output rescale is
//   rare; the final division uses the same reference, so the result is unchanged.
// * Masking touches only the sub-blocks that cross the diagonal, the key-padding bound
//   or the end of the sequence for a wave; tiles past the workgroup's last visible key
//   are not visited, and a wave skips the products of sub-blocks past its own last
//   visible key. Under the causal mask the two waves of each SIMD take a short and a
//   long row group, so the SIMDs share the diagonal tiles' work evenly.
// * Workgroups are ordered heaviest-first for causal attention; when B*H is a multiple
//   of 8, all query blocks of a head are placed on one XCD so its K/V tiles are shared
//   in that XCD's L2 (otherwise heads vary fastest, to keep every XCD busy).
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

// Item of round k for persistent workgroup p of P (-1 when done). Items u are numbered
// heaviest first; with xcd, the items of one XCD (u = 8 v + x) are dealt to that XCD's
// workgroups (p = 8 j + x) in a snake: v = k Px + j on even rounds, k Px + Px - 1 - j on
// odd ones, so heavy and light blocks pair up on every workgroup.
__device__ inline int snake_item(int p, int P, int n_items, int k, bool xcd) {
  if (xcd && P % 8 == 0) {
    const int x = p & 7, j = p >> 3, px = P >> 3;
    const int v = k * px + ((k & 1) ? px - 1 - j : j);
    const int u = 8 * v + x;
    return u < n_items ? u : -1;
  }
  const int u = k * P + ((k & 1) ? P - 1 - p : p);
  return u < n_items ? u : -1;
}
constexpr int kBN = 64;    // key rows per tile

// ---------------------------------------------------------------------------------
// 16-bit inputs (bf16 or f16)
// ---------------------------------------------------------------------------------
// W waves per workgroup (4 or 8), 32 query rows each. With 8 waves every K/V tile
// loaded into LDS serves 256 query rows, halving the tile traffic per FLOP; 4 waves
// keep enough workgroups for small problems.
//
// kMode 1, split-KV: workgroup index = split * per_split + (position as above); split p
// covers keys [p*split_len, (p+1)*split_len) and writes its normalised partial output
// and LSE at O + p*o_stride, LSE + p*lse_stride.
// kMode 2, block-sparse: bmask is an n_sb x n_sb byte matrix over 128-row query blocks
// and 128-key blocks; key blocks whose entry is 0 for the query block are hidden. Each
// workgroup first lists the key blocks enabled for any of its query blocks (the LDS
// list below) and streams only those tiles; a wave whose own query block leaves a
// listed key block disabled masks it.
// In both modes a row that sees no key gets O = 0 and LSE = -inf.
// kMode 3, dropout: the normalised probabilities are multiplied by Z / keep, Z_ij = 1
// iff random byte (i, j) >= drop_t, keep = (256 - drop_t) / 256 (keep_scale = 1/keep);
// byte (i, j) of head bh, with j = 32 g + u, is byte 8 (u / 16) + u % 8 of the
// Philox4x32-10 block at counter (i, 2 g + (u / 8) % 2, bh, offset) under the key
// (seed_lo, seed_hi). The statistics (and LSE) are those of the undropped scores.

template <typename T, int D, int W, int kMode>
__global__ __launch_bounds__(W * 64, 8 / W) void fwd_kernel_16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
    int BH, int H, int N, float scale, float sl2, int causal,
    const int* __restrict__ kv_len, int n_mblk, int heads_per_xcd, int split_len,
    int per_split, size_t o_stride, size_t lse_stride, const uint8_t* __restrict__ bmask,
    int n_sb, uint32_t seed_lo, uint32_t seed_hi, uint32_t offset, int drop_t,
    float keep_scale, int n_items) {
  constexpr bool kPartial = kMode == 1;
  constexpr bool kSparse = kMode == 2;
  constexpr bool kDropout = kMode == 3;
  constexpr bool kGuard = kMode != 0;  // rows may see no key at all
  constexpr int kTileBytes = kBN * D * 2;              // one K or V tile
  constexpr int kKC = D / 16;                          // 16-wide k-steps over head_dim
  constexpr int kDB = D / 32;                          // 32-row blocks of O^T
  constexpr int kCPR = D / 8;                          // 16-byte chunks per row
  constexpr int kThr = W * 64;
  constexpr int kBMw = W * 32;                         // query rows per workgroup
  constexpr int kVChunks = kTileBytes / 16 / kThr;     // K/V chunks per thread per tile
  // three buffers per tensor, as separate arrays so the compiler can tell the tiles
  // being read from the one being filled
  __shared__ __attribute__((aligned(1024))) uint8_t Kb0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t Kb1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t Kb2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t Vb0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t Vb1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t Vb2[kTileBytes];
  // block-sparse: enabled key blocks of this workgroup, each entry kb | (enabled for the
  // first query block) << 14 | (enabled for the second) << 15, then a sentinel 0
  __shared__ uint16_t blist[kSparse ? kSparseMaxBlocks + 1 : 1];
  __shared__ int blist_len;

  // Persistent grid: workgroup p walks a list of work items (query blocks), built so
  // that the blocks of a head stay on one XCD and each workgroup pairs heavy and light
  // blocks (a snake over the heaviest-first order); a barrier separates items.
  // (head_dim 64 runs one item per workgroup: the loop would cost it the registers
  // that let two workgroups share a compute unit)
  constexpr bool kPersist = D == 128;
  for (int kround = 0;; ++kround) {
    const int u = kPersist ? snake_item(blockIdx.x, gridDim.x, n_items, kround, heads_per_xcd != 0)
                           : (kround == 0 ? (int)blockIdx.x : -1);
    if (u < 0) break;
    [&]() {
      int split = 0, wid = u;
      if constexpr (kPartial) {
        split = u / per_split;
        wid = u - split * per_split;
      }
      const WgPos pos = wg_position(heads_per_xcd, wid, BH);
      if (pos.bh >= BH) return;
      const int mblk = n_mblk - 1 - pos.blk;  // heaviest query block first
      const int b = pos.bh / H;
      const size_t head = (size_t)pos.bh * N * D;
      const uint16_t* q = Q + head;
      const uint16_t* k = K + head;
      const uint16_t* v = V + head;
      float* const Op = kPartial ? O + split * o_stride : O;
      float* const LSEp = kPartial ? LSE + split * lse_stride : LSE;

      int kv_lim = N;
      if (kv_len != nullptr) kv_lim = min(N, max(1, kv_len[b]));
      const int m0 = mblk * kBMw;
      // keys [kbeg, kv_hi) of this workgroup's range can be visible: all of them, or one
      // split's range (its first key is a tile boundary)
      const int kbeg = kPartial ? split * split_len : 0;
      const int kv_hi = kPartial ? min(kv_lim, kbeg + split_len) : kv_lim;
      const int kend = causal ? min(kv_hi, m0 + kBMw) : kv_hi;
      // >= 1 without a split (key 0 is always visible); a split may hold no visible key
      int ntiles = kend > kbeg ? (kend - kbeg + kBN - 1) / kBN : 0;

      const int tid = threadIdx.x;
      const int lane = tid & 63;
      const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
      const int qi = lane & 31;
      const int hh = lane >> 5;
      // Waves w and w + 4 share a SIMD. With 8 waves the second four take the row groups in
      // reverse order (4 -> 7, ..., 7 -> 4), so under the causal mask each SIMD holds one
      // short and one long row group and the SIMDs finish the diagonal tiles together.
      const int wrow = (W == 8 && wave >= 4) ? 11 - wave : wave;
      const int wq0 = m0 + wrow * 32;              // first query row of this wave
      const int qrow = wq0 + qi;
      const int qrow_c = min(qrow, N - 1);

      // block-sparse: which of the workgroup's (one or two) query blocks this wave is in
      const int qb_lo = m0 / kSparseBlock;
      const int wave_flag = (wq0 / kSparseBlock == qb_lo) ? (1 << 14) : (1 << 15);
      if constexpr (kSparse) {
        // wave 0 compacts the enabled key blocks below the workgroup's last visible key
        if (wave == 0) {
          const int qb_hi = (m0 + kBMw - 1) / kSparseBlock;
          const int nkb = (kend + kSparseBlock - 1) / kSparseBlock;
          int count = 0;
          for (int base = 0; base < nkb; base += 64) {
            const int kb = base + lane;
            int entry = 0;
            if (kb < nkb) {
              const bool f0 = bmask[(size_t)qb_lo * n_sb + kb] != 0;
              const bool f1 = qb_hi != qb_lo && qb_hi < n_sb && bmask[(size_t)qb_hi * n_sb + kb] != 0;
              entry = kb | (f0 ? 1 << 14 : 0) | (f1 ? 1 << 15 : 0);
            }
            const uint64_t on = __ballot(entry >> 14);
            const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(on >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)on, 0));
            if (entry >> 14) blist[count + before] = (uint16_t)entry;
            count += __popcll(on);
          }
          if (lane == 0) {
            blist[count] = 0;  // sentinel: a block enabled for nobody
            blist_len = count;
          }
        }
        __syncthreads();
        ntiles = 2 * blist_len;
      }

      // 32-key sub-blocks (from kbeg) holding a key that some row of this wave can see:
      // under the causal mask or a key bound the trailing sub-blocks of the workgroup's
      // range may hold none, and the wave then skips their products and exponentials
      // (it still takes part in the tile staging and the barriers)
      int ns_live = 2 * ntiles;
      if constexpr (!kSparse) {
        const int wave_kend = causal ? min(kv_hi, wq0 + 32) : kv_hi;
        ns_live = __builtin_amdgcn_readfirstlane(min(ns_live, max(0, (wave_kend - kbeg + 31) / 32)));
      }

      if constexpr (kGuard) {
        if (ntiles == 0) {  // no key is visible to this block: empty rows
          if (qrow < N) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            float* orow = Op + head + (size_t)qrow * D;
#pragma unroll
            for (int c = 0; c < D / 8; ++c) *reinterpret_cast<f32x4*>(orow + 8 * c + 4 * hh) = z;
            if (hh == 0) LSEp[(size_t)pos.bh * N + qrow] = -INFINITY;
          }
          return;
        }
      }

      // K and V tiles -> registers with coalesced 16-byte loads, then -> LDS (V converted to
      // fp16), two tiles ahead of the one being computed. Loads go through a buffer resource
      // that starts at the tile, so rows past the end of the sequence read as zeros.
      u32x4 ks[kVChunks], vs[kVChunks];
      uint32_t ld_off[kVChunks];   // byte offset of this thread's chunks inside a tile
#pragma unroll
      for (int j = 0; j < kVChunks; ++j) {
        const int ci = tid + kThr * j;
        ld_off[j] = (uint32_t)((ci / kCPR) * D + (ci % kCPR) * 8) * 2;
      }
      // first key of tile t (64 keys) and of sub-block sb (32 keys)
      auto tile_key = [&](int t) {
        if constexpr (kSparse)
          return __builtin_amdgcn_readfirstlane((blist[t >> 1] & 0x1fff) * kSparseBlock + (t & 1) * kBN);
        else
          return kbeg + t * kBN;
      };
      auto load_kv_to = [&](int t, u32x4 (&kd)[kVChunks], u32x4 (&vd)[kVChunks]) {
        const int n0 = tile_key(t);
        // (a sparse list may name a tile past the end of the sequence: zero bytes)
        const uint32_t bytes = (uint32_t)max(N - n0, 0) * D * 2;
        const auto rk = buffer_rsrc(k + (size_t)n0 * D, bytes);
        const auto rv = buffer_rsrc(v + (size_t)n0 * D, bytes);
#pragma unroll
        for (int j = 0; j < kVChunks; ++j) {
          kd[j] = buffer_load16(rk, ld_off[j]);
          vd[j] = buffer_load16(rv, ld_off[j]);
        }
      };
      auto load_kv = [&](int t) { load_kv_to(t, ks, vs); };
      auto store_kv_from = [&](FA_LDS uint8_t* kb, FA_LDS uint8_t* vb, const u32x4 (&kd)[kVChunks],
                               const u32x4 (&vd)[kVChunks]) {
#pragma unroll
        for (int j = 0; j < kVChunks; ++j) {
          const int ci = tid + kThr * j;
          const int row = ci / kCPR, ch = ci % kCPR;
          lds_write16(kb + tile_off<D>(row, ch), kd[j]);
          lds_write16(vb + tile_off<D>(row, ch), to_f16x8<T>(vd[j]));
        }
      };
      auto store_kv = [&](FA_LDS uint8_t* kb, FA_LDS uint8_t* vb) { store_kv_from(kb, vb, ks, vs); };
      const int tlast = ntiles - 1;
      // tiles 0 and 1 are fetched together (tile 1 into registers used only here), so the
      // workgroup waits for one global-memory latency before its first product, not two
      u32x4 ks1[kVChunks], vs1[kVChunks];
      load_kv(0);
      load_kv_to(min(1, tlast), ks1, vs1);

      // Q fragment: B operand of S^T = K Q^T, lane (qi, hh) holds Q[qrow][16c + 8hh + 0..7]
      u32x4 qf[kKC];
#pragma unroll
      for (int c = 0; c < kKC; ++c)
        qf[c] = *reinterpret_cast<const u32x4*>(q + (size_t)qrow_c * D + 16 * c + 8 * hh);

      f32x16 oacc[kDB];
#pragma unroll
      for (int i = 0; i < kDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;

      float m_ref = -INFINITY;  // reference maximum used in the exponent (raw score units)
      float lsum = 0.f;         // this lane's half of the running denominator
      const int krow_base = kappa(qi);
      const int g = lane >> 4, gi = lane & 15;

      // Per-lane byte offsets inside a K or V tile, fixed for the whole loop. The swizzle
      // depends only on the low 4 bits of the row, so moving by 16 or 32 rows (and between
      // buffers) is a compile-time constant the LDS instructions take as an immediate offset.
      int koff[kKC];
#pragma unroll
      for (int c = 0; c < kKC; ++c) koff[c] = tile_off<D>(krow_base, 2 * c + hh);
      int voff[2][kDB];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int db = 0; db < kDB; ++db)
          voff[r][db] = tile_off<D>(8 * hh + (gi >> 2) + 4 * r, db * 4 + 2 * (g & 1) + ((gi & 3) >> 1)) +
                        8 * (gi & 1);

      store_kv((FA_LDS uint8_t*)Kb0, (FA_LDS uint8_t*)Vb0);  // tile 0
      load_kv(min(2, tlast));
      store_kv_from((FA_LDS uint8_t*)Kb1, (FA_LDS uint8_t*)Vb1, ks1, vs1);  // tile 1 (clamped)

      // The key axis is walked in 32-key sub-blocks (the tiled recurrence with tile width
      // 32), software-pipelined so each region pairs matrix-core work with vector work of
      // the neighbouring sub-block, while the LDS fragments of the next region are read:
      //   region A: scores of sub-block s+1 (MFMA) | P of sub-block s (exp, pack, sum)
      //             | V fragments of sub-block s
      //   region B: O^T += V^T P^T of sub-block s  | row maximum of sub-block s+1
      //             | K fragments of sub-block s+2
      // followed by the (rare) rescale for sub-block s+1. Hints interleave the streams
      // inside each region so the vector units and the LDS work while the matrix cores do.
      u32x4 kf[kKC];          // K fragments (A operand) of the next score product
      u32x2 vf[2][kDB][2];    // V^T fragments (A operand) of the next P V product
      auto read_k = [&](const FA_LDS uint8_t* Ks, int sub) {
#pragma unroll
        for (int c = 0; c < kKC; ++c) kf[c] = lds_read16(Ks + koff[c] + sub * 32 * D * 2);
      };
      auto read_v = [&](const FA_LDS uint8_t* Vs, int sub) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int db = 0; db < kDB; ++db) {
            const int rows = (32 * sub + 16 * c2) * D * 2;
            vf[c2][db][0] = lds_read_tr16(Vs + voff[0][db] + rows);
            vf[c2][db][1] = lds_read_tr16(Vs + voff[1][db] + rows);
          }
      };
      // S^T for 32 keys from the K fragments in kf
      auto scores = [&]() {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int c = 0; c < kKC; ++c) acc = Mfma<T>::run(kf[c], qf[c], acc);
        return acc;
      };
      // P = exp2(s*scale*log2e - m_ref*scale*log2e), rounded to fp16, and its row sum;
      // with dropout the product takes P * Z (the scale 1/keep is applied at the end) while
      // the row sum takes P. Sub-block sb: keys 32*sb .. 32*sb+31; this lane's register r
      // holds key 32*sb + 16*(r/8) + 8*hh + r%8, whose random byte is byte r of the Philox
      // block at counter (query, 2*sb + hh, head, offset): one block per lane and sub-block.
      auto expo = [&](const f32x16& s, uint32_t (&pk)[8], int sb) {
        uint32_t rnd[4] = {0, 0, 0, 0};
        if constexpr (kDropout) {
          const Philox4x32 ph = philox4x32((uint32_t)qrow, (uint32_t)(2 * sb + hh),
                                           (uint32_t)pos.bh, offset, seed_lo, seed_hi);
#pragma unroll
          for (int w = 0; w < 4; ++w) rnd[w] = ph.w[w];
        }
        // (a row that has seen no visible key yet -- possible in a split or a sparse
        // pattern -- keeps
        // m_ref = -inf; its scores are all -inf and must give P = 0, not NaN)
        const float nms = (kGuard && m_ref == -INFINITY) ? 0.f : -m_ref * sl2;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = exp2_fast(fmaf(s[2 * i], sl2, nms));
          const float p1 = exp2_fast(fmaf(s[2 * i + 1], sl2, nms));
          pk[i] = Mfma<F16>::pack(p0, p1);
          lsum = Mfma<F16>::dot_ones(pk[i], lsum);
          if constexpr (kDropout) {
            // registers 2i, 2i+1: bytes 2i and 2i+1, in word i/2
            const uint32_t wv = rnd[i >> 1] >> (16 * (i & 1));
            const bool keep0 = (int)(wv & 0xff) >= drop_t;
            const bool keep1 = (int)((wv >> 8) & 0xff) >= drop_t;
            pk[i] = Mfma<F16>::pack(keep0 ? p0 : 0.f, keep1 ? p1 : 0.f);
          }
        }
      };
      // two 16-key steps of O^T += V^T P^T from the V^T fragments in vf
      auto pv = [&](const uint32_t (&pk)[8]) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const u32x4 bp = {pk[4 * c2], pk[4 * c2 + 1], pk[4 * c2 + 2], pk[4 * c2 + 3]};
#pragma unroll
          for (int db = 0; db < kDB; ++db)
            oacc[db] = Mfma<F16>::run(u32x4{vf[c2][db][0][0], vf[c2][db][0][1],
                                            vf[c2][db][1][0], vf[c2][db][1][1]},
                                      bp, oacc[db]);
        }
      };
      auto rowmax = [&](const f32x16& s) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = max3f(mx, s[r], s[r + 1]);
        return max_halves(mx);  // both halves of the wave hold the same query rows
      };
      // a row raises its reference maximum only when the exponent would exceed 2^15 (P is
      // then at most 2^15, inside fp16); the decision is per row, so each row's arithmetic
      // depends on its own scores only
      auto rescale = [&](float mx) {
        const bool grow = (mx - m_ref) * sl2 > 15.0f;
        if (__any(grow)) {
          const float m_new = grow ? mx : m_ref;
          const float alpha = exp2_fast((m_ref - m_new) * sl2);  // 1 if kept, 0 from -inf
          m_ref = m_new;
          lsum *= alpha;
#pragma unroll
          for (int i = 0; i < kDB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
        }
      };
      // -inf where a key of sub-block `sb` is hidden from this lane's query (diagonal,
      // padding or sequence end); only sub-blocks that cross one of those bounds for this
      // wave are touched. Register r holds key 32*sb + 8*hh + 16*(r/8) + r%8, so one
      // per-lane bound (the last visible key, relative to the lane's first key) decides all
      // sixteen.
      const int last_vis = (causal ? min(kv_hi - 1, qrow) : kv_hi - 1) - 8 * hh;
      auto mask = [&](f32x16& s, int sb) {
        int n0 = kbeg + 32 * sb;
        bool off = false;  // block-sparse: the whole sub-block is disabled for this wave
        if constexpr (kSparse) {
          const int e = __builtin_amdgcn_readfirstlane(blist[sb >> 2]);
          n0 = (e & 0x1fff) * kSparseBlock + (sb & 3) * 32;
          off = (e & wave_flag) == 0;
        }
        if (off || (n0 + 32 > kv_hi) || (causal && n0 + 31 > wq0)) {
          const int lim = off ? -1 : last_vis - n0;
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = (16 * (r >> 3) + (r & 7) > lim) ? -INFINITY : s[r];
        }
      };
      // issue priority by region: a wave raises its priority for one of the two regions of
      // each half-step (head_dim 128: the score region, 64: the P V region), which favours
      // the SIMD's other wave when they meet in different regions (about 2% faster at both
      // head dims; the opposite choice was slower at 64)
      auto prio_scores = [&]() { __builtin_amdgcn_s_setprio(D == 128 ? 1 : 0); };
      auto prio_pv = [&]() { __builtin_amdgcn_s_setprio(D == 128 ? 0 : 1); };
      // keeps P in the region that computes it (the compiler would otherwise sink it into
      // the P V region, past the masking branch, and lose the overlap)
      auto pin = [&](const uint32_t (&pk)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(pk[i]));
      };
      // region A: each score MFMA followed by its share of the vector instructions (the 48
      // of expo, plus those of the tile store when one is in the region) and of the V
      // fragment reads
      auto hint_a = [&](auto nvalu) {
        constexpr int kPer = decltype(nvalu)::value / kKC;
#pragma unroll
        for (int c = 0; c < kKC; ++c) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, kPer, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 4 * kDB / kKC, 0);
        }
      };
      // region B: each P V MFMA followed by a K fragment read and a vector instruction of
      // the row maximum
      auto hint_b = [&]() {
#pragma unroll
        for (int c = 0; c < 2 * kDB; ++c) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, (kKC + 2 * kDB - 1) / (2 * kDB), 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
      };

      barrier_lds();  // tiles 0 and 1 visible
      read_k((const FA_LDS uint8_t*)Kb0, 0);
      f32x16 S;
      // (head_dim 64 runs every sub-block through the full step, so its first scores are
      // always formed; a sub-block nobody in the wave sees is masked to -inf there)
      if (D == 64 || ns_live > 0) {
        S = scores();
        mask(S, 0);
        rescale(rowmax(S));
      }
      read_k((const FA_LDS uint8_t*)Kb0, 1);

      // One key tile = two sub-blocks; tile t lives in buffers t%3. After the barrier that
      // opens step t every wave is done with tile t-1, so tile t+2 (held in registers) is
      // written into its buffers and tile t+3 is fetched. Every wave stages every tile of
      // the workgroup's range; inside its last tiles (step_tail below) it skips the
      // sub-blocks that hold no key visible to it and masks the rest.
      auto step = [&](int t, const FA_LDS uint8_t* Ka, const FA_LDS uint8_t* Va,
                      const FA_LDS uint8_t* Kn, FA_LDS uint8_t* Kw, FA_LDS uint8_t* Vw) {
        barrier_lds();
        store_kv(Kw, Vw);
        load_kv(min(t + 3, tlast));

        uint32_t pk[8];
        prio_scores();
        f32x16 Sn = scores();        // sub-block 2t+1 (K fragments read beforehand)
        expo(S, pk, 2 * t);          // P of sub-block 2t
        read_v(Va, 0);
        hint_a(std::integral_constant<int, 48 + 12 * kVChunks + 12>{});  // with the V conversion and the load addresses
        pin(pk);
        mask(Sn, 2 * t + 1);
        prio_pv();
        pv(pk);
        float mx = rowmax(Sn);
        read_k(Kn, 0);
        hint_b();
        rescale(mx);

        prio_scores();
        S = scores();                // sub-block 2t+2
        expo(Sn, pk, 2 * t + 1);     // P of sub-block 2t+1
        read_v(Va, 1);
        hint_a(std::integral_constant<int, 48>{});
        pin(pk);
        mask(S, 2 * t + 2);
        prio_pv();
        pv(pk);
        mx = rowmax(S);
        read_k(Kn, 1);
        hint_b();
        rescale(mx);
      };

      // The same step for the wave's last tiles, where a sub-block may hold no key visible
      // to the wave: each product and its vector work runs only for live sub-blocks, and
      // the buffers are chosen at run time (these steps are few, so they are not unrolled).
      auto step_tail = [&](int t) {
        const int r = t % 3;
        const FA_LDS uint8_t* Va = r == 0 ? (const FA_LDS uint8_t*)Vb0
                                 : r == 1 ? (const FA_LDS uint8_t*)Vb1 : (const FA_LDS uint8_t*)Vb2;
        const FA_LDS uint8_t* Kn = r == 0 ? (const FA_LDS uint8_t*)Kb1
                                 : r == 1 ? (const FA_LDS uint8_t*)Kb2 : (const FA_LDS uint8_t*)Kb0;
        FA_LDS uint8_t* Kw = r == 0 ? (FA_LDS uint8_t*)Kb2 : r == 1 ? (FA_LDS uint8_t*)Kb0 : (FA_LDS uint8_t*)Kb1;
        FA_LDS uint8_t* Vw = r == 0 ? (FA_LDS uint8_t*)Vb2 : r == 1 ? (FA_LDS uint8_t*)Vb0 : (FA_LDS uint8_t*)Vb1;
        const bool l0 = 2 * t < ns_live, l1 = 2 * t + 1 < ns_live, l2 = 2 * t + 2 < ns_live;
        barrier_lds();
        store_kv(Kw, Vw);
        load_kv(min(t + 3, tlast));

        uint32_t pk[8];
        f32x16 Sn = S;
        if (l1) Sn = scores();
        if (l0) expo(S, pk, 2 * t);
        read_v(Va, 0);
        if (l1) mask(Sn, 2 * t + 1);
        if (l0) pv(pk);
        read_k(Kn, 0);
        if (l1) rescale(rowmax(Sn));

        if (l2) S = scores();
        if (l1) expo(Sn, pk, 2 * t + 1);
        read_v(Va, 1);
        if (l2) mask(S, 2 * t + 2);
        if (l1) pv(pk);
        read_k(Kn, 1);
        if (l2) rescale(rowmax(S));
      };

      if constexpr (D == 64) {
        // head_dim 64 keeps every tile on the full step: the tail steps' extra registers
        // would push it past 128 VGPRs and halve its occupancy (two 8-wave workgroups per
        // CU); sub-blocks past a wave's diagonal are masked instead of skipped
        for (int t = 0; t < ntiles; t += 3) {
          step(t, (const FA_LDS uint8_t*)Kb0, (const FA_LDS uint8_t*)Vb0,
               (const FA_LDS uint8_t*)Kb1, (FA_LDS uint8_t*)Kb2, (FA_LDS uint8_t*)Vb2);
          if (t + 1 < ntiles)
            step(t + 1, (const FA_LDS uint8_t*)Kb1, (const FA_LDS uint8_t*)Vb1,
                 (const FA_LDS uint8_t*)Kb2, (FA_LDS uint8_t*)Kb0, (FA_LDS uint8_t*)Vb0);
          if (t + 2 < ntiles)
            step(t + 2, (const FA_LDS uint8_t*)Kb2, (const FA_LDS uint8_t*)Vb2,
                 (const FA_LDS uint8_t*)Kb0, (FA_LDS uint8_t*)Kb1, (FA_LDS uint8_t*)Vb1);
        }
      } else {
        // tiles t < t_hot have all three sub-blocks 2t, 2t+1, 2t+2 live for this wave
        const int t_hot = ns_live > 0 ? (ns_live - 1) / 2 : 0;
        int t = 0;
        for (; t < t_hot; t += 3) {
          step(t, (const FA_LDS uint8_t*)Kb0, (const FA_LDS uint8_t*)Vb0,
               (const FA_LDS uint8_t*)Kb1, (FA_LDS uint8_t*)Kb2, (FA_LDS uint8_t*)Vb2);
          if (t + 1 >= t_hot) { t += 1; break; }
          step(t + 1, (const FA_LDS uint8_t*)Kb1, (const FA_LDS uint8_t*)Vb1,
               (const FA_LDS uint8_t*)Kb2, (FA_LDS uint8_t*)Kb0, (FA_LDS uint8_t*)Vb0);
          if (t + 2 >= t_hot) { t += 2; break; }
          step(t + 2, (const FA_LDS uint8_t*)Kb2, (const FA_LDS uint8_t*)Vb2,
               (const FA_LDS uint8_t*)Kb0, (FA_LDS uint8_t*)Kb1, (FA_LDS uint8_t*)Vb1);
        }
        for (; t < ntiles; ++t) step_tail(t);
      }

      // epilogue: O = O_acc / l, LSE = scale*m_ref + ln(l)
      const float ltot = sum_halves(lsum);
      if (qrow < N) {
        // a row with no visible key (split or sparse pattern: ltot = 0) gets O = 0, LSE = -inf
        const bool empty = kGuard && !(ltot > 0.f);
        const float inv = empty ? 0.f : (kDropout ? keep_scale : 1.0f) / ltot;
        float* orow = Op + head + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const f32x4 val = {oacc[db][4 * a4 + 0] * inv, oacc[db][4 * a4 + 1] * inv,
                               oacc[db][4 * a4 + 2] * inv, oacc[db][4 * a4 + 3] * inv};
            *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * a4 + 4 * hh) = val;
          }
        if (hh == 0)
          LSEp[(size_t)pos.bh * N + qrow] =
              empty ? -INFINITY : m_ref * scale + log2_fast(ltot) * kLn2;
      }
    }();
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------
// fp32 inputs: 32x32x2 fp32 matrix cores, one workgroup per 32 query rows of a head.
// The key axis of the row group is split over the workgroup's KS waves: wave w takes the
// 32-key sub-blocks w, w + KS, w + 2 KS, ... and keeps its own reference maximum, row sum
// and unnormalised O^T; at the end the KS partial states are combined through LDS as
// split-KV partials are, M = max_w m_w, L = sum_w e^{m_w - M} l_w,
// O = sum_w e^{m_w - M} O_w / L, LSE = M + ln L (the same online-softmax identity the
// per-tile update uses). The fp32 products take 64 cycles each, so a row group's chain of
// products is the latency of a small problem; splitting its keys over KS SIMDs shortens
// that chain KS-fold. Each wave reads its K and V fragments straight from global memory.
// Head-dim order inside the score product: step c pairs element c of the lane half
// hh = 0 with element D/2 + c of the half hh = 1, so each lane's Q and K fragments are
// contiguous halves of their rows (any order of the head_dim sum gives S).
// ---------------------------------------------------------------------------------
template <int D, int KS>
__global__ __launch_bounds__(KS * 64, 1) void fwd_kernel_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int BH, int H, int N, float scale,
    float sl2, int causal, const int* __restrict__ kv_len, int n_rg, int heads_per_xcd) {
  constexpr int kDB = D / 32;   // 32-row blocks of O^T
  constexpr int kHalf = D / 2;  // head_dim elements per lane half
  constexpr int kLd = 33;       // padded query stride of the partial O^T in LDS
  __shared__ float so[KS][D * kLd];  // partial O^T of each wave, [d][query]
  __shared__ float sm[KS][32];       // reference maximum of each wave, per query
  __shared__ float sl[KS][32];       // row sum of each wave, per query

  const WgPos pos = wg_position(heads_per_xcd, blockIdx.x, BH);
  if (pos.bh >= BH) return;
  const int rg = n_rg - 1 - pos.blk;  // heaviest row group first
  const int b = pos.bh / H;
  const size_t head = (size_t)pos.bh * N * D;
  const float* q = Q + head;
  const float* k = K + head;
  const float* v = V + head;
  int kv_lim = N;
  if (kv_len != nullptr) kv_lim = min(N, max(1, kv_len[b]));
  const int r0 = rg * 32;
  // every sub-block below nsub holds a key that every row of the group can see (its first
  // key is below kv_lim and, under the causal mask, not after the group's first row)
  const int kend = causal ? min(kv_lim, r0 + 32) : kv_lim;
  const int nsub = (kend + 31) / 32;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int qi = lane & 31;
  const int hh = lane >> 5;
  const int qrow = r0 + qi;
  const int qrow_c = min(qrow, N - 1);

  // Q fragment (B operand): lane (qi, hh) holds Q[qrow][hh D/2 + c], c < D/2
  float qf[kHalf];
#pragma unroll
  for (int c = 0; c < kHalf; c += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(q + (size_t)qrow_c * D + hh * kHalf + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) qf[c + j] = x[j];
  }

  f32x16 oacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_ref = -INFINITY;  // raw score units
  float lsum = 0.f;         // this lane's half of the row sum

  for (int j = wave; j < nsub; j += KS) {
    const int n0 = 32 * j;
    // K fragment (A operand of S^T = K Q^T): row n0 + qi, the lane's half of head_dim.
    // Rows past the end of the sequence are clamped to the last row (finite values) and
    // masked below.
    float kf[kHalf];
    const float* krow = k + (size_t)min(n0 + qi, N - 1) * D + hh * kHalf;
#pragma unroll
    for (int c = 0; c < kHalf; c += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(krow + c);
#pragma unroll
      for (int t = 0; t < 4; ++t) kf[c + t] = x[t];
    }
    // V fragments (A operand of O^T += V^T P^T): accumulator register r of lane (qi, hh)
    // holds key n0 + 8 (r / 4) + 4 hh + r % 4, so the product's step r takes that key's V
    // row, element 32 db + qi
    float vf[kDB][16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float* vrow = v + (size_t)min(n0 + 8 * (r >> 2) + 4 * hh + (r & 3), N - 1) * D + qi;
#pragma unroll
      for (int db = 0; db < kDB; ++db) vf[db][r] = vrow[32 * db];
    }

    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int c = 0; c < kHalf; ++c) s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[c], qf[c], s, 0, 0, 0);

    if (n0 + 32 > kv_lim || (causal && n0 + 31 > r0)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = n0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        const bool hide = key >= kv_lim || (causal && key > qrow);
        s[r] = hide ? -INFINITY : s[r];
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = max3f(mx, s[r], s[r + 1]);
    mx = max_halves(mx);
    // the reference maximum is raised only when the exponent would exceed 2^8
    const bool grow = (mx - m_ref) * sl2 > 8.0f;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_ref;
      const float alpha = exp2_fast((m_ref - m_new) * sl2);  // 1 if kept, 0 from -inf
      m_ref = m_new;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < kDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }
    const float nms = -m_ref * sl2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = exp2_fast(fmaf(s[r], sl2, nms));
      lsum += s[r];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int db = 0; db < kDB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf[db][r], s[r], oacc[db], 0, 0, 0);
  }

  // partial states -> LDS (a wave that took no sub-block leaves m = -inf, l = 0, O = 0)
  const float ltot = sum_halves(lsum);
  if (hh == 0) {
    sm[wave][qi] = m_ref;
    sl[wave][qi] = ltot;
  }
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      so[wave][(32 * db + 8 * (r >> 2) + 4 * hh + (r & 3)) * kLd + qi] = oacc[db][r];
  __syncthreads();

  // combination: thread t owns query row t / TPR and EPT consecutive head_dim columns
  constexpr int kTPR = KS * 64 / 32;
  constexpr int kEPT = D / kTPR;
  static_assert(kEPT % 4 == 0, "16-byte output stores");
  const int row = threadIdx.x / kTPR;
  const int d0 = (threadIdx.x % kTPR) * kEPT;
  const int orow_i = r0 + row;
  if (orow_i < N) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < KS; ++w) M = fmaxf(M, sm[w][row]);
    float cw[KS];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < KS; ++w) {
      const float mw = sm[w][row];
      cw[w] = mw == -INFINITY ? 0.f : exp2_fast((mw - M) * sl2);
      L += cw[w] * sl[w][row];
    }
    const float inv = 1.0f / L;
    float* orow = O + head + (size_t)orow_i * D;
#pragma unroll
    for (int e = 0; e < kEPT; e += 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < KS; ++w) {
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] += cw[w] * so[w][(d0 + e + t) * kLd + row];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] *= inv;
      *reinterpret_cast<f32x4*>(orow + d0 + e) = acc;
    }
    if (d0 == 0) LSE[(size_t)pos.bh * N + orow_i] = M * scale + log2_fast(L) * kLn2;
  }
}

}  // namespace

FwdGrid fwd_grid(int B, int H, int N, int waves) {
  FwdGrid g;
  g.n_mblk = (N + 32 * waves - 1) / (32 * waves);
  g.heads_per_xcd = heads_per_xcd(B * H);
  g.blocks = B * H * g.n_mblk;
  return g;
}

int device_cu_count() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

// Workgroups of a persistent grid: the items, capped at per_cu resident workgroups on
// every compute unit (a multiple of 8, the XCD count).
static int persistent_grid(int items, int per_cu) {
  const int cap = device_cu_count() * per_cu;
  return items < cap ? items : cap;
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  const bool partial_or_sparse = a.split_len > 0 || a.block_mask != nullptr;
  const int waves = (a.d == 128 && partial_or_sparse)
                        ? 8 : fwd_waves(a.B, a.H, a.N, a.d, a.dtype, device_cu_count());
  const FwdGrid g = fwd_grid(a.B, a.H, a.N, waves);
  const auto* q16 = static_cast<const uint16_t*>(a.q);
  const auto* k16 = static_cast<const uint16_t*>(a.k);
  const auto* v16 = static_cast<const uint16_t*>(a.v);
  const float sl2 = a.scale * kLog2e;
  const int BH = a.B * a.H;
  const bool partial = a.split_len > 0;
  const bool sparse = a.block_mask != nullptr;
  const int n_splits = partial ? (a.N + a.split_len - 1) / a.split_len : 1;
  const size_t o_stride = (size_t)BH * a.N * a.d, lse_stride = (size_t)BH * a.N;
  const int n_sb = (a.N + kSparseBlock - 1) / kSparseBlock;
  const bool dropout = a.drop_t >= 0;
  const float keep_scale = dropout ? 256.0f / (float)(256 - a.drop_t) : 1.0f;
#define FA_LAUNCH16W(TAG, DIM, WV, MODE)                                                   \
  hipLaunchKernelGGL((fwd_kernel_16<TAG, DIM, WV, MODE>),                                   \
                     dim3(DIM == 128 ? persistent_grid(g.blocks * n_splits, 1)           \
                                     : g.blocks * n_splits),                                  \
                     dim3(WV * 64), 0, stream, q16, k16, v16, a.o, a.lse, BH, a.H, a.N,     \
                     a.scale, sl2, a.causal, a.kv_len, g.n_mblk, g.heads_per_xcd,           \
                     a.split_len, g.blocks, o_stride, lse_stride, a.block_mask, n_sb,      \
                     (uint32_t)a.seed, (uint32_t)(a.seed >> 32), a.offset, a.drop_t,       \
                     keep_scale, g.blocks * n_splits)
#define FA_LAUNCH16(TAG, DIM, MODE)                                 \
  do {                                                              \
    if (waves == 8) FA_LAUNCH16W(TAG, DIM, 8, MODE);                \
    else FA_LAUNCH16W(TAG, DIM, 4, MODE);                           \
  } while (0)
#define FA_LAUNCH16P(TAG, DIM)                       \
  do {                                               \
    if (partial) FA_LAUNCH16(TAG, DIM, 1);           \
    else if (sparse) FA_LAUNCH16(TAG, DIM, 2);       \
    else if (dropout) FA_LAUNCH16(TAG, DIM, 3);      \
    else FA_LAUNCH16(TAG, DIM, 0);                   \
  } while (0)
  // fp32: one workgroup per 32 query rows, the keys split over 8 waves at head_dim 64 and
  // over 4 at 128 (its fragments need more than the 256 registers of two waves per SIMD)
  const int n_rg = (a.N + 31) / 32;
#define FA_LAUNCH32(DIM, KS)                                                                \
  hipLaunchKernelGGL((fwd_kernel_f32<DIM, KS>), dim3(BH * n_rg), dim3(KS * 64), 0, stream,  \
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),         \
                     static_cast<const float*>(a.v), a.o, a.lse, BH, a.H, a.N, a.scale, sl2,   \
                     a.causal, a.kv_len, n_rg, g.heads_per_xcd)
  if (a.dtype == kDtypeBF16) {
    if (a.d == 64) FA_LAUNCH16P(BF16, 64); else FA_LAUNCH16P(BF16, 128);
  } else if (a.dtype == kDtypeF16) {
    if (a.d == 64) FA_LAUNCH16P(F16, 64); else FA_LAUNCH16P(F16, 128);
  } else {
    if (partial || sparse || dropout) return hipErrorNotSupported;  // rejected by the API
    if (a.d == 64) FA_LAUNCH32(64, 8); else FA_LAUNCH32(128, 4);
  }
#undef FA_LAUNCH16P
#undef FA_LAUNCH16
#undef FA_LAUNCH16W
#undef FA_LAUNCH32
  return hipGetLastError();
}

}  // namespace fa
