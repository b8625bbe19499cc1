// Index arithmetic shared by the kernels and their launchers: workgroup placement, the
// row order of matrix-core operands and the LDS tile swizzle. Plain integer functions
// that compile for the host too, so the host-side checks can enumerate them.
#pragma once

#if defined(__HIPCC__)
#define FA_HD __host__ __device__
#else
#define FA_HD
#endif

namespace fa {

// swap bits 2 and 3 of a row index in [0, 32): reading A-operand rows in this order
// makes accumulator register r of lane l hold row 16*(r/8) + 8*(l/32) + r%8, i.e. each
// lane's 8 consecutive registers cover 8 consecutive rows
FA_HD inline int kappa(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// blockIdx.x -> (head, block), block index `slot / heads_per_xcd` counted from 0. When
// B*H is a multiple of 8 (heads_per_xcd = B*H/8) the mapping is XCD-major: consecutive
// workgroups go to consecutive XCDs, and all blocks of a head land on one XCD so its
// K/V tiles are shared in that XCD's L2. Otherwise (heads_per_xcd = 0) heads vary
// fastest, so every XCD still gets an equal share of the work when there are fewer
// heads than XCDs or they do not divide evenly. Either way the grid is B*H x blocks.
struct WgPos {
  int bh, blk;
};
FA_HD inline WgPos wg_position(int heads_per_xcd, int w, int BH) {
  if (heads_per_xcd == 0) return {w % BH, w / BH};
  const int xcd = w & 7;
  const int slot = w >> 3;
  return {(slot % heads_per_xcd) * 8 + xcd, slot / heads_per_xcd};
}

// heads_per_xcd argument of the kernels: B*H/8 when B*H is a multiple of 8 (XCD-major
// placement), else 0 (heads vary fastest); the grid is B*H x blocks per head either way
inline int heads_per_xcd(int BH) { return BH % 8 == 0 ? BH / 8 : 0; }

// XOR swizzle of 16-byte chunks inside a 16-bit-element tile row, so that
// (a) 16 consecutive rows read at one logical chunk hit 16 distinct chunk slots and
// (b) 4 consecutive rows read through the transposing load hit distinct 64-byte groups.
template <int D> FA_HD constexpr int chunk_swizzle(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
}

// byte offset of (row, logical 16-byte chunk) in a swizzled [rows][D] 16-bit tile
template <int D> FA_HD constexpr int tile_off(int row, int chunk) {
  return row * (D * 2) + ((chunk ^ chunk_swizzle<D>(row)) << 4);
}

}  // namespace fa
