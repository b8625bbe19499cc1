// Device-side helpers shared by the forward and backward kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used throughout (checked on the device by a layout probe):
//   v_mfma_f32_32x32x16_{bf16,f16}: C[32x32] += A[32x16] * B[16x32].
//     lane l holds A[l%32][8*(l/32) + 0..7] and B[8*(l/32) + 0..7][l%32];
//     accumulator register r of lane l is C[8*(r/4) + 4*(l/32) + r%4][l%32].
//   v_mfma_f32_32x32x2f32: lane l holds A[l%32][l/32], B[l/32][l%32]; same C layout.
//   ds_read_b64_tr_b16: inside each group of 16 lanes, lanes 4e..4e+3 point at four
//     consecutive 4-element pieces of "row e"; lane i of the group receives element i
//     of rows 0..3. This reads a row-major [key][d] tile as the [d][key] operand.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_index.h"

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-bit element tag types: the storage is uint16_t; the tag selects the MFMA flavour.
struct BF16 {};
struct F16 {};

template <typename T> struct Mfma;
template <> struct Mfma<BF16> {
  __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two fp32 -> packed pair, round to nearest even
  __device__ static inline uint32_t pack(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
  // sum of a packed pair, accumulated in fp32
  __device__ static inline float dot_ones(uint32_t p, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), one, acc, false);
  }
};
template <> struct Mfma<F16> {
  __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack(float lo, float hi) {
    f16x2 r = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
  __device__ static inline float dot_ones(uint32_t p, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), one, acc, false);
  }
};

// bf16 pair -> f16 pair (exact for magnitudes in the fp16 normal range, and for 0)
__device__ inline uint32_t bf16x2_to_f16x2(uint32_t x) {
  const float lo = __uint_as_float(x << 16);
  const float hi = __uint_as_float(x & 0xffff0000u);
  f16x2 r = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

// 8 input elements (16 bytes of bf16 or f16) -> 8 fp16
template <typename T> __device__ inline u32x4 to_f16x8(u32x4 x);
template <> __device__ inline u32x4 to_f16x8<F16>(u32x4 x) { return x; }
template <> __device__ inline u32x4 to_f16x8<BF16>(u32x4 x) {
  return {bf16x2_to_f16x2(x[0]), bf16x2_to_f16x2(x[1]), bf16x2_to_f16x2(x[2]),
          bf16x2_to_f16x2(x[3])};
}

// the two elements of a packed bf16 or f16 pair as fp32
template <typename T> __device__ inline void unpack2(uint32_t x, float& lo, float& hi);
template <> __device__ inline void unpack2<BF16>(uint32_t x, float& lo, float& hi) {
  lo = __uint_as_float(x << 16);
  hi = __uint_as_float(x & 0xffff0000u);
}
template <> __device__ inline void unpack2<F16>(uint32_t x, float& lo, float& hi) {
  const f16x2 v = __builtin_bit_cast(f16x2, x);
  lo = (float)v[0];
  hi = (float)v[1];
}

// 8 input elements -> 8 fp16 of x * s, s a power of two (exact unless the product
// leaves the fp16 range)
template <typename T> __device__ inline u32x4 to_f16x8_scaled(u32x4 x, float s) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo, hi;
    unpack2<T>(x[i], lo, hi);
    r[i] = Mfma<F16>::pack(lo * s, hi * s);
  }
  return r;
}

// largest magnitude among the 8 elements of a 16-bit chunk, as fp32 (for non-NaN bf16
// and fp16 the magnitude bits order like unsigned integers)
template <typename T> __device__ inline float absmax8(u32x4 x) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = x[i] & 0x7fff7fffu;
    m = max(m, max(a & 0xffffu, a >> 16));
  }
  float lo, hi;
  unpack2<T>(m, lo, hi);
  return lo;
}

// Power-of-two scale for a largest magnitude m of dO: 1 while m lies in [2^-3, 2^4)
// (there fp16 already holds dO, dP and dS with its full 11-bit precision and no risk of
// overflow, since |dS| <= 2 max|dO|_2 max|V|_2), otherwise 2^(1 - e) for m = f 2^e,
// f in [0.5, 1), which brings m into [1, 2) (the exponent clamped so the scale stays a
// normal fp32); 1 for m = 0 or a non-finite m. The backward pass multiplies dO by it
// before rounding to fp16 and divides the gradients by it exactly in the fp32 epilogue,
// so small gradients do not sink into fp16 subnormals and large ones do not overflow.
__device__ inline float pow2_scale(float m) {
  if (!(m > 0.f) || !(m <= 3.4e38f)) return 1.0f;
  if (m >= 0.125f && m < 16.0f) return 1.0f;
  int e;
  (void)__builtin_frexpf(m, &e);
  const int x = min(126, max(-126, 1 - e));
  return __builtin_ldexpf(1.0f, x);
}


__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Reductions across the two 32-lane halves of the wave. v_permlane32_swap with both
// operands equal to x returns (lanes 0-31: x, x[l+32]; lanes 32-63: x[l-32], x), so
// combining its two results gives every lane the value over lanes l and l ^ 32.
__device__ inline float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// 16-byte LDS read / write
__device__ inline u32x4 lds_read16(const FA_LDS uint8_t* p) {
  return *reinterpret_cast<const FA_LDS u32x4*>(p);
}
__device__ inline void lds_write16(FA_LDS uint8_t* p, u32x4 v) {
  *reinterpret_cast<FA_LDS u32x4*>(p) = v;
}
// transposing 8-byte LDS read (see header comment)
__device__ inline u32x2 lds_read_tr16(const FA_LDS uint8_t* p) {
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<FA_LDS i16x4*>(const_cast<FA_LDS uint8_t*>(p)));
  return __builtin_bit_cast(u32x2, t);
}

// Workgroup barrier that hands LDS data between waves: it waits for this wave's LDS
// operations only, not for its outstanding global loads, so prefetches issued before it
// stay in flight across it (__syncthreads() also waits for every global load). The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ inline void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC11): ten rounds over a 4 x 32-bit counter with a
// 2 x 32-bit key; each round multiplies counter words 0 and 2 by fixed constants, keeps
// both 32-bit halves of the 64-bit products (one v_mad_u64_u32 each) and mixes them with
// words 1 and 3 and the round key; the key advances by fixed Weyl increments between
// rounds. The dropout mask is a pure function of (counter, key), so the backward pass
// regenerates it on chip.
struct Philox4x32 {
  uint32_t w[4];
};
__device__ inline Philox4x32 philox4x32(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                        uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)kM0 * c0, p1 = (uint64_t)kM1 * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c0 = n0;
    c1 = (uint32_t)p1;
    c2 = n2;
    c3 = (uint32_t)p0;
    k0 += kW0;
    k1 += kW1;
  }
  return {{c0, c1, c2, c3}};
}

// Buffer resource over `bytes` bytes from `base` (wave-uniform): a load through it at
// byte offset o >= bytes returns zeros instead of touching memory, so tiles that run
// past the end of a sequence need no clamping, and moving to the next tile is scalar
// arithmetic on the resource rather than per-lane address arithmetic.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ inline u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)offset, 0, 0);
}


}  // namespace fa
