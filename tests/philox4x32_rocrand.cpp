// Independent reference for the oracle's Philox4x32-10: the host-callable engine of the
// ROCm random-number library (rocRAND). The engine keys itself with the 64-bit seed,
// places the subsequence in counter words 2-3 and offset/4 in words 0-1, and returns the
// four words of the block in order; so block (c0, c1, c2, c3) under key (k0, k1) is the
// engine at seed k0 + 2^32 k1, subsequence c2 + 2^32 c3, offset 4 (c0 + 2^32 c1).
// Test infrastructure only: built by the oracle's pin tests with the host compiler.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdint>

extern "C" void philox4x32_rocrand(const uint32_t* ctr, const uint32_t* key, uint32_t* out,
                                   int n) {
  for (int b = 0; b < n; ++b) {
    const uint32_t* c = ctr + 4 * b;
    const unsigned long long seed = key[2 * b] | ((unsigned long long)key[2 * b + 1] << 32);
    const unsigned long long sub = c[2] | ((unsigned long long)c[3] << 32);
    const unsigned long long off = 4ull * (c[0] | ((unsigned long long)c[1] << 32));
    rocrand_device::philox4x32_10_engine e(seed, sub, off);
    for (int w = 0; w < 4; ++w) out[4 * b + w] = e.next();
  }
}
