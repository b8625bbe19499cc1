// Host-side safety tier: the C ABI layer (fa_api.cpp) and the launch index arithmetic
// built by g++ with AddressSanitizer and UndefinedBehaviorSanitizer and driven through
// every entry point. The kernel launchers are replaced by recorders, so nothing here
// touches a GPU: the test checks the host validation (codes, error strings, overflow
// guards, overlap and alignment checks), that accepted calls reach the launcher with the
// arguments given, and that the workgroup placement and the LDS swizzle used by the
// kernels are bijections that stay inside their ranges.
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../include/fa.h"
#include "../io_aware_softmax_tiled_amd/csrc/fa_internal.h"

static int g_fwd_calls = 0, g_bwd_calls = 0, g_merge_calls = 0, g_bwd_stages = -1;
static fa::FwdArgs g_last_fwd{};
static fa::BwdArgs g_last_bwd{};
static hipError_t g_launch_result = hipSuccess;

namespace fa {
hipError_t launch_fwd(const FwdArgs& a, hipStream_t) { ++g_fwd_calls; g_last_fwd = a; return g_launch_result; }
hipError_t launch_fwd_deferred(const FwdArgs& a, hipStream_t) { ++g_fwd_calls; g_last_fwd = a; return g_launch_result; }
hipError_t launch_bwd(const BwdArgs& a, hipStream_t, int stages) { ++g_bwd_calls; g_last_bwd = a; g_bwd_stages = stages; return g_launch_result; }
hipError_t launch_merge(const MergeArgs&, hipStream_t) { ++g_merge_calls; return g_launch_result; }
int device_cu_count() { return 256; }
size_t bwd_delta_bytes(int B, int H, int N) {
  const size_t bytes = (size_t)B * H * N * sizeof(float);
  return (bytes + 255) / 256 * 256;
}
size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  const size_t groups = (size_t)B * H * ((N + kDmaxRows - 1) / kDmaxRows);
  return bwd_delta_bytes(B, H, N) + (groups * sizeof(float) + 255) / 256 * 256;
}
}  // namespace fa

static int g_fail = 0;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, #c, fa_last_error()); ++g_fail; } } while (0)

// fake, well-aligned, non-overlapping device addresses: never dereferenced
static char* P(int i) { return reinterpret_cast<char*>((uintptr_t)0x7f0000000000ull + (uintptr_t)i * 0x10000000ull); }

static void abi_forward() {
  const int B = 2, H = 3, N = 100, d = 64;
  // accepted: reaches the launcher with the same arguments
  g_fwd_calls = 0;
  CHECK(fa_fwd(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B, H, N, d, 0.125f, 1, FA_BF16, nullptr, nullptr) == FA_OK);
  CHECK(g_fwd_calls == 1 && g_last_fwd.N == N && g_last_fwd.causal == 1 && g_last_fwd.dtype == FA_BF16 && g_last_fwd.q == P(0));
  // empty problems are no-ops
  CHECK(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, H, N, d, 0.125f, 0, FA_BF16, nullptr, nullptr) == FA_OK);
  CHECK(g_fwd_calls == 1);
  // rejections, each before any launch
  struct Bad { const void* q; int B, H, N, d; float scale; int dtype; int code; };
  const Bad bad[] = {
      {nullptr, B, H, N, d, 0.1f, FA_BF16, FA_EINVAL},
      {P(0), -1, H, N, d, 0.1f, FA_BF16, FA_EINVAL},
      {P(0), B, H, N, 96, 0.1f, FA_BF16, FA_EUNSUPPORTED},
      {P(0), B, H, N, d, 0.1f, 7, FA_EUNSUPPORTED},
      {P(0), B, H, N, d, -0.1f, FA_BF16, FA_EINVAL},
      {P(0), B, H, N, d, NAN, FA_BF16, FA_EINVAL},
      {P(0), B, H, N, d, INFINITY, FA_BF16, FA_EINVAL},
      {P(0), B, H, (1 << 22) + 1, d, 0.1f, FA_BF16, FA_EINVAL},
      {P(0), INT_MAX, INT_MAX, 1 << 22, 128, 0.1f, FA_BF16, FA_EINVAL},
      {P(0) + 2, B, H, N, d, 0.1f, FA_BF16, FA_EINVAL},
  };
  for (const Bad& b : bad) {
    CHECK(fa_fwd(b.q, P(1), P(2), (float*)P(3), (float*)P(4), b.B, b.H, b.N, b.d, b.scale, 0, b.dtype, nullptr, nullptr) == b.code);
    CHECK(std::strlen(fa_last_error()) > 0);
  }
  // overlapping output and input
  CHECK(fa_fwd(P(0), P(1), P(2), (float*)(P(0) + 64), (float*)P(4), B, H, N, d, 0.1f, 0, FA_BF16, nullptr, nullptr) == FA_EINVAL);
  CHECK(fa_fwd(P(0), P(1), P(2), (float*)P(3), (float*)(P(3) + 16), B, H, N, d, 0.1f, 0, FA_BF16, nullptr, nullptr) == FA_EINVAL);
  CHECK(g_fwd_calls == 1);
  // a launch failure is reported as FA_EHIP with the runtime's message
  g_launch_result = hipErrorInvalidValue;
  CHECK(fa_fwd(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B, H, N, d, 0.1f, 0, FA_F16, nullptr, nullptr) == FA_EHIP);
  g_launch_result = hipSuccess;
  // extensions: split-KV, sparse, dropout, deferred
  CHECK(fa_fwd_partial(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B, H, N, d, 0.1f, 0, FA_BF16, nullptr, 63, nullptr) == FA_EINVAL);
  CHECK(fa_fwd_partial(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B, H, N, d, 0.1f, 0, FA_F32, nullptr, 64, nullptr) == FA_EUNSUPPORTED);
  CHECK(fa_fwd_partial(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B, H, N, d, 0.1f, 0, FA_BF16, nullptr, 64, nullptr) == FA_OK);
  CHECK(g_last_fwd.split_len == 64);
  CHECK(fa_split_count(100, 64) == 2 && fa_split_count(INT_MAX, 64) == (int)((INT_MAX + 63LL) / 64) && fa_split_count(5, 0) == -1);
  // the split rule (256 compute units): two splits without the mask at <= 128 query-block
  // workgroups, four under it at <= 256, >= 2048 keys per split (1024 under the mask);
  // extremes stay in range
  CHECK(fa_split_hint(1, 4, 8192, 128, 0, FA_BF16) == 4096 && fa_split_hint(1, 4, 8192, 128, 1, FA_BF16) == 2048);
  CHECK(fa_split_hint(1, 2, 2048, 128, 1, FA_BF16) == 1024 && fa_split_hint(2, 16, 4096, 128, 1, FA_BF16) == 0);
  CHECK(fa_split_hint(1, 16, 2048, 128, 0, FA_BF16) == 0 && fa_split_hint(1, 8, 4096, 128, 0, FA_BF16) == 2048);
  CHECK(fa_split_hint(1, 4, 8192, 128, 0, FA_F32) == 0 && fa_split_hint(0, 4, 8192, 128, 0, FA_BF16) == 0);
  CHECK(fa_split_hint(1, 1, 65536, 128, 1, FA_F16) == 16384 && fa_split_hint(1, 1, 65536 + 256, 128, 1, FA_BF16) == 0);
  CHECK(fa_split_hint(1, 1, (1 << 22) - 1, 128, 0, FA_BF16) == 0 && fa_split_hint(65535, 1, 4096, 64, 1, FA_BF16) == 0);
  CHECK(fa_split_hint(-1, 4, 8192, 128, 0, FA_BF16) == -FA_EINVAL && fa_split_hint(1, 4, 8192, 96, 0, FA_BF16) == -FA_EUNSUPPORTED);
  CHECK(fa_split_hint(1, 4, (1 << 22) + 1, 128, 0, FA_BF16) == -FA_EINVAL);
  CHECK(fa_fwd_sparse(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B, H, N, d, 0.1f, 0, FA_BF16, nullptr, nullptr, nullptr) == FA_EINVAL);
  CHECK(fa_fwd_sparse(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B, H, N, d, 0.1f, 0, FA_BF16, nullptr, (const uint8_t*)P(5), nullptr) == FA_OK);
  CHECK(fa_fwd_sparse(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B, H, FA_SPARSE_MAX_N + 1, d, 0.1f, 0, FA_BF16, nullptr, (const uint8_t*)P(5), nullptr) == FA_EINVAL);
  for (float p : {-0.5f, 1.0f, NAN, INFINITY})
    CHECK(fa_fwd_dropout(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B, H, N, d, 0.1f, 0, FA_BF16, nullptr, p, 1, 2, nullptr) == FA_EINVAL);
  CHECK(fa_fwd_dropout(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B, H, N, d, 0.1f, 0, FA_BF16, nullptr, 0.17f, 1234, 5, nullptr) == FA_OK);
  CHECK(g_last_fwd.drop_t == 44 && g_last_fwd.seed == 1234 && g_last_fwd.offset == 5);
  CHECK(fa_fwd_deferred(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B, H, FA_DEFERRED_MAX_N + 1, d, 0.1f, 0, FA_BF16, nullptr, nullptr) == FA_EINVAL);
  CHECK(fa_dropout_threshold(0.0f) == 0 && fa_dropout_threshold(0.99999994f) == 255 && fa_dropout_threshold(1e-45f) == 0);
  // merge
  CHECK(fa_merge((const float*)P(0), (const float*)P(1), (float*)P(2), (float*)P(3), 0, B, H, N, d, nullptr) == FA_EINVAL);
  CHECK(fa_merge((const float*)P(0), (const float*)P(1), (float*)P(2), (float*)P(3), 3, B, H, N, d, nullptr) == FA_OK);
  CHECK(g_merge_calls == 1);
  // the forward with its split: unsplit without a workspace (or where no split pays),
  // else partials into the workspace and the merge into o and lse
  {
    const int B2 = 1, H2 = 4, N2 = 8192, d2 = 128;
    const size_t rows = (size_t)B2 * H2 * N2;
    const size_t need = fa_fwd_workspace_size(B2, H2, N2, d2, 0, FA_BF16);
    CHECK(need == (2 * rows * d2 * 4 + 255) / 256 * 256 + 2 * rows * 4);
    CHECK(fa_fwd_workspace_size(2, 16, 4096, 128, 1, FA_BF16) == 0 && fa_fwd_workspace_size(1, 4, 8192, 96, 0, FA_BF16) == 0);
    CHECK(fa_fwd_workspace_size(1, 4, 8192, 128, 0, FA_F32) == 0 && fa_fwd_workspace_size(0, 4, 8192, 128, 0, FA_BF16) == 0);
    g_fwd_calls = 0;
    g_merge_calls = 0;
    CHECK(fa_fwd_auto(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B2, H2, N2, d2, 0.1f, 0, FA_BF16, nullptr, nullptr, 0, nullptr) == FA_OK);
    CHECK(g_fwd_calls == 1 && g_merge_calls == 0 && g_last_fwd.split_len == 0 && g_last_fwd.o == (float*)P(3));
    CHECK(fa_fwd_auto(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B2, H2, N2, d2, 0.1f, 0, FA_BF16, nullptr, P(5), need, nullptr) == FA_OK);
    CHECK(g_fwd_calls == 2 && g_merge_calls == 1 && g_last_fwd.split_len == 4096 && g_last_fwd.o == (float*)P(5));
    CHECK(fa_fwd_auto(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B2, H2, N2, d2, 0.1f, 0, FA_BF16, nullptr, P(5), need - 1, nullptr) == FA_EINVAL);
    CHECK(fa_fwd_auto(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B2, H2, N2, d2, 0.1f, 0, FA_BF16, nullptr, P(5) + 16, need, nullptr) == FA_EINVAL);
    CHECK(fa_fwd_auto(P(0), P(1), P(2), (float*)P(3), (float*)P(4), B2, H2, N2, d2, 0.1f, 0, FA_BF16, nullptr, P(0), need, nullptr) == FA_EINVAL);
    CHECK(g_fwd_calls == 2 && g_merge_calls == 1);
  }
}

static void abi_backward() {
  const int B = 2, H = 3, N = 100, d = 128;
  const size_t ws = fa_bwd_workspace_size(B, H, N, d);
  CHECK(ws >= (size_t)B * H * N * 4 && ws % 256 == 0);
  CHECK(fa_bwd_workspace_size(0, H, N, d) == 0 && fa_bwd_workspace_size(-1, H, N, d) == 0);
  auto call = [&](void* w, size_t wb, int dtype, float* dq) {
    return fa_bwd(P(0), P(1), P(2), (const float*)P(3), P(4), (const float*)P(5), dq, (float*)P(7), (float*)P(8), B, H, N, d, 0.1f, 1, dtype, nullptr, w, wb, nullptr);
  };
  g_bwd_calls = 0;
  CHECK(call(P(9), ws, FA_BF16, (float*)P(6)) == FA_OK);
  CHECK(g_bwd_calls == 1 && g_last_bwd.delta == (float*)P(9) && g_bwd_stages == fa::kBwdAll);
  CHECK((char*)g_last_bwd.dmax == P(9) + fa::bwd_delta_bytes(B, H, N) && (uintptr_t)g_last_bwd.dmax % 256 == 0);
  CHECK(call(P(9), ws - 1, FA_BF16, (float*)P(6)) == FA_EWORKSPACE);
  CHECK(call(nullptr, ws, FA_BF16, (float*)P(6)) == FA_EWORKSPACE);
  CHECK(call(P(9) + 128, ws, FA_BF16, (float*)P(6)) == FA_EINVAL);   // 256-byte alignment
  CHECK(call(P(9), ws, FA_BF16, (float*)P(7)) == FA_EINVAL);         // dq aliases dk
  CHECK(call(P(9), ws, FA_BF16, (float*)P(0)) == FA_EINVAL);         // dq aliases q
  CHECK(g_bwd_calls == 1);
  for (int stage : {-1, 4})
    CHECK(fa_bwd_stage(stage, P(0), P(1), P(2), (const float*)P(3), P(4), (const float*)P(5), (float*)P(6), (float*)P(7), (float*)P(8), B, H, N, d, 0.1f, 1, FA_BF16, nullptr, P(9), ws, nullptr) == FA_EINVAL);
  CHECK(fa_bwd_stage(1, P(0), P(1), P(2), (const float*)P(3), P(4), (const float*)P(5), (float*)P(6), (float*)P(7), (float*)P(8), B, H, N, d, 0.1f, 1, FA_BF16, nullptr, P(9), ws, nullptr) == FA_OK);
  CHECK(g_bwd_stages == 2);
  CHECK(fa_bwd_sparse(P(0), P(1), P(2), (const float*)P(3), P(4), (const float*)P(5), (float*)P(6), (float*)P(7), (float*)P(8), B, H, N, d, 0.1f, 1, FA_BF16, nullptr, nullptr, P(9), ws, nullptr) == FA_EINVAL);
  CHECK(fa_bwd_dropout(P(0), P(1), P(2), (const float*)P(3), P(4), (const float*)P(5), (float*)P(6), (float*)P(7), (float*)P(8), B, H, N, d, 0.1f, 1, FA_BF16, nullptr, 0.5f, 9, 1, P(9), ws, nullptr) == FA_OK);
  CHECK(g_last_bwd.drop_t == 128);
  // fp32 inputs have a backward pass (its own kernels behind the same launcher); the
  // extensions do not
  CHECK(call(P(9), ws, FA_F32, (float*)P(6)) == FA_OK && g_last_bwd.dtype == FA_F32);
  CHECK(fa_bwd_dropout(P(0), P(1), P(2), (const float*)P(3), P(4), (const float*)P(5), (float*)P(6), (float*)P(7), (float*)P(8), B, H, N, d, 0.1f, 1, FA_F32, nullptr, 0.5f, 9, 1, P(9), ws, nullptr) == FA_EUNSUPPORTED);
  // status strings and the error buffer, including a message longer than the buffer
  for (int s = -1; s <= 5; ++s) CHECK(fa_status_str(s) != nullptr);
  CHECK(fa_version() > 0);
}

// workgroup placement: blockIdx -> (head, block) covers every (head, block) exactly once
static void placement() {
  for (int BH : {1, 2, 3, 7, 8, 9, 15, 16, 24, 32, 40, 64, 96, 128}) {
    for (int blocks : {1, 2, 3, 5, 16, 33}) {
      const int hpx = fa::heads_per_xcd(BH);
      std::vector<int> seen((size_t)BH * blocks, 0);
      for (int w = 0; w < BH * blocks; ++w) {
        const fa::WgPos p = fa::wg_position(hpx, w, BH);
        CHECK(p.bh >= 0 && p.bh < BH && p.blk >= 0 && p.blk < blocks);
        if (p.bh >= 0 && p.bh < BH && p.blk >= 0 && p.blk < blocks) ++seen[(size_t)p.bh * blocks + p.blk];
        if (hpx) CHECK(p.bh % 8 == w % 8);   // XCD-major: a head stays on one XCD
      }
      for (int c : seen) CHECK(c == 1);
    }
  }
  for (int m = 0; m < 32; ++m) CHECK(fa::kappa(fa::kappa(m)) == m && fa::kappa(m) >= 0 && fa::kappa(m) < 32);
}

// LDS swizzle: inside every row the 16-byte chunks are a permutation, rows stay inside
// their own bytes, and 16 consecutive rows read at one logical chunk hit 16 distinct slots
template <int D> static void swizzle() {
  constexpr int kChunks = D / 8;
  for (int row = 0; row < 64; ++row) {
    std::vector<int> hit(kChunks, 0);
    for (int c = 0; c < kChunks; ++c) {
      const int off = fa::tile_off<D>(row, c);
      CHECK(off >= row * D * 2 && off + 16 <= (row + 1) * D * 2 && off % 16 == 0);
      ++hit[(off - row * D * 2) / 16];
    }
    for (int h : hit) CHECK(h == 1);
  }
  for (int r0 = 0; r0 < 64; r0 += 16)
    for (int c = 0; c < kChunks; ++c) {
      std::vector<int> slot(kChunks > 16 ? kChunks : 16, 0);
      for (int r = r0; r < r0 + 16; ++r) ++slot[((fa::tile_off<D>(r, c) / 16) % 16)];
      int distinct = 0;
      for (int s : slot) distinct += s > 0;
      CHECK(distinct == 16);
    }
}

int main() {
  abi_forward();
  abi_backward();
  placement();
  swizzle<64>();
  swizzle<128>();
  if (g_fail) { std::printf("%d checks failed\n", g_fail); return 1; }
  std::printf("ALL OK\n");
  return 0;
}
