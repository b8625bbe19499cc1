// C ABI of the exact-attention library: host-side validation, workspace sizing,
// error strings, and dispatch to the kernel launchers. Nothing here allocates device
// memory or keeps state between calls. The operations and the contract of every
// entry point are documented in include/fa.h.
#include "../../include/fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "fa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_last_error[0] = '\0'; }

}  // namespace

namespace fa {
int api_fail(int status, const char* msg) {
  snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
  return status;
}
}  // namespace fa

namespace {

size_t elem_size(int dtype) { return dtype == FA_F32 ? 4 : 2; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Span {
  const void* p;
  size_t bytes;
  const char* name;
};

bool overlap(const Span& a, const Span& b) {
  if (a.bytes == 0 || b.bytes == 0) return false;
  const auto a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Shared checks of sizes, dtype, head_dim and scale. Returns FA_OK or an error.
int check_common(int B, int H, int N, int d, float scale, int dtype) {
  if (B < 0 || H < 0 || N < 0)
    return fail(FA_EINVAL, "sizes must be >= 0 (B=%d H=%d N=%d)", B, H, N);
  if (dtype != FA_F32 && dtype != FA_BF16 && dtype != FA_F16)
    return fail(FA_EUNSUPPORTED, "unknown dtype code %d (0=f32, 1=bf16, 2=f16)", dtype);
  if (d != 64 && d != 128) return fail(FA_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", d);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(FA_EINVAL, "scale must be finite and > 0 (got %g)", (double)scale);
  if (N > (1 << 22)) return fail(FA_EINVAL, "N=%d exceeds the limit 2^22", N);
  const double elems = (double)B * H * N * d;
  if (elems >= 1099511627776.0) return fail(FA_EINVAL, "B*H*N*d too large");
  // grid: 8 * ceil(B*H/8) * ceil(N/128) workgroups, and ceil(N/64) per head backward
  const double blocks = 8.0 * std::ceil((double)B * H / 8.0) * std::ceil(N / 64.0);
  if (blocks >= 2147483647.0) return fail(FA_EINVAL, "too many workgroups for one launch");
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_EINVAL: return "FA_EINVAL: invalid argument";
    case FA_EUNSUPPORTED: return "FA_EUNSUPPORTED: unsupported head_dim or dtype";
    case FA_EWORKSPACE: return "FA_EWORKSPACE: workspace missing or too small";
    case FA_EHIP: return "FA_EHIP: HIP runtime error at launch";
    default: return "unknown status";
  }
}

const char* fa_last_error(void) { return g_last_error; }

int fa_version(void) { return 100; /* 0.1.0 */ }

}  // extern "C"

namespace fa {
// the size, dtype and scale checks of the backward entry points, without any pointer
int bwd_check_sizes(int B, int H, int N, int d, float scale, int dtype) {
  clear_error();
  return check_common(B, H, N, d, scale, dtype);
}
}  // namespace fa

extern "C" int fa_dropout_threshold(float p) {
  if (!(p >= 0.0f && p < 1.0f)) return -1;
  const int t = (int)std::floor(256.0 * (double)p + 0.5);
  return t < 255 ? t : 255;
}

namespace {

size_t sparse_mask_bytes(int N) {
  const size_t n_sb = ((size_t)N + FA_SPARSE_BLOCK - 1) / FA_SPARSE_BLOCK;
  return n_sb * n_sb;
}

int check_sparse(int N, int dtype, const uint8_t* block_mask) {
  if (dtype == FA_F32)
    return fail(FA_EUNSUPPORTED, "block-sparse attention takes bf16 or f16 inputs, not f32");
  if (N > FA_SPARSE_MAX_N)
    return fail(FA_EINVAL, "N=%d exceeds the block-sparse limit %d", N, FA_SPARSE_MAX_N);
  if (N > 0 && !block_mask) return fail(FA_EINVAL, "null block_mask");
  return FA_OK;
}

// Dropout of the probabilities: byte threshold t (-1: none) and the generator key.
struct Drop {
  int t = -1;
  uint64_t seed = 0;
  uint32_t offset = 0;
};

// keep iff the element's random byte >= t = fa_dropout_threshold(p)
int check_dropout(int dtype, float p, Drop* out) {
  if (dtype == FA_F32)
    return fail(FA_EUNSUPPORTED, "attention with dropout takes bf16 or f16 inputs, not f32");
  const int t = fa_dropout_threshold(p);
  if (t < 0) return fail(FA_EINVAL, "dropout p=%g is not in [0, 1)", p);
  out->t = t;
  return FA_OK;
}

int fwd_impl(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H,
             int N, int d, float scale, int causal, int dtype, const int32_t* kv_len,
             const uint8_t* block_mask, void* stream, const Drop& drop = Drop(),
             bool deferred = false) {
  clear_error();
  int st = check_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  if ((size_t)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return fail(FA_EINVAL, "null tensor pointer");
  const size_t in_bytes = (size_t)B * H * N * d * elem_size(dtype);
  const size_t o_bytes = (size_t)B * H * N * d * 4;
  const size_t lse_bytes = (size_t)B * H * N * 4;
  const Span ins[] = {{q, in_bytes, "q"}, {k, in_bytes, "k"}, {v, in_bytes, "v"},
                      {kv_len, kv_len ? (size_t)B * 4 : 0, "kv_len"},
                      {block_mask, block_mask ? sparse_mask_bytes(N) : 0, "block_mask"}};
  const Span outs[] = {{o, o_bytes, "o"}, {lse, lse_bytes, "lse"}};
  for (const Span& s : ins) {
    const size_t al = s.p == kv_len ? 4 : s.p == block_mask ? 1 : 16;
    if (s.bytes && !aligned(s.p, al)) return fail(FA_EINVAL, "%s is not %zu-byte aligned", s.name, al);
  }
  if (!aligned(o, 16)) return fail(FA_EINVAL, "o is not 16-byte aligned");
  if (!aligned(lse, 4)) return fail(FA_EINVAL, "lse is not 4-byte aligned");
  for (const Span& a : outs) {
    for (const Span& b : ins)
      if (overlap(a, b)) return fail(FA_EINVAL, "output %s overlaps input %s", a.name, b.name);
  }
  if (overlap(outs[0], outs[1])) return fail(FA_EINVAL, "outputs o and lse overlap");

  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, scale, causal ? 1 : 0, dtype, kv_len};
  a.block_mask = block_mask;
  a.drop_t = drop.t;
  a.seed = drop.seed;
  a.offset = drop.offset;
  hipError_t e = deferred ? fa::launch_fwd_deferred(a, static_cast<hipStream_t>(stream))
                          : fa::launch_fwd(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_EHIP, "forward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H,
           int N, int d, float scale, int causal, int dtype, const int32_t* kv_len,
           void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, kv_len, nullptr, stream);
}

int fa_fwd_sparse(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                  int H, int N, int d, float scale, int causal, int dtype,
                  const int32_t* kv_len, const uint8_t* block_mask, void* stream) {
  clear_error();
  int st = check_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  st = check_sparse(N, dtype, block_mask);
  if (st != FA_OK) return st;
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, kv_len, block_mask,
                  stream);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                   int H, int N, int d, float scale, int causal, int dtype,
                   const int32_t* kv_len, float p, uint64_t seed, uint32_t offset,
                   void* stream) {
  clear_error();
  int st = check_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  Drop drop;
  st = check_dropout(dtype, p, &drop);
  if (st != FA_OK) return st;
  drop.seed = seed;
  drop.offset = offset;
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, kv_len, nullptr, stream,
                  drop);
}

int fa_fwd_deferred(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                    int H, int N, int d, float scale, int causal, int dtype,
                    const int32_t* kv_len, void* stream) {
  clear_error();
  int st = check_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_F32)
    return fail(FA_EUNSUPPORTED, "the deferred-PV forward takes bf16 or f16 inputs, not f32");
  if (N > FA_DEFERRED_MAX_N)
    return fail(FA_EINVAL, "N=%d exceeds the deferred-PV limit %d", N, FA_DEFERRED_MAX_N);
  static_assert(FA_DEFERRED_MAX_N == fa::kDeferredMaxN, "limit mismatch");
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, kv_len, nullptr, stream,
                  Drop(), true);
}

int fa_split_count(int N, int split_len) {
  if (split_len <= 0 || split_len % 64 != 0 || N < 0) return -1;
  return (int)(((long long)N + split_len - 1) / split_len);
}

int fa_split_hint(int B, int H, int N, int d, int causal, int dtype) {
  clear_error();
  const int st = check_common(B, H, N, d, 1.0f, dtype);
  if (st != FA_OK) return -st;
  return fa::fwd_split_hint(B, H, N, d, causal ? 1 : 0, dtype, fa::device_cu_count());
}

int fa_fwd_partial(const void* q, const void* k, const void* v, float* o_part,
                   float* lse_part, int B, int H, int N, int d, float scale, int causal,
                   int dtype, const int32_t* kv_len, int split_len, void* stream) {
  clear_error();
  int st = check_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_F32)
    return fail(FA_EUNSUPPORTED, "split-KV partials take bf16 or f16 inputs, not f32");
  if (split_len <= 0 || split_len % 64 != 0)
    return fail(FA_EINVAL, "split_len must be a positive multiple of 64 (got %d)", split_len);
  if ((size_t)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o_part || !lse_part) return fail(FA_EINVAL, "null tensor pointer");
  const int P = fa_split_count(N, split_len);
  if ((double)P * B * H * N * d >= 1099511627776.0)
    return fail(FA_EINVAL, "n_splits*B*H*N*d too large");
  const double blocks = (double)P * 8.0 * std::ceil((double)B * H / 8.0) * std::ceil(N / 64.0);
  if (blocks >= 2147483647.0) return fail(FA_EINVAL, "too many workgroups for one launch");
  const size_t in_bytes = (size_t)B * H * N * d * elem_size(dtype);
  const size_t o_bytes = (size_t)P * B * H * N * d * 4;
  const size_t lse_bytes = (size_t)P * B * H * N * 4;
  const Span ins[] = {{q, in_bytes, "q"}, {k, in_bytes, "k"}, {v, in_bytes, "v"},
                      {kv_len, kv_len ? (size_t)B * 4 : 0, "kv_len"}};
  const Span outs[] = {{o_part, o_bytes, "o_part"}, {lse_part, lse_bytes, "lse_part"}};
  for (const Span& s : ins)
    if (s.bytes && !aligned(s.p, s.p == kv_len ? 4 : 16))
      return fail(FA_EINVAL, "%s is not %d-byte aligned", s.name, s.p == kv_len ? 4 : 16);
  if (!aligned(o_part, 16)) return fail(FA_EINVAL, "o_part is not 16-byte aligned");
  if (!aligned(lse_part, 4)) return fail(FA_EINVAL, "lse_part is not 4-byte aligned");
  for (const Span& a : outs)
    for (const Span& b : ins)
      if (overlap(a, b)) return fail(FA_EINVAL, "output %s overlaps input %s", a.name, b.name);
  if (overlap(outs[0], outs[1])) return fail(FA_EINVAL, "outputs o_part and lse_part overlap");

  fa::FwdArgs a{q, k, v, o_part, lse_part, B, H, N, d, scale, causal ? 1 : 0, dtype, kv_len};
  a.split_len = split_len;
  hipError_t e = fa::launch_fwd(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(FA_EHIP, "partial forward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

int fa_merge(const float* o_part, const float* lse_part, float* o, float* lse, int n_splits,
             int B, int H, int N, int d, void* stream) {
  clear_error();
  if (B < 0 || H < 0 || N < 0)
    return fail(FA_EINVAL, "sizes must be >= 0 (B=%d H=%d N=%d)", B, H, N);
  if (d != 64 && d != 128) return fail(FA_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", d);
  if (n_splits < 1) return fail(FA_EINVAL, "n_splits must be >= 1 (got %d)", n_splits);
  if (n_splits > 65536) return fail(FA_EINVAL, "n_splits=%d exceeds the limit 65536", n_splits);
  if (N > (1 << 22)) return fail(FA_EINVAL, "N=%d exceeds the limit 2^22", N);
  if ((double)n_splits * B * H * N * d >= 1099511627776.0)
    return fail(FA_EINVAL, "n_splits*B*H*N*d too large");
  if ((double)B * H * N * (d / 4) / 256.0 >= 2147483647.0)
    return fail(FA_EINVAL, "too many workgroups for one launch");
  if ((size_t)B * H * N == 0) return FA_OK;
  if (!o_part || !lse_part || !o || !lse) return fail(FA_EINVAL, "null tensor pointer");
  const size_t rows = (size_t)B * H * N;
  const Span ins[] = {{o_part, (size_t)n_splits * rows * d * 4, "o_part"},
                      {lse_part, (size_t)n_splits * rows * 4, "lse_part"}};
  const Span outs[] = {{o, rows * d * 4, "o"}, {lse, rows * 4, "lse"}};
  if (!aligned(o_part, 16) || !aligned(o, 16))
    return fail(FA_EINVAL, "o_part and o must be 16-byte aligned");
  if (!aligned(lse_part, 4) || !aligned(lse, 4))
    return fail(FA_EINVAL, "lse_part and lse must be 4-byte aligned");
  for (const Span& a : outs)
    for (const Span& b : ins)
      if (overlap(a, b)) return fail(FA_EINVAL, "output %s overlaps input %s", a.name, b.name);
  if (overlap(outs[0], outs[1])) return fail(FA_EINVAL, "outputs o and lse overlap");

  fa::MergeArgs a{o_part, lse_part, o, lse, n_splits, B, H, N, d};
  hipError_t e = fa::launch_merge(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_EHIP, "merge launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

size_t fa_fwd_workspace_size(int B, int H, int N, int d, int causal, int dtype) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  if (check_common(B, H, N, d, 1.0f, dtype) != FA_OK) return 0;
  const int split_len = fa::fwd_split_hint(B, H, N, d, causal ? 1 : 0, dtype, fa::device_cu_count());
  if (split_len <= 0) return 0;
  const size_t P = (size_t)fa_split_count(N, split_len);
  const size_t rows = (size_t)B * H * N;
  return (P * rows * d * 4 + 255) / 256 * 256 + P * rows * 4;
}

int fa_fwd_auto(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                int H, int N, int d, float scale, int causal, int dtype, const int32_t* kv_len,
                void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int st = check_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  const size_t need = fa_fwd_workspace_size(B, H, N, d, causal, dtype);
  if (need == 0 || workspace == nullptr)
    return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, kv_len, nullptr, stream);
  if (workspace_bytes < need)
    return fail(FA_EINVAL, "workspace of %zu bytes is smaller than the %zu this shape needs",
                workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(FA_EINVAL, "workspace is not 256-byte aligned");
  const int split_len = fa::fwd_split_hint(B, H, N, d, causal ? 1 : 0, dtype, fa::device_cu_count());
  const int P = fa_split_count(N, split_len);
  const size_t rows = (size_t)B * H * N;
  float* o_part = static_cast<float*>(workspace);
  float* lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             ((size_t)P * rows * d * 4 + 255) / 256 * 256);
  // both calls check their own buffers: the partials (inside the workspace) against q, k,
  // v and kv_len, and o and lse against the partials
  st = fa_fwd_partial(q, k, v, o_part, lse_part, B, H, N, d, scale, causal, dtype, kv_len,
                      split_len, stream);
  if (st != FA_OK) return st;
  return fa_merge(o_part, lse_part, o, lse, P, B, H, N, d, stream);
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return 0;
  return fa::bwd_workspace_bytes(B, H, N, d);
}

}  // extern "C"

namespace {

int bwd_impl(const void* q, const void* k, const void* v, const float* o, const void* dout,
             const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
             float scale, int causal, int dtype, const int32_t* kv_len,
             const uint8_t* block_mask, void* workspace, size_t workspace_bytes,
             void* stream, int stages = fa::kBwdAll, const Drop& drop = Drop()) {
  clear_error();
  int st = check_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  if ((size_t)B * H * N == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(FA_EINVAL, "null tensor pointer");
  const size_t need = fa::bwd_workspace_bytes(B, H, N, d);
  if (!workspace || workspace_bytes < need)
    return fail(FA_EWORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(FA_EINVAL, "workspace is not 256-byte aligned");
  const size_t in_bytes = (size_t)B * H * N * d * elem_size(dtype);
  const size_t f_bytes = (size_t)B * H * N * d * 4;
  const size_t lse_bytes = (size_t)B * H * N * 4;
  const Span ins[] = {{q, in_bytes, "q"},       {k, in_bytes, "k"},         {v, in_bytes, "v"},
                      {o, f_bytes, "o"},        {dout, in_bytes, "dout"},   {lse, lse_bytes, "lse"},
                      {kv_len, kv_len ? (size_t)B * 4 : 0, "kv_len"},
                      {block_mask, block_mask ? sparse_mask_bytes(N) : 0, "block_mask"}};
  const Span outs[] = {{dq, f_bytes, "dq"}, {dk, f_bytes, "dk"}, {dv, f_bytes, "dv"},
                       {workspace, need, "workspace"}};
  for (const Span& s : ins) {
    const size_t al = (s.p == kv_len || s.p == lse) ? 4 : s.p == block_mask ? 1 : 16;
    if (s.bytes && !aligned(s.p, al)) return fail(FA_EINVAL, "%s is not %zu-byte aligned", s.name, al);
  }
  for (const Span& s : outs)
    if (!aligned(s.p, 16)) return fail(FA_EINVAL, "%s is not 16-byte aligned", s.name);
  for (int i = 0; i < 4; ++i) {
    for (const Span& b : ins)
      if (overlap(outs[i], b))
        return fail(FA_EINVAL, "output %s overlaps input %s", outs[i].name, b.name);
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j]))
        return fail(FA_EINVAL, "outputs %s and %s overlap", outs[i].name, outs[j].name);
  }

  fa::BwdArgs a{q,  k,  v,  o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal ? 1 : 0,
                dtype, kv_len, static_cast<float*>(workspace)};
  a.dmax = reinterpret_cast<float*>(static_cast<char*>(workspace) + fa::bwd_delta_bytes(B, H, N));
  a.block_mask = block_mask;
  a.drop_t = drop.t;
  a.seed = drop.seed;
  a.offset = drop.offset;
  hipError_t e = fa::launch_bwd(a, static_cast<hipStream_t>(stream), stages);
  if (e != hipSuccess) return fail(FA_EHIP, "backward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const float* o, const void* dout,
           const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
           float scale, int causal, int dtype, const int32_t* kv_len, void* workspace,
           size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, kv_len,
                  nullptr, workspace, workspace_bytes, stream);
}

int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const float* o,
                 const void* dout, const float* lse, float* dq, float* dk, float* dv, int B,
                 int H, int N, int d, float scale, int causal, int dtype,
                 const int32_t* kv_len, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (stage < 0 || stage > 3) {
    clear_error();
    return fail(FA_EINVAL, "stage must be 0 (D), 1 (dK/dV), 2 (dQ) or 3 (dQ and D), got %d",
                stage);
  }
  static const int kStageBits[4] = {1, 2, 4, 4 | 8};
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, kv_len,
                  nullptr, workspace, workspace_bytes, stream, kStageBits[stage]);
}

int fa_bwd_sparse(const void* q, const void* k, const void* v, const float* o,
                  const void* dout, const float* lse, float* dq, float* dk, float* dv, int B,
                  int H, int N, int d, float scale, int causal, int dtype,
                  const int32_t* kv_len, const uint8_t* block_mask, void* workspace,
                  size_t workspace_bytes, void* stream) {
  clear_error();
  int st = check_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  st = check_sparse(N, dtype, block_mask);
  if (st != FA_OK) return st;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, kv_len,
                  block_mask, workspace, workspace_bytes, stream);
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const float* o,
                   const void* dout, const float* lse, float* dq, float* dk, float* dv, int B,
                   int H, int N, int d, float scale, int causal, int dtype,
                   const int32_t* kv_len, float p, uint64_t seed, uint32_t offset,
                   void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int st = check_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  Drop drop;
  st = check_dropout(dtype, p, &drop);
  if (st != FA_OK) return st;
  drop.seed = seed;
  drop.offset = offset;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, kv_len,
                  nullptr, workspace, workspace_bytes, stream, fa::kBwdAll, drop);
}

}  // extern "C"
