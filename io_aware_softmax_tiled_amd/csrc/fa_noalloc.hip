// The backward pass without a caller workspace: its scratch (D and the 32-row maxima of
// |dO|) lives in one statically allocated device array of FA_NOALLOC_SCRATCH_BYTES per
// GPU, so the call allocates nothing. Meant for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that forbid it).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

// Every GPU the library runs on holds its own copy of this array until the process
// ends. Host code never passes its name to a kernel: the name is a host-side stand-in,
// so the device address is looked up once per device and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the device address of this device's scratch, looked up on the first call on it
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[256];
    snprintf(msg, sizeof msg, "fa_bwd_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
    return fa::api_fail(FA_EHIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) return fa::api_fail(FA_EHIP, "fa_bwd_noalloc: device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      char msg[256];
      snprintf(msg, sizeof msg, "fa_bwd_noalloc: hipGetSymbolAddress(scratch) failed: %s",
               hipGetErrorString(e));
      return fa::api_fail(FA_EHIP, msg);
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" int fa_bwd_noalloc(const void* q, const void* k, const void* v, const float* o,
                              const void* dout, const float* lse, float* dq, float* dk,
                              float* dv, int B, int H, int N, int d, float scale, int causal,
                              int dtype, const int32_t* kv_len, void* stream) {
  const int chk = fa::bwd_check_sizes(B, H, N, d, scale, dtype);
  if (chk != FA_OK) return chk;
  const size_t need = fa_bwd_workspace_size(B, H, N, d);
  if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "fa_bwd_noalloc: these sizes need %zu bytes of scratch, the static scratch holds %d "
             "(B*H*N at most about %d rows; use fa_bwd with a workspace)",
             need, FA_NOALLOC_SCRATCH_BYTES, FA_NOALLOC_SCRATCH_BYTES / 4 / 33 * 32);
    return fa::api_fail(FA_EWORKSPACE, msg);
  }
  void* ws = nullptr;
  if ((size_t)B * H * N > 0) {
    const int st = scratch_for_current_device(&ws);
    if (st != FA_OK) return st;
  }
  return fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, kv_len,
                ws, ws ? (size_t)FA_NOALLOC_SCRATCH_BYTES : 0, stream);
}
