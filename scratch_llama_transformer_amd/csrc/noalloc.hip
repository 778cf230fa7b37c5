// Entry point for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// fused softmax cross-entropy with its per-row loss scratch taken from a
// static device array instead of a caller-provided workspace.
#include <mutex>

#include "slt_internal.h"

// Per-row losses of one call (summed in a fixed order by the mean kernel):
// at most 2^20 rows, 4 MiB, held by each device the library runs on until the
// process ends.  In host code this name is a host-side stand-in, not a device
// address: host code uses the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) float scratch[1 << 20];

namespace {

constexpr int64_t kMaxRows = 1 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Address of this device's copy of `scratch`, looked up on the first call on
// the device (with that device current).
slt_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return slt::fail(SLT_EHIP, "softmax_xent_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return slt::fail(SLT_EUNSUPPORTED, "softmax_xent_noalloc: device index >= 64");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return slt::fail(SLT_EHIP, std::string("softmax_xent_noalloc: hipGetSymbolAddress: ") + hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SLT_OK;
}

}  // namespace

extern "C" slt_status slt_softmax_xent_noalloc(void* z, int64_t ldz, const int32_t* tokens, int32_t B, int32_t T,
                                               int64_t ld_tokens, int32_t V, float* loss, float* lse, int32_t dtype,
                                               void* stream) {
  if (B <= 0 || T <= 0 || V <= 0 || ldz < V || ld_tokens < T + 1 || (dtype != SLT_F32 && dtype != SLT_BF16))
    return slt::fail(SLT_EINVAL, "softmax_xent_noalloc: bad sizes");
  if ((int64_t)B * T > kMaxRows)
    return slt::fail(SLT_EINVAL, "softmax_xent_noalloc: B*T exceeds the 1048576 rows of the library's static scratch");
  if (!z || !tokens || !loss) return slt::fail(SLT_EINVAL, "softmax_xent_noalloc: NULL pointer");
  void* ws = nullptr;
  const slt_status st = scratch_address(&ws);
  if (st != SLT_OK) return st;
  return slt::launch_softmax_xent(z, ldz, tokens, B, T, ld_tokens, V, loss, lse, dtype, ws, slt::as_stream(stream));
}
