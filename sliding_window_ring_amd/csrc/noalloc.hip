// noalloc.hip -- swr_global_append_attend_noalloc: the fused global-layer
// call with its workspace in a static device array instead of caller memory,
// for callers that cannot allocate (code under graph capture, serving loops
// that forbid allocation).
//
// The array below is a file-scope device variable: every device the library
// runs on holds its own copy from module load until the process ends, at an
// address of its own.  Host code never passes the array's name to a kernel
// (on the host that name is a stand-in, not a device address); it looks the
// device address up once per device with hipGetSymbolAddress, with that
// device current, and passes that pointer instead.
#include <mutex>

#include "swr.h"
#include "swr_internal.h"

namespace swr {
namespace {

// Largest workspace the static array serves: 16 MiB, enough for the
// chunked global form of a 2-KV-head x 512-dim layer of 32 rows up to about
// 16,000 keys at B = 1 (64 KB of partials per 128 keys and KV head).  A
// streamed call (units x tiles >= 2048) keeps at least 512 partial slots,
// about 32 MiB at that shape, and gets SWR_ERR_WORKSPACE here.
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// The current device's address of `scratch` (looked up on the first call on
// that device).
hipError_t scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace swr

extern "C" swr_status swr_global_append_attend_noalloc(const swr_kv* kv, const void* k_new, const void* v_new,
                                                       const void* q, void* out, const int32_t* pos0,
                                                       int max_key_count, int B, int S, int Hq, int Hkv, int D,
                                                       float scale, hipStream_t stream) {
  if (B < 0 || S < 1 || Hq < 1 || Hkv < 1) return SWR_ERR_INVALID;
  const size_t need = swr_workspace_bytes(SWR_OP_GLOBAL_APPEND_ATTEND, B, S, Hq, Hkv, D, max_key_count);
  if (need > swr::kScratchBytes) return SWR_ERR_WORKSPACE;  // more than the static array holds
  // the lookup reads no device memory; the shared validation below runs
  // before anything is launched
  void* ws = nullptr;
  if (swr::scratch_address(&ws) != hipSuccess) return SWR_ERR_LAUNCH;
  return swr::attend(swr::MODE_GLOBAL, 1, kv, q, out, pos0, nullptr, k_new, v_new, max_key_count, B, S, Hq, Hkv,
                     D, scale, ws, swr::kScratchBytes, stream);
}
