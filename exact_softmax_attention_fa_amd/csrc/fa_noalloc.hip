// fa_fwd_splitkv_noalloc: the split-KV forward pass with its partial states in a fixed device
// buffer owned by the library, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc). Same kernels, same
// result as fa_fwd_splitkv.
//
// The buffer is the file-scope array `scratch` below: every GPU the library runs on holds its
// own copy (allocated when the code object is loaded on that GPU) until the process ends. In
// host code the name `scratch` is only a stand-in for the device symbol, never a device
// address: its address on each GPU comes from hipGetSymbolAddress, taken once per device with
// that device current and kept in `g_scratch`, and only that address is handed to kernels.
// Every call on one GPU uses the same buffer, so calls that overlap on one GPU (different
// streams, or several host threads without ordering) race. Nothing in the buffer needs to start
// at zero: the partial pass writes every entry the merge reads.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <mutex>

#include "fa.h"
#include "fa_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each GPU, null until first use

// Address of `scratch` on device `dev` (looked up once, with `dev` current). Returns an
// fa_status code.
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return FA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return FA_ERR_HIP;
    if (e != hipSuccess || p == nullptr || ((uintptr_t)p & 255) != 0) return FA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                      int B, int H, int N, int d, float scale, int causal, int dtype,
                                      int num_splits, hipStream_t stream) {
  fa::SplitPlan plan;
  fa::FwdArgs args;
  const int st = fa::splitkv_check(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, num_splits, &plan, &args);
  if (st != FA_OK) return st;
  void* ws = nullptr;
  if (plan.nsplit > 1) {
    if (plan.ws_bytes > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    // the buffer of the GPU the stream runs on (the current GPU for the null stream)
    int dev = -1;
    const hipError_t e = stream == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return FA_ERR_HIP;
    const int s2 = scratch_on(dev, &ws);
    if (s2 != FA_OK) return s2;
  }
  return fa::splitkv_run(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, plan, args, ws, stream);
}
