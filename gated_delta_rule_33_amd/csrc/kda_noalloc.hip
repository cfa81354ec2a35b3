// kda_noalloc.hip -- kda_prefill for callers that cannot allocate device
// memory: the workspace is a static device array that the library holds on
// every GPU it runs on, so the call itself allocates nothing.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include "kda.h"
#include "kda_internal.h"

namespace {

// The array itself.  In host code this name is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDev = 64;
std::mutex g_mu;
void* g_ptr[kMaxDev] = {};

// Device address of the current device's copy of `scratch`, resolved once
// per device (with that device current) and kept.
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" kda_status kda_prefill_noalloc(const kda_prefill_desc* d, const void* q, const void* k, const void* v,
                                          const float* log_alpha, const float* beta, const int32_t* cu_seqlens,
                                          const float* S0, void* o, float* S_T, void* stream) {
  if (!d) return KDA_ERR_INVALID_ARGUMENT;
  // the one-stream schedule: only kernel launches on `stream`, no library
  // streams or events, and nothing in the array has to start at zero (every
  // word a call reads it has written earlier in the same call)
  kda_prefill_desc one = *d;
  one.flags |= KDA_PREFILL_ONE_STREAM;
  const size_t need = kda_prefill_workspace_size(&one);
  if (need == 0) return kda_prefill(&one, q, k, v, log_alpha, beta, cu_seqlens, S0, o, S_T, nullptr, 0, stream);
  // larger problems run the bounded schedule, in segments that fit the
  // array; the call is refused (KDA_ERR_WORKSPACE_TOO_SMALL, nothing
  // launched) only when not even one chunk index per segment fits
  if (need > KDA_NOALLOC_SCRATCH_BYTES) one.flags |= KDA_PREFILL_BOUNDED;
  if (one.num_seqs == 0) return KDA_OK;
  void* ws = nullptr;
  if (scratch_ptr(&ws) != hipSuccess) return KDA_ERR_DEVICE;
  return kda::prefill_checked(&one, q, k, v, log_alpha, beta, cu_seqlens, S0, o, S_T, ws,
                              KDA_NOALLOC_SCRATCH_BYTES, stream);
}
