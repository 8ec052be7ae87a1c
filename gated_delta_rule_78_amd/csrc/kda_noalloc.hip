// kda_noalloc.hip -- the two-pass chunk forward (kda_chunk_fwd_ws) on a workspace that
// lives in a file-scope device array, for callers that may not allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a per-GPU global: every GPU the library runs on holds its own copy, at
// its own address, from the moment the code object is loaded until the process ends.
// Host code never passes the array's name to a kernel or a copy (on the host that name is
// only a stand-in, not a device address); the device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and used from then on.
// Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU
// (two streams, two host threads) race on it.  Nothing in it needs clearing between
// calls: every byte a call reads was written earlier in the same call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/kda.h"

static constexpr size_t kScratchBytes = (size_t)KDA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte units");

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// the device address of this device's copy of `scratch` (looked up on first use)
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return KDA_OK;
}

}  // namespace

extern "C" int kda_chunk_fwd_noalloc(const kda_shape* shape, const void* q, const void* k, const void* v,
                                     const void* alpha, const void* beta, const float* initial_state, void* o,
                                     float* final_state, void* stream) {
  if (!shape) return KDA_ERR_NULL;
  const size_t need = kda_chunk_fwd_workspace_size(shape);
  if (need > kScratchBytes) return KDA_ERR_SCRATCH;
  void* ws = nullptr;
  const int rc = scratch_of_current_device(&ws);
  if (rc) return rc;
  // (an invalid shape has need == 0 and is reported by kda_chunk_fwd_ws's own checks)
  return kda_chunk_fwd_ws(shape, q, k, v, alpha, beta, initial_state, o, final_state, ws, kScratchBytes, stream);
}
