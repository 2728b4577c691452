// ee_stack_extend_noalloc: an extend (decode) step that allocates nothing.
// Its workspace -- the new tokens' activations and the GEMMs' fp32 partial
// sums -- is `scratch`, a file-scope device array of EE_NOALLOC_SCRATCH_BYTES
// that every GPU the library runs this entry point on holds until the process
// ends.  For callers that cannot call hipMalloc: code under HIP graph capture,
// serving loops that forbid allocation.
//
// In host code `scratch` names a host-side stand-in, not device memory, so
// its device address is taken once per device with hipGetSymbolAddress (with
// that device current) and only that address is ever passed to kernels.
// Nothing in the buffer needs to start at zero: every byte a step reads was
// written earlier in the same step (the offsets, the activations, each
// partial-sum slot before its reduce).  Calls on one GPU share the buffer, so
// calls that overlap in time on one GPU (two streams, two threads) race.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "ee.h"
#include "internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)EE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` on each device

ee_status fail_msg(ee_status s, const char* fmt, long long a, long long b) {
  char buf[256];
  std::snprintf(buf, sizeof buf, fmt, a, b);
  return ee::set_error(s, buf);
}

// The current device's copy of `scratch`.
ee_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_msg(EE_ERR_HIP, "hipGetDevice failed (%lld)%lld", (long long)e, 0);
  if (dev < 0 || dev >= kMaxDevices)
    return fail_msg(EE_ERR_UNSUPPORTED, "device %lld above the %lld devices served", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail_msg(EE_ERR_HIP, "hipGetSymbolAddress of the scratch buffer failed (%lld) on device %lld",
                      (long long)e, dev);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return EE_OK;
}

}  // namespace

extern "C" {

ee_status ee_stack_extend_noalloc(ee_layer* const* layers, int32_t n_layers, const void* d_x, const int32_t* new_len,
                                  const int32_t* ctx_len, const int32_t* slot_base, int32_t batch, void* d_cache,
                                  int64_t capacity, void* d_y, void* stream) {
  // the step's size, from arguments checked just enough to read them; the
  // full validation runs in the shared implementation before any device work
  if (!layers || n_layers < 1 || !layers[0])
    return ee::set_error(EE_ERR_INVALID_ARG, "need at least one non-NULL layer");
  if (batch < 1 || batch > EE_MAX_EXTEND_BATCH)
    return fail_msg(EE_ERR_INVALID_ARG, "batch %lld not in [1, %lld]", batch, EE_MAX_EXTEND_BATCH);
  if (!new_len) return ee::set_error(EE_ERR_INVALID_ARG, "new_len is NULL");
  int64_t T = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (new_len[b] < 0) return fail_msg(EE_ERR_INVALID_ARG, "new_len[%lld] = %lld < 0", b, new_len[b]);
    T += new_len[b];
  }
  size_t need = 0;
  const ee_status st = ee_extend_workspace_size(layers[0], batch, T, &need);
  if (st != EE_OK) return st;
  if (need > kScratchBytes)
    return fail_msg(EE_ERR_WORKSPACE,
                    "a step of %lld new tokens needs %lld bytes of workspace, above the no-allocation scratch "
                    "buffer (EE_NOALLOC_SCRATCH_BYTES)",
                    (long long)T, (long long)need);
  void* ws = nullptr;
  const ee_status sa = scratch_address(&ws);
  if (sa != EE_OK) return sa;
  return ee::stack_extend_into(layers, n_layers, d_x, new_len, ctx_len, slot_base, batch, d_cache, capacity, d_y, ws,
                               kScratchBytes, stream);
}

}  // extern "C"
