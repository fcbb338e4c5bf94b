// ec_entropy_max_noalloc: the entropy pass and decision of ec_entropy_max with
// its per-segment partial statistics kept in a file-scope device array
// instead of a caller workspace, for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that
// forbid allocation).  Same kernels, same launch, same results bit for bit.
//
// `scratch` below is a host-side stand-in when named in host code; its device
// address is looked up once per device with hipGetSymbolAddress (that device
// current) and only that address is passed to kernels.  Each device holds its
// own copy of the array until the process ends.  Calls on one device share
// it: two calls that overlap in time on the same device race.  The partial
// statistics are fully written before they are read, so nothing needs
// clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ec.h"
#include "ec_launch.h"
#include "ec_validate.h"

static __device__ __align__(256) unsigned char scratch[EC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];        // device address of `scratch`, per device

// The device the stream runs on (the current device for the null stream).
hipError_t stream_device(hipStream_t s, int* dev) {
  if (s == nullptr) return hipGetDevice(dev);
  return hipStreamGetDevice(s, dev);
}

hipError_t scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t r = (cur != dev) ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (r != hipSuccess) return r;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int32_t ec_entropy_max_noalloc(const void* logits, int32_t dtype, int64_t n_rows,
                                          int64_t V, int64_t row_stride,
                                          const int32_t* decoded_rows, const int32_t* n_decoded,
                                          int32_t max_decoded, float tau, float* row_entropy,
                                          int32_t* row_argmax, float* row_top1, float* e_max,
                                          int32_t* full_flag, hipStream_t stream) {
  const int32_t st = ec::check_entropy(logits, dtype, n_rows, V, row_stride, decoded_rows,
                                       n_decoded, max_decoded, row_entropy, e_max, full_flag);
  if (st != EC_OK) return st;
  if (ec::entropy_ws_bytes(n_rows, V, dtype) > size_t(EC_NOALLOC_SCRATCH_BYTES))
    return EC_E_WORKSPACE;
  int dev = 0;
  void* ws = nullptr;
  if (stream_device(stream, &dev) != hipSuccess || scratch_on(dev, &ws) != hipSuccess)
    return EC_E_LAUNCH;
  const hipError_t e = ec::launch_entropy(logits, dtype, n_rows, nullptr, V, row_stride,
                                          row_entropy, row_argmax, row_top1, decoded_rows,
                                          n_decoded, max_decoded, tau, e_max, full_flag, ws, stream);
  return e == hipSuccess ? EC_OK : EC_E_LAUNCH;
}
