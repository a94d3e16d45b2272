// lora_noalloc.hip -- lora_sgmv_fused_noalloc: the fused shrink + expand
// call for callers that cannot allocate device memory or pass a workspace.
//
// The split-shrink hand-off of the fused kernel needs device scratch (the
// parts' stamps and partial sums). Here it lives in one file-scope device
// array, `scratch`, of kScratchBytes per GPU, which each GPU the library
// runs on holds until the process ends. Host code never passes the array's
// name to a kernel: on first use on a device, with that device current, the
// array's device address is looked up with hipGetSymbolAddress and kept per
// device, and only that address reaches the kernels.
//
// Every call on a GPU shares that GPU's array and leaves its contents
// behind: calls that overlap on one GPU (two streams, or two threads) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/lora_sgmv.h"
#include "lora_internal.h"
#include "lora_plan.h"

namespace lora {
namespace {

constexpr size_t kScratchBytes = LORA_NOALLOC_SCRATCH_BYTES;
// The hand-off words at the start of the scratch (fused-call workspace
// layout: tile counters, then one stamp per split-shrink part). Stamps must
// never equal a current launch's stamp, and launch ids are never 0, so the
// words are cleared once; partial sums need no clearing.
constexpr size_t kHandoffBytes = kStampOffset + (size_t)kMaxPartials * kStampStride;
static_assert(kHandoffBytes % 16 == 0 && kHandoffBytes < kScratchBytes, "hand-off words fit the scratch");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ __launch_bounds__(256) void scratch_clear_kernel(uint4* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kMaxDevices = 64;
struct DeviceScratch {
  std::mutex mu;
  void* ptr = nullptr;  // device address of `scratch` on this device (null until set up)
};
DeviceScratch g_scratch[kMaxDevices];

// The scratch of the current device: looked up (and its hand-off words
// cleared on `stream`) on the first call on that device.
struct StaticScratch final : WsSource {
  hipStream_t stream;
  explicit StaticScratch(void* s) : stream(static_cast<hipStream_t>(s)) { cap = kScratchBytes; }
  void* get() override {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
      set_error(LORA_DEVICE_ERROR, "hipGetDevice failed: %s", hipGetErrorString(e));
      return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
      set_error(LORA_DEVICE_ERROR, "device %d outside the %d devices the static scratch serves", dev, kMaxDevices);
      return nullptr;
    }
    DeviceScratch& d = g_scratch[dev];
    std::lock_guard<std::mutex> lock(d.mu);
    if (!d.ptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        set_error(LORA_DEVICE_ERROR, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
        return nullptr;
      }
      const int n = (int)(kHandoffBytes / 16);
      hipLaunchKernelGGL(scratch_clear_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                         static_cast<uint4*>(p), n);
      e = hipGetLastError();
      if (e != hipSuccess) {
        set_error(LORA_DEVICE_ERROR, "clearing the static scratch failed on device %d: %s", dev,
                  hipGetErrorString(e));
        return nullptr;
      }
      d.ptr = p;
    }
    return d.ptr;
  }
};

}  // namespace
}  // namespace lora

extern "C" int lora_sgmv_fused_noalloc(const void* x, int64_t ldx, const lora_adapters_t* adapters,
                                       const lora_segments_t* segments, void* y, int64_t ldy, float* u_save,
                                       int64_t ldu, void* stream) {
  lora::set_error(LORA_OK, "%s", "");
  lora::StaticScratch src(stream);
  return lora::sgmv_fused_from(x, ldx, adapters, segments, y, ldy, u_save, ldu, src, stream);
}
