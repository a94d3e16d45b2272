// lora_internal.h -- internal interfaces between the sources of the library
// (not part of the ABI).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/lora_sgmv.h"

namespace lora {

// A workspace owned by the library instead of the caller. After a call has
// validated its arguments and sized its workspace, get() returns the device
// address to use, or sets the call's error text and returns nullptr.
struct WsSource {
  size_t cap = 0;  // bytes available
  virtual ~WsSource() = default;
  virtual void* get() = 0;
};

// lora_sgmv_fused with its workspace taken from `src` (validation, errors and
// results as for lora_sgmv_fused; a batch needing more than src.cap bytes is
// refused with LORA_UNSUPPORTED before any HIP call).
int sgmv_fused_from(const void* x, int64_t ldx, const lora_adapters_t* adapters,
                    const lora_segments_t* segments, void* y, int64_t ldy, float* u_save, int64_t ldu,
                    WsSource& src, void* stream);

// Sets the calling thread's lora_last_error() text; returns `status`.
int set_error(int status, const char* fmt, ...);

}  // namespace lora
