// Host-side helpers shared by the C entry points: the thread-local error message,
// the device check and the HIP-call macros.  Every entry point returns PKM_OK or a
// negative code and leaves the reason for pkm_last_error(); nothing throws across
// the ABI and nothing aborts.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/pkm.h"

namespace pkm_abi {

// Records the message (printf format) and returns `code`.
int fail(int code, const char* fmt, ...);

// The message of the last failure on this thread.
const char* last_error();

// PKM_OK if the current device is a gfx950, else PKM_EUNSUPPORTED / PKM_EHIP.
int check_device();

// The address at which kernels read a table `p`: device memory as is, pinned host
// memory through its device mapping (the kernels then read it over the host link);
// anything else (pageable host memory) is refused with PKM_EINVAL naming `what`.
int device_view(const void* p, const char* what, const void** out);

// PKM_OK if `p` is device memory, else PKM_EINVAL naming `what`.
int require_device(const void* p, const char* what);

}  // namespace pkm_abi

#define PKM_HIP(call)                                                                                \
  do {                                                                                               \
    hipError_t e_ = (call);                                                                          \
    if (e_ != hipSuccess) return pkm_abi::fail(PKM_EHIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

#define PKM_LAUNCH(call)                                                                                       \
  do {                                                                                                         \
    hipError_t e_ = (call);                                                                                    \
    if (e_ != hipSuccess) return pkm_abi::fail(PKM_EHIP, "launch %s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)
