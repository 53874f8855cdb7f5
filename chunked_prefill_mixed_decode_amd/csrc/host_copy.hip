// Step metadata to the device with a kernel on the compute stream.
//
// "Chunked Prefill 的 Token 预算" §06: each round's rows carry positions and KV slots and each
// sequence its context length and block table; the host batch builder writes them into pinned
// memory once per step.  Copying them with the copy engine would make the compute queue wait on
// another queue every step; reading them from the kernel side keeps the whole step on one queue.
#include "cb.h"

#include <hip/hip_runtime.h>

#include <algorithm>

namespace cb {
namespace {

// System-scope loads: they bypass the GPU caches, so every launch sees what the host wrote last.
__global__ __launch_bounds__(256) void host_copy_kernel(const uint64_t* src, uint64_t* dst, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    dst[i] = __hip_atomic_load(const_cast<uint64_t*>(src) + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace
}  // namespace cb

extern "C" int cb_copy_host_to_device(void* stream, const void* src, void* dst, size_t nbytes) {
  if (nbytes == 0) return CB_OK;
  if (!src || !dst || (nbytes & 7) || (reinterpret_cast<uintptr_t>(src) & 7) || (reinterpret_cast<uintptr_t>(dst) & 7))
    return CB_ERR_INVALID;
  void* dsrc = nullptr;
  if (hipHostGetDevicePointer(&dsrc, const_cast<void*>(src), 0) != hipSuccess || !dsrc) {
    (void)hipGetLastError();
    return CB_ERR_INVALID;
  }
  const int64_t n = static_cast<int64_t>(nbytes / 8);
  const int64_t grid = std::min<int64_t>((n + 255) / 256, 256);
  cb::host_copy_kernel<<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint64_t*>(dsrc), static_cast<uint64_t*>(dst), n);
  return hipGetLastError() == hipSuccess ? CB_OK : CB_ERR_HIP;
}
