// w4a16_noalloc.hip -- the GEMM for callers that cannot allocate.
//
// w4a16_gemm_noalloc runs the same kernels as w4a16_gemm_ws, with the
// library's own static device array `scratch` in place of a caller workspace.
// Each GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends. Host code never uses the array's name as a
// device address: on first use on a device (with that device current) its
// address is taken with hipGetSymbolAddress and kept per device; kernels and
// the one-time clear receive that address.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/w4a16.h"
#include "w4a16_launch.h"

namespace w4a16_internal {
namespace {

constexpr size_t kScratchBytes = W4A16_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte lines");

// The scratch array. Zero-filled by the code-object loader, cleared once more
// per device at set-up, and left with zero counters and slots by every call.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

__global__ void zero_fill_kernel(uint4* p, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

// Address of this device's scratch array, set up on the first call on the
// device: the symbol's address, then one clear of the whole array with a fill
// kernel on `stream` (a kernel, not hipMemsetAsync, so that a first call made
// under graph capture records an ordinary kernel node). Returns nullptr when
// the runtime cannot give the address or launch the clear.
void* scratch_on_device(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] != nullptr) return g_ptr[dev];
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
  if ((reinterpret_cast<uintptr_t>(ptr) & 255u) != 0) return nullptr;
  const size_t n16 = kScratchBytes / 16;
  hipLaunchKernelGGL(zero_fill_kernel, dim3(1024), dim3(256), 0, stream, static_cast<uint4*>(ptr),
                     n16);
  if (hipGetLastError() != hipSuccess) return nullptr;
  g_ptr[dev] = ptr;
  return ptr;
}

}  // namespace
}  // namespace w4a16_internal

extern "C" int w4a16_gemm_noalloc(const void* x, const void* qweight, const void* scales, void* y,
                                  int M, int N, int K, int group, hipStream_t stream) {
  // Every check that does not need the device first: nothing is set up or
  // launched for a call that fails them.
  if (M < 0 || N < 0 || K < 0) return W4A16_ERR_INVALID_ARG;
  if (M == 0) return W4A16_OK;
  if (!x || !qweight || !scales || !y) return W4A16_ERR_INVALID_ARG;
  const bool group_ok = group == 32 || group == 64 || group == 128 || group == 256;
  if (N < 1 || K < 1 || !group_ok || K % group != 0) return W4A16_ERR_UNSUPPORTED;
  const uintptr_t any = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(qweight) |
                        reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(y);
  if ((any & 15u) != 0) return W4A16_ERR_MISALIGNED;
  const size_t need = w4a16_workspace_bytes(M, N);
  if (need > w4a16_internal::kScratchBytes) return W4A16_ERR_TOO_LARGE;
  void* ws = w4a16_internal::scratch_on_device(stream);
  if (ws == nullptr) return W4A16_ERR_LAUNCH;
  return w4a16_gemm_ws(x, qweight, scales, y, M, N, K, group, ws, w4a16_internal::kScratchBytes,
                       stream);
}
