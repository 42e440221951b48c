// w4a16_host.cpp -- host half of the W4A16 library: sizes, packing, argument
// checks and the M-dispatch. Nothing here touches a device except the launch
// calls at the very end of w4a16_gemm_ex.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "../../include/w4a16.h"
#include "w4a16_launch.h"

namespace {

bool pack_shape_ok(int N, int K, int group) {
  return N >= 0 && K >= 0 && group > 0 && K % 8 == 0 && group % 8 == 0 && K % group == 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool group_supported(int group) {
  return group == 32 || group == 64 || group == 128 || group == 256;
}

}  // namespace

extern "C" {

size_t w4a16_qweight_bytes(int N, int K) {
  if (N < 0 || K < 0 || K % 8 != 0) return 0;
  return static_cast<size_t>(N) * static_cast<size_t>(K) / 2;
}

size_t w4a16_scales_bytes(int N, int K, int group) {
  if (N < 0 || K < 0 || group <= 0 || K % group != 0) return 0;
  return static_cast<size_t>(N) * static_cast<size_t>(K / group) * 2;
}

int w4a16_pack(const int8_t* q, const uint16_t* scales_in, uint32_t* qweight_out,
               uint16_t* scales_out, int N, int K, int group) {
  if (!pack_shape_ok(N, K, group)) return W4A16_ERR_INVALID_ARG;
  const size_t total = static_cast<size_t>(N) * static_cast<size_t>(K);
  if (total == 0) return W4A16_OK;
  if (!q || !scales_in || !qweight_out || !scales_out) return W4A16_ERR_INVALID_ARG;
  // Validate everything before writing anything.
  for (size_t i = 0; i < total; ++i) {
    if (q[i] < -8 || q[i] > 7) return W4A16_ERR_INVALID_ARG;
  }
  const size_t words = static_cast<size_t>(K) / 8;
  for (int n = 0; n < N; ++n) {
    const int8_t* row = q + static_cast<size_t>(n) * K;
    uint32_t* out = qweight_out + static_cast<size_t>(n) * words;
    for (size_t j = 0; j < words; ++j) {
      const int8_t* c = row + 8 * j;
      uint32_t w = 0;
      for (int i = 7; i >= 0; --i) w = (w << 4) | (static_cast<uint32_t>(c[i]) & 0xFu);
      out[j] = w;
    }
  }
  const int G = K / group;
  for (int n = 0; n < N; ++n) {
    const uint16_t* src = scales_in + static_cast<size_t>(n) * G;
    for (int g = 0; g < G; ++g) scales_out[static_cast<size_t>(g) * N + n] = src[g];
  }
  return W4A16_OK;
}

int w4a16_select_path(int M, int N, int K, int group) {
  if (M < 0 || N < 1 || K < 1 || !group_supported(group) || K % group != 0) return -1;
  return w4a16_internal::choose_path(M, N, K, group);
}

int w4a16_gemm_ex(const void* x, const void* qweight, const void* scales, void* y, int M,
                  int N, int K, int group, int path, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return W4A16_ERR_INVALID_ARG;
  if (path != W4A16_PATH_AUTO && path != W4A16_PATH_SKINNY && path != W4A16_PATH_LARGE)
    return W4A16_ERR_INVALID_ARG;
  if (M == 0) return W4A16_OK;
  if (!x || !qweight || !scales || !y) return W4A16_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || !group_supported(group) || K % group != 0) return W4A16_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || !aligned16(y))
    return W4A16_ERR_MISALIGNED;
  if (path == W4A16_PATH_AUTO) path = w4a16_internal::choose_path(M, N, K, group);
  w4a16_internal::GemmArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.qweight = static_cast<const uint32_t*>(qweight);
  a.scales = static_cast<const uint16_t*>(scales);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.N = N;
  a.K = K;
  a.group = group;
  hipError_t err = path == W4A16_PATH_LARGE ? w4a16_internal::launch_large(a, stream)
                                            : w4a16_internal::launch_skinny(a, stream);
  return err == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

int w4a16_gemm(const void* x, const void* qweight, const void* scales, void* y, int M, int N,
               int K, int group, hipStream_t stream) {
  return w4a16_gemm_ex(x, qweight, scales, y, M, N, K, group, W4A16_PATH_AUTO, stream);
}

const char* w4a16_status_string(int status) {
  switch (status) {
    case W4A16_OK: return "W4A16_OK: success";
    case W4A16_ERR_INVALID_ARG: return "W4A16_ERR_INVALID_ARG: null pointer, bad size or code";
    case W4A16_ERR_UNSUPPORTED: return "W4A16_ERR_UNSUPPORTED: shape or group size not supported";
    case W4A16_ERR_MISALIGNED: return "W4A16_ERR_MISALIGNED: device pointer not 16-byte aligned";
    case W4A16_ERR_LAUNCH: return "W4A16_ERR_LAUNCH: kernel launch failed";
    default: return "unknown w4a16 status";
  }
}

int w4a16_version(void) { return 100; }

}  // extern "C"
