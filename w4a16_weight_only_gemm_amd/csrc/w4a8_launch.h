// w4a8_launch.h -- internal interface of the W4A8 kernels (int8 activations
// with one scale per row, 4-bit weights in the packed format of the W4A16
// kernels).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace w4a16_internal {

struct W4A8Args {
  const uint8_t* xq;        // int8 codes [M][K], 16-blocks in MFMA step order
  const float* sx;          // row scales [M]
  const uint32_t* qweight;  // packed weights (device arrangement)
  const uint16_t* scales;   // packed fp16 scales
  uint16_t* y;              // bf16 [M][N]
  int M, N, K, group;
};

// Shape-checked by the caller: M >= 1, K >= 16, K % 16 == 0, pointers 16-byte
// aligned. One workgroup per row.
hipError_t launch_w4a8_quantize(const uint16_t* x, uint8_t* xq, float* sx, int M, int K,
                                hipStream_t stream);
// Shape-checked by the caller: M >= 1, N >= 1, group 64 or 128, K % group == 0,
// packed weights below 4 GB, pointers 16-byte aligned.
hipError_t launch_w4a8_gemm(const W4A8Args& a, hipStream_t stream);

}  // namespace w4a16_internal
