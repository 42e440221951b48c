// w4a16_launch.h -- internal interface between the host half and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace w4a16_internal {

struct GemmArgs {
  const uint16_t* x;        // bf16 [M][K]
  const uint32_t* qweight;  // [N][K/8]
  const uint16_t* scales;   // fp16 [K/group][N]
  uint16_t* y;              // bf16 [M][N]
  int M, N, K, group;
};

// Shape-checked by the caller: M >= 1, N >= 1, K % group == 0, group in {32, 64, 128, 256},
// all pointers 16-byte aligned.
hipError_t launch_skinny(const GemmArgs& a, hipStream_t stream);
hipError_t launch_large(const GemmArgs& a, hipStream_t stream);

// M-dispatch: W4A16_PATH_SKINNY or W4A16_PATH_LARGE for a supported shape.
int choose_path(int M, int N, int K, int group);

}  // namespace w4a16_internal
