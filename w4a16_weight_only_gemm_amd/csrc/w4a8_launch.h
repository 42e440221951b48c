// w4a8_launch.h -- internal interface of the W4A8 kernels (int8 activations
// with one scale per row, 4-bit weights in the packed format of the W4A16
// kernels).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "w4a16_launch.h"

namespace w4a16_internal {

struct W4A8Args {
  const uint8_t* xq;        // int8 codes [M][K], 16-blocks in MFMA step order
  const float* sx;          // row scales [M]
  const uint32_t* qweight;  // packed weights (device arrangement)
  const uint16_t* scales;   // packed fp16 scales
  uint16_t* y;              // bf16 [M][N]
  int M, N, K, group;
};

struct W4A8QuantProblem {
  const uint16_t* x;        // bf16 [M][K]
  uint8_t* xq;              // int8 codes [M][K]
  float* sx;                // row scales [M]
  int K;
};

struct W4A8QuantBatch {
  W4A8QuantProblem prob[kMaxProblems];
  int M;
};

// Up to kMaxProblems GEMMs with the same M and group in one launch.
struct W4A8Batch {
  W4A8Args prob[kMaxProblems];
  int nprob;
  int MT;                       // row tiles (shared: same M)
  int tiles[kMaxProblems];      // tiles of each problem
  int begin[kMaxProblems];      // first block of each problem (multiple of 8)
};

// Shape-checked by the caller: M >= 1, count in 1..kMaxProblems, each K >= 16
// and K % 16 == 0, pointers 16-byte aligned. One workgroup per (problem, row).
hipError_t launch_w4a8_quantize(const W4A8QuantProblem* probs, int count, int M,
                                hipStream_t stream);
// Shape-checked by the caller: count in 1..kMaxProblems, all with the same
// M >= 1 and group (64 or 128), N >= 1, K % group == 0, packed weights below
// 4 GB, pointers 16-byte aligned. One launch; the K-deepest problems first.
hipError_t launch_w4a8_gemm(const W4A8Args* probs, int count, hipStream_t stream);

}  // namespace w4a16_internal
