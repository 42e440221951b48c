// w4a16_probe.hip -- a read-bandwidth probe: the practical ceiling of the
// weight stream.
//
// At small M the GEMM is bound by reading the packed weights once (ai.satyajit.si
// page, section "One weight read, shared by every stream", the bandwidth-ceiling
// equation). How close a kernel can come to the HBM peak depends on the access
// pattern as much as on the chip, so the measure of the streaming kernels is a
// plain read of the same number of bytes in the same pattern: a persistent grid
// of 8-wave workgroups, two per compute unit, each wave streaming one
// contiguous run of 16-byte words with non-temporal loads (1 KB per wave
// instruction, eight instructions in flight per wave), and no arithmetic beyond
// folding what it read into a 32-bit sum. The sums (one per workgroup) are
// written out, so no load can be dropped, and they let a test check that every
// word was read exactly once.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16_internal {
namespace {

constexpr int kProbeWaves = 8;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per lane

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v[0] + v[1] + v[2] + v[3]; }

// Wave w of nw reads words [n*w/nw, n*(w+1)/nw) of the buffer, lane l the
// words l, l + 64, ... of its run; the workgroup's wrapping sum goes to sink.
__global__ __launch_bounds__(64 * kProbeWaves) void read_probe_kernel(const u32x4* buf,
                                                                      long long n, int nw,
                                                                      uint32_t* sink) {
  __shared__ uint32_t wave_sum[kProbeWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x * kProbeWaves + wave;
  const long long r0 = w < nw ? n * w / nw : n, r1 = w < nw ? n * (w + 1) / nw : n;
  gptr<const u32x4> p = to_global(buf);
  uint32_t acc = 0;
  long long i = r0 + lane;
  // full rounds of kProbeUnroll loads per lane, all in flight together
  for (; i + 64LL * (kProbeUnroll - 1) < r1; i += 64LL * kProbeUnroll) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) v[k] = __builtin_nontemporal_load(p + i + 64LL * k);
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) acc += fold(v[k]);
  }
  for (; i < r1; i += 64) acc += fold(__builtin_nontemporal_load(p + i));
  // wave sum (wrapping), then workgroup sum in wave order
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) wave_sum[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int k = 0; k < kProbeWaves; ++k) s += wave_sum[k];
    sink[blockIdx.x] = s;
  }
}

}  // namespace

int read_probe_workgroups() {
  const int wgs = 2 * device_cus();
  return wgs < kReadProbeMaxWorkgroups ? wgs : kReadProbeMaxWorkgroups;
}

hipError_t launch_read_probe(const void* buf, long long words, uint32_t* sink, hipStream_t stream) {
  int wgs = read_probe_workgroups();
  long long nw = static_cast<long long>(wgs) * kProbeWaves;
  if (nw > words) {  // every wave reads at least one word
    wgs = static_cast<int>((words + kProbeWaves - 1) / kProbeWaves);
    nw = words;
  }
  if (wgs < 1) return hipSuccess;
  const u32x4* b = static_cast<const u32x4*>(buf);
  int nwi = static_cast<int>(nw);
  void* kargs[] = {&b, &words, &nwi, &sink};
  return hipLaunchKernel(reinterpret_cast<const void*>(&read_probe_kernel), dim3(wgs),
                         dim3(64 * kProbeWaves), kargs, 0, stream);
}

}  // namespace w4a16_internal
