// w4a16_skinny.hip -- the small-M path (decode and speculative-verify blocks).
//
// At small M the GEMM is bound by the weight stream: every packed weight is
// read from HBM exactly once and shared by all M rows (ai.satyajit.si page,
// section "One weight read, shared by every stream"). The kernel is built
// around that stream:
//
//  * A workgroup owns a 16-column tile and the whole K range, split evenly
//    over its WAVES waves (split-K inside the workgroup, reduced through LDS at
//    the end, so there is no cross-workgroup traffic and no workspace).
//  * Within a wave, lane l serves column (l % 16) and k-slice (l / 16) of
//    every MFMA step. Per group of GS weights a lane issues one vector load of
//    GS/32 consecutive packed words of its column (16 bytes at GS = 128);
//    those words are exactly its B operands for the GS/32 MFMA steps of the
//    group, so packed weights go HBM -> VGPR -> dequant -> MFMA without LDS.
//  * Dequantization is to the exact biased value 136 + q in bf16 (two VALU
//    ops per bf16 pair); after each step a second MFMA against a constant
//    -136 operand removes the bias, so the MFMA sees exact codes, products are
//    exact and the fp32 accumulator holds sum(x * q) for the group.
//  * The group's fp32 partial is scaled by s[group][n] and added to the
//    running fp32 result (one FMA per output element per group).
//  * Rows are padded to 16 (RB row blocks of 16 per workgroup); padded rows
//    repeat row M-1 and are never stored.
//
// Loads of weights and scales run P groups ahead of the math in a register
// ring; activations (L2-resident) are loaded at the top of their group and
// waited for after the dequantization. Weights use non-temporal loads since
// each byte is read once. Every load is unconditional (indices are clamped),
// which keeps the wait counters exact and the loop on scalar branches.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/w4a16.h"
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16_internal {

template <int WPL>
struct Words {
  uint32_t w[WPL];
};

template <int WPL>
__device__ __forceinline__ void load_words(Words<WPL>& out, const uint32_t* p) {
  if constexpr (WPL == 1) {
    out.w[0] = __builtin_nontemporal_load(p);
  } else if constexpr (WPL == 2) {
    u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    out.w[0] = v[0];
    out.w[1] = v[1];
  } else {
#pragma unroll
    for (int h = 0; h < WPL / 4; ++h) {
      u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + h);
      out.w[4 * h + 0] = v[0];
      out.w[4 * h + 1] = v[1];
      out.w[4 * h + 2] = v[2];
      out.w[4 * h + 3] = v[3];
    }
  }
}

template <int GS, int RB, int WAVES, int P>
__global__ __launch_bounds__(64 * WAVES) void skinny_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ sp, uint16_t* __restrict__ y, int M, int N, int K) {
  constexpr int WPL = GS / 32;  // packed words per lane per group = MFMA steps per group
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;  // B column / A row within the 16x16 tile
  const int lg = lane >> 4;   // k-slice of each MFMA step
  const int n0 = blockIdx.x * 16;
  const int m0 = blockIdx.y * 16 * RB;
  const int n = min(n0 + c16, N - 1);  // ragged column tile: clamp loads, mask stores
  const int G = K / GS;
  // This wave's groups [g0, g1); wave-uniform, so the loop runs on scalar branches.
  const int g0 = static_cast<int>(static_cast<long long>(G) * wave / WAVES);
  const int g1 = static_cast<int>(static_cast<long long>(G) * (wave + 1) / WAVES);

  const bf16x8 bias = bias_operand();
  f32x4 yacc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) yacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (g1 > g0) {
    const int glast = g1 - 1;
    const uint32_t* wp = qw + static_cast<size_t>(n) * (static_cast<size_t>(K) / 8) + lg * WPL;
    const uint16_t* sn = sp + n;
    // A rows of this lane. Rows past M read row M-1 instead: an MFMA output row
    // depends only on its own A row, and padded rows are never stored.
    const uint16_t* xr[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int m = min(m0 + 16 * rb + c16, M - 1);
      xr[rb] = x + static_cast<size_t>(m) * K + lg * WPL * 8;
    }
    // Loads past the wave's last group re-read that group (cache hits) so that
    // every load is unconditional; their results are never used.
    auto load_w = [&](Words<WPL>& o, uint16_t& s, int grp) {
      grp = min(grp, glast);
      load_words<WPL>(o, wp + static_cast<size_t>(grp) * (GS / 8));
      s = sn[static_cast<size_t>(grp) * N];
    };
    auto load_x = [&](u32x4 (&xa)[RB][WPL], int grp) {
      grp = min(grp, glast);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int t = 0; t < WPL; ++t)
          xa[rb][t] = *reinterpret_cast<const u32x4*>(xr[rb] + static_cast<size_t>(grp) * GS + 8 * t);
      }
    };

    Words<WPL> wq[P];
    uint16_t sq[P];
#pragma unroll
    for (int p = 0; p < P; ++p) load_w(wq[p], sq[p], g0 + p);

    for (int c = g0; c < g1; c += P) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int grp = c + p;
        if (grp < g1) {
          u32x4 xa[RB][WPL];
          load_x(xa, grp);
          f32x4 acc[RB];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < WPL; ++t) {
            const bf16x8 b = dequant_biased(wq[p].w[t]);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              const bf16x8 a = act_frag(xa[rb][t]);
              acc[rb] = mfma16(a, b, acc[rb]);
              acc[rb] = mfma16(a, bias, acc[rb]);
            }
          }
          const float s = fp16_bits_to_f32(sq[p]);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) yacc[rb][r] = __builtin_fmaf(s, acc[rb][r], yacc[rb][r]);
          }
          load_w(wq[p], sq[p], grp + P);
        }
      }
    }
  }

  // Split-K reduction over the waves of the workgroup. The accumulator of lane
  // l holds rows 4*(l/16)+r of column l%16 of each 16x16 row block.
  __shared__ float red[WAVES][RB][16][17];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][rb][4 * lg + r][c16] = yacc[rb][r];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < RB * 256; e += 64 * WAVES) {
    const int rb = e >> 8, row = (e >> 4) & 15, col = e & 15;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[w][rb][row][col];
    const int m = m0 + 16 * rb + row, nn = n0 + col;
    if (m < M && nn < N) y[static_cast<size_t>(m) * N + nn] = f32_to_bf16_bits(sum);
  }
}

namespace {

constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyPrefetch = 4;

template <int GS, int RB>
hipError_t launch_skinny_t(const GemmArgs& a, hipStream_t stream) {
  dim3 grid((a.N + 15) / 16, (a.M + 16 * RB - 1) / (16 * RB));
  dim3 block(64 * kSkinnyWaves);
  const uint16_t* x = a.x;
  const uint32_t* qw = a.qweight;
  const uint16_t* sp = a.scales;
  uint16_t* y = a.y;
  int M = a.M, N = a.N, K = a.K;
  void* args[] = {&x, &qw, &sp, &y, &M, &N, &K};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&skinny_kernel<GS, RB, kSkinnyWaves, kSkinnyPrefetch>),
      grid, block, args, 0, stream);
}

template <int GS>
hipError_t launch_skinny_g(const GemmArgs& a, hipStream_t stream) {
  if (a.M <= 16) return launch_skinny_t<GS, 1>(a, stream);
  if (a.M <= 32) return launch_skinny_t<GS, 2>(a, stream);
  return launch_skinny_t<GS, 4>(a, stream);
}

}  // namespace

hipError_t launch_skinny(const GemmArgs& a, hipStream_t stream) {
  switch (a.group) {
    case 32: return launch_skinny_g<32>(a, stream);
    case 64: return launch_skinny_g<64>(a, stream);
    case 128: return launch_skinny_g<128>(a, stream);
    case 256: return launch_skinny_g<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// Until the large-M kernel lands, large M runs the skinny kernel with 64-row
// tiles (grid.y covers M).
hipError_t launch_large(const GemmArgs& a, hipStream_t stream) { return launch_skinny(a, stream); }

int choose_path(int M, int N, int K, int group) {
  (void)N;
  (void)K;
  (void)group;
  return M <= 64 ? W4A16_PATH_SKINNY : W4A16_PATH_LARGE;
}

}  // namespace w4a16_internal
