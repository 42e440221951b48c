// w4a16_large.hip -- the large-M path (batched decode, prefill-sized blocks).
//
// Past the point where the weight stream stops being the bottleneck, the
// GEMM is bound by matrix arithmetic (ai.satyajit.si page, section "What one
// more stream costs on this model": once the rows' arithmetic catches up with
// the weight traffic, each extra row adds its full share of compute). This
// kernel is therefore a tiled MFMA GEMM in which every operand byte is reused
// as often as registers and LDS allow:
//
//  * A workgroup computes a 128 x 256 output tile with 8 waves (2 x 4), each
//    wave a 64 x 64 sub-tile: 4 x 4 blocks of v_mfma_f32_16x16x32_bf16.
//  * K advances in tiles of 128. The workgroup stages the 128 x 128 bf16
//    activation tile into LDS (double-buffered, one barrier per tile),
//    reordered into the k-slot order of the weight dequantization and
//    XOR-swizzled by row so that both the staging writes and the fragment
//    reads are free of bank conflicts.
//  * Packed weights go straight from the tiled format into registers: a
//    lane's words of one (16-column block, group) tile are its B operands
//    for that group's MFMA steps. Each wave dequantizes its own 4 column
//    blocks and reuses each B operand for its 4 row blocks.
//  * Dequantization yields the exact biased value 136 + q (as in the small-M
//    kernels). Instead of a second MFMA against a -136 operand, the bias is
//    removed by starting each group's accumulation from -136 * sum_k x[m][k]
//    over the group: those row sums are formed once per workgroup while the
//    activation tile is staged (8 values per lane, then a DPP reduction) and
//    kept in LDS next to the tile. Every MFMA then does useful work.
//  * The group's fp32 partial is scaled by its fp16 scale and added to the
//    running fp32 result, as in the other kernels.
//  * Workgroups are numbered so that the 8 XCDs (which take workgroups round
//    robin) each own a contiguous range of tiles, row tiles fastest: the row
//    tiles that share a column tile's weights run together on one XCD and
//    find those weights in its L2.
//
// Group sizes 32, 64 and 128 are handled here (a k-tile holds 4, 2 or 1
// whole groups). Rows beyond M and column blocks beyond N are clamped on load
// and never stored.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16_internal {
namespace {

constexpr int kLgWaves = 8;
constexpr int kLgWN = 4;                      // waves along N (2 along M)
constexpr int kLgMB = 4;                      // 16-row blocks per wave
constexpr int kLgNB = 4;                      // 16-column blocks per wave
constexpr int kLgRows = 2 * kLgMB * 16;       // 128 rows per workgroup tile
constexpr int kLgBlocks = kLgWN * kLgNB;      // 16 column blocks = 256 columns
constexpr int kLgThreads = kLgWaves * 64;
constexpr int kLgKT = 128;                    // k per tile
constexpr int kLgPieces = kLgKT / 8;          // 16-byte pieces per row per tile
constexpr int kLgLoads = kLgRows * kLgPieces / kLgThreads;  // pieces staged per thread
constexpr int kLgRowBytes = kLgKT * 2;
constexpr int kLgABytes = kLgRows * kLgRowBytes;            // 32 KB per buffer

template <int GS>
struct LgCfg {
  static constexpr int T = kLgKT / GS;        // groups per k-tile
  static constexpr int WPL = GS / 32;         // MFMA steps (words per lane) per group
  static constexpr int LPG = GS / 8;          // staging lanes per group
  static constexpr int SBytes = T * kLgRows * 4;
  static constexpr int BufBytes = kLgABytes + SBytes;
  static constexpr size_t Lds = 2 * static_cast<size_t>(BufBytes);
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  // Out-of-row sources read as zero (bound_ctrl).
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, true));
}

// Sum of the 8 bf16 values of a 16-byte piece, in fp32.
__device__ __forceinline__ float sum8(u32x4 d) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += __builtin_bit_cast(float, d[i] << 16);
    s += __builtin_bit_cast(float, d[i] & 0xFFFF0000u);
  }
  return s;
}

// Windowed sum over the LPG consecutive lanes ending at this lane (lanes of a
// group are consecutive and aligned, so the group's last lane holds its sum).
template <int LPG>
__device__ __forceinline__ float group_lane_sum(float v) {
  static_assert(LPG == 4 || LPG == 8 || LPG == 16, "group of 32, 64 or 128");
  v += dpp_f32<0x111>(v);                          // row_shr:1
  v += dpp_f32<0x112>(v);                          // row_shr:2
  if constexpr (LPG >= 8) v += dpp_f32<0x114>(v);  // row_shr:4
  if constexpr (LPG >= 16) v += dpp_f32<0x118>(v); // row_shr:8
  return v;
}

struct StageRegs {
  u32x4 d[kLgLoads];
};

template <int GS>
struct BRegs {
  uint32_t w[kLgNB][LgCfg<GS>::T * LgCfg<GS>::WPL];  // 4 words per block per tile
  uint32_t s[kLgNB][LgCfg<GS>::T];                   // scale pairs (fp16 x 2)
};

template <int GS>
__global__ __launch_bounds__(kLgThreads, 1) void large_kernel(GemmArgs a, int MT, int NT) {
  using C = LgCfg<GS>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lg_lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave / kLgWN, wn = wave % kLgWN;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K / GS;
  const int NCB = (N + 15) / 16;
  const int ntiles = (G + C::T - 1) / C::T;

  // Tile of this workgroup: XCD x (= blockIdx % 8) owns a contiguous range of
  // the MT * NT tiles, row tiles fastest.
  const int total = MT * NT;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = total >> 3, rem = total & 7;
  const int tile = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int mt = tile % MT, nt = tile / MT;
  const int m0 = mt * kLgRows;

  gptr<const uint16_t> xg = to_global(a.x);
  gptr<const uint32_t> qg = to_global(a.qweight);
  gptr<const uint16_t> sg = to_global(a.scales);

  // ---- staging assignment: piece `spiece` of rows srow0 + i * (512 / 16) ----
  const int spiece = tid % kLgPieces;
  const int srow0 = tid / kLgPieces;
  constexpr int kRowStep = kLgThreads / kLgPieces;   // 32

  auto stage_load = [&](StageRegs& r, int t) {
    int k = t * kLgKT + spiece * 8;
    if (k > K - 8) k = K - 8;  // beyond the last group: any valid piece (unused)
#pragma unroll
    for (int i = 0; i < kLgLoads; ++i) {
      int row = m0 + srow0 + i * kRowStep;
      if (row > M - 1) row = M - 1;
      r.d[i] = *reinterpret_cast<gptr<const u32x4>>(xg + static_cast<size_t>(row) * K + k);
    }
  };
  auto stage_store = [&](const StageRegs& r, int buf) {
    unsigned char* base = lg_lds + buf * C::BufBytes;
    float* sums = reinterpret_cast<float*>(base + kLgABytes);
#pragma unroll
    for (int i = 0; i < kLgLoads; ++i) {
      const int row = srow0 + i * kRowStep;
      float s = group_lane_sum<C::LPG>(sum8(r.d[i]));
      if ((spiece % C::LPG) == C::LPG - 1) sums[(spiece / C::LPG) * kLgRows + row] = s;
      const int sl = spiece ^ (row & 15);
      *reinterpret_cast<bf16x8*>(base + row * kLgRowBytes + sl * 16) = act_frag(r.d[i]);
    }
  };

  // ---- weights and scales of this wave's 4 column blocks ----
  int blk[kLgNB];
#pragma unroll
  for (int nb = 0; nb < kLgNB; ++nb) {
    int b = nt * kLgBlocks + wn * kLgNB + nb;
    blk[nb] = b < NCB ? b : NCB - 1;
  }
  auto load_b = [&](BRegs<GS>& r, int t) {
#pragma unroll
    for (int gi = 0; gi < C::T; ++gi) {
      int grp = t * C::T + gi;
      if (grp > G - 1) grp = G - 1;
#pragma unroll
      for (int nb = 0; nb < kLgNB; ++nb) {
        const size_t tile_idx = static_cast<size_t>(blk[nb]) * G + grp;
        gptr<const uint32_t> p = qg + (tile_idx * 64 + lane) * C::WPL;
        if constexpr (C::WPL == 4) {
          u32x4 v = *reinterpret_cast<gptr<const u32x4>>(p);
#pragma unroll
          for (int w = 0; w < 4; ++w) r.w[nb][gi * 4 + w] = v[w];
        } else if constexpr (C::WPL == 2) {
          u32x2 v = *reinterpret_cast<gptr<const u32x2>>(p);
          r.w[nb][gi * 2 + 0] = v[0];
          r.w[nb][gi * 2 + 1] = v[1];
        } else {
          r.w[nb][gi] = *p;
        }
        r.s[nb][gi] = *reinterpret_cast<gptr<const uint32_t>>(sg + tile_idx * 16 + (lane & 14));
      }
    }
  };

  f32x4 yacc[kLgMB][kLgNB];
#pragma unroll
  for (int mb = 0; mb < kLgMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kLgNB; ++nb) yacc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int arow = wm * (kLgMB * 16) + (lane & 15);     // A fragment row (block 0)
  const int jgrp = lane >> 4;                            // k-slice of the lane
  const int shalf = (lane & 1) * 16;                     // scale half of the pair

  auto compute = [&](const BRegs<GS>& b, int t, int buf) {
    const unsigned char* base = lg_lds + buf * C::BufBytes;
    const float* sums = reinterpret_cast<const float*>(base + kLgABytes);
    // A fragments of all 4 steps of the tile
    bf16x8 af[4][kLgMB];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int gi = st / C::WPL, w = st % C::WPL;
      const int piece = gi * C::LPG + jgrp * C::WPL + w;
#pragma unroll
      for (int mb = 0; mb < kLgMB; ++mb) {
        const int row = arow + mb * 16;
        af[st][mb] = *reinterpret_cast<const bf16x8*>(base + row * kLgRowBytes +
                                                     ((piece ^ (lane & 15)) * 16));
      }
    }
#pragma unroll
    for (int gi = 0; gi < C::T; ++gi) {
      if (C::T > 1 && t * C::T + gi >= G) break;  // ragged last tile (uniform)
      // -136 * (row sums of this group) for the rows this lane accumulates
      f32x4 bias[kLgMB];
#pragma unroll
      for (int mb = 0; mb < kLgMB; ++mb) {
        f32x4 s = *reinterpret_cast<const f32x4*>(sums + gi * kLgRows + wm * (kLgMB * 16) +
                                                  mb * 16 + 4 * jgrp);
        bias[mb] = s * -136.0f;
      }
#pragma unroll
      for (int nb = 0; nb < kLgNB; ++nb) {
        f32x4 acc[kLgMB];
#pragma unroll
        for (int w = 0; w < C::WPL; ++w) {
          const bf16x8 bq = dequant_biased(b.w[nb][gi * C::WPL + w]);
#pragma unroll
          for (int mb = 0; mb < kLgMB; ++mb)
            acc[mb] = mfma16(af[gi * C::WPL + w][mb], bq, w == 0 ? bias[mb] : acc[mb]);
        }
        const float sc = fp16_bits_to_f32(static_cast<uint16_t>(b.s[nb][gi] >> shalf));
#pragma unroll
        for (int mb = 0; mb < kLgMB; ++mb) yacc[mb][nb] += sc * acc[mb];
      }
    }
  };

  // ---- pipeline: tile t computes from LDS buffer t & 1 while tile t + 1 is
  // loaded into registers and then staged into the other buffer ----
  StageRegs sr;
  BRegs<GS> bcur, bnxt;
  stage_load(sr, 0);
  load_b(bcur, 0);
  stage_store(sr, 0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int tn = t + 1 < ntiles ? t + 1 : t;   // the last iteration reloads (unused)
    stage_load(sr, tn);
    load_b(bnxt, tn);
    compute(bcur, t, t & 1);
    stage_store(sr, (t + 1) & 1);
    // LDS-only barrier: global loads of the next tile may stay in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    bcur = bnxt;
  }

  // ---- epilogue: bf16 (RNE) stores of the rows and columns that exist ----
  gptr<uint16_t> yg = to_global(a.y);
#pragma unroll
  for (int nb = 0; nb < kLgNB; ++nb) {
    const int col = (nt * kLgBlocks + wn * kLgNB + nb) * 16 + (lane & 15);
    if (col >= N) continue;
#pragma unroll
    for (int mb = 0; mb < kLgMB; ++mb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * (kLgMB * 16) + mb * 16 + 4 * jgrp + r;
        if (row < M) yg[static_cast<size_t>(row) * N + col] = f32_to_bf16_bits(yacc[mb][nb][r]);
      }
    }
  }
}

template <int GS>
hipError_t launch_large_t(const GemmArgs& a, hipStream_t stream) {
  const int MT = (a.M + kLgRows - 1) / kLgRows;
  const int NCB = (a.N + 15) / 16;
  const int NT = (NCB + kLgBlocks - 1) / kLgBlocks;
  const long long total = static_cast<long long>(MT) * NT;
  if (total < 1 || total > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const void* fn = reinterpret_cast<const void*>(&large_kernel<GS>);
  const size_t lds = LgCfg<GS>::Lds;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  GemmArgs copy = a;
  int mt = MT, ntc = NT;
  void* kargs[] = {&copy, &mt, &ntc};
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(total)), dim3(kLgThreads), kargs, lds,
                         stream);
}

}  // namespace

bool large_supported(int group) { return group == 32 || group == 64 || group == 128; }

hipError_t launch_large(const GemmArgs& a, hipStream_t stream) {
  switch (a.group) {
    case 32: return launch_large_t<32>(a, stream);
    case 64: return launch_large_t<64>(a, stream);
    case 128: return launch_large_t<128>(a, stream);
    default: return launch_skinny(a, stream);  // group 256: split-K kernel
  }
}

}  // namespace w4a16_internal
