// w4a16_plain.hip -- the kernel behind w4a16_gemm for small M (no workspace).
//
// Without a workspace no output can be summed across workgroups, so a
// workgroup owns whole output tiles: NB consecutive 16-column blocks (16 NB
// columns) and MB 16-row blocks, over the whole of K. Its waves split K into
// equal contiguous ranges of groups and are summed through LDS at the end.
//
//  * Weights: per group a wave loads one tile of the packed format for each
//    of its NB column blocks (the lane's words are its MFMA B operands), P
//    groups ahead, non-temporal: every weight byte is read from HBM once.
//  * Activations: one fragment per row block and MFMA step feeds NB column
//    blocks, so the activation bytes a workgroup reads per weight byte fall as
//    1/NB (each activation element is read once per workgroup: the waves
//    cover disjoint K ranges). With XLDS (M <= 16 rows whose whole K fits),
//    the workgroup stages its rows in LDS once, with each group's -24 * row
//    sums, and the waves read fragments from there.
//  * Dequantization to the exact biased codes 24 + q, MFMA 16x16x32 bf16; the
//    bias leaves through the accumulator start: -24 * (row sums), from LDS
//    with XLDS, else one MFMA chain against a -24 operand per row block,
//    shared by the NB column blocks. Then one fp32 FMA per output and group
//    applies the group's scale.
//
// The host picks (MB, NB, waves, groups in flight, staging) from M, N and K
// (plain_form) so that the grid has enough workgroups for the compute units,
// no compute unit holds more than it must, and each wave keeps enough bytes
// in flight.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/w4a16.h"
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16_internal {
namespace {

constexpr size_t kPlainLdsLimit = 160 * 1024;  // LDS of one compute unit

template <int WPL>
struct PWords {
  uint32_t w[WPL];
};

template <int WPL>
__device__ __forceinline__ void load_tile_words(PWords<WPL>& out, gptr<const uint32_t> p) {
  if constexpr (WPL == 1) {
    out.w[0] = __builtin_nontemporal_load(p);
  } else if constexpr (WPL == 2) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<gptr<const u32x2>>(p));
    out.w[0] = v[0];
    out.w[1] = v[1];
  } else {
#pragma unroll
    for (int h = 0; h < WPL / 4; ++h) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<gptr<const u32x4>>(p) + h);
      out.w[4 * h + 0] = v[0];
      out.w[4 * h + 1] = v[1];
      out.w[4 * h + 2] = v[2];
      out.w[4 * h + 3] = v[3];
    }
  }
}

// One group's loads for this lane: NB weight tiles, NB scale pairs and (without
// XLDS) the MB x WPL activation fragments.
template <int WPL, int MB, int NB, bool XLDS>
struct PStage {
  PWords<WPL> w[NB];
  uint32_t s2[NB];
  u32x4 x[XLDS ? 1 : MB][WPL];
};

// WM: waves along the rows. The workgroup's WAVES waves form WM x (WAVES / WM):
// wave w takes row blocks [(w % WM) MB / WM, ...) and the (w / WM)-th of the
// WAVES / WM ranges of K. With WM > 1 the waves of one K range share each
// weight tile (one is read from HBM, the others hit the caches: the loads are
// then ordinary, not non-temporal) and each holds the activations of fewer
// rows, which leaves registers for more groups in flight.
//
// XS (group 128, no XLDS): the activation fragments are loaded coalesced --
// 16 lanes read one row's 256 contiguous bytes of the group, so every load
// instruction uses whole 128-byte lines -- and turned into the MFMA operand
// arrangement through a wave-private LDS area (row-swizzled, lg_slot, so both
// the writes and the 16-row fragment reads are free of bank conflicts). Read
// directly in operand order, the four lanes of a row sit 64 bytes apart and a
// load instruction touches 32 lines, a quarter of each.
template <int GS, int MB, int NB, int WAVES, int P, bool XLDS, int WM = 1, bool XS = false>
__global__ __launch_bounds__(64 * WAVES) void plain_kernel(const uint16_t* __restrict__ x,
                                                          const uint32_t* __restrict__ qw,
                                                          const uint16_t* __restrict__ sp,
                                                          uint16_t* __restrict__ y, int M, int N,
                                                          int K) {
  constexpr int WPL = GS / 32;  // MFMA steps per group = packed words per lane per tile
  constexpr int LPG = GS / 8;   // 16-byte pieces of a row per group
  constexpr int WK = WAVES / WM;  // waves along K
  constexpr int MBW = MB / WM;    // row blocks per wave
  static_assert(!XLDS || MB == 1, "staged activations: one row block");
  static_assert(WK * WM == WAVES && MBW * WM == MB, "waves and row blocks divide evenly");
  static_assert(!XS || (GS == 128 && !XLDS), "coalesced staging: group 128, rows not in LDS");
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int c16 = lane & 15, lg = lane >> 4;
  const int G = K / GS;
  const int NCB = (N + 15) / 16;
  const int b0 = blockIdx.x * NB;
  const int m0 = blockIdx.y * 16 * MB;
  const int Mr = min(M - m0, 16 * MB);  // rows of this row tile
  const int wm = wave % WM, wk = wave / WM;
  const int mbw0 = wm * MBW;             // this wave's first row block
  // this wave's groups [g0, g1) (wave-uniform)
  const int g0 = static_cast<int>(static_cast<long long>(G) * wk / WK);
  const int g1 = static_cast<int>(static_cast<long long>(G) * (wk + 1) / WK);

  extern __shared__ __attribute__((aligned(16))) uint32_t plds[];
  // XLDS layout: rows [Mr][K + 8] bf16 (16 bytes of padding per row against
  // bank conflicts), then [G][16] fp32 -24 * row sums (rows past Mr repeat
  // row Mr - 1), then the reduction area.
  const int xstride = K + 8;                        // bf16 elements
  const int sum_off = XLDS ? (Mr * xstride) / 2 : 0;  // 4-byte words; Mr * xstride is even
  float* const xsum = reinterpret_cast<float*>(plds + sum_off);
  // XS: this wave's staging area, MBW row blocks of 16 rows x 256 bytes, after
  // the reduction area
  constexpr int kXsWaveBytes = XS ? MBW * 16 * 256 : 0;
  float* const red = reinterpret_cast<float*>(plds + (XLDS ? sum_off + G * 16 : 0));
  unsigned char* const xs_lds = reinterpret_cast<unsigned char*>(plds) +
                                static_cast<size_t>(WK) * MB * NB * 1024 + wave * kXsWaveBytes;

  // Column blocks past the last are clamped on load (their results are not stored).
  gptr<const uint32_t> wbase[NB];
  gptr<const uint32_t> sbase[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int b = min(b0 + nb, NCB - 1);
    wbase[nb] = to_global(qw) + static_cast<size_t>(b) * G * 64 * WPL + lane * WPL;
    sbase[nb] = reinterpret_cast<gptr<const uint32_t>>(to_global(sp) + static_cast<size_t>(b) * G * 16 +
                                                       (c16 & ~1));
  }
  // activation rows of this lane's A operand, one per row block (rows past M
  // repeat the last row; their MFMA output rows are never stored)
  // XS: load instruction i of a row block covers rows 4i + lane / 16, each
  // 16-lane row reading its 16 pieces of 16 bytes
  gptr<const uint16_t> xrow[XS ? MBW * 4 : MBW];
  if constexpr (XS) {
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = min(m0 + 16 * (mbw0 + mb) + 4 * i + lg, M - 1);
        xrow[mb * 4 + i] = to_global(x) + static_cast<size_t>(m) * K + 8 * c16;
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
      const int m = min(m0 + 16 * (mbw0 + mb) + c16, M - 1);
      xrow[mb] = to_global(x) + static_cast<size_t>(m) * K + lg * WPL * 8;
    }
  }

  const int glast = g1 - 1;
  auto load_stage = [&](PStage<WPL, MBW, NB, XLDS>& st, int grp) {
    grp = min(grp, glast);  // past the wave's last group: re-read it (cache hits, unused)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const gptr<const uint32_t> wp = wbase[nb] + static_cast<size_t>(grp) * 64 * WPL;
      if constexpr (WM == 1) {
        load_tile_words<WPL>(st.w[nb], wp);
      } else {
#pragma unroll
        for (int i = 0; i < WPL; ++i) st.w[nb].w[i] = wp[i];
      }
      st.s2[nb] = sbase[nb][static_cast<size_t>(grp) * 8];
    }
    if constexpr (XS) {
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          st.x[mb][i] = *reinterpret_cast<gptr<const u32x4>>(xrow[mb * 4 + i] + static_cast<size_t>(grp) * GS);
    } else if constexpr (!XLDS) {
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int t = 0; t < WPL; ++t)
          st.x[mb][t] = *reinterpret_cast<gptr<const u32x4>>(xrow[mb] + static_cast<size_t>(grp) * GS + 8 * t);
    }
  };

  PStage<WPL, MBW, NB, XLDS> stage[P];
  const bool active = g1 > g0;
  if (active) {
#pragma unroll
    for (int p = 0; p < P; ++p) load_stage(stage[p], g0 + p);
  }

  if constexpr (XLDS) {
    // Stage the row tile's activations and each group's -24 * row sums. A
    // group's LPG pieces of a row are consecutive elements of the loop (Mr *
    // K / 8 is a multiple of LPG, each pass a multiple of 64), so they sit in
    // consecutive lanes of one pass, all active together.
    const int chunks = K / 8;
    for (int e = threadIdx.x; e < Mr * chunks; e += 64 * WAVES) {
      const int row = e / chunks, c8 = e - row * chunks;
      const u32x4 d = *reinterpret_cast<gptr<const u32x4>>(to_global(x) +
                                                          static_cast<size_t>(m0 + row) * K + 8 * c8);
      *reinterpret_cast<u32x4*>(plds + (row * xstride + 8 * c8) / 2) = d;
      const float bsum = group_lane_sum<LPG>(neg_bias_sum8(d));
      if ((c8 % LPG) == 0) {
        float* dst = xsum + (c8 / LPG) * 16;
        dst[row] = bsum;
        if (row == Mr - 1)
          for (int m = Mr; m < 16; ++m) dst[m] = bsum;
      }
    }
    lds_barrier();  // LDS only: the weight loads in flight keep flying
  }

  const bf16x8 bias = bias_operand();
  f32x4 yacc[MBW][NB];
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) yacc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (active) {
    const int xl = (min(c16, Mr - 1) * xstride + lg * WPL * 8) / 2;  // XLDS: this lane's row, 4-byte words
    for (int c = g0; c < g1; c += P) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int grp = c + p;
        if (grp < g1) {
          PStage<WPL, MBW, NB, XLDS>& st = stage[p];
#pragma unroll
          for (int mb = 0; mb < MBW; ++mb) {
            bf16x8 a[WPL];
            f32x4 accb;
            if constexpr (XLDS) {
              const uint32_t* xp = plds + xl + (grp * GS) / 2;
#pragma unroll
              for (int t = 0; t < WPL; ++t)
                a[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xp + 4 * t));
              accb = *reinterpret_cast<const f32x4*>(xsum + grp * 16 + 4 * lg);
            } else {
              if constexpr (XS) {
                // coalesced pieces into the wave's area, then operand fragments
                // out of it (the same wave writes and reads: LDS keeps order)
                unsigned char* area = xs_lds + mb * 16 * 256;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int row = 4 * i + lg;
                  *reinterpret_cast<u32x4*>(area + row * 256 + lg_slot(c16, row) * 16) = st.x[mb][i];
                }
#pragma unroll
                for (int t = 0; t < WPL; ++t)
                  a[t] = *reinterpret_cast<const bf16x8*>(area + c16 * 256 + lg_slot(lg * WPL + t, c16) * 16);
              } else {
#pragma unroll
                for (int t = 0; t < WPL; ++t) a[t] = act_frag(st.x[mb][t]);
              }
              accb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int t = 0; t < WPL; ++t) accb = mfma16(a[t], bias, accb);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              f32x4 acc = accb;
#pragma unroll
              for (int t = 0; t < WPL; ++t) acc = mfma16(a[t], dequant_biased(st.w[nb].w[t]), acc);
              const float s = fp16_bits_to_f32(static_cast<uint16_t>(st.s2[nb] >> (16 * (c16 & 1))));
#pragma unroll
              for (int r = 0; r < 4; ++r) yacc[mb][nb][r] = __builtin_fmaf(s, acc[r], yacc[mb][nb][r]);
            }
          }
          load_stage(st, grp + P);
        }
      }
    }
  }

  // K reduction over the waves of each K range, through LDS: the value of
  // register r of (row block mb, column block nb) of lane l from the waves of
  // K range k at red[((k * MB + mb) * NB + nb) * 4 + r][l]; then each thread
  // sums the K ranges of its outputs in order. The accumulator of lane l holds
  // rows 4 (l / 16) + r of column l % 16 of its 16 x 16 block.
  if constexpr (XLDS) __syncthreads();  // the staged rows are no longer read
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[(((wk * MB + mbw0 + mb) * NB + nb) * 4 + r) * 64 + lane] = yacc[mb][nb][r];
  __syncthreads();
  constexpr int OUTS = MB * NB * 256;
  for (int e = threadIdx.x; e < OUTS; e += 64 * WAVES) {
    // e = ((mb * NB + nb) * 4 + r) * 64 + l
    const int l = e & 63, r = (e >> 6) & 3, blk = e >> 8;
    const int mb = blk / NB, nb = blk - mb * NB;
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < WK; ++k) sum += red[((k * MB + mb) * NB + nb) * 256 + r * 64 + l];
    const int m = m0 + 16 * mb + 4 * (l >> 4) + r;
    const int n = (b0 + nb) * 16 + (l & 15);
    if (m < M && n < N) to_global(y)[static_cast<size_t>(m) * N + n] = f32_to_bf16_bits(sum);
  }
}

template <int GS, int MB, int NB, int WAVES, int P, bool XLDS, int WM = 1, bool XS = false>
hipError_t launch_plain_t(const GemmArgs& a, hipStream_t stream) {
  const int NCB = (a.N + 15) / 16;
  if ((static_cast<long long>(a.M) + 16 * MB - 1) / (16 * MB) > 65535)
    return hipErrorInvalidValue;  // grid.y holds at most 65535 row tiles
  dim3 grid((NCB + NB - 1) / NB, (a.M + 16 * MB - 1) / (16 * MB));
  const int Mr = a.M < 16 * MB ? a.M : 16 * MB;
  size_t lds = static_cast<size_t>(WAVES / WM) * MB * NB * 256 * sizeof(float);
  if (XLDS) lds += static_cast<size_t>(Mr) * (a.K + 8) * 2 + static_cast<size_t>(a.K / GS) * 16 * 4;
  if (XS) lds += static_cast<size_t>(WAVES) * (MB / WM) * 16 * 256;
  const void* fn = reinterpret_cast<const void*>(&plain_kernel<GS, MB, NB, WAVES, P, XLDS, WM, XS>);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  const uint16_t* x = a.x;
  const uint32_t* qw = a.qweight;
  const uint16_t* sp = a.scales;
  uint16_t* y = a.y;
  int M = a.M, N = a.N, K = a.K;
  void* kargs[] = {&x, &qw, &sp, &y, &M, &N, &K};
  return hipLaunchKernel(fn, grid, dim3(64 * WAVES), kargs, lds, stream);
}

// The forms w4a16_gemm runs, by index (plain_form picks one per shape).
enum PlainForm : int {
  // up to 16 rows (one row block): measured on the decode layer set (qkv
  // 5120x7168, o 6144x5120, gate_up 5120x34816, down 17408x5120, group 128)
  // over every (column blocks, waves, groups in flight, staging) form that
  // fits: wide N (2176 column blocks) prefers 4-wave workgroups with 2 to 4
  // column blocks (at group 128 the 4-wave XS forms below); deep K at one or two rows 16 waves and staged rows; the
  // rest 8 waves below 9 rows, 4 waves above (at groups 32, 64 and 256; group
  // 128 takes the XS forms from 9 rows). Group 256 (twice the registers per
  // group) keeps fewer groups in flight. Few column blocks (the tensor-parallel
  // shard's qkv 5120x896: 56) take one block per 16-wave workgroup, and so does
  // one row whose K fits LDS (qkv and o of the layer set: 6.75 -> 6.29 and
  // 6.88 -> 6.47 us).
  kWideStaged,   // 1 x 2 blocks, 4 waves, rows in LDS
  kWide2,        // 1 x 2, 4 waves
  kWide4,        // 1 x 4, 4 waves
  kDeepStaged,   // 1 x 2, 16 waves, rows in LDS
  kSmall8,       // 1 x 2, 8 waves
  kOne16Staged,  // 1 x 1, 16 waves, rows in LDS
  kOne16,        // 1 x 1, 16 waves
  // more rows at group 128, activation fragments through a wave-private LDS
  // area (XS); MB x NB blocks, waves (along rows x along K)
  kXs1x2,        // 1 x 2, 8 waves (1 x 8)
  kXs1x4,        // 1 x 4, 8 waves (1 x 8)
  kXs1x5,        // 1 x 5, 8 waves (1 x 8)
  kXs2x2,        // 2 x 2, 16 waves (2 x 8)
  kXs2x3,        // 2 x 3, 16 waves (2 x 8)
  kXs2x4,        // 2 x 4, 16 waves (2 x 8)
  kXs2x5,        // 2 x 5, 8 waves (2 x 4)
  kXs4x4,        // 4 x 4, 16 waves (4 x 4)
  // up to 16 rows at group 128 with wide N (2176 column blocks): 4-wave
  // workgroups, 3 column blocks up to 4 rows and 5 above (gate_up 5120x34816:
  // 20.5 -> 17.9 us at M = 1, 26.0 -> 19.3 at 8, 24.5 -> 21.6 at 16)
  kXs1x3w4,      // 1 x 3, 4 waves
  kXs1x5w4,      // 1 x 5, 4 waves
  // and at 17 to 32 rows, where the time model puts it ahead of the tile
  // engine (gate_up: 31.8 -> 25.8 us at M = 17, 32.7 -> 28.9 at 32)
  kXs2x5w4,      // 2 x 5, 4 waves (1 x 4)
  // at 7 to 12 rows with K above 1024, two groups in flight (down 17408x5120:
  // 17.2 -> 16.5 us at M = 8, 19.1 -> 16.9 at 9; 16 rows: the same)
  kXs1x2p2,      // 1 x 2, 8 waves, P = 2
  // more rows at groups 32, 64 and 256, fragments loaded in operand order
  kOp2x2,        // 2 x 2, 4 waves
  kOp2x4,        // 2 x 4, 4 waves
  kOp4x2,        // 4 x 2, 4 waves
  kOp4x4,        // 4 x 4, 4 waves
  kPlainForms
};

struct PlainFormInfo {
  int mb, nb, waves;
};
constexpr PlainFormInfo kPlainFormInfo[kPlainForms] = {
    {1, 2, 4}, {1, 2, 4}, {1, 4, 4}, {1, 2, 16}, {1, 2, 8}, {1, 1, 16}, {1, 1, 16},
    {1, 2, 8}, {1, 4, 8}, {1, 5, 8}, {2, 2, 16}, {2, 3, 16}, {2, 4, 16}, {2, 5, 8}, {4, 4, 16},
    {1, 3, 4}, {1, 5, 4}, {2, 5, 4}, {1, 2, 8},
    {2, 2, 4}, {2, 4, 4}, {4, 2, 4}, {4, 4, 4}};

constexpr PlainForm kXsForms[] = {kXs1x2, kXs1x4, kXs1x5, kXs2x2,
                                  kXs2x3, kXs2x4, kXs2x5, kXs4x4};

// Modelled time of an XS form (microseconds): from 9 rows each
// workgroup streams its MB x 16 activation rows (from L2) and NB weight
// columns over all of K at about 45 GB/s per compute unit, after a fixed
// start of 4 us (8 waves), 1.5 us (16 waves: more loads in flight from the
// first group) or 2 us (4 waves); a compute unit that holds n workgroups takes
// n times as long. Fitted to the decode layer set and its tensor-parallel
// shard (qkv 5120x896, o 768x5120, gate_up 5120x4352, down 2176x5120) at M =
// 17 to 320, where the form it puts first is within 1 % of the fastest of
// every form measured, summed over the shapes (above 320 rows it runs 5-11 %
// under the measured time of the shard's qkv, 12.4 and 19.7 against 13.0 and
// 22.1 us at 512 and 1024 rows, still far from the tile engine's 30 us); at 9
// to 16 rows (the rows past M repeat row M - 1 and are read from the caches)
// it puts first the fastest XS form of each decode projection.
double xs_estimate_us(PlainForm f, int M, int N, int K) {
  const PlainFormInfo& i = kPlainFormInfo[f];
  const long long ncb = (static_cast<long long>(N) + 15) / 16;
  const long long wgs = (ncb + i.nb - 1) / i.nb * ((static_cast<long long>(M) + 16 * i.mb - 1) / (16 * i.mb));
  const long long rounds = (wgs + kModelCUs - 1) / kModelCUs;
  const double bytes = static_cast<double>(K) * (32.0 * i.mb + 8.0 * i.nb);
  const double t0 = i.waves == 16 ? 1.5 : i.waves == 4 ? 2.0 : 4.0;
  return static_cast<double>(rounds) * (bytes / 45000.0 + t0);
}

// The XS form of least modelled time; with wide4 and wide N (1024 column
// blocks or more) the 4-wave 32-row form is a candidate too.
PlainForm best_xs_form(int M, int N, int K, bool wide4, double* est_out) {
  PlainForm best = kXsForms[0];
  double best_est = xs_estimate_us(best, M, N, K);
  for (PlainForm f : kXsForms) {
    const double e = xs_estimate_us(f, M, N, K);
    if (e < best_est) {
      best_est = e;
      best = f;
    }
  }
  if (wide4 && (N + 15) / 16 >= 1024) {
    const double e = xs_estimate_us(kXs2x5w4, M, N, K);
    if (e < best_est) {
      best_est = e;
      best = kXs2x5w4;
    }
  }
  if (est_out) *est_out = best_est;
  return best;
}

template <int GS>
hipError_t launch_plain_g(const GemmArgs& a, hipStream_t s) {
  constexpr int P2 = GS >= 256 ? 1 : 2;
  constexpr int P4 = GS >= 256 ? 2 : 4;
  // the one-block 16-wave forms keep 128 k (one group of 128 or more) in flight
  constexpr int P1 = GS >= 128 ? 1 : 128 / GS;
  switch (plain_form(a.M, a.N, a.K, GS)) {
    case kWideStaged: return launch_plain_t<GS, 1, 2, 4, P4, true>(a, s);
    case kWide2: return launch_plain_t<GS, 1, 2, 4, P2, false>(a, s);
    case kWide4: return launch_plain_t<GS, 1, 4, 4, P2, false>(a, s);
    case kDeepStaged: return launch_plain_t<GS, 1, 2, 16, P2, true>(a, s);
    case kSmall8: return launch_plain_t<GS, 1, 2, 8, P2, false>(a, s);
    case kOne16Staged: return launch_plain_t<GS, 1, 1, 16, P1, true>(a, s);
    case kOne16: return launch_plain_t<GS, 1, 1, 16, P1, false>(a, s);
    case kOp2x2: return launch_plain_t<GS, 2, 2, 4, P2, false>(a, s);
    case kOp2x4: return launch_plain_t<GS, 2, 4, 4, P2, false>(a, s);
    case kOp4x2: return launch_plain_t<GS, 4, 2, 4, 1, false>(a, s);
    case kOp4x4: return launch_plain_t<GS, 4, 4, 4, 1, false>(a, s);
    default: break;
  }
  if constexpr (GS == 128) {
    switch (plain_form(a.M, a.N, a.K, GS)) {
      case kXs1x2: return launch_plain_t<GS, 1, 2, 8, 1, false, 1, true>(a, s);
      case kXs1x4: return launch_plain_t<GS, 1, 4, 8, 1, false, 1, true>(a, s);
      case kXs1x5: return launch_plain_t<GS, 1, 5, 8, 1, false, 1, true>(a, s);
      case kXs2x2: return launch_plain_t<GS, 2, 2, 16, 1, false, 2, true>(a, s);
      case kXs2x3: return launch_plain_t<GS, 2, 3, 16, 1, false, 2, true>(a, s);
      case kXs2x4: return launch_plain_t<GS, 2, 4, 16, 1, false, 2, true>(a, s);
      case kXs2x5: return launch_plain_t<GS, 2, 5, 8, 1, false, 2, true>(a, s);
      case kXs4x4: return launch_plain_t<GS, 4, 4, 16, 1, false, 4, true>(a, s);
      case kXs1x3w4: return launch_plain_t<GS, 1, 3, 4, 1, false, 1, true>(a, s);
      case kXs1x5w4: return launch_plain_t<GS, 1, 5, 4, 1, false, 1, true>(a, s);
      case kXs2x5w4: return launch_plain_t<GS, 2, 5, 4, 1, false, 1, true>(a, s);
      case kXs1x2p2: return launch_plain_t<GS, 1, 2, 8, 2, false, 1, true>(a, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

int plain_form(int M, int N, int K, int group) {
  const bool wide = (N + 15) / 16 >= 1024;
  const size_t xlds_rows = static_cast<size_t>(M < 16 ? M : 16) * (static_cast<size_t>(K) + 8) * 2 +
                           static_cast<size_t>(K / group) * 64;
  // From 9 rows at group 128 the XS forms win on the decode layer set and its
  // tensor-parallel shard (M = 16: 76.6 -> 61.8 us per layer set as four
  // calls); at 8 rows and fewer the forms below (measured at M = 4, 6 and 8).
  // At group 128 and up to 16 rows, wide N takes the 4-wave XS forms, and a
  // short K (at most 8 groups: the shard's o 768x5120, 4.2-4.4 -> 3.6-3.8 us)
  // the 8-wave two-block XS form, at every row count.
  if (group == 128 && M <= 16) {
    if (wide) return M <= 4 ? kXs1x3w4 : kXs1x5w4;
    if (K <= 1024 && (N + 15) / 16 >= 128) return kXs1x2;
  }
  if (group == 128 && M >= 9) {
    const PlainForm f = best_xs_form(M, N, K, true, nullptr);
    return f == kXs1x2 && M <= 12 && K > 1024 ? kXs1x2p2 : f;
  }
  if (M <= 16) {
    if (wide) {
      if (M <= 2 && xlds_rows + 4 * 2 * 1024 <= kPlainLdsLimit) return kWideStaged;
      return M <= 4 ? kWide2 : kWide4;
    }
    if (M <= 2 && K >= 12288 && xlds_rows + 16 * 2 * 1024 <= kPlainLdsLimit) return kDeepStaged;
    if (M <= 8 && (N + 15) / 16 < 128) return kOne16;
    if (M == 1 && xlds_rows + 16 * 1024 <= kPlainLdsLimit) return kOne16Staged;
    if (group == 128 && M >= 7 && K > 1024) return kXs1x2p2;
    return M <= 8 ? kSmall8 : kWide2;
  }
  if (M <= 32) return wide ? kOp2x4 : kOp2x2;
  return wide ? kOp4x4 : kOp4x2;
}

void plain_form_shape(int form, int* rows, int* cols, int* waves) {
  const PlainFormInfo& i = kPlainFormInfo[form >= 0 && form < kPlainForms ? form : 0];
  *rows = 16 * i.mb;
  *cols = 16 * i.nb;
  *waves = i.waves;
}

// The best XS form's modelled time; at other group sizes the forms load their
// activation fragments in operand order, measured 1.3x slower than XS at 64
// rows on the decode layer set.
double plain_estimate_us(int M, int N, int K, int group) {
  double est = 0.0;
  best_xs_form(M, N, K, group == 128, &est);
  return group == 128 ? est : 1.3 * est;
}

hipError_t launch_skinny(const GemmArgs& a, hipStream_t stream) {
  switch (a.group) {
    case 32: return launch_plain_g<32>(a, stream);
    case 64: return launch_plain_g<64>(a, stream);
    case 128: return launch_plain_g<128>(a, stream);
    case 256: return launch_plain_g<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a16_internal
