// w4a16_large.hip -- the large-M path (batched decode, prefill-sized blocks).
//
// Past the point where the weight stream stops being the bottleneck, the
// GEMM is bound by matrix arithmetic (ai.satyajit.si page, section "What one
// more stream costs on this model": once the rows' arithmetic catches up with
// the weight traffic, each extra row adds its full share of compute). This
// kernel is therefore a tiled MFMA GEMM in which every operand byte is reused
// as often as registers and LDS allow:
//
//  * A workgroup computes a 128 x 256 output tile with 8 waves side by side
//    along N, each a 128 x 32 sub-tile: 8 x 2 blocks of
//    v_mfma_f32_16x16x32_bf16. Every dequantized weight register feeds 8
//    MFMAs, and no two waves dequantize the same weights.
//  * K advances in tiles of 128. The workgroup stages the 128 x 128 bf16
//    activation tile into LDS (double-buffered, one barrier per tile),
//    XOR-swizzled by row so that both the staging writes and the fragment
//    reads are free of bank conflicts.
//  * Packed weights go straight from the tiled format into registers: a
//    lane's words of one (16-column block, group) tile are its B operands
//    for that group's MFMA steps.
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
// whole groups). Rows beyond M read as zero (buffer range), column blocks
// beyond N are clamped on load; neither is stored.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16_internal {
namespace {

constexpr int kLgWaves = 8;                   // all along N
constexpr int kLgMB = 8;                      // 16-row blocks per wave (all 128 rows)
constexpr int kLgNB = 2;                      // 16-column blocks per wave
constexpr int kLgRows = kLgMB * 16;           // 128 rows per workgroup tile
constexpr int kLgBlocks = kLgWaves * kLgNB;   // 16 column blocks = 256 columns
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
  // Lane permutations within rows of 16 lanes whose sources all exist.
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF,
                                                     true));
}

// -136 times the sum of the 8 bf16 values of a 16-byte piece, in fp32: four
// bf16 dot products against the pair (-136, -136). Each product is exact in
// fp32 (8-bit by 8-bit significands); only the additions round.
__device__ __forceinline__ float neg136_sum8(u32x4 d) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 k = __builtin_bit_cast(bf16x2, kBiasPair);
  // Elements are copied to scalars first: this compiler's __builtin_bit_cast
  // of a vector-element expression (d[1]) reads the vector's first element.
  const uint32_t e0 = d[0], e1 = d[1], e2 = d[2], e3 = d[3];
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, e0), k, 0.f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, e1), k, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, e2), k, s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, e3), k, s, false);
}

// Sum over the aligned group of LPG consecutive lanes containing this lane,
// returned in every lane of the group (butterfly within quads, half rows and
// rows of 16 lanes).
template <int LPG>
__device__ __forceinline__ float group_lane_sum(float v) {
  static_assert(LPG == 4 || LPG == 8 || LPG == 16, "group of 32, 64 or 128");
  v += dpp_f32<0xB1>(v);                           // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);                           // quad_perm [2,3,0,1]
  if constexpr (LPG >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror
  if constexpr (LPG >= 16) v += dpp_f32<0x140>(v); // row_mirror
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

// Buffer resource over [base, base + bytes): loads at offsets at or beyond
// `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

template <int GS>
__global__ __launch_bounds__(kLgThreads, 1) void large_kernel(GemmArgs a, int MT, int NT) {
  using C = LgCfg<GS>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lg_lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wn = wave;
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

  // ---- activation staging: thread stages piece `spiece` (8 values) of rows
  // srow0 + 32 i. Loads go through a buffer resource based at (row m0, k of
  // the tile) and ending at the end of x, so rows beyond M read as zero. ----
  const int spiece = tid % kLgPieces;
  const int srow0 = tid / kLgPieces;
  constexpr int kRowStep = kLgThreads / kLgPieces;   // 32
  const uint32_t xbytes = static_cast<uint32_t>(M - m0) * static_cast<uint32_t>(K) * 2u;
  const uint16_t* xrow0 = a.x + static_cast<size_t>(m0) * K;
  uint32_t voff[kLgLoads];
#pragma unroll
  for (int i = 0; i < kLgLoads; ++i)
    voff[i] = (static_cast<uint32_t>(srow0 + i * kRowStep) * K + spiece * 8) * 2u;

  auto stage_load = [&](StageRegs& r, int t) {
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(xrow0 + t * kLgKT, xbytes - static_cast<uint32_t>(t) * (kLgKT * 2));
#pragma unroll
    for (int i = 0; i < kLgLoads; ++i) r.d[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, voff[i], 0, 0);
  };
  auto stage_store = [&](const StageRegs& r, int buf) {
    unsigned char* base = lg_lds + buf * C::BufBytes;
    float* sums = reinterpret_cast<float*>(base + kLgABytes);
#pragma unroll
    for (int i = 0; i < kLgLoads; ++i) {
      const int row = srow0 + i * kRowStep;
      const float s = group_lane_sum<C::LPG>(neg136_sum8(r.d[i]));
      sums[(spiece / C::LPG) * kLgRows + row] = s;  // every lane of the group: same value
      const int sl = spiece ^ (row & 15);
      *reinterpret_cast<u32x4*>(base + row * kLgRowBytes + sl * 16) = r.d[i];
    }
  };

  // ---- weights and scales of this wave's 4 column blocks: wave-uniform tile
  // offsets, one lane offset ----
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(a.qweight, static_cast<uint32_t>(NCB) * 16u * static_cast<uint32_t>(K) / 2u);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(a.scales, static_cast<uint32_t>(NCB) * 16u * static_cast<uint32_t>(G) * 2u);
  const uint32_t qlane = static_cast<uint32_t>(lane) * C::WPL * 4u;
  const uint32_t slane = static_cast<uint32_t>(lane & 14) * 2u;
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
        const uint32_t tile_idx = static_cast<uint32_t>(blk[nb]) * G + grp;
        const int qoff = static_cast<int>(tile_idx * (64u * C::WPL * 4u));
        if constexpr (C::WPL == 4) {
          u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rq, qlane, qoff, 0);
#pragma unroll
          for (int w = 0; w < 4; ++w) r.w[nb][gi * 4 + w] = v[w];
        } else if constexpr (C::WPL == 2) {
          u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rq, qlane, qoff, 0);
          r.w[nb][gi * 2 + 0] = v[0];
          r.w[nb][gi * 2 + 1] = v[1];
        } else {
          r.w[nb][gi] = __builtin_amdgcn_raw_buffer_load_b32(rq, qlane, qoff, 0);
        }
        r.s[nb][gi] =
            __builtin_amdgcn_raw_buffer_load_b32(rs, slane, static_cast<int>(tile_idx * 32u), 0);
      }
    }
  };

  f32x4 yacc[kLgMB][kLgNB];
#pragma unroll
  for (int mb = 0; mb < kLgMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kLgNB; ++nb) yacc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int arow = lane & 15;                            // A fragment row (block 0)
  const int jgrp = lane >> 4;                            // k-slice of the lane
  const int shalf = (lane & 1) * 16;                     // scale half of the pair

  // One k-tile: 4 MFMA steps of 32 k. Step st belongs to group st / WPL of the
  // tile; a group's accumulation starts from its -136 * row-sum tile and ends
  // with the scaled add into yacc.
  auto compute = [&](const BRegs<GS>& b, int t, int buf) {
    const unsigned char* base = lg_lds + buf * C::BufBytes;
    const float* sums = reinterpret_cast<const float*>(base + kLgABytes);
    f32x4 acc[kLgNB][kLgMB];
    f32x4 bias[kLgMB];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int gi = st / C::WPL, w = st % C::WPL;
      if (C::T > 1 && t * C::T + gi >= G) break;  // ragged last tile (uniform)
      if (w == 0) {
#pragma unroll
        for (int mb = 0; mb < kLgMB; ++mb)
          bias[mb] = *reinterpret_cast<const f32x4*>(sums + gi * kLgRows + mb * 16 + 4 * jgrp);
      }
      const int piece = gi * C::LPG + jgrp * C::WPL + w;
      bf16x8 af[kLgMB];
#pragma unroll
      for (int mb = 0; mb < kLgMB; ++mb)
        af[mb] = *reinterpret_cast<const bf16x8*>(base + (arow + mb * 16) * kLgRowBytes +
                                                 ((piece ^ (lane & 15)) * 16));
#pragma unroll
      for (int nb = 0; nb < kLgNB; ++nb) {
        const bf16x8 bq = dequant_biased(b.w[nb][st]);
#pragma unroll
        for (int mb = 0; mb < kLgMB; ++mb)
          acc[nb][mb] = mfma16(af[mb], bq, w == 0 ? bias[mb] : acc[nb][mb]);
      }
      if (w == C::WPL - 1) {
#pragma unroll
        for (int nb = 0; nb < kLgNB; ++nb) {
          const float sc = fp16_bits_to_f32(static_cast<uint16_t>(b.s[nb][gi] >> shalf));
#pragma unroll
          for (int mb = 0; mb < kLgMB; ++mb) yacc[mb][nb] += sc * acc[nb][mb];
        }
      }
    }
  };

  // ---- pipeline: tile t computes from LDS buffer t & 1 while tile t + 1 is
  // loaded into registers and then staged into the other buffer. Weight
  // registers alternate between two sets (no copies). ----
  StageRegs sr;
  BRegs<GS> b0, b1;
  stage_load(sr, 0);
  load_b(b0, 0);
  stage_store(sr, 0);
  __syncthreads();
  auto iter = [&](int t, const BRegs<GS>& cur, BRegs<GS>& nxt) {
    const int tn = t + 1 < ntiles ? t + 1 : t;   // the last iteration reloads (unused)
    stage_load(sr, tn);
    load_b(nxt, tn);
    __builtin_amdgcn_sched_barrier(0);            // issue the loads before the math
    compute(cur, t, t & 1);
    stage_store(sr, (t + 1) & 1);
    // LDS-only barrier: global loads of the next tile may stay in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  for (int t = 0; t < ntiles; t += 2) {
    iter(t, b0, b1);
    if (t + 1 >= ntiles) break;
    iter(t + 1, b1, b0);
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
        const int row = m0 + mb * 16 + 4 * jgrp + r;
        if (row < M) yg[static_cast<size_t>(row) * N + col] = f32_to_bf16_bits(yacc[mb][nb][r]);
      }
    }
  }
}

template <int GS>
hipError_t launch_large_t(const GemmArgs& a, hipStream_t stream) {
  const int NCB = (a.N + 15) / 16;
  const int NT = (NCB + kLgBlocks - 1) / kLgBlocks;
  const void* fn = reinterpret_cast<const void*>(&large_kernel<GS>);
  const size_t lds = LgCfg<GS>::Lds;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  // Buffer offsets are 32-bit: each launch covers at most rows_per_launch rows
  // of x (and the packed weights must stay below 4 GB, checked by the caller).
  const long long row_bytes = 2LL * a.K;
  long long rows_per_launch = (0xFFFFFFFFLL - 16) / row_bytes;
  rows_per_launch -= rows_per_launch % kLgRows;
  if (rows_per_launch < kLgRows) return hipErrorInvalidValue;
  for (long long r0 = 0; r0 < a.M; r0 += rows_per_launch) {
    GemmArgs part = a;
    part.M = static_cast<int>(a.M - r0 < rows_per_launch ? a.M - r0 : rows_per_launch);
    part.x = a.x + r0 * a.K;
    part.y = a.y + r0 * a.N;
    int MT = (part.M + kLgRows - 1) / kLgRows;
    const long long total = static_cast<long long>(MT) * NT;
    if (total < 1 || total > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    int ntc = NT;
    void* kargs[] = {&part, &MT, &ntc};
    e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(total)), dim3(kLgThreads), kargs, lds,
                        stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool large_supported(int group) { return group == 32 || group == 64 || group == 128; }

hipError_t launch_large(const GemmArgs& a, hipStream_t stream) {
  // packed weights and scales are addressed with 32-bit buffer offsets
  const long long qbytes = static_cast<long long>((a.N + 15) / 16) * 16 * a.K / 2;
  if (qbytes > 0xFFFFFFF0LL) return launch_skinny(a, stream);
  switch (a.group) {
    case 32: return launch_large_t<32>(a, stream);
    case 64: return launch_large_t<64>(a, stream);
    case 128: return launch_large_t<128>(a, stream);
    default: return launch_skinny(a, stream);  // group 256: split-K kernel
  }
}

}  // namespace w4a16_internal
