// w4a16_large.hip -- the large-M path (batched decode, prefill-sized blocks).
//
// Past the point where the weight stream stops being the bottleneck, the
// GEMM is bound by matrix arithmetic (ai.satyajit.si page, section "What one
// more stream costs on this model": once the rows' arithmetic catches up with
// the weight traffic, each extra row adds its full share of compute). The
// kernels here are therefore tiled MFMA GEMMs in which every operand byte is
// reused as often as registers and LDS allow:
//
//  * An output tile is R x 256 (R = 32, 64 or 128 rows) and belongs to one
//    workgroup of 8 waves side by side along N, each an R x 32 sub-tile of
//    (R/16) x 2 blocks of v_mfma_f32_16x16x32_bf16. Every dequantized weight
//    register feeds R/16 MFMAs, and no two waves dequantize the same weights.
//  * K advances in k-tiles of 128. The workgroup stages the R x 128 bf16
//    activation tile into LDS (double-buffered, one barrier per k-tile),
//    XOR-swizzled by row (lg_slot) so that both the staging writes and the
//    fragment reads are free of bank conflicts on gfx950's LDS.
//  * Packed weights go straight from the tiled format into registers: a
//    lane's words of one (16-column block, group) tile are its B operands
//    for that group's MFMA steps.
//  * Dequantization yields the exact biased value 24 + q (as in the small-M
//    kernels). Instead of a second MFMA against a -24 operand, the bias is
//    removed by starting each group's accumulation from -24 * sum_k x[m][k]
//    over the group: those row sums are formed once per workgroup while the
//    activation tile is staged (bf16 dot products, then a DPP reduction) and
//    kept in LDS next to the tile. Every MFMA then does useful work.
//  * The group's fp32 partial is scaled by its fp16 scale and added to the
//    running fp32 result, as in the other kernels.
//
// Two schedules share that tile engine:
//  * tile_kernel: one workgroup per 32, 64 or 128 x 256 tile, the whole K
//    range; needs no workspace. The tile height is the one a time model of
//    the three forms puts first for the shape (tile_estimate_us); at 32 and
//    64 rows the loads run three k-tiles ahead. Workgroups are numbered so
//    that the 8 XCDs (which take workgroups round robin) each own a
//    contiguous range of tiles, row tiles fastest: the row tiles that share a
//    column tile's weights run together on one XCD and find those weights in
//    its L2.
//  * large_streamk_kernel: a persistent grid splits the (problem, tile,
//    k-tile) iterations of up to 8 problems evenly, so the machine stays full
//    whatever the tile count (at M = 128 one layer has only about 200 tiles
//    for 256 compute units). Tiles cut between workgroups are combined
//    through a caller workspace: each workgroup publishes its part, and the
//    last to arrive (an atomic counter per tile) sums the parts in workgroup
//    order, so the result does not depend on timing.
//
// Group sizes 32, 64 and 128 are handled here (a k-tile holds 4, 2 or 1
// whole groups). Rows beyond M read as zero (buffer range), column blocks
// beyond N are clamped on load; neither is stored.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16_internal {
namespace {

constexpr int kLgWaves = 8;                   // all along N
constexpr int kLgNB = 2;                      // 16-column blocks per wave
constexpr int kLgBlocks = kLgWaves * kLgNB;   // 16 column blocks = 256 columns
constexpr int kLgThreads = kLgWaves * 64;
constexpr int kLgKT = 128;                    // k per k-tile
constexpr int kLgPieces = kLgKT / 8;          // 16-byte pieces per row per k-tile
constexpr int kLgRowBytes = kLgKT * 2;
constexpr int kLgRowStep = kLgThreads / kLgPieces;  // 32 rows staged per pass

// Tile geometry and LDS layout for group size GS and MB 16-row blocks.
template <int GS, int MB>
struct LgCfg {
  static_assert(MB == 2 || MB == 4 || MB == 8, "32, 64 or 128 rows per tile");
  static constexpr int Rows = MB * 16;
  static constexpr int Loads = Rows * kLgPieces / kLgThreads;  // pieces staged per thread
  static constexpr int ABytes = Rows * kLgRowBytes;
  static constexpr int T = kLgKT / GS;        // groups per k-tile
  static constexpr int WPL = GS / 32;         // MFMA steps (words per lane) per group
  static constexpr int LPG = GS / 8;          // staging lanes per group
  static constexpr int SBytes = T * Rows * 4;
  static constexpr int BufBytes = ABytes + SBytes;
  static constexpr size_t Lds = 2 * static_cast<size_t>(BufBytes);
  static constexpr int Regs = MB * kLgNB * 4;  // accumulator floats per lane
};


template <int GS, int MB>
struct StageRegs {
  u32x4 d[LgCfg<GS, MB>::Loads];
};

template <int GS>
struct BRegs {
  uint32_t w[kLgNB][kLgKT / 32];    // 4 words per block per k-tile
  uint32_t s[kLgNB][kLgKT / GS];    // scale pairs (fp16 x 2) per group
};

template <int MB>
struct Acc {
  f32x4 v[MB][kLgNB];
};

template <int MB>
__device__ __forceinline__ void zero(Acc<MB>& a) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kLgNB; ++nb) a.v[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ------------------------------------------------------------------ tile engine
//
// One workgroup's view of one output tile: rows m0 .. m0 + Rows - 1, column
// blocks 16 nt .. 16 nt + 15 (wave w owns blocks 16 nt + 2w, 16 nt + 2w + 1).
// kloop() accumulates k-tiles [k0, k1) into acc; every wave of the workgroup
// must call it with the same arguments (it holds workgroup barriers).
template <int GS, int MB>
struct TileEngine {
  using C = LgCfg<GS, MB>;
  unsigned char* lds;
  int tid, lane, wave;
  int M, N, K, G, NCB, m0, nt;
  const uint16_t* xrow0;
  uint32_t xbytes;
  __amdgpu_buffer_rsrc_t rq, rs;
  int blk[kLgNB];

  __device__ __forceinline__ void setup(unsigned char* lds_, const uint16_t* x, const uint32_t* qw,
                                        const uint16_t* sp, int M_, int N_, int K_, int m0_,
                                        int nt_) {
    lds = lds_;
    tid = threadIdx.x;
    lane = tid & 63;
    wave = uniform(tid >> 6);
    M = M_;
    N = N_;
    K = K_;
    G = K / GS;
    NCB = (N + 15) / 16;
    m0 = m0_;
    nt = nt_;
    xbytes = static_cast<uint32_t>(M - m0) * static_cast<uint32_t>(K) * 2u;
    xrow0 = x + static_cast<size_t>(m0) * K;
    rq = make_rsrc(qw, static_cast<uint32_t>(NCB) * 16u * static_cast<uint32_t>(K) / 2u);
    rs = make_rsrc(sp, static_cast<uint32_t>(NCB) * 16u * static_cast<uint32_t>(G) * 2u);
#pragma unroll
    for (int nb = 0; nb < kLgNB; ++nb) {
      const int b = nt * kLgBlocks + wave * kLgNB + nb;
      blk[nb] = b < NCB ? b : NCB - 1;
    }
  }

  // ---- activation staging: thread stages piece tid % 16 (8 values) of rows
  // tid / 16 + 32 i, through a buffer resource based at (row m0, k of the
  // k-tile) and ending at the end of x, so rows beyond M read as zero ----
  __device__ __forceinline__ void stage_load(StageRegs<GS, MB>& r, int t) const {
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(xrow0 + t * kLgKT, xbytes - static_cast<uint32_t>(t) * (kLgKT * 2));
    const int spiece = tid % kLgPieces, srow0 = tid / kLgPieces;
#pragma unroll
    for (int i = 0; i < C::Loads; ++i) {
      const uint32_t voff =
          (static_cast<uint32_t>(srow0 + i * kLgRowStep) * K + spiece * 8) * 2u;
      r.d[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, voff, 0, 0);
    }
  }
  __device__ __forceinline__ void stage_store(const StageRegs<GS, MB>& r, int buf) const {
    unsigned char* base = lds + buf * C::BufBytes;
    float* sums = reinterpret_cast<float*>(base + C::ABytes);
    const int spiece = tid % kLgPieces, srow0 = tid / kLgPieces;
#pragma unroll
    for (int i = 0; i < C::Loads; ++i) {
      const int row = srow0 + i * kLgRowStep;
      const float s = group_lane_sum<C::LPG>(neg_bias_sum8(r.d[i]));
      sums[(spiece / C::LPG) * C::Rows + row] = s;  // every lane of the group: same value
      const int sl = lg_slot(spiece, row);
      *reinterpret_cast<u32x4*>(base + row * kLgRowBytes + sl * 16) = r.d[i];
    }
  }

  // ---- this wave's weights and scales of k-tile t ----
  __device__ __forceinline__ void load_b(BRegs<GS>& r, int t) const {
    const uint32_t qlane = static_cast<uint32_t>(lane) * C::WPL * 4u;
    const uint32_t slane = static_cast<uint32_t>(lane & 14) * 2u;
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
  }

  // One k-tile: 4 MFMA steps of 32 k. Step st belongs to group st / WPL of the
  // k-tile; a group's accumulation starts from its -24 * row-sum tile and
  // ends with the scaled add into acc_out.
  __device__ __forceinline__ void compute(Acc<MB>& acc_out, const BRegs<GS>& b, int t,
                                          int buf) const {
    const unsigned char* base = lds + buf * C::BufBytes;
    const float* sums = reinterpret_cast<const float*>(base + C::ABytes);
    const int arow = lane & 15, jgrp = lane >> 4;
    const int shalf = (lane & 1) * 16;
    f32x4 acc[kLgNB][MB];
    f32x4 bias[MB];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int gi = st / C::WPL, w = st % C::WPL;
      if (C::T > 1 && t * C::T + gi >= G) break;  // ragged last k-tile (uniform)
      if (w == 0) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          bias[mb] = *reinterpret_cast<const f32x4*>(sums + gi * C::Rows + mb * 16 + 4 * jgrp);
      }
      const int piece = gi * C::LPG + jgrp * C::WPL + w;
      bf16x8 af[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[mb] = *reinterpret_cast<const bf16x8*>(base + (arow + mb * 16) * kLgRowBytes +
                                                 lg_slot(piece, arow) * 16);
      // Both blocks' operands are dequantized first and the step's
      // 2 x MB MFMAs then issue as one uninterrupted run (the scheduling
      // fences keep the compiler from spreading them among the VALU work),
      // row block by row block so that each A fragment is done with after
      // two MFMAs: 3 to 4 % faster at 512 to 1024 rows, 6 % at 64.
      bf16x8 bq[kLgNB];
#pragma unroll
      for (int nb = 0; nb < kLgNB; ++nb) bq[nb] = dequant_biased(b.w[nb][st]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < kLgNB; ++nb)
          acc[nb][mb] = mfma16(af[mb], bq[nb], w == 0 ? bias[mb] : acc[nb][mb]);
      __builtin_amdgcn_sched_barrier(0);
      if (w == C::WPL - 1) {
#pragma unroll
        for (int nb = 0; nb < kLgNB; ++nb) {
          const float sc = fp16_bits_to_f32(static_cast<uint16_t>(b.s[nb][gi] >> shalf));
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc_out.v[mb][nb] += sc * acc[nb][mb];
        }
      }
    }
  }

  // k-tiles [k0, k1): k-tile t computes from LDS buffer (t - k0) & 1 while
  // k-tile t + 1 is loaded into registers and then staged into the other
  // buffer. Weight registers alternate between two sets (no copies). Every
  // k-tile ends with a workgroup barrier, so the LDS buffers are free on
  // return.
  __device__ __forceinline__ void kloop(Acc<MB>& acc, int k0, int k1) const {
    StageRegs<GS, MB> sr;
    BRegs<GS> b0, b1;
    stage_load(sr, k0);
    load_b(b0, k0);
    stage_store(sr, 0);
    lds_barrier();
    auto iter = [&](int t, const BRegs<GS>& cur, BRegs<GS>& nxt) {
      const int tn = t + 1 < k1 ? t + 1 : t;   // the last iteration reloads (unused)
      const int buf = (t - k0) & 1;
      stage_load(sr, tn);
      load_b(nxt, tn);
      __builtin_amdgcn_sched_barrier(0);       // issue the loads before the math
      compute(acc, cur, t, buf);
      stage_store(sr, buf ^ 1);
      lds_barrier();
    };
    for (int t = k0; t < k1; t += 2) {
      iter(t, b0, b1);
      if (t + 1 >= k1) break;
      iter(t + 1, b1, b0);
    }
  }

  // k-tiles [k0, k1) with the loads of k-tile t + D issued before k-tile t
  // computes: D register sets of activation pieces and D + 1 of weights (the
  // LDS double buffer as in kloop). For workgroups that each own a whole K
  // range at tile counts near the number of compute units, where one
  // workgroup's k-tiles follow each other on load latency rather than on
  // arithmetic. The step is unrolled over D (D + 1) k-tiles so that every
  // register set has a fixed name (an indexed copy would wait for its loads).
  template <int D>
  __device__ __forceinline__ void kloop_deep(Acc<MB>& acc, int k0, int k1) const {
    constexpr int PER = D * (D + 1);  // a multiple of D, D + 1 and 2
    StageRegs<GS, MB> sr[D];
    BRegs<GS> b[D + 1];
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int t = k0 + j < k1 ? k0 + j : k1 - 1;  // past the end: reload (unused)
      stage_load(sr[j], t);
      load_b(b[j], t);
    }
    stage_store(sr[0], 0);
    lds_barrier();
    for (int t0 = k0; t0 < k1; t0 += PER) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        // k-tile t = t0 + j: its weights are b[j % (D + 1)], its activations
        // sit in LDS buffer j & 1; sr[j % D] and b[(j + D) % (D + 1)] are free
        const int t = t0 + j;
        if (t >= k1) break;
        const int tl = t + D < k1 ? t + D : k1 - 1;
        stage_load(sr[j % D], tl);
        load_b(b[(j + D) % (D + 1)], tl);
        __builtin_amdgcn_sched_barrier(0);  // issue the loads before the math
        compute(acc, b[j % (D + 1)], t, j & 1);
        stage_store(sr[(j + 1) % D], (j + 1) & 1);
        lds_barrier();
      }
    }
  }

  // bf16 (RNE) stores of the rows and columns that exist.
  __device__ __forceinline__ void store(const Acc<MB>& acc, uint16_t* y) const {
    gptr<uint16_t> yg = to_global(y);
    const int jgrp = lane >> 4;
#pragma unroll
    for (int nb = 0; nb < kLgNB; ++nb) {
      const int col = (nt * kLgBlocks + wave * kLgNB + nb) * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + mb * 16 + 4 * jgrp + r;
          if (row < M) yg[static_cast<size_t>(row) * N + col] = f32_to_bf16_bits(acc.v[mb][nb][r]);
        }
      }
    }
  }
};

// =================================================== one workgroup per tile

// MB x 16 rows by 256 columns per workgroup over the whole K range, loads
// issued D k-tiles ahead (D = 1: kloop).
template <int GS, int MB, int D>
__global__ __launch_bounds__(kLgThreads, 1) void tile_kernel(GemmArgs a, int MT, int NT) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lg_lds[];
  const int tile = xcd_grouped(blockIdx.x, MT * NT);
  const int mt = tile % MT, nt = tile / MT;
  TileEngine<GS, MB> e;
  e.setup(lg_lds, a.x, a.qweight, a.scales, a.M, a.N, a.K, mt * LgCfg<GS, MB>::Rows, nt);
  Acc<MB> acc;
  zero(acc);
  const int kt = (e.G + LgCfg<GS, MB>::T - 1) / LgCfg<GS, MB>::T;
  if constexpr (D == 1)
    e.kloop(acc, 0, kt);
  else
    e.template kloop_deep<D>(acc, 0, kt);
  e.store(acc, a.y);
}

// ============================================================ stream-K grid

// The stream-K and whole-tile schedules keep loads two k-tiles ahead at 32 and
// 64 rows (grouped decode layer set: 54.7 -> 48.4 us at M = 17, 55.6 -> 50.5
// at M = 32, unchanged at 64) and one at 128 rows, whose registers are full.
template <int MB, int GS>
__device__ __forceinline__ void kloop_for(const TileEngine<GS, MB>& e, Acc<MB>& acc, int k0,
                                          int k1) {
  if constexpr (MB <= 4)
    e.template kloop_deep<2>(acc, k0, k1);
  else
    e.kloop(acc, k0, k1);
}

// Workgroup w of NW owns units [U*w/NW, U*(w+1)/NW) of U.
__device__ __forceinline__ long long lg_first_unit(int w, long long U, int NW) {
  return U * w / NW;
}
// Owner of unit u: the largest w with floor(U*w/NW) <= u.
__device__ __forceinline__ int lg_unit_owner(long long u, long long U, int NW) {
  return static_cast<int>(((u + 1) * NW - 1) / U);
}

// Cross-workgroup hand-off of a tile's parts, without device-wide fences (a
// device-scope fence writes back and invalidates the whole L2 of this chip):
//   writer: every wave stores its part with agent-scope atomic stores and
//           waits for them (vmcnt 0); after a workgroup barrier one lane
//           increments the tile's counter (agent-scope atomic).
//   reader: the workgroup whose increment completes the count reads every
//           part with agent-scope atomic loads, issued only after the
//           increment returned (its result is handed over through LDS).
// A part is stored register-major (float r of lane l at r * 64 + l of the
// wave's region), the layout every workgroup shares for a tile, so each
// store and load instruction covers 256 contiguous bytes.
// TILES (planned calls with many tiles): no stream-K split; logical
// workgroup w runs whole tiles w, w + NW, w + 2 NW, ... of the plan's tile
// sequence (problem by problem, row tiles of a column tile consecutive), so
// the row tiles that share a column tile's weights run at the same time on
// workgroups of one XCD and read those weights once through its L2. Needs no
// workspace; used when there are enough tiles to balance the workgroups.
template <int GS, int MB, bool TABLE, bool TILES>
__global__ __launch_bounds__(kLgThreads, 1) void large_streamk_kernel(const LargeSKArgs args) {
  using C = LgCfg<GS, MB>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lg_lds[];
  __shared__ int last_flag;
  // A planned call whose device plan is not the one the host launched from
  // does nothing (every workgroup takes the same exit, before any barrier).
  if constexpr (TABLE) {
    if (load_const(args.plan_checksum) != args.checksum) return;
  }
  const long long U = args.units;
  const int NW = args.nwg;
  const int wg = xcd_grouped(blockIdx.x, NW);
  const long long u0 = lg_first_unit(wg, U, NW);
  const long long u1 = lg_first_unit(wg + 1, U, NW);
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);

  // Descriptor of problem p: in the kernel arguments, or in the device table
  // of a planned call.
  auto prob_at = [&](int p) -> LargeProblem {
    {
      // field by field, as scalar loads from the table or the kernel
      // arguments (both read-only here)
      const LargeProblem* e = (TABLE ? args.table : args.prob) + p;
      LargeProblem r;
      r.x = load_const(&e->x);
      r.qw = load_const(&e->qw);
      r.sp = load_const(&e->sp);
      r.y = load_const(&e->y);
      r.N = load_const(&e->N);
      r.K = load_const(&e->K);
      r.G = load_const(&e->G);
      r.NCB = load_const(&e->NCB);
      r.MT = load_const(&e->MT);
      r.NT = load_const(&e->NT);
      r.KT = load_const(&e->KT);
      r.u_begin = load_const(&e->u_begin);
      r.t_begin = load_const(&e->t_begin);
      return r;
    }
  };
  // Problem of a unit of this workgroup's range (uniform): a forward scan
  // over the problems' first units, from problem 0 or, in a table, from the
  // problem holding the workgroup's first unit. One scalar load per step, so
  // no descriptor stays live in registers (an unrolled compare over all eight
  // kept them in SGPRs, which spilled 16 bytes per lane at 128-row tiles).
  auto problem_of = [&](long long u) {
    const auto* tab = TABLE ? args.table : args.prob;
    int p = TABLE ? load_const(args.wgfirst + wg) : 0;
    while (p + 1 < args.nprob && load_const(&tab[p + 1].u_begin) <= u) ++p;
    return p;
  };
  auto part_of = [&](int w, int slot) {
    return args.part + ((static_cast<size_t>(w) * 2 + slot) * kLgWaves + wave) * C::Regs * 64;
  };

  TileEngine<GS, MB> e;
  Acc<MB> acc;
  if constexpr (TILES) {
    // args.units counts tiles here; the problem index only moves forward
    const auto* tab = args.table;
    int p = 0;
    for (long long t = wg; t < U; t += NW) {
      while (p + 1 < args.nprob && load_const(&tab[p + 1].t_begin) <= t) p = uniform(p + 1);
      const LargeProblem pr = prob_at(p);
      const int tile = uniform(static_cast<int>(t - pr.t_begin));
      e.setup(lg_lds, pr.x, pr.qw, pr.sp, args.M, pr.N, pr.K, (tile % pr.MT) * C::Rows,
              tile / pr.MT);
      zero(acc);
      kloop_for<MB>(e, acc, 0, pr.KT);
      e.store(acc, pr.y);
    }
    return;
  }
  int fin_p[2] = {-1, -1}, fin_tile[2] = {0, 0};
  int nfin = 0;
  for (long long u = u0; u < u1;) {
    const int p = problem_of(u);
    const LargeProblem& pr = prob_at(p);
    const int v = uniform(static_cast<int>(u - pr.u_begin));
    const int tile = uniform(v / pr.KT);
    const int k0 = v - tile * pr.KT;
    const long long tile_u0 = pr.u_begin + static_cast<long long>(tile) * pr.KT;
    const long long seg_end = tile_u0 + pr.KT < u1 ? tile_u0 + pr.KT : u1;
    const int k1 = k0 + static_cast<int>(seg_end - u);
    e.setup(lg_lds, pr.x, pr.qw, pr.sp, args.M, pr.N, pr.K, (tile % pr.MT) * C::Rows,
            tile / pr.MT);
    zero(acc);
    kloop_for<MB>(e, acc, k0, k1);
    if (k0 == 0 && k1 == pr.KT) {
      e.store(acc, pr.y);
    } else {
      // publish this workgroup's part of the tile and count it
      const int slot = u0 >= tile_u0 ? 0 : 1;
      float* mine = part_of(wg, slot);
      const float* flat = reinterpret_cast<const float*>(&acc);
#pragma unroll
      for (int r = 0; r < C::Regs; ++r)
        __hip_atomic_store(mine + r * 64 + lane, flat[r], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      wait_vmem_all();  // this wave's part is complete
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();  // ... and so is every wave's
      if (tid == 0) {
        const int nseg =
            lg_unit_owner(tile_u0 + pr.KT - 1, U, NW) - lg_unit_owner(tile_u0, U, NW) + 1;
        const int old = __hip_atomic_fetch_add(args.counters + pr.t_begin + tile, 1,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = old == nseg - 1;
      }
      lds_barrier();
      if (last_flag) {
        fin_p[nfin] = p;
        fin_tile[nfin] = tile;
        ++nfin;
      }
      lds_barrier();  // the flag is read before it is rewritten
    }
    u = seg_end;
  }

  // Finalize the tiles whose last part arrived here: sum the parts in
  // workgroup order, store bf16, reset the counter for the next call.
  for (int i = 0; i < nfin; ++i) {
    const LargeProblem& pr = prob_at(fin_p[i]);
    const int tile = fin_tile[i];
    const long long tile_u0 = pr.u_begin + static_cast<long long>(tile) * pr.KT;
    const int wfirst = lg_unit_owner(tile_u0, U, NW);
    const int wlast = lg_unit_owner(tile_u0 + pr.KT - 1, U, NW);
    zero(acc);
    float* sum = reinterpret_cast<float*>(&acc);
    // B parts at a time (64 floats per lane), their loads all in flight together:
    // at 32 rows a tile cut among ten workgroups is summed in three round trips
    // instead of ten (one projection alone at M = 17: 28 -> 23 us). Past the
    // last part the loads re-read it and are not added; the parts are added in
    // workgroup order, one at a time, as before.
    constexpr int B = C::Regs >= 64 ? 1 : 64 / C::Regs;
    for (int w0 = wfirst; w0 <= wlast; w0 += B) {
      float v[B][C::Regs];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int w = w0 + b <= wlast ? w0 + b : wlast;
        const float* part = part_of(w, lg_first_unit(w, U, NW) >= tile_u0 ? 0 : 1);
#pragma unroll
        for (int r = 0; r < C::Regs; ++r)
          v[b][r] = __hip_atomic_load(part + r * 64 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (w0 + b > wlast) break;
#pragma unroll
        for (int r = 0; r < C::Regs; ++r) sum[r] += v[b][r];
      }
      // cleared once read (the sum above used every loaded value), so the call
      // leaves the whole workspace at zero and calls of every kind can share
      // it. The stores follow the sum, so every load has returned; nothing
      // reads the part again in this call, so plain stores of 16 bytes per
      // lane do (the wave's Regs x 64 floats in Regs / 4 instructions)
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (w0 + b > wlast) break;
        float* part = part_of(w0 + b, lg_first_unit(w0 + b, U, NW) >= tile_u0 ? 0 : 1);
#pragma unroll
        for (int j = 0; j < C::Regs / 4; ++j)
          __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u},
                                      reinterpret_cast<gptr<u32x4>>(to_global(part)) + j * 64 + lane);
      }
    }
    e.setup(lg_lds, pr.x, pr.qw, pr.sp, args.M, pr.N, pr.K, (tile % pr.MT) * C::Rows,
            tile / pr.MT);
    e.store(acc, pr.y);
    if (tid == 0)
      __hip_atomic_store(args.counters + pr.t_begin + tile, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ================================================================ launchers

template <int GS, int MB, int D>
hipError_t launch_tile_t(const GemmArgs& a, hipStream_t stream) {
  using C = LgCfg<GS, MB>;
  const int NCB = (a.N + 15) / 16;
  const int NT = (NCB + kLgBlocks - 1) / kLgBlocks;
  const void* fn = reinterpret_cast<const void*>(&tile_kernel<GS, MB, D>);
  const size_t lds = C::Lds;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  // Buffer offsets are 32-bit: each launch covers at most rows_per_launch rows
  // of x (and the packed weights must stay below 4 GB, checked by the caller).
  const long long row_bytes = 2LL * a.K;
  long long rows_per_launch = (0xFFFFFFFFLL - 16) / row_bytes;
  rows_per_launch -= rows_per_launch % C::Rows;
  if (rows_per_launch < C::Rows) return hipErrorInvalidValue;
  for (long long r0 = 0; r0 < a.M; r0 += rows_per_launch) {
    GemmArgs part = a;
    part.M = static_cast<int>(a.M - r0 < rows_per_launch ? a.M - r0 : rows_per_launch);
    part.x = a.x + r0 * a.K;
    part.y = a.y + r0 * a.N;
    int MT = (part.M + C::Rows - 1) / C::Rows;
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

// 32- and 64-row tiles keep loads three k-tiles ahead (at those tile counts a
// workgroup's k-tiles wait on load latency); 128-row tiles have the
// arithmetic to cover one.
template <int GS>
hipError_t launch_tile_g(const GemmArgs& a, int rows, hipStream_t stream) {
  switch (rows) {
    case 32: return launch_tile_t<GS, 2, 3>(a, stream);
    case 64: return launch_tile_t<GS, 4, 3>(a, stream);
    default: return launch_tile_t<GS, 8, 1>(a, stream);
  }
}

// Stream-K cost figures (one MI355X, decode layer-set projections launched
// alone and grouped): one k-tile of 128 per workgroup costs about 0.6, 0.75 and
// 2.2 us at 32, 64 and 128 rows, and the workgroup that finishes a cut tile
// reads each part (8 waves x 16, 32 or 64 floats per lane: 32, 64 or 128 KB)
// at about 55 GB/s.
double streamk_ktile_us(int rows) { return rows <= 32 ? 0.6 : (rows <= 64 ? 0.75 : 2.2); }
double streamk_part_us(int rows) { return 2048.0 * (rows / 16) * 8 / 55000.0; }

long long streamk_max_ways(int rows, int max_kt) {
  const double s = std::sqrt(static_cast<double>(max_kt) * streamk_ktile_us(rows) / streamk_part_us(rows));
  const long long w = static_cast<long long>(std::ceil(s));
  return w < 2 ? 2 : w;
}

// Units and tiles of the problems for tiles of `rows` rows (group GS): fills
// the problems' offsets and returns the unit count; *tiles_out is the tile
// count, *nwg_out the workgroups of the persistent grid.
long long plan_large_probs(LargeProblem* probs, int count, int M, int group, int rows,
                           long long* tiles_out, int* nwg_out) {
  const int T = kLgKT / group;  // groups per k-tile
  long long units = 0, tiles = 0;
  int max_kt = 1;
  for (int i = 0; i < count; ++i) {
    LargeProblem& p = probs[i];
    p.G = p.K / group;
    p.NCB = (p.N + 15) / 16;
    p.MT = (M + rows - 1) / rows;
    p.NT = (p.NCB + kLgBlocks - 1) / kLgBlocks;
    p.KT = (p.G + T - 1) / T;
    p.u_begin = units;
    p.t_begin = static_cast<int>(tiles);
    units += static_cast<long long>(p.MT) * p.NT * p.KT;
    tiles += static_cast<long long>(p.MT) * p.NT;
    if (p.KT > max_kt) max_kt = p.KT;
  }
  long long nwg = static_cast<long long>(device_cus());
  if (nwg > kLargeMaxWorkgroups) nwg = kLargeMaxWorkgroups;
  // A tile cut among S workgroups is summed by one of them, which reads the S
  // parts; beyond about sqrt(k-tiles x cost per k-tile / time per part) ways
  // that read costs more than the split saves. A launch of few, deep tiles
  // (one 64-column problem with K = 65536 has one tile of 512 k-tiles) would
  // otherwise cut each tile among every workgroup.
  const long long cap = tiles * streamk_max_ways(rows, max_kt);
  if (nwg > cap) nwg = cap;
  if (nwg > units) nwg = units;  // every workgroup owns at least one unit
  *tiles_out = tiles;
  *nwg_out = static_cast<int>(nwg);
  return units;
}

template <int GS, int MB, bool TABLE = false, bool TILES = false>
hipError_t launch_large_sk_t(LargeSKArgs& sk, hipStream_t stream) {
  using C = LgCfg<GS, MB>;
  if constexpr (!TABLE) {
    long long tiles = 0;
    sk.units = plan_large_probs(sk.prob, sk.nprob, sk.M, GS, C::Rows, &tiles, &sk.nwg);
  }
  const void* fn = reinterpret_cast<const void*>(&large_streamk_kernel<GS, MB, TABLE, TILES>);
  const size_t lds = C::Lds;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  void* kargs[] = {&sk};
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(sk.nwg)), dim3(kLgThreads), kargs, lds,
                         stream);
}

template <int MB, bool TABLE = false, bool TILES = false>
hipError_t launch_large_sk_g(LargeSKArgs& sk, int group, hipStream_t stream) {
  switch (group) {
    case 32: return launch_large_sk_t<32, MB, TABLE, TILES>(sk, stream);
    case 64: return launch_large_sk_t<64, MB, TABLE, TILES>(sk, stream);
    case 128: return launch_large_sk_t<128, MB, TABLE, TILES>(sk, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool large_supported(int group) { return group == 32 || group == 64 || group == 128; }

bool large_runs(int N, int K, int group) {
  const long long qbytes = static_cast<long long>((N + 15) / 16) * 16 * K / 2;
  return large_supported(group) && qbytes <= 0xFFFFFFF0LL;
}

// Whole-K tile forms, per k-tile of 128 (microseconds, one MI355X, decode
// layer set and its tensor-parallel shard at M = 17 to 512): one workgroup of
// 32, 64 or 128 rows per compute unit takes 0.75, 1.08 or 1.9; a second round
// of workgroups costs as much again, except at 32 rows, where two workgroups
// share a compute unit and n rounds cost about 0.8 n.
double tile_estimate_us(int M, int N, int K, int group, int* rows_out) {
  const long long NT = ((static_cast<long long>(N) + 15) / 16 + kLgBlocks - 1) / kLgBlocks;
  const long long G = K / group;
  const long long T = kLgKT / group;
  const double kt = static_cast<double>((G + T - 1) / T);
  const int rows_opt[3] = {32, 64, 128};
  const double per_ktile[3] = {0.75, 1.08, 1.9};
  double best = 0.0;
  int best_rows = 128;
  for (int i = 0; i < 3; ++i) {
    const long long tiles = (static_cast<long long>(M) + rows_opt[i] - 1) / rows_opt[i] * NT;
    const long long n = (tiles + kModelCUs - 1) / kModelCUs;
    const double rounds = i == 0 && n > 1 ? 0.8 * static_cast<double>(n) : static_cast<double>(n);
    const double est = kt * per_ktile[i] * rounds + 1.0;
    if (i == 0 || est < best) {
      best = est;
      best_rows = rows_opt[i];
    }
  }
  if (rows_out) *rows_out = best_rows;
  return best;
}

hipError_t launch_large(const GemmArgs& a, hipStream_t stream) {
  // packed weights and scales are addressed with 32-bit buffer offsets
  if (!large_runs(a.N, a.K, a.group)) return launch_skinny(a, stream);
  int rows = 128;
  tile_estimate_us(a.M, a.N, a.K, a.group, &rows);
  switch (a.group) {
    case 32: return launch_tile_g<32>(a, rows, stream);
    case 64: return launch_tile_g<64>(a, rows, stream);
    default: return launch_tile_g<128>(a, rows, stream);
  }
}

// Tile height of the stream-K schedules: the fewest row tiles times the cost
// of one k-tile at that height (0.75, 1.08 and 1.9 us for 32, 64 and 128 rows,
// the whole-K tile forms' figures), a lower tile only when it saves more than
// 3 %. 32 rows up to 32, 64 up to 64, then 128 except at 129-192 and 257-320
// rows, where 64-row tiles waste fewer rows: grouped decode layer set 174.5 ->
// 155.8 us at M = 160, 179.5 -> 162.2 at 192, 258.9 -> 253.0 at 320.
int large_streamk_rows(int M) {
  const int rows[3] = {128, 64, 32};
  const double per_ktile[3] = {1.9, 1.08, 0.75};
  int best = 128;
  double best_cost = 0.0;
  for (int i = 0; i < 3; ++i) {
    const double cost = static_cast<double>((M + rows[i] - 1) / rows[i]) * per_ktile[i];
    if (i == 0 || cost < 0.97 * best_cost) {
      best_cost = cost;
      best = rows[i];
    }
  }
  return best;
}

size_t large_streamk_counter_bytes(int M, long long total_columns) {
  const long long rows = large_streamk_rows(M);
  const long long mt = (static_cast<long long>(M) + rows - 1) / rows;
  const long long ints = mt * (kMaxProblems + (total_columns + 255) / 256);
  return static_cast<size_t>((ints * 4 + 255) / 256 * 256);
}

size_t large_streamk_part_bytes(int M) {
  const int regs = large_streamk_rows(M) / 16 * kLgNB * 4;
  return static_cast<size_t>(kLargeMaxWorkgroups) * 2 * kLgWaves * regs * 64 * sizeof(float);
}

// One problem above 16 rows: whether the kernels of w4a16_gemm (whole K per
// workgroup, no workspace) are expected to beat the stream-K schedule. The
// stream-K time: a workgroup's k-tiles at their cost, the finisher's reads of
// the parts of a cut tile, and about 15 us of launch, first loads and hand-off;
// it must win by 10 % to be chosen. On the decode layer set's projections
// alone it wins only for down (17408 x 5120) from M = 256 (1024 rows: 217
// against 241 us); at M = 64 every projection is about twice as fast whole
// (qkv 15.5 against 33.8 us).
bool single_prefers_whole_k(int M, int N, int K, int group) {
  if (M <= 16 || !large_supported(group)) return false;
  const int rows = large_streamk_rows(M);
  LargeProblem p = {};
  p.N = N;
  p.K = K;
  long long tiles = 0;
  int nwg = 0;
  const long long units = plan_large_probs(&p, 1, M, group, rows, &tiles, &nwg);
  if (nwg < 1) return true;
  const double u = static_cast<double>(units) / nwg;
  const double kt = static_cast<double>(p.KT);
  double ways = u < kt ? std::ceil(kt / u) + 1.0 : 2.0;
  if (ways > nwg) ways = nwg;
  const double sk = u * streamk_ktile_us(rows) + ways * streamk_part_us(rows) + 15.0;
  double whole = tile_estimate_us(M, N, K, group, nullptr);
  if (M <= kPlainMaxRows) {
    const double plain = plain_estimate_us(M, N, K, group);
    if (plain < whole) whole = plain;
  }
  return !(sk < 0.9 * whole);
}

bool large_streamk_fits(const StreamKProblem* probs, int count, int M, int group) {
  if (!large_supported(group)) return false;
  for (int i = 0; i < count; ++i) {
    const long long xbytes = 2LL * M * probs[i].K;
    const long long qbytes = static_cast<long long>((probs[i].N + 15) / 16) * 16 * probs[i].K / 2;
    if (xbytes > 0xFFFFFFF0LL || qbytes > 0xFFFFFFF0LL) return false;
  }
  return true;
}

hipError_t launch_large_streamk(const StreamKProblem* probs, int count, int M, int group,
                                float* part, int* counters, hipStream_t stream) {
  if (count < 1 || count > kMaxProblems || M < 1) return hipErrorInvalidValue;
  LargeSKArgs sk = {};
  for (int i = 0; i < count; ++i) {
    sk.prob[i].x = probs[i].x;
    sk.prob[i].qw = probs[i].qw;
    sk.prob[i].sp = probs[i].sp;
    sk.prob[i].y = probs[i].y;
    sk.prob[i].N = probs[i].N;
    sk.prob[i].K = probs[i].K;
  }
  sk.nprob = count;
  sk.M = M;
  sk.part = part;
  sk.counters = counters;
  switch (large_streamk_rows(M)) {
    case 32: return launch_large_sk_g<2>(sk, group, stream);
    case 64: return launch_large_sk_g<4>(sk, group, stream);
    default: return launch_large_sk_g<8>(sk, group, stream);
  }
}

int build_large_plan(LargeProblem* probs, int count, int M, int group, PlanHeader& h,
                     int* wgfirst) {
  if (!large_supported(group)) return -1;
  const int rows = large_streamk_rows(M);
  long long tiles = 0;
  int nwg = 0;
  const long long units = plan_large_probs(probs, count, M, group, rows, &tiles, &nwg);
  if (nwg < 1 || nwg > kPlanMaxWorkgroups) return -1;
  h.kind = kPlanKindLarge;
  h.rows = rows;
  h.grid = nwg;
  h.nwaves = nwg;
  h.units = units;
  // Enough tiles (at least kPlanTilesPerWorkgroup per workgroup): whole tiles
  // round robin, no workspace. The grid never exceeds the tile count.
  if (tiles >= static_cast<long long>(kPlanTilesPerWorkgroup) * nwg) {
    h.tiles = 1;
    h.units = tiles;
    for (int w = 0; w < nwg; ++w) wgfirst[w] = 0;  // unused in this form
    h.counters_off = h.slots_off = h.part_off = 0;
    h.workspace_bytes = 0;
    return 0;
  }
  h.tiles = 0;
  h.lds_bytes = 0;  // fixed by the kernel's group size and tile rows
  // logical workgroup w's first unit is units * w / nwg
  int p = 0;
  for (int w = 0; w < nwg; ++w) {
    const long long u = units * w / nwg;
    while (p + 1 < count && probs[p + 1].u_begin <= u) ++p;
    wgfirst[w] = p;
  }
  h.counters_off = 0;
  h.slots_off = 0;
  h.part_off = (tiles * 4 + 255) / 256 * 256;
  h.workspace_bytes = h.part_off + static_cast<long long>(large_streamk_part_bytes(M));
  return 0;
}

hipError_t launch_large_planned(const PlanHeader& h, const unsigned char* plan_dev, char* ws,
                                hipStream_t stream) {
  LargeSKArgs sk = {};
  sk.table = reinterpret_cast<const LargeProblem*>(plan_dev + h.table_off);
  sk.wgfirst = reinterpret_cast<const int*>(plan_dev + h.wgfirst_off);
  sk.plan_checksum =
      reinterpret_cast<const unsigned long long*>(plan_dev + offsetof(PlanHeader, checksum));
  sk.checksum = h.checksum;
  sk.nprob = h.count;
  sk.M = h.M;
  sk.units = h.units;
  sk.nwg = h.grid;
  sk.part = reinterpret_cast<float*>(ws + h.part_off);
  sk.counters = reinterpret_cast<int*>(ws + h.counters_off);
  if (h.tiles) {
    switch (h.rows) {
      case 32: return launch_large_sk_g<2, true, true>(sk, h.group, stream);
      case 64: return launch_large_sk_g<4, true, true>(sk, h.group, stream);
      default: return launch_large_sk_g<8, true, true>(sk, h.group, stream);
    }
  }
  switch (h.rows) {
    case 32: return launch_large_sk_g<2, true>(sk, h.group, stream);
    case 64: return launch_large_sk_g<4, true>(sk, h.group, stream);
    default: return launch_large_sk_g<8, true>(sk, h.group, stream);
  }
}

}  // namespace w4a16_internal
