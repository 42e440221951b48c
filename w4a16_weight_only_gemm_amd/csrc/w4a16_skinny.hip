// w4a16_skinny.hip -- the streaming kernel for small M (decode and
// speculative-verify blocks) behind the workspace entry points and planned
// calls.
//
// At small M the GEMM is bound by the weight stream: every packed weight is
// read from HBM exactly once and shared by all M rows (ai.satyajit.si page,
// section "One weight read, shared by every stream"). The inner step:
//
//  * A unit is one tile of the packed format: 16 output columns x one group
//    (1 KB of packed weights at group 128), stored contiguously in the order
//    lane l of a wavefront needs it: its words are exactly its B operands for
//    the group's MFMA steps (lane l serves column l % 16 and k-slice l / 16 of
//    every step). A wave therefore loads a unit with one contiguous vector load
//    and feeds it HBM -> VGPR -> dequant -> MFMA without LDS.
//  * Dequantization is to the exact biased value 24 + q in bf16 (two VALU
//    ops per bf16 pair); the bias is removed through the accumulator start
//    (-24 times the group's row sums, or an MFMA chain against a constant -24
//    operand), so the MFMA sees exact codes, products are exact and the fp32
//    accumulator holds sum(x * q) over the group. The group's partial is then
//    scaled by its fp16 scale and added to the running fp32 result.
//  * Rows are padded to 16: padded rows repeat row M-1 and are never stored
//    (an MFMA output row depends only on its own A row).
//
// streamk_kernel: a persistent grid of long-lived waves splits the linear
//   sequence of units (problem, column block, group) -- contiguous in memory --
//   evenly, so every wave streams one long contiguous run of weights. Column
//   blocks cut between waves are combined through a caller-provided workspace
//   in a fixed order, so the result does not depend on timing (see the
//   hand-off below). Several problems (the four projections of a layer, or a
//   whole planned step) share one launch.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/w4a16.h"
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16_internal {

template <int WPL>
struct Words {
  uint32_t w[WPL];
};

// One unit's packed words for this lane (WPL consecutive words), non-temporal:
// every weight byte is read once.
template <int WPL>
__device__ __forceinline__ void load_words_g(Words<WPL>& out, gptr<const uint32_t> p) {
  if constexpr (WPL == 1) {
    out.w[0] = __builtin_nontemporal_load(p);
  } else if constexpr (WPL == 2) {
    u32x2 v = __builtin_nontemporal_load(reinterpret_cast<gptr<const u32x2>>(p));
    out.w[0] = v[0];
    out.w[1] = v[1];
  } else {
#pragma unroll
    for (int h = 0; h < WPL / 4; ++h) {
      u32x4 v = __builtin_nontemporal_load(reinterpret_cast<gptr<const u32x4>>(p) + h);
      out.w[4 * h + 0] = v[0];
      out.w[4 * h + 1] = v[1];
      out.w[4 * h + 2] = v[2];
      out.w[4 * h + 3] = v[3];
    }
  }
}

// ============================================================= stream-K kernel

// Wave w of NW owns units [U*w/NW, U*(w+1)/NW) of U.
__device__ __forceinline__ long long wave_first_unit(int w, long long U, int NW) {
  return U * w / NW;
}

// Owner of unit u: the largest w with floor(U*w/NW) <= u.
__device__ __forceinline__ int unit_owner(long long u, long long U, int NW) {
  return static_cast<int>(((u + 1) * NW - 1) / U);
}

// Hand-off of the super-blocks that stream-K cuts, in two levels, both after
// the stream, so that no wave waits on memory while it streams:
//  1. inside the workgroup: a wave keeps its part of a super-block cut at the
//     start or end of its run in LDS (slot 0 for the first super-block of its
//     run, 1 for the last); after the stream, one barrier, and the first wave
//     of the workgroup that overlaps such a super-block sums the parts of the
//     workgroup's waves in wave order;
//  2. across workgroups, for a super-block that extends past the workgroup's
//     units, one part per workgroup:
//     a. shared by exactly two workgroups (the usual case: a workgroup's run
//        is longer than a super-block): each swaps its part into the
//        super-block's slots in the workspace with one atomic exchange per
//        value; per value, the exchange that returns the other part finishes
//        it (see swap_part). One memory round trip.
//     b. shared by three or more: published through the workspace and counted
//        by an atomic counter per super-block; the workgroup whose increment
//        completes the count sums the parts in workgroup order.
// The summation order is fixed (two addends sum the same in either order), so
// the result does not depend on timing. Level 2 uses no device-wide fences (on
// this chip a device-scope fence writes back and invalidates the whole L2,
// which costs more than the GEMM itself). Every access that crosses
// workgroups is an agent-scope atomic, coherent across the L2s of all XCDs.
// In 2b:
//   writer: atomic stores of the part; wait until they complete (vmcnt 0);
//           atomic increment of the super-block's counter.
//   reader: the wave whose increment completes the count reads every part
//           with atomic loads, issued only after the increment returned.
// The writer's stores are complete, hence visible device-wide, before its
// increment is issued; the reader's loads depend on its increment's result
// and so happen after it. Compiler barriers keep the generated order.

// Index of this lane's value (column block j, row m, column c16) in a part of
// NBW x Mr x 16 floats. Rows at or past Mr are padding rows, computed from a
// repeat of row M - 1 and so equal to row Mr - 1: they map there (same value),
// which keeps every part access unconditional.
template <int NBW>
__device__ __forceinline__ int part_index(int j, int m, int c16, int Mr) {
  return (j * Mr + min(m, Mr - 1)) * 16 + c16;
}

// Store the bf16 results of super-block sb (rows 4*lg + r of column c16 of
// each of its NBW column blocks).
template <int NBW>
__device__ __forceinline__ void store_block(const StreamKProblem& pr, int sb, const float (&v)[NBW][4],
                                            int lg, int c16, int M) {
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int n = (sb * NBW + j) * 16 + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * lg + r;
      if (m < M && n < pr.N) to_global(pr.y)[static_cast<size_t>(m) * pr.N + n] = f32_to_bf16_bits(v[j][r]);
    }
  }
}

// Workgroup of the wave that owns unit u.
template <int WAVES>
__device__ __forceinline__ int unit_wg(long long u, long long U, int NW) {
  return unit_owner(u, U, NW) / WAVES;
}

// A part value as stored in a swap slot: its bit pattern XOR a signalling-NaN
// pattern. Arithmetic never yields a signalling NaN, so a stored value is
// never 0, and 0 marks an empty slot.
constexpr uint32_t kSlotMask = 0x7FA5A5A5u;

// Level 2a: finish super-block sb (shared by exactly two workgroups) with
// this workgroup's part v. The slots of the super-block hold 0 between calls.
// For each value, the two workgroups' exchanges are ordered by the atomic:
// the first gets 0 back and is done; the second gets the first's part, adds
// its own (the sum of two addends does not depend on their order), stores
// the bf16 result and empties the slot. Rows at or past Mr are padding: their
// lanes take no part.
template <int NBW>
__device__ __forceinline__ void swap_part(const StreamKArgs& args, const StreamKProblem& pr, int sb,
                                          int lg, int c16, int M, int Mr, const float (&v)[NBW][4]) {
  uint32_t* slots = args.slots + static_cast<size_t>(pr.sb_begin + sb) * NBW * Mr * 16;
  uint32_t old[NBW][4];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      old[j][r] = 0;
      const int m = 4 * lg + r;
      if (m < Mr)
        old[j][r] = __hip_atomic_exchange(slots + (j * Mr + m) * 16 + c16,
                                          __builtin_bit_cast(uint32_t, v[j][r]) ^ kSlotMask,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int n = (sb * NBW + j) * 16 + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * lg + r;
      if (old[j][r] != 0) {
        const float sum = v[j][r] + __builtin_bit_cast(float, old[j][r] ^ kSlotMask);
        if (m < M && n < pr.N) to_global(pr.y)[static_cast<size_t>(m) * pr.N + n] = f32_to_bf16_bits(sum);
        __hip_atomic_store(slots + (j * Mr + m) * 16 + c16, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// Level 2b, writer: publish workgroup b's part v of super-block sb in its
// slot (0 for the super-block holding the workgroup's first unit, 1 for the
// one holding its last) and count it; nseg workgroups share the super-block.
// Returns true when it was the last part to arrive; the caller then finalizes
// the super-block.
template <int NBW>
__device__ __forceinline__ bool publish_wg_part(const StreamKArgs& args, const StreamKProblem& pr,
                                                int b, int slot, int nseg, int sb, int lane, int lg,
                                                int c16, int Mr, const float (&v)[NBW][4]) {
  float* mine = args.part + (static_cast<size_t>(b) * 2 + slot) * NBW * Mr * 16;
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      __hip_atomic_store(mine + part_index<NBW>(j, 4 * lg + r, c16, Mr), v[j][r], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_vmem_all();  // the part is complete before it is counted
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  int old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_add(args.counters + pr.sb_begin + sb, 1, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  const bool last = uniform(__shfl(old, 0)) == nseg - 1;
  wait_vmem_all();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return last;
}

// Level 2b, reader: sum the parts of workgroups bfirst..blast of super-block
// sb (workgroup c's in slot slot_of(c)) in workgroup order, store the bf16
// results and reset the super-block's counter for the next call.
template <int NBW, typename SlotOf>
__device__ __forceinline__ void finalize_block(const StreamKArgs& args, const StreamKProblem& pr,
                                               int bfirst, int blast, SlotOf slot_of, int sb,
                                               int lane, int lg, int c16, int M, int Mr) {
  float sum[NBW][4];
#pragma unroll
  for (int j = 0; j < NBW; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) sum[j][r] = 0.f;
  // Two parts at a time, so their loads are all in flight together; the sum
  // runs in workgroup order. Each part is cleared once read, so that the call
  // leaves the whole workspace at zero (calls of every kind can then share it).
  auto load_part = [&](float (&v)[NBW][4], int c) {
    float* part = args.part + (static_cast<size_t>(c) * 2 + slot_of(c)) * NBW * Mr * 16;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        v[j][r] = __hip_atomic_load(part + part_index<NBW>(j, 4 * lg + r, c16, Mr), __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  auto clear_part = [&](int c) {
    float* part = args.part + (static_cast<size_t>(c) * 2 + slot_of(c)) * NBW * Mr * 16;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __hip_atomic_store(part + part_index<NBW>(j, 4 * lg + r, c16, Mr), 0.f, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  int c = bfirst;
  for (; c + 1 <= blast; c += 2) {
    float v0[NBW][4], v1[NBW][4];
    load_part(v0, c);
    load_part(v1, c + 1);
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) sum[j][r] = (sum[j][r] + v0[j][r]) + v1[j][r];
  }
  if (c <= blast) {
    float v0[NBW][4];
    load_part(v0, c);
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) sum[j][r] += v0[j][r];
  }
  store_block<NBW>(pr, sb, sum, lg, c16, M);
  // the loads above have returned (their values were summed), so the parts
  // can be overwritten now
  for (c = bfirst; c <= blast; ++c) clear_part(c);
  if (lane == 0)
    __hip_atomic_store(args.counters + pr.sb_begin + sb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Level 2 for a super-block that extends past workgroup b's part of the
// sequence: workgroups bfirst..blast share it; slot_of(c) is workgroup c's slot.
template <int NBW, typename SlotOf>
__device__ __forceinline__ void hand_off_across(const StreamKArgs& args, const StreamKProblem& pr,
                                                int b, int bfirst, int blast, SlotOf slot_of, int sb,
                                                int lane, int lg, int c16, int M, int Mr,
                                                const float (&v)[NBW][4]) {
  if (blast - bfirst == 1) {
    swap_part<NBW>(args, pr, sb, lg, c16, M, Mr, v);  // level 2a
  } else if (publish_wg_part<NBW>(args, pr, b, slot_of(b), blast - bfirst + 1, sb, lane, lg, c16, Mr,
                                  v)) {
    finalize_block<NBW>(args, pr, bfirst, blast, slot_of, sb, lane, lg, c16, M, Mr);  // level 2b
  }
}

// Loads of one unit for one lane: for each of its NBW column blocks the packed
// words and the 32-bit word holding this lane's column scale (with its
// neighbour column's, so the load is 32-bit: 16-bit loads would be packed two
// to a register and tie their waits together) and, without staged
// activations, its A-operand activations (shared by the NBW blocks).
template <int WPL, int NBW>
struct UnitLoads {
  Words<WPL> w[NBW];
  uint32_t s2[NBW];
  u32x4 x[WPL];
};

// With staged activations (one column block per unit) the kernel runs two
// 8-wave workgroups per compute unit, i.e. four waves per SIMD: at most 128
// VGPRs (the table form would otherwise take a few more).
template <int GS, int WAVES, int P, bool XLDS, int NBW, bool TABLE>
__global__ __launch_bounds__(64 * WAVES, (XLDS && GS <= 128) ? 4 : 1) void streamk_kernel(
    const StreamKArgs args) {
  constexpr int WPL = GS / 32;
  // A planned call whose device plan is not the one the host launched from
  // does nothing (every wave of the grid takes the same exit).
  if constexpr (TABLE) {
    if (load_const(args.plan_checksum) != args.checksum) return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int lg = lane >> 4;
  const int M = args.M;
  const int Mr = min(M, 16);
  const long long U = args.units;
  const int NW = args.nwaves;
  const int wg = blockIdx.x * WAVES + wave;  // waves wg >= NW of the last workgroup own nothing
  const long long u0 = wg < NW ? wave_first_unit(wg, U, NW) : U;
  const long long u1 = wg < NW ? wave_first_unit(wg + 1, U, NW) : U;

  // Descriptor of problem p: in the kernel arguments, or in the device table
  // of a planned call.
  auto prob_at = [&](int p) -> StreamKProblem {
    {
      // field by field, as scalar loads from the table or the kernel
      // arguments (both read-only here)
      const StreamKProblem* e = (TABLE ? args.table : args.prob) + p;
      StreamKProblem r;
      r.x = load_const(&e->x);
      r.qw = load_const(&e->qw);
      r.sp = load_const(&e->sp);
      r.y = load_const(&e->y);
      r.N = load_const(&e->N);
      r.K = load_const(&e->K);
      r.G = load_const(&e->G);
      r.NCB = load_const(&e->NCB);
      r.NSB = load_const(&e->NSB);
      r.u_begin = load_const(&e->u_begin);
      r.sb_begin = load_const(&e->sb_begin);
      return r;
    }
  };
  // Problem of a global unit of this workgroup's range (wave-uniform): a
  // forward scan over the problems' first units, from problem 0 or, in a
  // table, from the problem holding the workgroup's first unit. The scan reads
  // one field per step as a scalar load, so no descriptor stays live in
  // registers (an unrolled compare over all eight made the compiler keep
  // them in SGPRs and spill).
  auto problem_of = [&](long long u) {
    const auto* tab = TABLE ? args.table : args.prob;
    int p = TABLE ? load_const(args.wgfirst + blockIdx.x) : 0;
    while (p + 1 < args.nprob && load_const(&tab[p + 1].u_begin) <= u) ++p;
    return p;
  };

  // ---- per-problem stream state of the wave's current sub-run ----
  struct Run {
    int p, v0, v1, G, NCB;         // problem, its units [v0, v1), groups, column blocks
    gptr<const uint16_t> xrow;     // activations of this lane's A row
    gptr<const uint32_t> wbase;    // this lane's words of tile 0
    gptr<const uint32_t> sbase;    // this lane's scale pair of tile 0
  };
  auto make_run = [&](long long u) {
    Run r;
    r.p = problem_of(u);
    const StreamKProblem& pr = prob_at(r.p);
    const long long pend = pr.u_begin + static_cast<long long>(pr.NSB) * pr.G;
    r.v0 = uniform(static_cast<int>(u - pr.u_begin));
    r.v1 = uniform(static_cast<int>((u1 < pend ? u1 : pend) - pr.u_begin));
    r.G = uniform(pr.G);
    r.NCB = uniform(pr.NCB);
    r.xrow = to_global(pr.x) + static_cast<size_t>(min(c16, M - 1)) * pr.K + lg * WPL * 8;
    r.wbase = to_global(pr.qw) + lane * WPL;
    r.sbase = reinterpret_cast<gptr<const uint32_t>>(to_global(pr.sp) + (c16 & ~1));
    return r;
  };
  // Loads of unit v of the run (clamped to its last unit: loads past it re-read
  // that unit, cache hits never used, so every load is unconditional). Unit v
  // is group v % G of super-block v / G; with NBW = 1 it is tile v itself.
  auto load_unit = [&](UnitLoads<WPL, NBW>& d, const Run& r, int v) {
    v = min(v, r.v1 - 1);
    const int sb = NBW == 1 ? 0 : uniform(v / r.G);
    const int g = NBW == 1 ? 0 : v - sb * r.G;
    if constexpr (!XLDS) {
      const int gx = NBW == 1 ? v % r.G : g;
#pragma unroll
      for (int t = 0; t < WPL; ++t)
        d.x[t] = *reinterpret_cast<gptr<const u32x4>>(r.xrow + static_cast<size_t>(gx) * GS + 8 * t);
    }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      // tile of column block sb*NBW + j (blocks past the last re-read it)
      const size_t tile = NBW == 1 ? static_cast<size_t>(v)
                                   : static_cast<size_t>(min(sb * NBW + j, r.NCB - 1)) * r.G + g;
      load_words_g<WPL>(d.w[j], r.wbase + tile * 64 * WPL);
      d.s2[j] = r.sbase[tile * 8];
    }
  };

  UnitLoads<WPL, NBW> bufA[P], bufB[P];
  Run run;
  const bool active = u1 > u0;
  if (active) {
    // The first chunk's weights go out before the activation staging below,
    // so the two latencies overlap.
    run = make_run(u0);
#pragma unroll
    for (int i = 0; i < P; ++i) load_unit(bufA[i], run, run.v0 + i);
  }

  // Activations for the A operand. With XLDS the workgroup stages the x rows
  // (min(M,16) rows) of every problem its units touch into LDS once;
  // otherwise each lane reads them from global memory.
  extern __shared__ __attribute__((aligned(16))) uint32_t xlds[];  // 16-byte aligned: read as 128-bit words
  int lds_base[kMaxProblems];
  int lds_stride[kMaxProblems];
#pragma unroll
  for (int i = 0; i < kMaxProblems; ++i) {
    lds_base[i] = 0;
    lds_stride[i] = 0;
  }
  // Per-problem LDS offsets are indexed by p - plo, plo the workgroup's first
  // problem (at most kMaxProblems problems per workgroup, checked on the host).
  int plo = 0;
  // With XLDS, LDS also holds per problem and group the bias term -24 *
  // (sum of the group's activations) of each row, as [G][SS] fp32 after the
  // activation rows: an MFMA chain started from it sums a * q with the codes'
  // bias already removed. SS = 16 holds rows 0..15 (rows past Mr repeat row
  // Mr - 1); with at most 4 rows SS = 8: rows 0..3, then row Mr - 1 four
  // times, which lanes of rows 4..15 (all padding) read.
  const int SS = streamk_sum_stride(M);
  int xs_base[kMaxProblems];
#pragma unroll
  for (int i = 0; i < kMaxProblems; ++i) xs_base[i] = 0;
  float* const xsum = reinterpret_cast<float*>(xlds);
  if constexpr (XLDS) {
    const long long wu0 = wave_first_unit(blockIdx.x * WAVES, U, NW);
    const long long wu1 = wave_first_unit(min((blockIdx.x + 1) * WAVES, NW), U, NW);
    if (wu1 > wu0) {
      plo = problem_of(wu0);
      const int phi = problem_of(wu1 - 1);
      int off = 0;  // in bf16 elements
#pragma unroll
      for (int j = 0; j < kMaxProblems; ++j) {
        if (plo + j <= phi) {
          lds_base[j] = off;
          lds_stride[j] = prob_at(plo + j).K + 8;  // 16 bytes of padding per row against bank conflicts
          off += Mr * lds_stride[j];
        }
      }
      int xoff = off / 2;  // in 4-byte words; a multiple of 4
#pragma unroll
      for (int j = 0; j < kMaxProblems; ++j) {
        if (plo + j <= phi) {
          xs_base[j] = xoff;
          xoff += prob_at(plo + j).G * SS;
        }
      }
#pragma unroll
      for (int j = 0; j < kMaxProblems; ++j) {
        if (plo + j <= phi) {
          const int i = j;  // slot of problem plo + j in the LDS offset arrays
          const StreamKProblem& pr = prob_at(plo + j);
          constexpr int LPG = GS / 8;  // 16-byte pieces per group
          const int chunks = pr.K / 8;
          // Mr * chunks is a multiple of LPG and each pass starts at a
          // multiple of 64: a group's pieces are in consecutive lanes of one
          // pass, all active together.
          for (int e = threadIdx.x; e < Mr * chunks; e += 64 * WAVES) {
            const int row = e / chunks, c8 = e - row * chunks;
            const u32x4 d =
                *reinterpret_cast<gptr<const u32x4>>(to_global(pr.x) + static_cast<size_t>(row) * pr.K + 8 * c8);
            *reinterpret_cast<u32x4*>(xlds + (lds_base[i] + row * lds_stride[i] + 8 * c8) / 2) = d;
            const float bsum = group_lane_sum<LPG>(neg_bias_sum8(d));  // the group's first lane stores
            if ((c8 % LPG) == 0) {
              float* dst = xsum + xs_base[i] + (c8 / LPG) * SS;
              dst[row] = bsum;
              if (row == Mr - 1)
                for (int m = Mr; m < SS; ++m) dst[m] = bsum;
            }
          }
        }
      }
    }
    lds_barrier();  // LDS only: the weight loads already in flight keep flying
  }
  // This wave's LDS parts: [2 slots][NBW][Mr][16] fp32 (level 1 of the hand-off).
  float* const lparts = reinterpret_cast<float*>(xlds + args.lds_part_off);
  float* const mylds = lparts + wave * 2 * NBW * Mr * 16;

  if (active) {
    const bf16x8 bias = bias_operand();
    f32x4 yacc[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) yacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The wave's run, one problem at a time. Within a problem consecutive units
    // are consecutive groups of a super-block, so the cursors are plain offsets.
    for (bool first = true;; first = false) {
      if (!first) {
#pragma unroll
        for (int i = 0; i < P; ++i) load_unit(bufA[i], run, run.v0 + i);
      }
      const StreamKProblem& pr = prob_at(run.p);
      const int G = run.G;
      const int rp = run.p - plo;  // slot of the problem in the LDS offset arrays (with XLDS)
      const int xbase = XLDS ? (lds_base[rp] + min(c16, M - 1) * lds_stride[rp] + lg * WPL * 8) / 2 : 0;
      // with XLDS: this lane's rows of group 0
      const float* const xs = xsum + xs_base[rp] + 4 * (SS == 16 ? lg : min(lg, 1));
      int sb = uniform(run.v0 / G);
      int g = uniform(run.v0 - sb * G);
      int seg_g0 = g;  // first group of the current super-block segment

      // Compute the units of one chunk (buf holds units v .. v+P-1). Units
      // past the run's end (clamped re-loads of its last unit) are computed
      // too, with their contribution scaled by zero: every path then consumes
      // every loaded register, so no load can still be pending when the
      // buffer is reloaded, and the compiler's waits stay exact (a skipped
      // unit would make it drain all loads before each reload).
      auto compute_chunk = [&](UnitLoads<WPL, NBW> (&buf)[P], int v) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
          const int vv = v + i;
          const bool live = vv < run.v1;
          {
            bf16x8 a[WPL];
            if constexpr (XLDS) {
              const uint32_t* xl = xlds + xbase + (g * GS) / 2;
#pragma unroll
              for (int t = 0; t < WPL; ++t)
                a[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xl + 4 * t));
            } else {
#pragma unroll
              for (int t = 0; t < WPL; ++t) a[t] = act_frag(buf[i].x[t]);
            }
            if constexpr (NBW == 1) {
              // from -24 * (row sums): sum of a * q (exact products)
              f32x4 acc = *reinterpret_cast<const f32x4*>(xs + g * SS);
#pragma unroll
              for (int t = 0; t < WPL; ++t) acc = mfma16(a[t], dequant_biased(buf[i].w[0].w[t]), acc);
              const float sc =
                  live ? fp16_bits_to_f32(static_cast<uint16_t>(buf[i].s2[0] >> (16 * (c16 & 1)))) : 0.f;
#pragma unroll
              for (int r = 0; r < 4; ++r) yacc[0][r] = __builtin_fmaf(sc, acc[r], yacc[0][r]);
            } else {
              // -24 * (row sums of the group) once, as the start of every block's sum
              f32x4 accb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int t = 0; t < WPL; ++t) accb = mfma16(a[t], bias, accb);
#pragma unroll
              for (int j = 0; j < NBW; ++j) {
                f32x4 acc = accb;
#pragma unroll
                for (int t = 0; t < WPL; ++t) acc = mfma16(a[t], dequant_biased(buf[i].w[j].w[t]), acc);
                const float sc =
                    live ? fp16_bits_to_f32(static_cast<uint16_t>(buf[i].s2[j] >> (16 * (c16 & 1)))) : 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) yacc[j][r] = __builtin_fmaf(sc, acc[r], yacc[j][r]);
              }
            }

            if (live && (g == G - 1 || vv == run.v1 - 1)) {
              // End of this wave's segment of super-block sb.
              if (seg_g0 == 0 && g == G - 1) {
                // The whole super-block was ours: store the results. The wait
                // keeps the compiler's later load waits exact (see wait_vmem_all).
                float out[NBW][4];
#pragma unroll
                for (int j = 0; j < NBW; ++j)
#pragma unroll
                  for (int r = 0; r < 4; ++r) out[j][r] = yacc[j][r];
                store_block<NBW>(pr, sb, out, lg, c16, M);
                wait_vmem_all();
              } else {
                // Cut: keep the part in LDS (slot 0 for the first super-block
                // of the run, 1 for the last) until the stream has ended.
                const long long usb0 = pr.u_begin + static_cast<long long>(sb) * G;
                float* mine = mylds + (u0 >= usb0 ? 0 : NBW * Mr * 16);
#pragma unroll
                for (int j = 0; j < NBW; ++j)
#pragma unroll
                  for (int r = 0; r < 4; ++r) mine[part_index<NBW>(j, 4 * lg + r, c16, Mr)] = yacc[j][r];
              }
#pragma unroll
              for (int j = 0; j < NBW; ++j) yacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
              seg_g0 = 0;
            }
            if (live && ++g == G) {
              g = 0;
              ++sb;
            }
          }
        }
      };

      // Double-buffered chunks: the next chunk's loads are issued before the
      // current chunk is computed, so P to 2P units stay in flight. The
      // compiled loop routes the early exit through its header, so the exit
      // waits for the unused loads in flight: otherwise the header would have
      // to drain every load before each reload.
      for (int v = run.v0; v < run.v1; v += 2 * P) {
#pragma unroll
        for (int i = 0; i < P; ++i) load_unit(bufB[i], run, v + P + i);
        compute_chunk(bufA, v);
        if (v + P >= run.v1) {
          wait_vmem_all();
          break;
        }
#pragma unroll
        for (int i = 0; i < P; ++i) load_unit(bufA[i], run, v + 2 * P + i);
        compute_chunk(bufB, v + P);
      }

      const long long next = prob_at(run.p).u_begin + run.v1;
      if (next >= u1) break;
      run = make_run(next);
    }
  }

  // ---- hand-off of the cut super-blocks (after every wave's stream) ----
  lds_barrier();  // every wave's LDS parts are in place
  if (!active) return;
  const int b = blockIdx.x;
  const long long W0 = wave_first_unit(b * WAVES, U, NW);
  const long long W1 = wave_first_unit(min((b + 1) * WAVES, NW), U, NW);
  // A wave leads the cut super-blocks that it is the workgroup's first wave
  // to overlap: the one holding its first unit (unless an earlier wave of the
  // workgroup overlaps it too) and the one holding its last unit.
  for (int k = 0; k < 2; ++k) {
    const long long u = k == 0 ? u0 : u1 - 1;
    const int p = problem_of(u);
    const StreamKProblem& pr = prob_at(p);
    const int G = uniform(pr.G);
    const int sb = uniform(static_cast<int>((u - pr.u_begin) / G));
    const long long s0 = pr.u_begin + static_cast<long long>(sb) * G;
    const long long s1 = s0 + G;
    if (k == 1 && s0 <= u0) break;             // the run's last super-block is its first
    if (k == 0 && s0 < u0 && wave > 0) continue;  // led by an earlier wave of the workgroup
    if (s0 >= u0 && s1 <= u1) continue;        // whole: stored during the stream
    // Level 1: the parts of this workgroup's waves, in wave order.
    float sum[NBW][4];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) sum[j][r] = 0.f;
    const int vlast = unit_owner((s1 < W1 ? s1 : W1) - 1, U, NW);
    for (int v = wg; v <= vlast; ++v) {
      const float* part = lparts + ((v - b * WAVES) * 2 + (wave_first_unit(v, U, NW) >= s0 ? 0 : 1)) *
                                       NBW * Mr * 16;
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) sum[j][r] += part[part_index<NBW>(j, 4 * lg + r, c16, Mr)];
    }
    if (s0 >= W0 && s1 <= W1) {
      store_block<NBW>(pr, sb, sum, lg, c16, M);  // the workgroup owns it whole
    } else {
      // a workgroup's slot: 0 when the super-block holds its first unit
      auto slot_of = [&](int c) { return wave_first_unit(c * WAVES, U, NW) >= s0 ? 0 : 1; };
      hand_off_across<NBW>(args, pr, b, unit_wg<WAVES>(s0, U, NW), unit_wg<WAVES>(s1 - 1, U, NW),
                           slot_of, sb, lane, lg, c16, M, Mr, sum);
    }
  }
}

// =============================================================== launchers

namespace {

#ifndef W4A16_STREAMK_PREFETCH
#define W4A16_STREAMK_PREFETCH 4
#endif
#ifndef W4A16_STREAMK_WG_PER_CU
#define W4A16_STREAMK_WG_PER_CU 2
#endif

#ifndef W4A16_STREAMK_WIDE_PREFETCH
#define W4A16_STREAMK_WIDE_PREFETCH 1
#endif
#ifndef W4A16_STREAMK_WIDE_WG_PER_CU
#define W4A16_STREAMK_WIDE_WG_PER_CU 1
#endif

// Units in flight per wave: a wide unit carries NBW weight tiles, so fewer of
// them keep the same bytes in flight within the register budget.
template <int NBW>
constexpr int streamk_prefetch() {
  return NBW == 1 ? W4A16_STREAMK_PREFETCH : W4A16_STREAMK_WIDE_PREFETCH;
}

template <int GS, bool XLDS, int NBW, bool TABLE>
hipError_t launch_streamk_t(const StreamKArgs& sk, int wgs, size_t lds, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(
      &streamk_kernel<GS, kStreamKWaves, streamk_prefetch<NBW>(), XLDS, NBW, TABLE>);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  StreamKArgs copy = sk;
  void* kargs[] = {&copy};
  return hipLaunchKernel(fn, dim3(wgs), dim3(64 * kStreamKWaves), kargs, lds, stream);
}

// Activations staged in LDS: one column block per unit. Read by each wave:
// streamk_wide_blocks(group) column blocks per unit.
template <bool XLDS, bool TABLE = false>
hipError_t launch_streamk_x(const StreamKArgs& sk, int group, int wgs, size_t lds, hipStream_t s) {
  switch (group) {
    case 32: return launch_streamk_t<32, XLDS, XLDS ? 1 : streamk_wide_blocks(32), TABLE>(sk, wgs, lds, s);
    case 64: return launch_streamk_t<64, XLDS, XLDS ? 1 : streamk_wide_blocks(64), TABLE>(sk, wgs, lds, s);
    case 128: return launch_streamk_t<128, XLDS, XLDS ? 1 : streamk_wide_blocks(128), TABLE>(sk, wgs, lds, s);
    case 256: return launch_streamk_t<256, XLDS, XLDS ? 1 : streamk_wide_blocks(256), TABLE>(sk, wgs, lds, s);
    default: return hipErrorInvalidValue;
  }
}

// LDS for the waves' parts of cut super-blocks: [waves][2][nbw][min(M,16)][16] fp32.
size_t streamk_lds_part_bytes(int M, int nbw) {
  return static_cast<size_t>(kStreamKWaves) * 2 * nbw * (M < 16 ? M : 16) * 16 * sizeof(float);
}

// Units of the problems with NBW column blocks per super-block, and the grid:
// fills the problems' offsets, *units and *nwaves and returns the workgroup
// count; *sbs is the total number of super-blocks.
int plan_streamk_probs(StreamKProblem* probs, int count, int nbw, long long* units_out,
                       int* nwaves_out, long long* sbs_out) {
  long long units = 0, sbs = 0;
  for (int i = 0; i < count; ++i) {
    StreamKProblem& p = probs[i];
    p.NSB = (p.NCB + nbw - 1) / nbw;
    p.u_begin = units;
    p.sb_begin = static_cast<int>(sbs);
    units += static_cast<long long>(p.NSB) * p.G;
    sbs += p.NSB;
  }
  int wgs = device_cus() * (nbw == 1 ? W4A16_STREAMK_WG_PER_CU : W4A16_STREAMK_WIDE_WG_PER_CU);
  const int max_waves = nbw == 1 ? kStreamKMaxWaves : kStreamKWideMaxWaves;
  if (wgs * kStreamKWaves > max_waves) wgs = max_waves / kStreamKWaves;
  // Every counted wave must own at least one unit (NW <= units): the parts of
  // a super-block are then produced by consecutive non-empty waves.
  long long nw = static_cast<long long>(wgs) * kStreamKWaves;
  if (nw > units) nw = units;
  *units_out = units;
  *nwaves_out = static_cast<int>(nw);
  if (sbs_out) *sbs_out = sbs;
  return static_cast<int>((nw + kStreamKWaves - 1) / kStreamKWaves);
}

int plan_streamk(StreamKArgs& sk, int nbw) {
  return plan_streamk_probs(sk.prob, sk.nprob, nbw, &sk.units, &sk.nwaves, nullptr);
}

// The most LDS any workgroup needs for staged activations (Mr rows of K + 8
// bf16 and G x 16 fp32 group sums of every problem its units touch), and the
// most problems one workgroup touches.
void streamk_lds_need(const StreamKProblem* probs, int count, int M, long long units, long long nw,
                      int wgs, long long* need_out, int* touch_out) {
  const int Mr = M < 16 ? M : 16;
  long long need = 0;
  int touch = 0;
  int p = 0;  // first problem overlapping the current workgroup (ranges increase with b)
  for (int b = 0; b < wgs; ++b) {
    const long long wb0 = static_cast<long long>(b) * kStreamKWaves;
    const long long wb1 = wb0 + kStreamKWaves < nw ? wb0 + kStreamKWaves : nw;
    const long long wu0 = units * wb0 / nw;
    const long long wu1 = units * wb1 / nw;
    if (wu1 <= wu0) continue;
    while (p + 1 < count && probs[p + 1].u_begin <= wu0) ++p;
    long long bytes = 0;
    int n = 0;
    for (int i = p; i < count && probs[i].u_begin < wu1; ++i) {
      bytes += static_cast<long long>(Mr) * (probs[i].K + 8) * 2 +
               static_cast<long long>(probs[i].G) * streamk_sum_stride(M) * 4;
      ++n;
    }
    if (bytes > need) need = bytes;
    if (n > touch) touch = n;
  }
  *need_out = need;
  *touch_out = touch;
}

}  // namespace

// Compute units of the current device (cached per device).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

hipError_t launch_streamk(const StreamKProblem* probs, int count, int M, int group, float* part,
                          uint32_t* slots, int* counters, hipStream_t stream) {
  if (count < 1 || count > kMaxProblems || M < 1 || M > 16) return hipErrorInvalidValue;
  StreamKArgs sk = {};
  for (int i = 0; i < count; ++i) {
    StreamKProblem p = probs[i];
    p.G = p.K / group;
    p.NCB = (p.N + 15) / 16;
    sk.prob[i] = p;
  }
  sk.nprob = count;
  sk.M = M;
  sk.part = part;
  sk.slots = slots;
  sk.counters = counters;
  // LDS for staged activations (one column block per unit): the most any
  // workgroup needs (Mr rows of K + 8 and G x 16 group sums of each problem
  // its units touch). Beyond the budget, each wave reads activations itself
  // and takes streamk_wide_blocks(group) column blocks per unit instead.
  int wgs = plan_streamk(sk, 1);
  long long need = 0;
  int touch = 0;
  streamk_lds_need(sk.prob, count, M, sk.units, sk.nwaves, wgs, &need, &touch);
  // The waves' parts (level 1 of the hand-off) follow the staged activations.
  const size_t x_bytes = (static_cast<size_t>(need) + 15) / 16 * 16;
  const size_t lds = x_bytes + streamk_lds_part_bytes(M, 1);
  if (lds <= kStreamKLdsBudget) {
    sk.lds_part_off = static_cast<int>(x_bytes / 4);
    return launch_streamk_x<true>(sk, group, wgs, lds, stream);
  }
  const int nbw = streamk_wide_blocks(group);
  wgs = plan_streamk(sk, nbw);
  sk.lds_part_off = 0;
  return launch_streamk_x<false>(sk, group, wgs, streamk_lds_part_bytes(M, nbw), stream);
}

// Stream-K plan of validated problems (N, K, pointers set): fills the
// problems' offsets, the header's launch and workspace fields and the first
// problem of every workgroup.
int build_streamk_plan(StreamKProblem* probs, int count, int M, int group, PlanHeader& h,
                       int* wgfirst) {
  for (int i = 0; i < count; ++i) {
    probs[i].G = probs[i].K / group;
    probs[i].NCB = (probs[i].N + 15) / 16;
  }
  long long units = 0, sbs = 0;
  int nw = 0;
  int wgs = plan_streamk_probs(probs, count, 1, &units, &nw, &sbs);
  long long need = 0;
  int touch = 0;
  streamk_lds_need(probs, count, M, units, nw, wgs, &need, &touch);
  const size_t x_bytes = (static_cast<size_t>(need) + 15) / 16 * 16;
  const size_t lds = x_bytes + streamk_lds_part_bytes(M, 1);
  int nbw = 1;
  if (lds <= kStreamKLdsBudget && touch <= kMaxProblems) {
    h.xlds = 1;
    h.lds_part_off = static_cast<int>(x_bytes / 4);
    h.lds_bytes = static_cast<int>(lds);
  } else {
    nbw = streamk_wide_blocks(group);
    wgs = plan_streamk_probs(probs, count, nbw, &units, &nw, &sbs);
    h.xlds = 0;
    h.lds_part_off = 0;
    h.lds_bytes = static_cast<int>(streamk_lds_part_bytes(M, nbw));
  }
  if (wgs < 1 || wgs > kPlanMaxWorkgroups) return -1;
  h.kind = kPlanKindStreamK;
  h.nbw = nbw;
  h.grid = wgs;
  h.nwaves = nw;
  h.units = units;
  // workgroup b's first unit is that of its first wave, units * 8b / nw
  int p = 0;
  for (int b = 0; b < wgs; ++b) {
    const long long u = units * (static_cast<long long>(b) * kStreamKWaves) / nw;
    while (p + 1 < count && probs[p + 1].u_begin <= u) ++p;
    wgfirst[b] = p;
  }
  const int Mr = M < 16 ? M : 16;
  const long long counter_bytes = (sbs * 4 + 255) / 256 * 256;
  const long long slot_bytes = (sbs * nbw * Mr * 16 * 4 + 255) / 256 * 256;
  h.counters_off = 0;
  h.slots_off = counter_bytes;
  h.part_off = counter_bytes + slot_bytes;
  h.workspace_bytes = h.part_off + static_cast<long long>(streamk_part_bytes(M));
  return 0;
}

hipError_t launch_streamk_planned(const PlanHeader& h, const unsigned char* plan_dev, char* ws,
                                  hipStream_t stream) {
  StreamKArgs sk = {};
  sk.table = reinterpret_cast<const StreamKProblem*>(plan_dev + h.table_off);
  sk.wgfirst = reinterpret_cast<const int*>(plan_dev + h.wgfirst_off);
  sk.plan_checksum =
      reinterpret_cast<const unsigned long long*>(plan_dev + offsetof(PlanHeader, checksum));
  sk.checksum = h.checksum;
  sk.nprob = h.count;
  sk.M = h.M;
  sk.units = h.units;
  sk.nwaves = h.nwaves;
  sk.part = reinterpret_cast<float*>(ws + h.part_off);
  sk.slots = reinterpret_cast<uint32_t*>(ws + h.slots_off);
  sk.counters = reinterpret_cast<int*>(ws + h.counters_off);
  sk.lds_part_off = h.lds_part_off;
  return h.xlds ? launch_streamk_x<true, true>(sk, h.group, h.grid, h.lds_bytes, stream)
                : launch_streamk_x<false, true>(sk, h.group, h.grid, h.lds_bytes, stream);
}

// w4a16_gemm's M-dispatch: up to 16 rows the small-M forms of plain_kernel;
// above, whichever of the two families the time models put first (the tile
// engine needs enough 256-column tiles to fill the compute units: on the
// decode layer set gate_up from 33 rows, qkv from 160, o and down from 224;
// a narrow projection such as the tensor-parallel shard's qkv 5120x896 stays
// on plain_kernel at 1024 rows, 22 against 30 us). Beyond 65535 row tiles of
// 16 (the grid's second dimension) only the tile engine runs.
int choose_path(int M, int N, int K, int group) {
  if (M > kPlainMaxRows) return W4A16_PATH_LARGE;
  if (M <= 16 || !large_supported(group)) return W4A16_PATH_SKINNY;
  return tile_estimate_us(M, N, K, group, nullptr) < plain_estimate_us(M, N, K, group)
             ? W4A16_PATH_LARGE
             : W4A16_PATH_SKINNY;
}

int describe_form(int M, int N, int K, int group, int path, int* rows, int* cols, int* waves) {
  if (path == W4A16_PATH_AUTO || M > kPlainMaxRows) path = choose_path(M, N, K, group);
  if (path == W4A16_PATH_LARGE && large_runs(N, K, group)) {
    tile_estimate_us(M, N, K, group, rows);
    *cols = 256;
    *waves = 8;
    return W4A16_PATH_LARGE;
  }
  if (M > kPlainMaxRows) return -1;  // no kernel takes that many rows of this shape
  plain_form_shape(plain_form(M, N, K, group), rows, cols, waves);
  return W4A16_PATH_SKINNY;
}

}  // namespace w4a16_internal
