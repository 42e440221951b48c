// w4a8.hip -- the W4A8 variant: int8 activations with one scale per row,
// 4-bit weights, int8 MFMA.
//
// Past the bend where the rows' arithmetic overtakes the weight stream, the
// only way to a higher rate is cheaper arithmetic (ai.satyajit.si page,
// section "What one more stream costs on this model"); the int8 path of
// gfx950 (v_mfma_i32_16x16x64_i8) does twice the multiply-adds per cycle of
// the bf16 one. Two kernels:
//
//  * w4a8_quantize_kernel: one workgroup per activation row. Pass 1 finds
//    a = max |x| (as the integer maximum of the bf16 magnitude bits, which
//    orders finite values exactly); pass 2 forms t = x * (127 / a) in fp32,
//    rounds to the nearest integer (ties to even, v_rndne), clamps to
//    [-127, 127] and stores the codes; the row scale is a / 127. Codes are
//    stored row-major, each aligned block of 16 k in the order in which one
//    MFMA step consumes the weight codes of two packed words:
//    0,4,1,5,2,6,3,7, 8,12,9,13,10,14,11,15.
//
//  * w4a8_gemm_kernel: one workgroup per 128 x 256 output tile (8 waves), or
//    128 x 128 (4 waves, two workgroups per CU) for M <= 256, where the wider
//    tiles leave compute units idle; tiles in XCD-grouped order. K advances
//    in k-tiles of 128: the workgroup stages the 128 x 128-byte code tile in
//    LDS (double-buffered, 16-byte pieces XOR-swizzled by row). The waves sit
//    side by side along N, each owning a 128 x 32 sub-tile: 8 x 2 blocks of
//    16 x 16, so every weight operand feeds eight MFMAs and no two waves load
//    or convert the same weights. Loads run
//    two k-tiles ahead of the math (three rotating weight register sets, two
//    staging sets). A packed 4-bit code moved into the high nibble of a byte
//    (low nibble zero) is the signed byte 16 q, so a packed word becomes two
//    int8 operand registers with one and (odd nibbles, in place) and one
//    shift and and (even nibbles): the int32 MFMA sums are 16 times the exact
//    sums of products, with no offset to remove. At the end of a group the
//    int32 sum is converted to fp32 and multiplied by the group's fp16 scale
//    times 1/16 (exact), then added to the fp32 result; the epilogue
//    multiplies by the row scale and rounds to bf16.
//
// Group sizes 64 and 128 (a k-tile holds two or one whole groups; a group
// fills whole 64-deep MFMA steps in every lane group). Rows beyond M read as
// zero (buffer range) and are not stored; column blocks beyond N are clamped
// on load and not stored.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "w4a16_device.h"
#include "w4a8_launch.h"

namespace w4a16_internal {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ quantization

constexpr int kQThreads = 256;

// Maximum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t u = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o));
    v = u > v ? u : v;
  }
  return v;
}

// Code of one value: nearest integer of x * inv (ties to even), clamped.
__device__ __forceinline__ uint32_t code_byte(uint32_t bf16_bits, float inv) {
  const float x = __builtin_bit_cast(float, bf16_bits << 16);
  float r = __builtin_rintf(x * inv);
  r = r > 127.f ? 127.f : r;
  r = r < -127.f ? -127.f : r;
  return static_cast<uint32_t>(static_cast<int>(r)) & 0xFFu;
}

__global__ __launch_bounds__(kQThreads) void w4a8_quantize_kernel(const W4A8QuantBatch bt) {
  const int p = uniform(static_cast<int>(blockIdx.x) / bt.M);
  const W4A8QuantProblem& pr = bt.prob[p];
  const uint16_t* x = pr.x;
  uint32_t* xq = reinterpret_cast<uint32_t*>(pr.xq);
  float* sx = pr.sx;
  const int K = pr.K;
  __shared__ uint32_t wmax[kQThreads / 64];
  const int m = static_cast<int>(blockIdx.x) - p * bt.M;
  const int tid = threadIdx.x;
  const int nblk = K / 16;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(m) * K);
  // pass 1: the largest magnitude, as bf16 bits without the sign
  uint32_t amax = 0;
  for (int i = tid; i < nblk; i += kQThreads) {
    const u32x4 lo = xr[2 * i], hi = xr[2 * i + 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a0 = lo[j] & 0x7FFF7FFFu, a1 = hi[j] & 0x7FFF7FFFu;
      const uint32_t l0 = a0 & 0xFFFFu, h0 = a0 >> 16, l1 = a1 & 0xFFFFu, h1 = a1 >> 16;
      const uint32_t m0 = l0 > h0 ? l0 : h0, m1 = l1 > h1 ? l1 : h1;
      const uint32_t mm = m0 > m1 ? m0 : m1;
      amax = mm > amax ? mm : amax;
    }
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = wmax[0];
#pragma unroll
  for (int w = 1; w < kQThreads / 64; ++w) amax = wmax[w] > amax ? wmax[w] : amax;
  const float a = __builtin_bit_cast(float, amax << 16);
  const float inv = a > 0.f ? 127.f / a : 0.f;
  if (tid == 0) sx[m] = a / 127.f;
  // pass 2: codes of each block of 16, stored in MFMA step order
  u32x4* out = reinterpret_cast<u32x4*>(xq) + static_cast<size_t>(m) * nblk;
  for (int i = tid; i < nblk; i += kQThreads) {
    const u32x4 lo = xr[2 * i], hi = xr[2 * i + 1];
    uint32_t c[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[2 * j] = code_byte(lo[j] & 0xFFFFu, inv);
      c[2 * j + 1] = code_byte(lo[j] >> 16, inv);
      c[8 + 2 * j] = code_byte(hi[j] & 0xFFFFu, inv);
      c[8 + 2 * j + 1] = code_byte(hi[j] >> 16, inv);
    }
    // byte p of each half holds offset 0,4,1,5,2,6,3,7 of that half
    u32x4 o;
    o[0] = c[0] | (c[4] << 8) | (c[1] << 16) | (c[5] << 24);
    o[1] = c[2] | (c[6] << 8) | (c[3] << 16) | (c[7] << 24);
    o[2] = c[8] | (c[12] << 8) | (c[9] << 16) | (c[13] << 24);
    o[3] = c[10] | (c[14] << 8) | (c[11] << 16) | (c[15] << 24);
    out[i] = o;
  }
}

// -------------------------------------------------------------------- GEMM

constexpr int kQ8KT = 128;       // k per k-tile (bytes of a row's codes)
constexpr int kQ8Pieces = kQ8KT / 16;

// Tile geometry: WAVES = WM x WN waves, each MB x NB blocks of 16 x 16.
template <int GS, int WAVES, int WM, int MB, int NB>
struct Q8Cfg {
  static_assert(GS == 64 || GS == 128, "group 64 or 128");
  static_assert(WAVES % WM == 0, "whole wave rows");
  static constexpr int Threads = 64 * WAVES;
  static constexpr int WN = WAVES / WM;
  static constexpr int Rows = WM * MB * 16;
  static constexpr int Blocks = WN * NB;                  // 16-column blocks per tile
  static constexpr int Loads = Rows * kQ8Pieces / Threads;
  static_assert(Loads >= 1 && Rows * kQ8Pieces % Threads == 0, "whole staging passes");
  static constexpr int RowStep = Threads / kQ8Pieces;  // rows staged per pass
  static constexpr int T = kQ8KT / GS;                    // groups per k-tile
  static constexpr int WPL = GS / 32;                     // words per lane per group
  static constexpr int Steps = GS / 64;                   // MFMA steps per group
  static constexpr int ABytes = Rows * kQ8KT;
  static constexpr size_t Lds = 2 * static_cast<size_t>(ABytes);
};

// LDS slot of 16-byte piece p of a row: p ^ (r & 7) ^ ((r >> 3) & 1), r the
// row mod 16. For a fixed p, rows 0..7 (and 8..15) take eight distinct slots,
// and so do the eight even (odd) rows of a 16-row block, so the staging
// writes (eight rows) and the fragment reads (sixteen rows, two 128-byte rows
// per 256-byte line of banks) are free of bank conflicts.
__device__ __forceinline__ int q8_slot(int piece, int row) {
  return piece ^ (row & 7) ^ ((row >> 3) & 1);
}

// The codes of two packed words as one int8 operand, each byte 16 q: a 4-bit
// two's-complement code moved into the high nibble of a byte, low nibble
// zero, is the signed byte 16 q. Bytes in the order even nibbles of w0
// (shifted up), odd nibbles of w0 (in place), then the same for w1.
__device__ __forceinline__ i32x4 dequant_i8x16(uint32_t w0, uint32_t w1) {
  i32x4 r;
  r[0] = static_cast<int>((w0 << 4) & 0xF0F0F0F0u);
  r[1] = static_cast<int>(w0 & 0xF0F0F0F0u);
  r[2] = static_cast<int>((w1 << 4) & 0xF0F0F0F0u);
  r[3] = static_cast<int>(w1 & 0xF0F0F0F0u);
  return r;
}

__device__ __forceinline__ i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

template <int GS, int WAVES, int WM, int MB, int NB>
struct Q8Stage {
  u32x4 d[Q8Cfg<GS, WAVES, WM, MB, NB>::Loads];
};

template <int NB>
struct Q8B {
  uint32_t w[NB][kQ8KT / 32];  // 4 words per block per k-tile
  uint32_t s[NB][2];           // scale pairs (fp16 x 2) per group (T <= 2)
};

template <int MB, int NB>
struct Q8Acc {
  f32x4 v[MB][NB];
};

template <int GS, int WAVES, int WM, int MB, int NB>
struct Q8Engine {
  using C = Q8Cfg<GS, WAVES, WM, MB, NB>;
  unsigned char* lds;
  int tid, lane, wave, wm, wn;
  int M, N, K, G, NCB, m0, nt;
  const uint8_t* xrow0;
  uint32_t xbytes;
  __amdgpu_buffer_rsrc_t rq, rs;
  int blk[NB];

  __device__ __forceinline__ void setup(unsigned char* lds_, const W4A8Args& a, int m0_,
                                        int nt_) {
    lds = lds_;
    tid = threadIdx.x;
    lane = tid & 63;
    wave = uniform(tid >> 6);
    wm = wave % WM;
    wn = wave / WM;
    M = a.M;
    N = a.N;
    K = a.K;
    G = K / GS;
    NCB = (N + 15) / 16;
    m0 = m0_;
    nt = nt_;
    xbytes = static_cast<uint32_t>(M - m0) * static_cast<uint32_t>(K);
    xrow0 = a.xq + static_cast<size_t>(m0) * K;
    rq = make_rsrc(a.qweight, static_cast<uint32_t>(NCB) * 16u * static_cast<uint32_t>(K) / 2u);
    rs = make_rsrc(a.scales, static_cast<uint32_t>(NCB) * 16u * static_cast<uint32_t>(G) * 2u);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = nt * C::Blocks + wn * NB + nb;
      blk[nb] = b < NCB ? b : NCB - 1;
    }
  }

  // Thread stages piece tid % 8 of rows tid / 8 + 64 i, through a buffer
  // resource based at (row m0, k-tile t) that ends at the end of xq.
  __device__ __forceinline__ void stage_load(Q8Stage<GS, WAVES, WM, MB, NB>& r, int t) const {
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(xrow0 + t * kQ8KT, xbytes - static_cast<uint32_t>(t) * kQ8KT);
    const int spiece = tid % kQ8Pieces, srow0 = tid / kQ8Pieces;
#pragma unroll
    for (int i = 0; i < C::Loads; ++i) {
      const uint32_t voff = static_cast<uint32_t>(srow0 + i * C::RowStep) * K + spiece * 16;
      r.d[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, voff, 0, 0);
    }
  }
  __device__ __forceinline__ void stage_store(const Q8Stage<GS, WAVES, WM, MB, NB>& r, int buf) const {
    unsigned char* base = lds + buf * C::ABytes;
    const int spiece = tid % kQ8Pieces, srow0 = tid / kQ8Pieces;
#pragma unroll
    for (int i = 0; i < C::Loads; ++i) {
      const int row = srow0 + i * C::RowStep;
      *reinterpret_cast<u32x4*>(base + row * kQ8KT + q8_slot(spiece, row) * 16) = r.d[i];
    }
  }

  // This wave's weight words and scales of k-tile t.
  __device__ __forceinline__ void load_b(Q8B<NB>& r, int t) const {
    const uint32_t qlane = static_cast<uint32_t>(lane) * C::WPL * 4u;
    const uint32_t slane = static_cast<uint32_t>(lane & 14) * 2u;
#pragma unroll
    for (int gi = 0; gi < C::T; ++gi) {
      int grp = t * C::T + gi;
      if (grp > G - 1) grp = G - 1;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t tile_idx = static_cast<uint32_t>(blk[nb]) * G + grp;
        const int qoff = static_cast<int>(tile_idx * (64u * C::WPL * 4u));
        if constexpr (C::WPL == 4) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rq, qlane, qoff, 0);
#pragma unroll
          for (int w = 0; w < 4; ++w) r.w[nb][w] = v[w];
        } else {
          const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rq, qlane, qoff, 0);
          r.w[nb][gi * 2 + 0] = v[0];
          r.w[nb][gi * 2 + 1] = v[1];
        }
        r.s[nb][gi] =
            __builtin_amdgcn_raw_buffer_load_b32(rs, slane, static_cast<int>(tile_idx * 32u), 0);
      }
    }
  }

  // One k-tile: for each group, Steps MFMA steps of 64 k per 16 x 16 block
  // (one column block at a time, its MB row blocks side by side), then the
  // block's scaled add into acc_out. The integer sums are 16 times the
  // products of codes; the 1/16 goes into the scale.
  __device__ __forceinline__ void compute(Q8Acc<MB, NB>& acc_out, const Q8B<NB>& b, int t,
                                          int buf) const {
    const unsigned char* base = lds + buf * C::ABytes;
    const int arow = lane & 15, lg = lane >> 4;
    const int shalf = (lane & 1) * 16;
    const int rbase = wm * MB * 16;
#pragma unroll
    for (int gi = 0; gi < C::T; ++gi) {
      if (C::T > 1 && t * C::T + gi >= G) break;  // ragged last k-tile (uniform)
      i32x4 af[C::Steps][MB];
#pragma unroll
      for (int s = 0; s < C::Steps; ++s) {
        const int piece = gi * (GS / 16) + lg * (GS / 64) + s;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int row = rbase + mb * 16 + arow;
          af[s][mb] =
              *reinterpret_cast<const i32x4*>(base + row * kQ8KT + q8_slot(piece, arow) * 16);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        i32x4 acc[MB];
#pragma unroll
        for (int s = 0; s < C::Steps; ++s) {
          const int w0 = gi * C::WPL + 2 * s;
          const i32x4 bq = dequant_i8x16(b.w[nb][w0], b.w[nb][w0 + 1]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[mb] = mfma_i8(af[s][mb], bq, s == 0 ? i32x4{0, 0, 0, 0} : acc[mb]);
        }
        const float sc =
            fp16_bits_to_f32(static_cast<uint16_t>(b.s[nb][gi] >> shalf)) * 0.0625f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc_out.v[mb][nb][r] += sc * static_cast<float>(acc[mb][r]);
      }
    }
  }

  // k-tiles [0, kt), two k-tiles ahead: while k-tile t computes from LDS
  // buffer t & 1, the codes and weights of k-tile t + 2 are loaded into
  // registers and the codes of k-tile t + 1 (loaded one iteration earlier)
  // are staged into the other buffer; one workgroup barrier per k-tile.
  // Three weight sets and two staging sets rotate through six unrolled
  // iterations (no register copies). Loads past the last k-tile repeat it.
  __device__ __forceinline__ void kloop(Q8Acc<MB, NB>& acc, int kt) const {
    Q8Stage<GS, WAVES, WM, MB, NB> sa, sb;
    Q8B<NB> b0, b1, b2;
    const int t1 = kt > 1 ? 1 : 0;
    stage_load(sa, 0);
    load_b(b0, 0);
    stage_load(sb, t1);
    load_b(b1, t1);
    stage_store(sa, 0);
    lds_barrier();
    // s_next holds k-tile t + 1; s_next2 and nxt2 receive k-tile t + 2
    auto iter = [&](int t, const Q8B<NB>& cur, Q8B<NB>& nxt2, const Q8Stage<GS, WAVES, WM, MB, NB>& s_next,
                    Q8Stage<GS, WAVES, WM, MB, NB>& s_next2) {
      const int t2 = t + 2 < kt ? t + 2 : kt - 1;
      stage_load(s_next2, t2);
      load_b(nxt2, t2);
      __builtin_amdgcn_sched_barrier(0);  // issue the loads before the math
      compute(acc, cur, t, t & 1);
      stage_store(s_next, (t + 1) & 1);
      lds_barrier();
    };
    // A single exit, at the top: an iteration past the last k-tile is
    // skipped rather than left through a break (exits from the middle of the
    // unrolled body make the compiler copy the accumulators at every exit).
    for (int t = 0; t < kt; t += 6) {
      iter(t, b0, b2, sb, sa);
      if (t + 1 < kt) iter(t + 1, b1, b0, sa, sb);
      if (t + 2 < kt) iter(t + 2, b2, b1, sb, sa);
      if (t + 3 < kt) iter(t + 3, b0, b2, sa, sb);
      if (t + 4 < kt) iter(t + 4, b1, b0, sb, sa);
      if (t + 5 < kt) iter(t + 5, b2, b1, sa, sb);
    }
  }

  // y = acc * sx[row], rounded to bf16, for the rows and columns that exist.
  __device__ __forceinline__ void store(const Q8Acc<MB, NB>& acc, const float* sx,
                                        uint16_t* y) const {
    gptr<uint16_t> yg = to_global(y);
    const gptr<const float> sxg = to_global(sx);
    const int lg = lane >> 4;
    float rs[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + (wm * MB + mb) * 16 + 4 * lg + r;
        rs[mb][r] = row < M ? sxg[row] : 0.f;
      }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = (nt * C::Blocks + wn * NB + nb) * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + (wm * MB + mb) * 16 + 4 * lg + r;
          if (row < M)
            yg[static_cast<size_t>(row) * N + col] = f32_to_bf16_bits(acc.v[mb][nb][r] * rs[mb][r]);
        }
      }
    }
  }
};

// Workgroups of problem p are blocks [begin[p], begin[p] + tiles[p]) of the
// grid; begin[p] is a multiple of 8, so the hardware's round-robin XCD of a
// block is also its XCD within the problem, and each XCD owns a contiguous
// range of the problem's tiles (row tiles of a column tile together). Blocks
// past a problem's tiles (padding to the next multiple of 8) exit at once.
template <int GS, int WAVES, int WM, int MB, int NB>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void w4a8_gemm_kernel(const W4A8Batch bt) {
  using C = Q8Cfg<GS, WAVES, WM, MB, NB>;
  extern __shared__ __attribute__((aligned(16))) unsigned char q8_lds[];
  const int b = blockIdx.x;
  int p = 0;
#pragma unroll
  for (int i = 1; i < kMaxProblems; ++i)
    if (i < bt.nprob && b >= bt.begin[i]) p = i;
  const int local = b - bt.begin[p];
  if (local >= bt.tiles[p]) return;
  const int tile = xcd_grouped(local, bt.tiles[p]);
  const int MT = bt.MT;
  const int mt = tile % MT, nt = tile / MT;
  const W4A8Args& a = bt.prob[p];
  Q8Engine<GS, WAVES, WM, MB, NB> e;
  e.setup(q8_lds, a, mt * C::Rows, nt);
  Q8Acc<MB, NB> acc;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc.v[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  e.kloop(acc, (e.G + C::T - 1) / C::T);
  e.store(acc, a.sx, a.y);
}

// Wave tiles of 128 x 32 (8 x 2 MFMA blocks), all waves along N: 8 waves
// (128 x 256 workgroup tiles, one workgroup per CU) or, for small M where
// 256-column tiles leave compute units idle, 4 waves (128 x 128 tiles, two
// workgroups per CU).
constexpr int kQ8WM = 1, kQ8MB = 8, kQ8NB = 2;
#ifndef W4A8_SMALL_TILE_MAX_M
#define W4A8_SMALL_TILE_MAX_M 256
#endif

// One launch over bt.prob[0 .. nprob), all with M rows; fills MT, tiles and
// begin. Problems are dispatched in the order given.
template <int GS, int WAVES>
hipError_t launch_w4a8_batch(W4A8Batch& bt, hipStream_t stream) {
  using C = Q8Cfg<GS, WAVES, kQ8WM, kQ8MB, kQ8NB>;
  const void* fn =
      reinterpret_cast<const void*>(&w4a8_gemm_kernel<GS, WAVES, kQ8WM, kQ8MB, kQ8NB>);
  const size_t lds = C::Lds;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  bt.MT = (bt.prob[0].M + C::Rows - 1) / C::Rows;
  long long blocks = 0;
  for (int i = 0; i < bt.nprob; ++i) {
    const int NCB = (bt.prob[i].N + 15) / 16;
    const long long tiles = static_cast<long long>(bt.MT) * ((NCB + C::Blocks - 1) / C::Blocks);
    if (tiles < 1 || blocks + tiles > 0x7FFFFFF0LL) return hipErrorInvalidValue;
    bt.begin[i] = static_cast<int>(blocks);
    bt.tiles[i] = static_cast<int>(tiles);
    blocks += (tiles + 7) / 8 * 8;
  }
  void* kargs[] = {&bt};
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(blocks)), dim3(C::Threads), kargs, lds,
                         stream);
}

template <int GS>
hipError_t launch_w4a8_batch_m(W4A8Batch& bt, hipStream_t stream) {
  return bt.prob[0].M <= W4A8_SMALL_TILE_MAX_M ? launch_w4a8_batch<GS, 4>(bt, stream)
                                               : launch_w4a8_batch<GS, 8>(bt, stream);
}

template <int GS>
hipError_t launch_w4a8_t(const W4A8Args* probs, int count, hipStream_t stream) {
  constexpr int kRows = kQ8WM * kQ8MB * 16;  // tile rows (both wave counts)
  // Code offsets are 32-bit: a problem with M * K beyond that runs by itself,
  // in row chunks of at most rows_per_launch rows.
  bool fits = true;
  for (int i = 0; i < count; ++i)
    fits = fits && static_cast<long long>(probs[i].M) * probs[i].K <= 0xFFFFFF00LL;
  if (fits) {
    W4A8Batch bt = {};
    // longest tiles first: the K-deepest problems start before the rest
    int order[kMaxProblems];
    for (int i = 0; i < count; ++i) order[i] = i;
    for (int i = 1; i < count; ++i)
      for (int j = i; j > 0 && probs[order[j]].K > probs[order[j - 1]].K; --j) {
        const int t = order[j];
        order[j] = order[j - 1];
        order[j - 1] = t;
      }
    for (int i = 0; i < count; ++i) bt.prob[i] = probs[order[i]];
    bt.nprob = count;
    return launch_w4a8_batch_m<GS>(bt, stream);
  }
  for (int i = 0; i < count; ++i) {
    const W4A8Args& a = probs[i];
    long long rows_per_launch = (0xFFFFFF00LL) / a.K;
    rows_per_launch -= rows_per_launch % kRows;
    if (rows_per_launch < kRows) return hipErrorInvalidValue;
    for (long long r0 = 0; r0 < a.M; r0 += rows_per_launch) {
      W4A8Batch bt = {};
      W4A8Args& part = bt.prob[0];
      part = a;
      part.M = static_cast<int>(a.M - r0 < rows_per_launch ? a.M - r0 : rows_per_launch);
      part.xq = a.xq + r0 * a.K;
      part.sx = a.sx + r0;
      part.y = a.y + r0 * a.N;
      bt.nprob = 1;
      const hipError_t e = launch_w4a8_batch_m<GS>(bt, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_w4a8_quantize(const W4A8QuantProblem* probs, int count, int M,
                                hipStream_t stream) {
  if (count < 1 || count > kMaxProblems || M < 1 ||
      static_cast<long long>(M) * count > 0x7FFFFFFFLL)
    return hipErrorInvalidValue;
  W4A8QuantBatch bt = {};
  for (int i = 0; i < count; ++i) bt.prob[i] = probs[i];
  bt.M = M;
  const void* fn = reinterpret_cast<const void*>(&w4a8_quantize_kernel);
  void* kargs[] = {&bt};
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(M * count)), dim3(kQThreads), kargs, 0,
                         stream);
}

hipError_t launch_w4a8_gemm(const W4A8Args* probs, int count, hipStream_t stream) {
  if (count < 1 || count > kMaxProblems) return hipErrorInvalidValue;
  switch (probs[0].group) {
    case 64: return launch_w4a8_t<64>(probs, count, stream);
    case 128: return launch_w4a8_t<128>(probs, count, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a16_internal
