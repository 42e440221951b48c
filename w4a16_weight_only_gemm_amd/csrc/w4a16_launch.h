// w4a16_launch.h -- internal interface between the host half and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace w4a16_internal {

struct GemmArgs {
  const uint16_t* x;        // bf16 [M][K], row-major
  const uint32_t* qweight;  // packed tiles [ceil(N/16)][K/group][64 lanes][group/32 words]
  const uint16_t* scales;   // fp16 [ceil(N/16)][K/group][16]
  uint16_t* y;              // bf16 [M][N], row-major
  int M, N, K, group;
};

// Shape-checked by the caller: M >= 1, N >= 1, K % group == 0, group in {32, 64, 128, 256},
// all pointers 16-byte aligned.
hipError_t launch_skinny(const GemmArgs& a, hipStream_t stream);
hipError_t launch_large(const GemmArgs& a, hipStream_t stream);
// Group sizes the MFMA tile engine handles (others run the plain kernel).
bool large_supported(int group);
// Whether the tile engine runs the shape: a group it handles and packed
// weights below 4 GB (32-bit buffer offsets); launch_large falls back to
// plain_kernel otherwise.
bool large_runs(int N, int K, int group);

// ---- w4a16_gemm's choice of kernel form (host arithmetic only) ----
// Compute units the time models below assume (one MI355X); the choice is a
// pure function of the shape, so it is the same on every device and call.
constexpr int kModelCUs = 256;
// Rows plain_kernel takes: its grid's second dimension counts row tiles of at
// least 16 rows and holds at most 65535.
constexpr int kPlainMaxRows = 65535 * 16;
// Modelled time (microseconds) of the best whole-K tile form (tile_kernel) for
// the shape, and its tile height (32, 64 or 128 rows) in *rows_out.
double tile_estimate_us(int M, int N, int K, int group, int* rows_out);
// plain_kernel forms (w4a16_plain.hip); the form launch_skinny runs for a
// shape, its workgroup geometry, and the modelled time of the best form at
// more than 16 rows.
int plain_form(int M, int N, int K, int group);
void plain_form_shape(int form, int* rows, int* cols, int* waves);
double plain_estimate_us(int M, int N, int K, int group);
// A single problem above 16 rows that the workspace entry points run with the
// kernels of w4a16_gemm instead of the stream-K schedule.
bool single_prefers_whole_k(int M, int N, int K, int group);

// ---- stream-K (persistent, several problems per launch, M <= 16) ----
constexpr int kMaxProblems = 8;
constexpr int kStreamKWaves = 8;                // waves per workgroup
constexpr int kStreamKMaxWaves = 8192;          // grid never exceeds this many waves
// Staged activations, their row sums and the waves' parts per workgroup: two
// workgroups fit in a compute unit's 160 KB.
constexpr size_t kStreamKLdsBudget = 78 * 1024;
// Floats per group in the staged row sums: rows 0..15, or with at most 4 rows
// rows 0..3 and then the last row four times (the padding rows' value).
__host__ __device__ constexpr int streamk_sum_stride(int M) { return M <= 4 ? 8 : 16; }

struct StreamKProblem {
  const uint16_t* x;        // bf16 [M][K]
  const uint32_t* qw;       // packed weights (device arrangement)
  const uint16_t* sp;       // packed scales
  uint16_t* y;              // bf16 [M][N]
  int N, K;
  // filled in by launch_streamk
  int G, NCB;               // groups per column, 16-column blocks
  int NSB;                  // super-blocks (NBW consecutive column blocks each)
  long long u_begin;        // first unit (super-block, group) of this problem
  int sb_begin;             // first super-block (index of its counter)
};

struct StreamKArgs {
  StreamKProblem prob[kMaxProblems];  // the problems, unless `table` is set
  // Planned calls: the problems in a device table (nprob entries) and, per
  // workgroup, the problem holding its first unit; the kernel checks the
  // device plan's checksum against `checksum` before doing anything.
  const StreamKProblem* table;
  const int* wgfirst;
  const unsigned long long* plan_checksum;
  unsigned long long checksum;
  int nprob;
  int M;
  long long units;          // total units over all problems
  int nwaves;               // waves that own units (<= units)
  float* part;              // [workgroups][2][NBW][min(M,16)][16] fp32 parts
  uint32_t* slots;          // [super-blocks][NBW][min(M,16)][16] swap slots, zero between calls
  int* counters;            // one per super-block, zero between calls
  int lds_part_off;         // LDS offset (in 4-byte words) of the waves' parts
};

// Column blocks per stream-K unit: 1 when the activations are staged in LDS,
// streamk_wide_blocks(group) when each wave reads them itself (then one
// activation fragment serves that many weight tiles: the wider, the less
// activation traffic per weight byte, up to what the registers hold without
// spilling at two waves per SIMD).
constexpr int streamk_wide_blocks(int group) { return group == 256 ? 3 : 6; }
constexpr int kStreamKWideMaxBlocks = 6;
constexpr int kStreamKWideMaxWaves = 4096;      // grid cap with wide units

// Workspace layout: counters first (kMaxProblems + ceil(columns/16) ints),
// then the swap slots (one value per output of every super-block), then the
// per-workgroup parts, each region rounded up to 256 bytes.
size_t streamk_counter_bytes(long long total_columns);
size_t streamk_slot_bytes(int M, long long total_columns);
size_t streamk_part_bytes(int M);

hipError_t launch_streamk(const StreamKProblem* probs, int count, int M, int group, float* part,
                          uint32_t* slots, int* counters, hipStream_t stream);

// ---- stream-K large-M path (tiles of 32, 64 or 128 rows x 256 columns) ----
constexpr int kLargeMaxWorkgroups = 320;  // persistent grid never exceeds this

struct LargeProblem {
  const uint16_t* x;
  const uint32_t* qw;
  const uint16_t* sp;
  uint16_t* y;
  int N, K;
  // filled in by launch_large_streamk
  int G, NCB;               // groups per column, 16-column blocks
  int MT, NT, KT;           // row tiles, column tiles, k-tiles per tile
  long long u_begin;        // first unit (tile, k-tile) of this problem
  int t_begin;              // first tile (index of its counter)
};

struct LargeSKArgs {
  LargeProblem prob[kMaxProblems];  // the problems, unless `table` is set
  const LargeProblem* table;        // planned calls, as in StreamKArgs
  const int* wgfirst;
  const unsigned long long* plan_checksum;
  unsigned long long checksum;
  int nprob;
  int M;
  long long units;          // total units over all problems
  int nwg;                  // workgroups, each owning at least one unit
  float* part;              // [kLargeMaxWorkgroups][2][8 waves][regs][64 lanes] fp32 parts
  int* counters;            // one per tile, zero between calls
};

// Tile rows used for M rows, and the workspace layout: counters first
// (rounded up to 256 bytes), then the parts.
int large_streamk_rows(int M);
size_t large_streamk_counter_bytes(int M, long long total_columns);
size_t large_streamk_part_bytes(int M);
// True when the problems can run on the stream-K large path (group size and
// 32-bit buffer ranges).
bool large_streamk_fits(const StreamKProblem* probs, int count, int M, int group);
hipError_t launch_large_streamk(const StreamKProblem* probs, int count, int M, int group,
                                float* part, int* counters, hipStream_t stream);

// ---- planned calls: many problems, descriptors in device memory ----
//
// A plan is a byte image built on the host (w4a16_plan_build) and copied by
// the caller to device memory: a header, then the problem table (StreamKProblem
// or LargeProblem entries, as the kernel reads them), then the first problem
// of every workgroup. The host launches from its copy; the kernels read the
// table from the device copy.
constexpr uint32_t kPlanMagic = 0x4C503457u;  // "W4PL"
constexpr uint32_t kPlanVersion = 1;
constexpr int kPlanKindStreamK = 1;  // M <= 16: streaming kernel
constexpr int kPlanKindLarge = 2;    // M > 16: MFMA tile engine
constexpr int kPlanMaxProblems = 4096;
constexpr int kPlanMaxWorkgroups = 1024;  // both grids stay below this
constexpr int kPlanTilesPerWorkgroup = 16;  // large plans: whole tiles from this many per workgroup

struct PlanHeader {
  uint32_t magic, version;
  int kind, count, M, group;
  int grid;          // workgroups launched
  int nwaves;        // stream-K: waves owning units; large: workgroups owning units
  int nbw;           // stream-K: column blocks per super-block
  int rows;          // large: tile rows
  int xlds;          // stream-K: activations staged in LDS
  int lds_bytes;     // dynamic LDS per workgroup
  int lds_part_off;  // stream-K: LDS offset (4-byte words) of the waves' parts
  int table_off;     // byte offset of the problem table
  int wgfirst_off;   // byte offset of the per-workgroup first problem
  int tiles;         // large: whole tiles dealt round robin (no workspace), else stream-K
  long long units;
  long long total_columns;
  long long counters_off, slots_off, part_off;  // byte offsets in the workspace
  long long workspace_bytes;
  unsigned long long checksum;  // FNV-1a (64-bit) of every plan byte, this field read as 0
  unsigned long long pad1[5];
};
static_assert(sizeof(PlanHeader) % 16 == 0, "16-byte multiple");
constexpr size_t kPlanHeaderBytes = 256;
static_assert(sizeof(PlanHeader) <= kPlanHeaderBytes, "header fits its slot");

// Plans of validated problems (pointers, N and K set): fill the problems'
// offsets, the header's launch and workspace fields and the first problem of
// every workgroup (at most kPlanMaxWorkgroups). Return 0, or -1 when the
// problems do not fit the form.
int build_streamk_plan(StreamKProblem* probs, int count, int M, int group, PlanHeader& h,
                       int* wgfirst);
int build_large_plan(LargeProblem* probs, int count, int M, int group, PlanHeader& h,
                     int* wgfirst);
hipError_t launch_streamk_planned(const PlanHeader& h, const unsigned char* plan_dev, char* ws,
                                  hipStream_t stream);
hipError_t launch_large_planned(const PlanHeader& h, const unsigned char* plan_dev, char* ws,
                                hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cus();

// ---- read-bandwidth probe (w4a16_probe.hip) ----
constexpr int kReadProbeMaxWorkgroups = 2048;  // sink words the probe may write
int read_probe_workgroups();
hipError_t launch_read_probe(const void* buf, long long words, uint32_t* sink, hipStream_t stream);

// M-dispatch: W4A16_PATH_SKINNY or W4A16_PATH_LARGE for a supported shape.
int choose_path(int M, int N, int K, int group);
// The workgroup tile (rows x columns, waves) that w4a16_gemm_ex runs for a
// supported shape on `path` (W4A16_PATH_AUTO resolved first); returns the path.
int describe_form(int M, int N, int K, int group, int path, int* rows, int* cols, int* waves);

}  // namespace w4a16_internal
