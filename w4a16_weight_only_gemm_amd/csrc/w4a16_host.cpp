// w4a16_host.cpp -- host half of the W4A16 library: sizes, packing, argument
// checks and the M-dispatch. Nothing here touches a device except the launch
// calls at the very end of w4a16_gemm_ex.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/w4a16.h"
#include "w4a16_launch.h"
#include "w4a8_launch.h"

namespace {

bool pack_shape_ok(int N, int K, int group) {
  return N >= 0 && K >= 0 && group > 0 && group % 32 == 0 && K % group == 0;
}

size_t column_blocks(int N) { return (static_cast<size_t>(N) + 15) / 16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool group_supported(int group) {
  return group == 32 || group == 64 || group == 128 || group == 256;
}

// Byte layout of a plan of `count` problems: header, problem table (room for
// the larger of the two entry types), first problem per workgroup.
struct PlanLayout {
  size_t table_off, wgfirst_off, total;
};

PlanLayout plan_layout(int count) {
  using namespace w4a16_internal;
  const size_t entry = sizeof(StreamKProblem) > sizeof(LargeProblem) ? sizeof(StreamKProblem)
                                                                      : sizeof(LargeProblem);
  PlanLayout l;
  l.table_off = kPlanHeaderBytes;
  l.wgfirst_off = l.table_off + (entry * count + 255) / 256 * 256;
  l.total = l.wgfirst_off + static_cast<size_t>(kPlanMaxWorkgroups) * sizeof(int);
  return l;
}

// FNV-1a, 64-bit.
uint64_t fnv1a64(const unsigned char* p, size_t n) {
  uint64_t h = 0xcbf29ce484222325ull;
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 0x100000001b3ull;
  }
  return h;
}

// The header of a host plan, or nullptr if it is not one this library built.
const w4a16_internal::PlanHeader* plan_header(const void* plan) {
  using namespace w4a16_internal;
  if (!plan || (reinterpret_cast<uintptr_t>(plan) & 7u) != 0) return nullptr;
  const PlanHeader* h = static_cast<const PlanHeader*>(plan);
  if (h->magic != kPlanMagic || h->version != kPlanVersion) return nullptr;
  if (h->kind != kPlanKindStreamK && h->kind != kPlanKindLarge) return nullptr;
  return h;
}

}  // namespace

extern "C" {

size_t w4a16_qweight_bytes(int N, int K) {
  if (N < 0 || K < 0 || K % 32 != 0) return 0;
  return column_blocks(N) * 16 * static_cast<size_t>(K) / 2;
}

size_t w4a16_scales_bytes(int N, int K, int group) {
  if (N < 0 || K < 0 || group <= 0 || group % 32 != 0 || K % group != 0) return 0;
  return column_blocks(N) * 16 * static_cast<size_t>(K / group) * 2;
}

int w4a16_pack(const int8_t* q, const uint16_t* scales_in, uint32_t* qweight_out,
               uint16_t* scales_out, int N, int K, int group) {
  if (!pack_shape_ok(N, K, group)) return W4A16_ERR_INVALID_ARG;
  if (N == 0 || K == 0) return W4A16_OK;
  if (!q || !scales_in || !qweight_out || !scales_out) return W4A16_ERR_INVALID_ARG;
  const size_t total = static_cast<size_t>(N) * static_cast<size_t>(K);
  // Validate everything before writing anything.
  for (size_t i = 0; i < total; ++i) {
    if (q[i] < -8 || q[i] > 7) return W4A16_ERR_INVALID_ARG;
  }
  const int G = K / group;
  const int wpl = group / 32;           // words per lane per tile
  const size_t blocks = column_blocks(N);
  uint32_t* out = qweight_out;
  uint16_t* sout = scales_out;
  for (size_t b = 0; b < blocks; ++b) {
    for (int t = 0; t < G; ++t) {
      // tile (b, t): lane l = 16 * slice + column, holding wpl consecutive words
      for (int slice = 0; slice < 4; ++slice) {
        for (int col = 0; col < 16; ++col) {
          const size_t n = b * 16 + col;
          for (int w = 0; w < wpl; ++w) {
            uint32_t word = 0;
            if (n < static_cast<size_t>(N)) {  // padding columns of the last block: zero codes
              const int8_t* codes = q + n * K + static_cast<size_t>(t) * group + slice * wpl * 8;
              // nibble v holds the code of k = 2v, nibble v + 4 that of k = 2v + 1
              for (int v = 3; v >= 0; --v)
                word = (word << 4) | (static_cast<uint32_t>(codes[8 * w + 2 * v + 1]) & 0xFu);
              for (int v = 3; v >= 0; --v)
                word = (word << 4) | (static_cast<uint32_t>(codes[8 * w + 2 * v]) & 0xFu);
            }
            out[(slice * 16 + col) * wpl + w] = word;
          }
        }
      }
      out += 64 * wpl;
      for (int col = 0; col < 16; ++col) {
        const size_t n = b * 16 + col;
        sout[col] = n < static_cast<size_t>(N) ? scales_in[n * G + t] : static_cast<uint16_t>(0);
      }
      sout += 16;
    }
  }
  return W4A16_OK;
}

int w4a16_select_path(int M, int N, int K, int group) {
  if (M < 0 || N < 1 || K < 1 || !group_supported(group) || K % group != 0) return -1;
  if (M > w4a16_internal::kPlainMaxRows && !w4a16_internal::large_runs(N, K, group)) return -1;
  return w4a16_internal::choose_path(M, N, K, group);
}

int w4a16_select_form(int M, int N, int K, int group, int path, int* rows, int* cols, int* waves) {
  if (M < 0 || N < 1 || K < 1 || !group_supported(group) || K % group != 0) return -1;
  if (path != W4A16_PATH_AUTO && path != W4A16_PATH_SKINNY && path != W4A16_PATH_LARGE) return -1;
  if (!rows || !cols || !waves) return -1;
  return w4a16_internal::describe_form(M, N, K, group, path, rows, cols, waves);
}

int w4a16_gemm_ex(const void* x, const void* qweight, const void* scales, void* y, int M,
                  int N, int K, int group, int path, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return W4A16_ERR_INVALID_ARG;
  if (path != W4A16_PATH_AUTO && path != W4A16_PATH_SKINNY && path != W4A16_PATH_LARGE)
    return W4A16_ERR_INVALID_ARG;
  if (M == 0) return W4A16_OK;
  if (!x || !qweight || !scales || !y) return W4A16_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || !group_supported(group) || K % group != 0) return W4A16_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || !aligned16(y))
    return W4A16_ERR_MISALIGNED;
  if (path == W4A16_PATH_AUTO) path = w4a16_internal::choose_path(M, N, K, group);
  if (M > w4a16_internal::kPlainMaxRows) {
    // plain_kernel's grid holds at most that many rows: the tile engine, or nothing
    if (!w4a16_internal::large_runs(N, K, group)) return W4A16_ERR_UNSUPPORTED;
    path = W4A16_PATH_LARGE;
  }
  w4a16_internal::GemmArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.qweight = static_cast<const uint32_t*>(qweight);
  a.scales = static_cast<const uint16_t*>(scales);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.N = N;
  a.K = K;
  a.group = group;
  hipError_t err = path == W4A16_PATH_LARGE ? w4a16_internal::launch_large(a, stream)
                                            : w4a16_internal::launch_skinny(a, stream);
  return err == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

int w4a16_gemm(const void* x, const void* qweight, const void* scales, void* y, int M, int N,
               int K, int group, hipStream_t stream) {
  return w4a16_gemm_ex(x, qweight, scales, y, M, N, K, group, W4A16_PATH_AUTO, stream);
}

size_t w4a16_workspace_bytes(int M, long long total_columns) {
  if (M < 0 || total_columns < 0) return 0;
  if (M > 16)
    return w4a16_internal::large_streamk_counter_bytes(M, total_columns) +
           w4a16_internal::large_streamk_part_bytes(M);
  return w4a16_internal::streamk_counter_bytes(total_columns) +
         w4a16_internal::streamk_slot_bytes(M, total_columns) +
         w4a16_internal::streamk_part_bytes(M);
}

int w4a16_gemm_grouped(const w4a16_problem* problems, int count, int M, int group,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!problems || count < 1 || count > W4A16_MAX_PROBLEMS || M < 0)
    return W4A16_ERR_INVALID_ARG;
  if (M == 0) return W4A16_OK;
  if (!group_supported(group)) return W4A16_ERR_UNSUPPORTED;
  long long columns = 0;
  for (int i = 0; i < count; ++i) {
    const w4a16_problem& p = problems[i];
    if (p.N < 0 || p.K < 0) return W4A16_ERR_INVALID_ARG;
    if (!p.x || !p.qweight || !p.scales || !p.y) return W4A16_ERR_INVALID_ARG;
    if (p.N < 1 || p.K < 1 || p.K % group != 0) return W4A16_ERR_UNSUPPORTED;
    if (!aligned16(p.x) || !aligned16(p.qweight) || !aligned16(p.scales) || !aligned16(p.y))
      return W4A16_ERR_MISALIGNED;
    columns += p.N;
  }
  // One problem above 16 rows: w4a16_gemm's kernels when the time models put
  // them ahead (they need no workspace, which is then left untouched).
  if (count == 1 && w4a16_internal::single_prefers_whole_k(M, problems[0].N, problems[0].K, group)) {
    const w4a16_problem& p = problems[0];
    return w4a16_gemm_ex(p.x, p.qweight, p.scales, p.y, M, p.N, p.K, group, W4A16_PATH_AUTO,
                         stream);
  }
  w4a16_internal::StreamKProblem probs[W4A16_MAX_PROBLEMS] = {};
  for (int i = 0; i < count; ++i) {
    probs[i].x = static_cast<const uint16_t*>(problems[i].x);
    probs[i].qw = static_cast<const uint32_t*>(problems[i].qweight);
    probs[i].sp = static_cast<const uint16_t*>(problems[i].scales);
    probs[i].y = static_cast<uint16_t*>(problems[i].y);
    probs[i].N = problems[i].N;
    probs[i].K = problems[i].K;
  }
  if (M > 16 && !w4a16_internal::large_streamk_fits(probs, count, M, group)) {
    // Group 256 or 32-bit buffer ranges exceeded: the per-problem kernels,
    // one launch each, no workspace.
    for (int i = 0; i < count; ++i) {
      const w4a16_problem& p = problems[i];
      const int rc = w4a16_gemm_ex(p.x, p.qweight, p.scales, p.y, M, p.N, p.K, group,
                                   W4A16_PATH_AUTO, stream);
      if (rc != W4A16_OK) return rc;
    }
    return W4A16_OK;
  }
  if (!workspace || workspace_bytes < w4a16_workspace_bytes(M, columns))
    return W4A16_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return W4A16_ERR_MISALIGNED;
  char* ws = static_cast<char*>(workspace);
  int* counters = reinterpret_cast<int*>(ws);
  hipError_t err;
  if (M > 16) {
    float* part = reinterpret_cast<float*>(
        ws + w4a16_internal::large_streamk_counter_bytes(M, columns));
    err = w4a16_internal::launch_large_streamk(probs, count, M, group, part, counters, stream);
  } else {
    char* slots = ws + w4a16_internal::streamk_counter_bytes(columns);
    float* part = reinterpret_cast<float*>(slots + w4a16_internal::streamk_slot_bytes(M, columns));
    err = w4a16_internal::launch_streamk(probs, count, M, group, part,
                                         reinterpret_cast<uint32_t*>(slots), counters, stream);
  }
  return err == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

size_t w4a16_plan_bytes(int count) {
  if (count < 1 || count > w4a16_internal::kPlanMaxProblems) return 0;
  return plan_layout(count).total;
}

int w4a16_plan_build(const w4a16_problem* problems, int count, int M, int group, void* plan,
                     size_t plan_bytes) {
  using namespace w4a16_internal;
  if (!problems || !plan || count < 1 || count > kPlanMaxProblems || M < 1)
    return W4A16_ERR_INVALID_ARG;
  const PlanLayout lay = plan_layout(count);
  if (plan_bytes < lay.total) return W4A16_ERR_INVALID_ARG;
  if (!group_supported(group)) return W4A16_ERR_UNSUPPORTED;
  long long columns = 0;
  for (int i = 0; i < count; ++i) {
    const w4a16_problem& p = problems[i];
    if (p.N < 0 || p.K < 0) return W4A16_ERR_INVALID_ARG;
    if (!p.x || !p.qweight || !p.scales || !p.y) return W4A16_ERR_INVALID_ARG;
    if (p.N < 1 || p.K < 1 || p.K % group != 0) return W4A16_ERR_UNSUPPORTED;
    if (!aligned16(p.x) || !aligned16(p.qweight) || !aligned16(p.scales) || !aligned16(p.y))
      return W4A16_ERR_MISALIGNED;
    columns += p.N;
  }
  std::vector<StreamKProblem> sk(count);
  for (int i = 0; i < count; ++i) {
    sk[i] = StreamKProblem{};
    sk[i].x = static_cast<const uint16_t*>(problems[i].x);
    sk[i].qw = static_cast<const uint32_t*>(problems[i].qweight);
    sk[i].sp = static_cast<const uint16_t*>(problems[i].scales);
    sk[i].y = static_cast<uint16_t*>(problems[i].y);
    sk[i].N = problems[i].N;
    sk[i].K = problems[i].K;
  }
  unsigned char* out = static_cast<unsigned char*>(plan);
  std::memset(out, 0, lay.total);
  PlanHeader h = {};
  h.magic = kPlanMagic;
  h.version = kPlanVersion;
  h.count = count;
  h.M = M;
  h.group = group;
  h.table_off = static_cast<int>(lay.table_off);
  h.wgfirst_off = static_cast<int>(lay.wgfirst_off);
  h.total_columns = columns;
  int* wgfirst = reinterpret_cast<int*>(out + lay.wgfirst_off);
  if (M <= 16) {
    if (build_streamk_plan(sk.data(), count, M, group, h, wgfirst) != 0)
      return W4A16_ERR_UNSUPPORTED;
    std::memcpy(out + lay.table_off, sk.data(), sizeof(StreamKProblem) * count);
  } else {
    // the MFMA tile engine: groups 32, 64 and 128 and 32-bit buffer ranges
    if (!large_streamk_fits(sk.data(), count, M, group)) return W4A16_ERR_UNSUPPORTED;
    std::vector<LargeProblem> lg(count);
    for (int i = 0; i < count; ++i) {
      lg[i] = LargeProblem{};
      lg[i].x = sk[i].x;
      lg[i].qw = sk[i].qw;
      lg[i].sp = sk[i].sp;
      lg[i].y = sk[i].y;
      lg[i].N = sk[i].N;
      lg[i].K = sk[i].K;
    }
    if (build_large_plan(lg.data(), count, M, group, h, wgfirst) != 0)
      return W4A16_ERR_UNSUPPORTED;
    std::memcpy(out + lay.table_off, lg.data(), sizeof(LargeProblem) * count);
  }
  // the checksum covers every byte of the plan, its own field read as zero
  h.checksum = 0;
  std::memcpy(out, &h, sizeof(h));
  h.checksum = fnv1a64(out, lay.total);
  std::memcpy(out, &h, sizeof(h));
  return W4A16_OK;
}

size_t w4a16_plan_workspace_bytes(const void* plan) {
  const w4a16_internal::PlanHeader* h = plan_header(plan);
  return h ? static_cast<size_t>(h->workspace_bytes) : 0;
}

int w4a16_gemm_planned(const void* plan, const void* plan_dev, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  using namespace w4a16_internal;
  const PlanHeader* hp = plan_header(plan);
  if (!hp || !plan_dev) return W4A16_ERR_INVALID_ARG;
  const PlanHeader h = *hp;
  if (!aligned16(plan_dev)) return W4A16_ERR_MISALIGNED;
  if (h.workspace_bytes > 0) {  // a plan of whole tiles needs none
    if (!workspace || workspace_bytes < static_cast<size_t>(h.workspace_bytes))
      return W4A16_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return W4A16_ERR_MISALIGNED;
  }
  const unsigned char* dev = static_cast<const unsigned char*>(plan_dev);
  char* ws = static_cast<char*>(workspace);
  const hipError_t err = h.kind == kPlanKindStreamK ? launch_streamk_planned(h, dev, ws, stream)
                                                    : launch_large_planned(h, dev, ws, stream);
  return err == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

int w4a16_gemm_ws(const void* x, const void* qweight, const void* scales, void* y, int M, int N,
                  int K, int group, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return W4A16_ERR_INVALID_ARG;
  w4a16_problem p = {x, qweight, scales, y, N, K};
  if (M == 0) return W4A16_OK;
  if (!x || !qweight || !scales || !y) return W4A16_ERR_INVALID_ARG;
  return w4a16_gemm_grouped(&p, 1, M, group, workspace, workspace_bytes, stream);
}

int w4a8_quantize_grouped(const w4a8_quantize_problem* problems, int count, int M,
                          hipStream_t stream) {
  if (!problems || count < 1 || count > W4A16_MAX_PROBLEMS || M < 0) return W4A16_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i)
    if (problems[i].K < 0) return W4A16_ERR_INVALID_ARG;
  if (M == 0) return W4A16_OK;
  w4a16_internal::W4A8QuantProblem probs[W4A16_MAX_PROBLEMS] = {};
  for (int i = 0; i < count; ++i) {
    const w4a8_quantize_problem& p = problems[i];
    if (!p.x || !p.xq || !p.sx) return W4A16_ERR_INVALID_ARG;
    if (p.K < 16 || p.K % 16 != 0) return W4A16_ERR_UNSUPPORTED;
    if (!aligned16(p.x) || !aligned16(p.xq) || !aligned16(p.sx)) return W4A16_ERR_MISALIGNED;
    probs[i].x = static_cast<const uint16_t*>(p.x);
    probs[i].xq = static_cast<uint8_t*>(p.xq);
    probs[i].sx = static_cast<float*>(p.sx);
    probs[i].K = p.K;
  }
  if (static_cast<long long>(M) * count > 0x7FFFFFFFLL) return W4A16_ERR_UNSUPPORTED;
  const hipError_t err = w4a16_internal::launch_w4a8_quantize(probs, count, M, stream);
  return err == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

int w4a8_quantize(const void* x, void* xq, void* sx, int M, int K, hipStream_t stream) {
  if (M < 0 || K < 0) return W4A16_ERR_INVALID_ARG;
  if (M == 0) return W4A16_OK;
  const w4a8_quantize_problem p = {x, xq, sx, K};
  return w4a8_quantize_grouped(&p, 1, M, stream);
}

int w4a8_gemm_grouped(const w4a8_problem* problems, int count, int M, int group,
                      hipStream_t stream) {
  if (!problems || count < 1 || count > W4A16_MAX_PROBLEMS || M < 0) return W4A16_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i)
    if (problems[i].N < 0 || problems[i].K < 0) return W4A16_ERR_INVALID_ARG;
  if (M == 0) return W4A16_OK;
  w4a16_internal::W4A8Args probs[W4A16_MAX_PROBLEMS] = {};
  for (int i = 0; i < count; ++i) {
    const w4a8_problem& p = problems[i];
    if (!p.xq || !p.sx || !p.qweight || !p.scales || !p.y) return W4A16_ERR_INVALID_ARG;
    if (p.N < 1 || p.K < 1 || (group != 64 && group != 128) || p.K % group != 0)
      return W4A16_ERR_UNSUPPORTED;
    // packed weights and scales are addressed with 32-bit buffer offsets
    if (w4a16_qweight_bytes(p.N, p.K) > 0xFFFFFFF0u) return W4A16_ERR_UNSUPPORTED;
    if (!aligned16(p.xq) || !aligned16(p.sx) || !aligned16(p.qweight) || !aligned16(p.scales) ||
        !aligned16(p.y))
      return W4A16_ERR_MISALIGNED;
    w4a16_internal::W4A8Args& a = probs[i];
    a.xq = static_cast<const uint8_t*>(p.xq);
    a.sx = static_cast<const float*>(p.sx);
    a.qweight = static_cast<const uint32_t*>(p.qweight);
    a.scales = static_cast<const uint16_t*>(p.scales);
    a.y = static_cast<uint16_t*>(p.y);
    a.M = M;
    a.N = p.N;
    a.K = p.K;
    a.group = group;
  }
  const hipError_t err = w4a16_internal::launch_w4a8_gemm(probs, count, stream);
  return err == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

int w4a8_gemm(const void* xq, const void* sx, const void* qweight, const void* scales, void* y,
              int M, int N, int K, int group, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return W4A16_ERR_INVALID_ARG;
  if (M == 0) return W4A16_OK;
  const w4a8_problem p = {xq, sx, qweight, scales, y, N, K};
  return w4a8_gemm_grouped(&p, 1, M, group, stream);
}

const char* w4a16_status_string(int status) {
  switch (status) {
    case W4A16_OK: return "W4A16_OK: success";
    case W4A16_ERR_INVALID_ARG: return "W4A16_ERR_INVALID_ARG: null pointer, bad size or code";
    case W4A16_ERR_UNSUPPORTED: return "W4A16_ERR_UNSUPPORTED: shape or group size not supported";
    case W4A16_ERR_MISALIGNED: return "W4A16_ERR_MISALIGNED: device pointer not 16-byte aligned";
    case W4A16_ERR_LAUNCH: return "W4A16_ERR_LAUNCH: kernel launch failed";
    case W4A16_ERR_TOO_LARGE:
      return "W4A16_ERR_TOO_LARGE: shape needs more scratch than the static array holds";
    default: return "unknown w4a16 status";
  }
}

int w4a16_version(void) { return 100; }

int w4a16_read_probe(const void* buf, size_t bytes, void* sink, size_t sink_bytes,
                     hipStream_t stream) {
  if (bytes % 16 != 0) return W4A16_ERR_INVALID_ARG;
  if (sink == nullptr ||
      sink_bytes < static_cast<size_t>(w4a16_internal::kReadProbeMaxWorkgroups) * 4)
    return W4A16_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return W4A16_ERR_MISALIGNED;
  if (bytes == 0) return W4A16_OK;
  if (buf == nullptr) return W4A16_ERR_INVALID_ARG;
  if (!aligned16(buf)) return W4A16_ERR_MISALIGNED;
  const long long words = static_cast<long long>(bytes / 16);
  return w4a16_internal::launch_read_probe(buf, words, static_cast<uint32_t*>(sink), stream) ==
                 hipSuccess
             ? W4A16_OK
             : W4A16_ERR_LAUNCH;
}

}  // extern "C"

namespace w4a16_internal {

size_t streamk_counter_bytes(long long total_columns) {
  const long long ints = kMaxProblems + (total_columns + 15) / 16;
  return static_cast<size_t>((ints * 4 + 255) / 256 * 256);
}

size_t streamk_slot_bytes(int M, long long total_columns) {
  const int rows = M < 16 ? M : 16;
  // super-blocks x NBW column blocks <= column blocks + problems x NBW
  const long long blocks = (total_columns + 15) / 16 + kMaxProblems * (1 + kStreamKWideMaxBlocks);
  return static_cast<size_t>((blocks * 16 * rows * 4 + 255) / 256 * 256);
}

size_t streamk_part_bytes(int M) {
  const int rows = M < 16 ? M : 16;
  // per workgroup, the larger of the two layouts: narrow units (one block) or
  // wide ones
  const size_t narrow = static_cast<size_t>(kStreamKMaxWaves / kStreamKWaves) * 2;
  const size_t wide =
      static_cast<size_t>(kStreamKWideMaxWaves / kStreamKWaves) * 2 * kStreamKWideMaxBlocks;
  return (narrow > wide ? narrow : wide) * rows * 16 * sizeof(float);
}

}  // namespace w4a16_internal
