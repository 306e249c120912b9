// C ABI of libpkv: argument validation, launch sizing and the stream/merge plumbing.
// Every check runs on the host before any HIP call; kernels only ever see validated shapes.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <climits>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <unordered_set>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_kernels.h"

namespace {
thread_local char g_last_error[256] = "";
}  // namespace

void pkv::note_message(const char* what) { snprintf(g_last_error, sizeof g_last_error, "%s", what); }

hipError_t pkv::note_error(const char* what, hipError_t err) {
  if (err != hipSuccess)
    snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what, hipGetErrorString(err),
             static_cast<int>(err));
  return err;
}

namespace {

using pkv::kBlockSize;

std::atomic<int32_t> g_kernel_choice{pkv::kAuto};

// PKV_CHECK=1 in the environment turns on host validation of device indices (read per call).
bool check_mode() {
  const char* e = std::getenv("PKV_CHECK");
  return e && e[0] == '1';
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int elem_bytes(pkv_dtype dt) { return dt == PKV_F32 ? 4 : 2; }

bool dtype_ok(pkv_dtype dt) { return dt == PKV_F32 || dt == PKV_F16 || dt == PKV_BF16; }

bool head_dim_ok(int32_t hd) { return hd == 64 || hd == 128; }

size_t round_up256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

constexpr int32_t kMaxBatch = 8192;  // sequences per stream launch (LDS holds B+1 prefix sums)

// Waves of the stream pass on the current device: the kernel's occupancy at the largest
// launch-time LDS, times the compute units. Independent of B, so one workspace size serves
// every sub-batch of a call.
int32_t device_workers(pkv_dtype dt, int32_t hd, int32_t kernel) {
  return pkv::default_workers(dt, hd, kernel, kMaxBatch);
}

int32_t current_kernel(pkv_dtype dt, int32_t Hq, int32_t Hkv) {
  return pkv::select_kernel(dt, Hq / Hkv, g_kernel_choice.load());
}

struct Layout {
  int32_t H, GS;          // head slots per sequence, q heads per slot
  size_t seg, ml, bytes;  // byte offsets of the (m, l) and o arrays; total size
};

// extra: cells past the workers' 2W (a plan's B*H private cells plus its shared cells).
Layout stream_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t hd, int32_t kernel,
                     int32_t W, int64_t extra = 0) {
  Layout L{};
  L.H = kernel == pkv::kMatrix ? Hkv : Hq;
  L.GS = kernel == pkv::kMatrix ? Hq / Hkv : 1;
  const size_t cells = (static_cast<size_t>(W) * 2 + static_cast<size_t>(extra)) * L.GS;
  L.seg = round_up256(static_cast<size_t>(B + 1) * sizeof(int32_t));
  L.ml = L.seg + round_up256(cells * 2 * sizeof(float));
  L.bytes = L.ml + cells * hd * sizeof(float);
  return L;
}

// Prefill workspace: (m, l) then o of the plan's cells (GS rows each); 0 bytes without cells.
struct PrefillLayout {
  size_t ml, o, bytes;
};

PrefillLayout prefill_layout(int64_t cells, int32_t GS, int32_t hd) {
  PrefillLayout L{};
  const size_t rows = static_cast<size_t>(cells) * GS;
  L.ml = 0;
  L.o = round_up256(rows * 2 * sizeof(float));
  L.bytes = rows == 0 ? 0 : L.o + rows * hd * sizeof(float);
  return L;
}

// Tile positions of a launch stay in int32: T + W <= B * max_blocks * H + W < 2^31.
bool stream_fits(int32_t B, int32_t max_blocks, int32_t H, int32_t W) {
  return B <= kMaxBatch &&
         static_cast<int64_t>(B) * max_blocks * H + W < (int64_t{1} << 31);
}

// Host-side validation of device indices (PKV_CHECK=1 only; synchronous).
template <typename T>
bool copy_to_host(std::vector<T>* dst, const T* src, size_t n, hipStream_t stream) {
  dst->resize(n);
  if (n == 0) return true;
  if (pkv::note_error("index check copy", hipMemcpyAsync(dst->data(), src, n * sizeof(T),
                                                        hipMemcpyDeviceToHost, stream)) != hipSuccess)
    return false;
  return pkv::note_error("index check sync", hipStreamSynchronize(stream)) == hipSuccess;
}

pkv_status check_decode_indices(const int32_t* tables, const int32_t* lens, int32_t B,
                                int32_t NB, int32_t max_blocks, int32_t max_ctx,
                                hipStream_t stream) {
  std::vector<int32_t> t, l;
  if (!copy_to_host(&l, lens, B, stream)) return PKV_ERR_HIP;
  if (!copy_to_host(&t, tables, static_cast<size_t>(B) * max_blocks, stream)) return PKV_ERR_HIP;
  for (int32_t i = 0; i < B; ++i) {
    if (l[i] < 0 || l[i] > max_ctx) return PKV_ERR_INDEX;
    const int32_t nb = ceil_div(l[i], kBlockSize);
    for (int32_t j = 0; j < nb; ++j) {
      const int32_t e = t[static_cast<size_t>(i) * max_blocks + j];
      if (e < 0 || (e & ~pkv::kSharedBit) >= NB) return PKV_ERR_INDEX;
    }
  }
  return PKV_OK;
}

pkv_status validate_decode(const void* out, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                           int32_t hd, int32_t bs, int32_t NB, int32_t max_blocks,
                           int32_t max_ctx, float scale, pkv_dtype dtype) {
  if (!dtype_ok(dtype)) return PKV_ERR_UNSUPPORTED;
  if (bs != kBlockSize || !head_dim_ok(hd)) return PKV_ERR_UNSUPPORTED;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || NB <= 0 || max_blocks <= 0 ||
      max_ctx < 0 || static_cast<int64_t>(max_blocks) * kBlockSize < max_ctx ||
      static_cast<int64_t>(NB) * kBlockSize >= (int64_t{1} << 31) || !std::isfinite(scale))
    return PKV_ERR_INVALID_ARG;
  // Head slots travel in the upper half of a signed 32-bit tile word (at most 32767), and the
  // merge grid's rows are q heads plus kv heads (at most 65535): Hq <= 32767 covers both.
  if (Hq > 32767) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
      (reinterpret_cast<uintptr_t>(context_lens) & 3u))
    return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

pkv::StreamParams make_params(void* out, const void* q, const void* k_new, const void* v_new,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_tables,
                              const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                              int32_t hd, int32_t NB, int32_t max_blocks, int32_t max_ctx,
                              float scale, int32_t W, const Layout& L, void* workspace) {
  pkv::StreamParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.k_new = k_new;
  p.v_new = v_new;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.hd = hd;
  p.NB = NB;
  p.max_blocks = max_blocks;
  p.max_ctx = max_ctx;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  p.num_workers = W;
  char* base = static_cast<char*>(workspace);
  p.ws_seg = reinterpret_cast<int32_t*>(base);
  p.ws_ml = reinterpret_cast<float*>(base + L.seg);
  p.ws_o = reinterpret_cast<float*>(base + L.ml);
  p.table_rows = B;
  return p;
}

// One stream pass (and, if asked, its merge) over B <= kMaxBatch sequences.
pkv_status stream_impl(void* out, const void* q, const void* k_new, const void* v_new,
                       const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                       int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs, int32_t NB,
                       int32_t max_blocks, int32_t max_ctx, float scale, pkv_dtype dtype,
                       int32_t W, void* workspace, size_t workspace_bytes, void* stream,
                       bool merge_after, bool index_checks = true) {
  pkv_status st = validate_decode(out, q, k_cache, v_cache, block_tables, context_lens, B, Hq,
                                  Hkv, hd, bs, NB, max_blocks, max_ctx, scale, dtype);
  if (st != PKV_OK) return st;
  if ((k_new == nullptr) != (v_new == nullptr)) return PKV_ERR_INVALID_ARG;
  if (k_new && B > 0 && (!aligned16(k_new) || !aligned16(v_new))) return PKV_ERR_INVALID_ARG;
  if (W <= 0 || W % pkv::kWaves != 0) return PKV_ERR_INVALID_ARG;
  const int32_t kernel = current_kernel(dtype, Hq, Hkv);
  const Layout L = stream_layout(B, Hq, Hkv, hd, kernel, W);
  if (!stream_fits(B, max_blocks, L.H, W)) return PKV_ERR_UNSUPPORTED;
  if (B == 0) return PKV_OK;
  if (!workspace || workspace_bytes < L.bytes) return PKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PKV_ERR_INVALID_ARG;
  auto hs = static_cast<hipStream_t>(stream);
  if (index_checks && check_mode()) {
    st = check_decode_indices(block_tables, context_lens, B, NB, max_blocks, max_ctx, hs);
    if (st != PKV_OK) return st;
  }
  const pkv::StreamParams p = make_params(out, q, k_new, v_new, k_cache, v_cache, block_tables,
                                          context_lens, B, Hq, Hkv, hd, NB, max_blocks, max_ctx,
                                          scale, W, L, workspace);
  if (pkv::launch_stream(p, dtype, kernel, hs) != hipSuccess) return PKV_ERR_HIP;
  if (merge_after && pkv::launch_merge(p, dtype, kernel, hs) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_last_error; }

const char* pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_OUT_OF_BLOCKS: return "PKV_ERR_OUT_OF_BLOCKS";
    case PKV_ERR_UNKNOWN_SEQ: return "PKV_ERR_UNKNOWN_SEQ";
    case PKV_ERR_SEQ_EXISTS: return "PKV_ERR_SEQ_EXISTS";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_INDEX: return "PKV_ERR_INDEX";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    default: return "PKV_ERR_UNKNOWN_STATUS";
  }
}

size_t pkv_cache_bytes(int32_t NB, int32_t Hkv, int32_t hd, int32_t bs, pkv_dtype dtype) {
  if (NB <= 0 || Hkv <= 0 || hd <= 0 || bs <= 0 || !dtype_ok(dtype)) return 0;
  return static_cast<size_t>(NB) * Hkv * hd * bs * elem_bytes(dtype);
}

pkv_status pkv_write(const void* k, const void* v, void* k_cache, void* v_cache,
                     const int32_t* slot_mapping, int32_t T, int32_t Hkv, int32_t hd, int32_t bs,
                     int32_t NB, pkv_dtype dtype, void* stream) {
  if (!dtype_ok(dtype) || bs != kBlockSize || !head_dim_ok(hd)) return PKV_ERR_UNSUPPORTED;
  if (T < 0 || Hkv <= 0 || NB <= 0 || static_cast<int64_t>(NB) * kBlockSize >= (int64_t{1} << 31))
    return PKV_ERR_INVALID_ARG;
  if (Hkv > 65535) return PKV_ERR_UNSUPPORTED;  // one grid row per kv head
  if (T == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 3u))
    return PKV_ERR_INVALID_ARG;
  auto hs = static_cast<hipStream_t>(stream);
  if (check_mode()) {
    std::vector<int32_t> s;
    if (!copy_to_host(&s, slot_mapping, T, hs)) return PKV_ERR_HIP;
    std::unordered_set<int32_t> seen;
    for (int32_t x : s) {
      if (x >= NB * kBlockSize) return PKV_ERR_INDEX;
      if (x >= 0 && !seen.insert(x).second) return PKV_ERR_INDEX;
    }
  }
  pkv::WriteParams p{k, v, k_cache, v_cache, slot_mapping, T, Hkv, hd, NB};
  return pkv::launch_write(p, dtype, hs) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_probe_read(const void* base, size_t base_bytes, const int32_t* tile_ids,
                          int32_t n, int32_t num_workers, uint32_t* sink, void* stream) {
  if (n < 0 || num_workers <= 0 || num_workers % pkv::kWaves != 0) return PKV_ERR_INVALID_ARG;
  if (n == 0) return PKV_OK;
  const size_t tiles = base_bytes / 4096;
  if (!base || !tile_ids || !sink || tiles == 0 || tiles > static_cast<size_t>(INT32_MAX) ||
      !aligned16(base) || (reinterpret_cast<uintptr_t>(tile_ids) & 3u) ||
      (reinterpret_cast<uintptr_t>(sink) & 3u))
    return PKV_ERR_INVALID_ARG;
  return pkv::launch_probe_read(base, static_cast<int32_t>(tiles), tile_ids, n, num_workers, sink,
                                static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                           int32_t n, int32_t Hkv, int32_t hd, int32_t bs, int32_t NB,
                           pkv_dtype dtype, void* stream) {
  if (!dtype_ok(dtype) || bs != kBlockSize || !head_dim_ok(hd)) return PKV_ERR_UNSUPPORTED;
  if (n < 0 || Hkv <= 0 || NB <= 0 || static_cast<int64_t>(NB) * kBlockSize >= (int64_t{1} << 31))
    return PKV_ERR_INVALID_ARG;
  if (pkv::copy_blocks_grid_y(Hkv, hd, dtype) > 65535) return PKV_ERR_UNSUPPORTED;
  if (n == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src || !dst) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache) || (reinterpret_cast<uintptr_t>(src) & 3u) ||
      (reinterpret_cast<uintptr_t>(dst) & 3u))
    return PKV_ERR_INVALID_ARG;
  auto hs = static_cast<hipStream_t>(stream);
  if (check_mode()) {
    std::vector<int32_t> s, d;
    if (!copy_to_host(&s, src, n, hs) || !copy_to_host(&d, dst, n, hs)) return PKV_ERR_HIP;
    std::unordered_set<int32_t> targets, sources;
    for (int32_t i = 0; i < n; ++i) {
      if (s[i] >= NB || d[i] >= NB) return PKV_ERR_INDEX;
      if (s[i] < 0 || d[i] < 0) continue;  // padding pair
      if (!targets.insert(d[i]).second) return PKV_ERR_INDEX;
      sources.insert(s[i]);
    }
    for (int32_t t : targets)
      if (sources.count(t)) return PKV_ERR_INDEX;
  }
  pkv::CopyParams p{k_cache, v_cache, src, dst, n, Hkv, hd, NB};
  return pkv::launch_copy_blocks(p, dtype, hs) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

size_t pkv_decode_plan_max_ints(int32_t B, int32_t max_blocks) {
  if (B < 0 || max_blocks <= 0) return 0;
  return pkv::kPlanHeader + 3 * static_cast<size_t>(B) + 1 +
         static_cast<size_t>(pkv::kUnitInts + 2) * B * max_blocks;
}

pkv_status pkv_decode_plan(const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                           int32_t max_blocks, int32_t max_context_len, int32_t Hq, int32_t Hkv,
                           int32_t NB, pkv_dtype dtype, int32_t max_group, int32_t* plan,
                           size_t capacity, size_t* plan_ints) {
  if (!dtype_ok(dtype)) return PKV_ERR_UNSUPPORTED;
  if (max_group < 0 || max_group > pkv::kRowsPerTile) return PKV_ERR_INVALID_ARG;
  if (B < 0 || B > kMaxBatch || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_blocks <= 0 ||
      NB <= 0 || max_context_len < 0 ||
      static_cast<int64_t>(max_blocks) * kBlockSize < max_context_len || !plan_ints)
    return PKV_ERR_INVALID_ARG;
  if (B > 0 && (!block_tables || !context_lens)) return PKV_ERR_INVALID_ARG;
  const int32_t G = Hq / Hkv;
  const int32_t kernel = current_kernel(dtype, Hq, Hkv);
  const int32_t H = kernel == pkv::kMatrix ? Hkv : Hq;
  const int32_t GS = kernel == pkv::kMatrix ? G : 1;
  // The shared pass reads a chunk once per tile of 16 / G members: for G > 4 (two sequences
  // or fewer per tile) the matrix-core stream kernel, whose sharers re-read the blocks from
  // the L2, is faster, so such batches get no runs.
  const bool share = dtype != PKV_F32 && G <= (max_group ? max_group : pkv::kMaxPlannedGroup);
  std::vector<int32_t> v;
  pkv::plan_build(block_tables, context_lens, B, max_blocks, max_context_len, NB, H, GS, G,
                  pkv::kPlanChunk, share, &v);
  *plan_ints = v.size();
  if (!plan || capacity < v.size()) return PKV_ERR_WORKSPACE;
  std::memcpy(plan, v.data(), v.size() * sizeof(int32_t));
  return PKV_OK;
}

}  // extern "C"

namespace pkv {

// Launches of a validated plan's shared and stream passes under the automatic choice: one
// where the one-launch kernel exists and the shared pass reads at least as many (block, head)
// tiles as the stream pass, else two (one when the plan has no units: no shared pass). In the
// one launch the shared pass's work-groups start first and the stream pass's short ranges
// fill its tail; where the stream pass dominates, the two passes in one launch measured no
// faster than apart (they compete for the same memory path), so they stay apart.
int32_t planned_launches(const int32_t* plan, int32_t B, int32_t Hkv, int32_t dtype,
                         int32_t kernel, int32_t W) {
  const int32_t H = plan[2], U = plan[4];
  if (U == 0) return 1;
  if (!fused_kernel_exists(dtype, kernel, W)) return 2;
  const int32_t* skip = plan + kPlanHeader;
  const int32_t* blocks = skip + B;
  const int32_t* units = blocks + 2 * static_cast<size_t>(B) + 1;  // past sh_ptr[B + 1]
  int64_t stream_tiles = 0, shared_tiles = 0;
  for (int32_t s = 0; s < B; ++s) stream_tiles += std::max(0, blocks[s] - skip[s]);
  for (int32_t u = 0; u < U; ++u)
    shared_tiles += units[static_cast<size_t>(u) * kUnitInts + 2] -
                    units[static_cast<size_t>(u) * kUnitInts + 1];
  return shared_tiles * Hkv >= stream_tiles * H ? 1 : 2;
}

}  // namespace pkv

extern "C" {

int32_t pkv_decode_planned_launches(const int32_t* plan, size_t plan_ints, int32_t B,
                                    int32_t Hq, int32_t Hkv, int32_t max_blocks,
                                    pkv_dtype dtype, int32_t num_workers) {
  if (!plan || B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_blocks <= 0 ||
      !dtype_ok(dtype) || num_workers <= 0 || num_workers % pkv::kWaves != 0)
    return 0;
  const int32_t kernel = current_kernel(dtype, Hq, Hkv);
  const int32_t G = Hq / Hkv;
  const int32_t H = kernel == pkv::kMatrix ? Hkv : Hq;
  const int32_t GS = kernel == pkv::kMatrix ? G : 1;
  pkv::PlanView pv;
  if (!pkv::plan_check(plan, plan_ints, B, max_blocks, H, GS, G, false, &pv)) return 0;
  return pkv::planned_launches(plan, B, Hkv, dtype, kernel, num_workers);
}

size_t pkv_decode_planned_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t hd,
                                          pkv_dtype dtype, int32_t num_workers,
                                          const int32_t* plan, size_t plan_ints) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || !dtype_ok(dtype) || !head_dim_ok(hd) ||
      num_workers <= 0 || num_workers % pkv::kWaves != 0 || !plan ||
      plan_ints < static_cast<size_t>(pkv::kPlanHeader))
    return 0;
  const int32_t kernel = current_kernel(dtype, Hq, Hkv);
  const Layout L0 = stream_layout(B, Hq, Hkv, hd, kernel, num_workers);
  if (plan[0] != pkv::kPlanMagic || plan[1] != B || plan[2] != L0.H || plan[3] != L0.GS ||
      plan[7] < 0)
    return 0;
  const int64_t extra = static_cast<int64_t>(B) * L0.H + plan[7];
  return stream_layout(B, Hq, Hkv, hd, kernel, num_workers, extra).bytes;
}

pkv_status pkv_decode_planned(int32_t pass, void* out, const void* q, const void* k_new,
                              const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                              int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs, int32_t NB,
                              int32_t max_blocks, int32_t max_context_len, float scale,
                              pkv_dtype dtype, const int32_t* plan_host, const int32_t* plan_dev,
                              size_t plan_ints, int32_t num_workers, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (pass < 0 || pass > 5) return PKV_ERR_INVALID_ARG;
  pkv_status st = validate_decode(out, q, k_cache, v_cache, block_tables, context_lens, B, Hq,
                                  Hkv, hd, bs, NB, max_blocks, max_context_len, scale, dtype);
  if (st != PKV_OK) return st;
  if ((k_new == nullptr) != (v_new == nullptr)) return PKV_ERR_INVALID_ARG;
  if (k_new && B > 0 && (!aligned16(k_new) || !aligned16(v_new))) return PKV_ERR_INVALID_ARG;
  if (num_workers <= 0 || num_workers % pkv::kWaves != 0) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  const int32_t W = num_workers;
  const int32_t G = Hq / Hkv;
  const int32_t kernel = current_kernel(dtype, Hq, Hkv);
  const Layout L0 = stream_layout(B, Hq, Hkv, hd, kernel, W);
  if (!stream_fits(B, max_blocks, L0.H, W)) return PKV_ERR_UNSUPPORTED;
  if (!plan_host || !plan_dev || (reinterpret_cast<uintptr_t>(plan_dev) & 3u))
    return PKV_ERR_INVALID_ARG;
  pkv::PlanView pv;
  if (!pkv::plan_check(plan_host, plan_ints, B, max_blocks, L0.H, L0.GS, G, k_new != nullptr,
                       &pv))
    return PKV_ERR_INVALID_ARG;
  if (pv.U > 0 && (dtype == PKV_F32 || G > pkv::kRowsPerTile)) return PKV_ERR_UNSUPPORTED;
  // one wave per (unit, kv head), plus the stream workers in the one-launch form: the launch's
  // work-items must stay within 32-bit grid indexing
  if ((static_cast<int64_t>(pv.U) * Hkv + W + 8 * pkv::kWaves) * 64 > INT32_MAX)
    return PKV_ERR_UNSUPPORTED;
  const Layout L = stream_layout(B, Hq, Hkv, hd, kernel, W, static_cast<int64_t>(B) * L0.H + pv.cells);
  if (!workspace || workspace_bytes < L.bytes) return PKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PKV_ERR_INVALID_ARG;
  auto hs = static_cast<hipStream_t>(stream);
  if (check_mode()) {
    st = check_decode_indices(block_tables, context_lens, B, NB, max_blocks, max_context_len, hs);
    if (st != PKV_OK) return st;
  }
  pkv::StreamParams p = make_params(out, q, k_new, v_new, k_cache, v_cache, block_tables,
                                    context_lens, B, Hq, Hkv, hd, NB, max_blocks,
                                    max_context_len, scale, W, L, workspace);
  const int32_t* base = plan_dev + pkv::kPlanHeader;
  p.skip = base;
  p.sh_ptr = base + 2 * static_cast<size_t>(B);
  p.units = p.sh_ptr + B + 1;
  p.members = p.units + static_cast<size_t>(pv.U) * pkv::kUnitInts;
  p.sh_list = p.members + plan_host[5];
  p.num_units = pv.U;
  p.shared_cells = pv.cells;
  p.shared_base = 2 * W + B * L0.H;
  const bool one = pass == 5 || ((pass == 0 || pass == 4) &&
                                 pkv::planned_launches(plan_host, B, Hkv, dtype, kernel, W) == 1);
  if (one && pkv::launch_fused(p, dtype, kernel, hs) != hipSuccess) return PKV_ERR_HIP;
  if ((pass == 1 || (!one && (pass == 0 || pass == 4))) &&
      pkv::launch_shared(p, dtype, kernel, hs) != hipSuccess)
    return PKV_ERR_HIP;
  if ((pass == 2 || (!one && (pass == 0 || pass == 4))) &&
      pkv::launch_stream(p, dtype, kernel, hs) != hipSuccess)
    return PKV_ERR_HIP;
  if ((pass == 0 || pass == 3) && pkv::launch_merge(p, dtype, kernel, hs) != hipSuccess)
    return PKV_ERR_HIP;
  return PKV_OK;
}

pkv_status pkv_prefill_plan(const int32_t* query_start, const int32_t* context_lens, int32_t S,
                            int32_t max_blocks, int32_t max_context_len, int32_t Hq, int32_t Hkv,
                            pkv_dtype dtype, int32_t* plan, size_t capacity, size_t* plan_ints) {
  if (!dtype_ok(dtype)) return PKV_ERR_UNSUPPORTED;
  if (S < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_blocks <= 0 || max_context_len < 0 ||
      static_cast<int64_t>(max_blocks) * kBlockSize < max_context_len || !plan_ints ||
      (S > 0 && (!query_start || !context_lens)))
    return PKV_ERR_INVALID_ARG;
  if (dtype == PKV_F32 || Hq / Hkv > pkv::kRowsPerTile) return PKV_ERR_UNSUPPORTED;
  if (S == 0 ? (query_start && query_start[0] != 0) : query_start[0] != 0)
    return PKV_ERR_INVALID_ARG;
  for (int32_t s = 0; s < S; ++s) {
    const int64_t q = static_cast<int64_t>(query_start[s + 1]) - query_start[s];
    if (q < 0 || context_lens[s] < q || context_lens[s] > max_context_len)
      return PKV_ERR_INVALID_ARG;
  }
  const int32_t T = S > 0 ? query_start[S] : 0;
  if (static_cast<int64_t>(T) * Hq * 64 >= (int64_t{1} << 31)) return PKV_ERR_UNSUPPORTED;
  const int32_t G = Hq / Hkv;
  std::vector<int32_t> v;
  const int32_t zero = 0;
  const int32_t* qsp = S > 0 ? query_start : &zero;
  const int32_t chunk = pkv::prefill_chunk(qsp, context_lens, S, Hkv, pkv::prefill_tile_rows(G),
                                           pkv::kPrefillMaxBlocks, pkv::kPrefillMinGroups);
  pkv::prefill_plan_build(qsp, context_lens, S, Hkv, G, pkv::prefill_tile_rows(G), chunk, &v);
  *plan_ints = v.size();
  if (!plan || capacity < v.size()) return PKV_ERR_WORKSPACE;
  std::memcpy(plan, v.data(), v.size() * sizeof(int32_t));
  return PKV_OK;
}

size_t pkv_prefill_workspace_bytes(int32_t Hq, int32_t Hkv, int32_t hd, const int32_t* plan,
                                   size_t plan_ints) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || !head_dim_ok(hd) || !plan ||
      plan_ints < static_cast<size_t>(pkv::kPlanHeader) || plan[0] != pkv::kPrefillMagic ||
      plan[2] != Hkv || plan[3] != Hq / Hkv || plan[7] < 0)
    return static_cast<size_t>(-1);
  return prefill_layout(plan[7], Hq / Hkv, hd).bytes;
}

pkv_status pkv_prefill_attn(int32_t pass, void* out, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables, int32_t S,
                            int32_t T, int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs,
                            int32_t NB, int32_t max_blocks, int32_t max_context_len, float scale,
                            pkv_dtype dtype, const int32_t* plan_host, const int32_t* plan_dev,
                            size_t plan_ints, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (pass < 0 || pass > 2) return PKV_ERR_INVALID_ARG;
  if (!dtype_ok(dtype) || bs != kBlockSize || !head_dim_ok(hd)) return PKV_ERR_UNSUPPORTED;
  if (S < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Hq > 65535 || NB <= 0 ||
      max_blocks <= 0 || max_context_len < 0 ||
      static_cast<int64_t>(max_blocks) * kBlockSize < max_context_len ||
      static_cast<int64_t>(NB) * kBlockSize >= (int64_t{1} << 31) || !std::isfinite(scale))
    return PKV_ERR_INVALID_ARG;
  if (dtype == PKV_F32 || Hq / Hkv > pkv::kRowsPerTile) return PKV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(T) * Hq * 64 >= (int64_t{1} << 31)) return PKV_ERR_UNSUPPORTED;
  if (T == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !plan_host || !plan_dev)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
      (reinterpret_cast<uintptr_t>(plan_dev) & 3u))
    return PKV_ERR_INVALID_ARG;
  const int32_t G = Hq / Hkv;
  pkv::PlanView pv;
  if (!pkv::prefill_plan_check(plan_host, plan_ints, T, S, max_blocks, max_context_len, Hkv, G,
                               pkv::prefill_tile_rows(G), pkv::kPrefillMaxBlocks, &pv))
    return PKV_ERR_INVALID_ARG;
  // one work-group of 256 work-items per (unit, kv head): within 32-bit grid indexing
  if (static_cast<int64_t>(pv.U) * Hkv * 256 > INT32_MAX) return PKV_ERR_UNSUPPORTED;
  const PrefillLayout L = prefill_layout(pv.cells, G, hd);
  if (L.bytes > 0 && (!workspace || workspace_bytes < L.bytes)) return PKV_ERR_WORKSPACE;
  if (L.bytes > 0 && !aligned16(workspace)) return PKV_ERR_INVALID_ARG;
  auto hs = static_cast<hipStream_t>(stream);
  pkv::StreamParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.B = T;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.hd = hd;
  p.NB = NB;
  p.max_blocks = max_blocks;
  p.max_ctx = max_context_len;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  char* ws = static_cast<char*>(workspace);
  p.ws_ml = L.bytes > 0 ? reinterpret_cast<float*>(ws + L.ml) : nullptr;
  p.ws_o = L.bytes > 0 ? reinterpret_cast<float*>(ws + L.o) : nullptr;
  const int32_t* base = plan_dev + pkv::kPlanHeader;
  p.skip = base;
  p.row_vis = base + T;
  p.sh_ptr = base + 2 * static_cast<size_t>(T);
  p.units = p.sh_ptr + T + 1;
  p.members = p.units + static_cast<size_t>(pv.U) * pkv::kUnitInts;
  p.sh_list = p.members + plan_host[5];
  p.num_units = pv.U;
  p.shared_cells = pv.cells;
  p.shared_base = 0;
  p.table_rows = S;
  if ((pass == 0 || pass == 1) && pkv::launch_prefill(p, dtype, hs) != hipSuccess)
    return PKV_ERR_HIP;
  if ((pass == 0 || pass == 2) && pv.has_shared &&
      pkv::launch_merge(p, dtype, pkv::kMatrix, hs) != hipSuccess)
    return PKV_ERR_HIP;
  return PKV_OK;
}

int32_t pkv_decode_kernel(int32_t Hq, int32_t Hkv, pkv_dtype dtype) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || !dtype_ok(dtype)) return 0;
  return current_kernel(dtype, Hq, Hkv);
}

int32_t pkv_decode_num_workers(int32_t Hq, int32_t Hkv, int32_t hd, pkv_dtype dtype) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || !dtype_ok(dtype) || !head_dim_ok(hd)) return 0;
  return device_workers(dtype, hd, current_kernel(dtype, Hq, Hkv));
}

size_t pkv_decode_stream_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t hd,
                                         pkv_dtype dtype, int32_t num_workers) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || !dtype_ok(dtype) || !head_dim_ok(hd) ||
      num_workers <= 0 || num_workers % pkv::kWaves != 0)
    return 0;
  return stream_layout(B, Hq, Hkv, hd, current_kernel(dtype, Hq, Hkv), num_workers).bytes;
}

size_t pkv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t hd,
                                  int32_t max_context_len, pkv_dtype dtype) {
  if (B <= 0 || max_context_len < 0) return 0;
  const int32_t W = pkv_decode_num_workers(Hq, Hkv, hd, dtype);
  if (W == 0) return 0;
  return pkv_decode_stream_workspace_bytes(B < kMaxBatch ? B : kMaxBatch, Hq, Hkv, hd, dtype, W);
}

}  // extern "C"

namespace {

// pkv_decode_attn and pkv_decode_append_attn: stream + merge per sub-batch.
pkv_status decode_all(void* out, const void* q, const void* k_new, const void* v_new,
                      const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                      int32_t hd, int32_t bs, int32_t NB, int32_t max_blocks,
                      int32_t max_context_len, float scale, pkv_dtype dtype, void* workspace,
                      size_t workspace_bytes, void* stream, bool index_checks = true) {
  pkv_status st = validate_decode(out, q, k_cache, v_cache, block_tables, context_lens, B, Hq,
                                  Hkv, hd, bs, NB, max_blocks, max_context_len, scale, dtype);
  if (st != PKV_OK || B == 0) return st;
  const int32_t W = pkv_decode_num_workers(Hq, Hkv, hd, dtype);
  if (W == 0) {
    (void)pkv::note_error("device occupancy query", hipErrorInvalidDevice);
    return PKV_ERR_HIP;
  }
  const Layout L = stream_layout(1, Hq, Hkv, hd, current_kernel(dtype, Hq, Hkv), W);
  // Sub-batches: at most kMaxBatch sequences, and few enough tiles for int32 positions.
  int32_t chunk = B < kMaxBatch ? B : kMaxBatch;
  while (chunk > 0 && !stream_fits(chunk, max_blocks, L.H, W)) chunk /= 2;
  if (chunk == 0) return PKV_ERR_UNSUPPORTED;
  const size_t row_bytes = static_cast<size_t>(Hq) * hd * elem_bytes(dtype);
  const size_t new_bytes = static_cast<size_t>(Hkv) * hd * elem_bytes(dtype);
  for (int32_t i0 = 0; i0 < B; i0 += chunk) {
    const int32_t n = B - i0 < chunk ? B - i0 : chunk;
    st = stream_impl(static_cast<char*>(out) + i0 * row_bytes,
                     static_cast<const char*>(q) + i0 * row_bytes,
                     k_new ? static_cast<const char*>(k_new) + i0 * new_bytes : nullptr,
                     v_new ? static_cast<const char*>(v_new) + i0 * new_bytes : nullptr,
                     k_cache, v_cache, block_tables + static_cast<size_t>(i0) * max_blocks,
                     context_lens + i0, n, Hq, Hkv, hd, bs, NB, max_blocks, max_context_len,
                     scale, dtype, W, workspace, workspace_bytes, stream, /*merge_after=*/true,
                     index_checks);
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_decode_attn(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                           int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs, int32_t NB,
                           int32_t max_blocks, int32_t max_context_len, float scale,
                           pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return decode_all(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, B,
                    Hq, Hkv, hd, bs, NB, max_blocks, max_context_len, scale, dtype, workspace,
                    workspace_bytes, stream);
}

pkv_status pkv_decode_append_attn(void* out, const void* q, const void* k_new,
                                  const void* v_new, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs,
                                  int32_t NB, int32_t max_blocks, int32_t max_context_len,
                                  float scale, pkv_dtype dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (B > 0 && (!k_new || !v_new)) return PKV_ERR_INVALID_ARG;
  return decode_all(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, B, Hq,
                    Hkv, hd, bs, NB, max_blocks, max_context_len, scale, dtype, workspace,
                    workspace_bytes, stream);
}

pkv_status pkv_decode_append_attn_noalloc(void* out, const void* q, const void* k_new,
                                          const void* v_new, void* k_cache, void* v_cache,
                                          const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t B, int32_t Hq,
                                          int32_t Hkv, int32_t hd, int32_t bs, int32_t NB,
                                          int32_t max_blocks, int32_t max_context_len,
                                          float scale, pkv_dtype dtype, void* stream) {
  if (B > 0 && (!k_new || !v_new)) return PKV_ERR_INVALID_ARG;
  pkv_status st = validate_decode(out, q, k_cache, v_cache, block_tables, context_lens, B, Hq,
                                  Hkv, hd, bs, NB, max_blocks, max_context_len, scale, dtype);
  if (st != PKV_OK || B == 0) return st;
  const size_t need = pkv_decode_workspace_bytes(B, Hq, Hkv, hd, max_context_len, dtype);
  if (need > pkv::kStaticScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof msg,
             "pkv_decode_append_attn_noalloc: this shape needs %zu bytes of scratch, more than "
             "the %zu the library holds per device",
             need, pkv::kStaticScratchBytes);
    pkv::note_message(msg);
    return PKV_ERR_WORKSPACE;
  }
  void* scratch = pkv::static_scratch();
  if (scratch == nullptr) return PKV_ERR_HIP;
  return decode_all(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, B, Hq,
                    Hkv, hd, bs, NB, max_blocks, max_context_len, scale, dtype, scratch,
                    pkv::kStaticScratchBytes, stream, /*index_checks=*/false);
}

pkv_status pkv_decode_stream(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs,
                             int32_t NB, int32_t max_blocks, int32_t max_context_len,
                             float scale, pkv_dtype dtype, int32_t num_workers, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return stream_impl(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, B,
                     Hq, Hkv, hd, bs, NB, max_blocks, max_context_len, scale, dtype,
                     num_workers, workspace, workspace_bytes, stream, /*merge_after=*/false);
}

pkv_status pkv_decode_append_stream(void* out, const void* q, const void* k_new,
                                    const void* v_new, void* k_cache, void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    int32_t B, int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs,
                                    int32_t NB, int32_t max_blocks, int32_t max_context_len,
                                    float scale, pkv_dtype dtype, int32_t num_workers,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (B > 0 && (!k_new || !v_new)) return PKV_ERR_INVALID_ARG;
  return stream_impl(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, B, Hq,
                     Hkv, hd, bs, NB, max_blocks, max_context_len, scale, dtype, num_workers,
                     workspace, workspace_bytes, stream, /*merge_after=*/false);
}

}  // extern "C"

namespace {

pkv_status merge_impl(void* out, const void* k_new, const void* v_new, void* k_cache,
                      void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                      int32_t NB, int32_t max_blocks, int32_t max_ctx, const void* workspace,
                      size_t workspace_bytes, int32_t B, int32_t Hq, int32_t Hkv, int32_t hd,
                      pkv_dtype dtype, int32_t num_workers, void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(hd)) return PKV_ERR_UNSUPPORTED;
  if (B < 0 || B > kMaxBatch || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Hq > 32767 ||
      num_workers <= 0 || num_workers % pkv::kWaves != 0)
    return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (!out || !aligned16(out)) return PKV_ERR_INVALID_ARG;
  const int32_t kernel = current_kernel(dtype, Hq, Hkv);
  const Layout L = stream_layout(B, Hq, Hkv, hd, kernel, num_workers);
  if (!workspace || workspace_bytes < L.bytes) return PKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PKV_ERR_INVALID_ARG;
  const pkv::StreamParams p = make_params(out, nullptr, k_new, v_new, k_cache, v_cache,
                                          block_tables, context_lens, B, Hq, Hkv, hd, NB,
                                          max_blocks, max_ctx, 1.0f, num_workers, L,
                                          const_cast<void*>(workspace));
  return pkv::launch_merge(p, dtype, kernel, static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

}  // namespace

extern "C" {

pkv_status pkv_decode_merge(void* out, const void* workspace, size_t workspace_bytes, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t hd, pkv_dtype dtype,
                            int32_t num_workers, void* stream) {
  return merge_impl(out, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 1, 0,
                    workspace, workspace_bytes, B, Hq, Hkv, hd, dtype, num_workers, stream);
}

pkv_status pkv_decode_append_merge(void* out, const void* k_new, const void* v_new,
                                   void* k_cache, void* v_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, int32_t NB, int32_t max_blocks,
                                   int32_t max_context_len, const void* workspace,
                                   size_t workspace_bytes, int32_t B, int32_t Hq, int32_t Hkv,
                                   int32_t hd, pkv_dtype dtype, int32_t num_workers,
                                   void* stream) {
  if (B > 0 && (!k_new || !v_new || !k_cache || !v_cache || !block_tables || !context_lens ||
                !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
                !aligned16(v_cache) || NB <= 0 || max_blocks <= 0 || max_context_len < 0 ||
                static_cast<int64_t>(max_blocks) * kBlockSize < max_context_len ||
                (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
                (reinterpret_cast<uintptr_t>(context_lens) & 3u)))
    return PKV_ERR_INVALID_ARG;
  return merge_impl(out, k_new, v_new, k_cache, v_cache, block_tables, context_lens, NB,
                    max_blocks, max_context_len, workspace, workspace_bytes, B, Hq, Hkv, hd,
                    dtype, num_workers, stream);
}

int32_t pkv_set_attn_kernel(int32_t which) {
  if (which < pkv::kAuto || which > pkv::kMatrix) return -1;
  return g_kernel_choice.exchange(which);
}

}  // extern "C"
