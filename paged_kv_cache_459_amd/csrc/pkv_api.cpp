// C ABI of libpkv: argument validation, launch heuristics and the split-context plumbing.
// Every check runs on the host before any HIP call; kernels only ever see validated shapes.

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdint>
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

// Partition length for pkv_decode_attn. Every partition of P tokens becomes one work-group of
// four waves, so P trades parallelism (short partitions) against per-wave pipeline length and
// merge traffic (long partitions).
int32_t choose_partition(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_ctx, pkv_dtype dt) {
  (void)B;
  (void)Hq;
  (void)Hkv;
  (void)dt;
  (void)max_ctx;
  return 512;
}

struct Split {
  int32_t P, MP;
  size_t bytes_ml, bytes;  // size of m (and l) region, rounded; total bytes
};

Split split_layout(int32_t B, int32_t Hq, int32_t hd, int32_t max_ctx, int32_t P) {
  Split s{};
  s.P = P;
  s.MP = max_ctx > 0 ? ceil_div(max_ctx, P) : 1;
  const size_t cells = static_cast<size_t>(B) * Hq * s.MP;
  s.bytes_ml = round_up256(cells * sizeof(float));
  s.bytes = 2 * s.bytes_ml + cells * hd * sizeof(float);
  return s;
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
      const int32_t b = t[static_cast<size_t>(i) * max_blocks + j];
      if (b < 0 || b >= NB) return PKV_ERR_INDEX;
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
  if (Hq > 65535) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
      (reinterpret_cast<uintptr_t>(context_lens) & 3u))
    return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

pkv::AttnParams make_params(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t hd, int32_t NB, int32_t max_blocks,
                            int32_t max_ctx, float scale, const Split& s, void* partials) {
  pkv::AttnParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.hd = hd;
  p.NB = NB;
  p.max_blocks = max_blocks;
  p.max_ctx = max_ctx;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  p.part_tokens = s.P;
  p.max_parts = s.MP;
  if (partials && s.MP > 1) {
    char* base = static_cast<char*>(partials);
    p.ws_m = reinterpret_cast<float*>(base);
    p.ws_l = reinterpret_cast<float*>(base + s.bytes_ml);
    p.ws_o = reinterpret_cast<float*>(base + 2 * s.bytes_ml);
  }
  return p;
}

pkv_status partition_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                          int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs, int32_t NB,
                          int32_t max_blocks, int32_t max_ctx, float scale, pkv_dtype dtype,
                          int32_t P, void* partials, size_t partials_bytes, void* stream,
                          bool merge_after) {
  pkv_status st = validate_decode(out, q, k_cache, v_cache, block_tables, context_lens, B, Hq,
                                  Hkv, hd, bs, NB, max_blocks, max_ctx, scale, dtype);
  if (st != PKV_OK) return st;
  if (P <= 0 || P % kBlockSize != 0 || P > kBlockSize * pkv::kMaxPartBlocks)
    return PKV_ERR_INVALID_ARG;
  const Split s = split_layout(B, Hq, hd, max_ctx, P);
  if (s.MP > 65535) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (s.MP > 1 && (!partials || partials_bytes < s.bytes)) return PKV_ERR_WORKSPACE;
  if (partials && !aligned16(partials)) return PKV_ERR_INVALID_ARG;
  auto hs = static_cast<hipStream_t>(stream);
  if (check_mode()) {
    st = check_decode_indices(block_tables, context_lens, B, NB, max_blocks, max_ctx, hs);
    if (st != PKV_OK) return st;
  }
  const pkv::AttnParams p = make_params(out, q, k_cache, v_cache, block_tables, context_lens, B,
                                        Hq, Hkv, hd, NB, max_blocks, max_ctx, scale, s, partials);
  const int32_t kernel = pkv::select_kernel(dtype, Hq / Hkv, g_kernel_choice.load());
  if (pkv::launch_partition(p, dtype, kernel, hs) != hipSuccess) return PKV_ERR_HIP;
  if (merge_after && s.MP > 1) {
    if (pkv::launch_merge(p, dtype, hs) != hipSuccess) return PKV_ERR_HIP;
  }
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

int32_t pkv_decode_partition_tokens(int32_t B, int32_t Hq, int32_t Hkv, int32_t hd,
                                    int32_t max_context_len, pkv_dtype dtype) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || !head_dim_ok(hd) || max_context_len < 0 ||
      !dtype_ok(dtype))
    return 0;
  return choose_partition(B, Hq, Hkv, max_context_len, dtype);
}

size_t pkv_decode_partials_bytes(int32_t B, int32_t Hq, int32_t hd, int32_t max_context_len,
                                 int32_t part_tokens) {
  if (B < 0 || Hq <= 0 || hd <= 0 || max_context_len < 0 || part_tokens <= 0) return 0;
  const Split s = split_layout(B, Hq, hd, max_context_len, part_tokens);
  return s.MP > 1 ? s.bytes : 0;
}

size_t pkv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t hd,
                                  int32_t max_context_len, pkv_dtype dtype) {
  const int32_t P = pkv_decode_partition_tokens(B, Hq, Hkv, hd, max_context_len, dtype);
  if (P == 0) return 0;
  return pkv_decode_partials_bytes(B, Hq, hd, max_context_len, P);
}

pkv_status pkv_decode_attn(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                           int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs, int32_t NB,
                           int32_t max_blocks, int32_t max_context_len, float scale,
                           pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(hd)) return PKV_ERR_UNSUPPORTED;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || max_context_len < 0 || B < 0) return PKV_ERR_INVALID_ARG;
  const int32_t P = choose_partition(B, Hq, Hkv, max_context_len, dtype);
  return partition_impl(out, q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, hd, bs,
                        NB, max_blocks, max_context_len, scale, dtype, P, workspace,
                        workspace_bytes, stream, /*merge_after=*/true);
}

pkv_status pkv_decode_partition(void* out, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables,
                                const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                int32_t hd, int32_t bs, int32_t NB, int32_t max_blocks,
                                int32_t max_context_len, float scale, pkv_dtype dtype,
                                int32_t part_tokens, void* partials, size_t partials_bytes,
                                void* stream) {
  return partition_impl(out, q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, hd, bs,
                        NB, max_blocks, max_context_len, scale, dtype, part_tokens, partials,
                        partials_bytes, stream, /*merge_after=*/false);
}

pkv_status pkv_decode_merge(void* out, const void* partials, size_t partials_bytes,
                            const int32_t* context_lens, int32_t B, int32_t Hq, int32_t hd,
                            int32_t max_context_len, pkv_dtype dtype, int32_t part_tokens,
                            void* stream) {
  if (!dtype_ok(dtype) || !head_dim_ok(hd)) return PKV_ERR_UNSUPPORTED;
  if (B < 0 || Hq <= 0 || Hq > 65535 || max_context_len < 0 || part_tokens <= 0 ||
      part_tokens % kBlockSize)
    return PKV_ERR_INVALID_ARG;
  const Split s = split_layout(B, Hq, hd, max_context_len, part_tokens);
  if (B == 0 || s.MP <= 1) return PKV_OK;  // nothing was split
  if (!out || !context_lens || !aligned16(out) || (reinterpret_cast<uintptr_t>(context_lens) & 3u))
    return PKV_ERR_INVALID_ARG;
  if (!partials || partials_bytes < s.bytes) return PKV_ERR_WORKSPACE;
  if (!aligned16(partials)) return PKV_ERR_INVALID_ARG;
  auto hs = static_cast<hipStream_t>(stream);
  if (check_mode()) {
    std::vector<int32_t> l;
    if (!copy_to_host(&l, context_lens, B, hs)) return PKV_ERR_HIP;
    for (int32_t x : l)
      if (x < 0 || x > max_context_len) return PKV_ERR_INDEX;
  }
  const pkv::AttnParams p = make_params(out, nullptr, nullptr, nullptr, nullptr, context_lens, B,
                                        Hq, Hq, hd, 1, 1, max_context_len, 1.0f, s,
                                        const_cast<void*>(partials));
  return pkv::launch_merge(p, dtype, hs) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int32_t pkv_set_attn_kernel(int32_t which) {
  if (which < pkv::kAuto || which > pkv::kMatrix) return -1;
  return g_kernel_choice.exchange(which);
}

}  // extern "C"
