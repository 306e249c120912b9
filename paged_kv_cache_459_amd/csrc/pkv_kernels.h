// Internal launcher interface between the C ABI (pkv_api.cpp) and the HIP kernels.
// Not installed; callers use include/pkv.h.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace pkv {

constexpr int kBlockSize = 16;      // tokens per block ([P3] §3.2; [P1] §二 example)
constexpr int kMaxPartBlocks = 256;  // largest partition: 256 blocks = 4096 tokens

enum AttnKernel : int32_t { kAuto = 0, kVector = 1, kMatrix = 2 };

struct WriteParams {
  const void* k;
  const void* v;
  void* k_cache;
  void* v_cache;
  const int32_t* slots;
  int32_t T, Hkv, hd, NB;
};

struct AttnParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t B, Hq, Hkv, hd, NB, max_blocks, max_ctx;
  float scale_log2;     // softmax scale times log2(e): scores are kept in base-2 units
  int32_t part_tokens;  // P, a multiple of 16, at most 16 * kMaxPartBlocks
  int32_t max_parts;    // MP = ceil(max_ctx / P), at least 1
  float* ws_m;          // [B][Hq][MP] (natural-log units), null if MP == 1
  float* ws_l;          // [B][Hq][MP]
  float* ws_o;          // [B][Hq][MP][hd]
};

// dtype: 0 f32, 1 f16, 2 bf16 (pkv_dtype). Return the launch status (hipGetLastError).
hipError_t launch_write(const WriteParams& p, int32_t dtype, hipStream_t stream);
hipError_t launch_partition(const AttnParams& p, int32_t dtype, int32_t kernel,
                            hipStream_t stream);
hipError_t launch_merge(const AttnParams& p, int32_t dtype, hipStream_t stream);

// Records the failing step and the HIP error text for pkv_last_error(); returns err.
hipError_t note_error(const char* what, hipError_t err);

// Which kernel launch_partition runs for this shape and request (kVector or kMatrix).
int32_t select_kernel(int32_t dtype, int32_t G, int32_t request);

}  // namespace pkv
