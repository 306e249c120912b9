// Internal launcher interface between the C ABI (pkv_api.cpp) and the HIP kernels.
// Not installed; callers use include/pkv.h.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

namespace pkv {

constexpr int kBlockSize = 16;  // tokens per block ([P3] §3.2; [P1] §二 example)
constexpr int kWaves = 4;       // waves per work-group of the attention stream kernels
// Block-table entry bit marking a block that several sequences of the batch read (the
// allocator's marked export sets it); the block id is the entry without it.
constexpr int32_t kSharedBit = 0x40000000;

enum AttnKernel : int32_t { kAuto = 0, kVector = 1, kMatrix = 2 };

struct WriteParams {
  const void* k;
  const void* v;
  void* k_cache;
  void* v_cache;
  const int32_t* slots;
  int32_t T, Hkv, hd, NB;
};

struct CopyParams {
  void* k_cache;
  void* v_cache;
  const int32_t* src;  // [n] device: block copied from
  const int32_t* dst;  // [n] device: block copied to
  int32_t n, Hkv, hd, NB;
};

// Arguments of the attention stream pass and of the merge pass.
struct StreamParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  // Append mode (both non-null): [B][Hkv][hd], the K/V of each sequence's newest token
  // (position n_i - 1). The stream pass uses them in place of the slot's old contents; the
  // merge pass stores them into the slot. Null: plain attention over the cache.
  const void* k_new;
  const void* v_new;
  int32_t B, Hq, Hkv, hd, NB, max_blocks, max_ctx;
  float scale_log2;     // softmax scale times log2(e): scores are kept in base-2 units
  int32_t num_workers;  // W: waves of the stream pass, a positive multiple of kWaves
  int32_t* ws_seg;      // [B + 1] prefix sums of block counts (written by the stream pass)
  float* ws_ml;         // [W][2][GS][2]: (m, l) of each piece
  float* ws_o;          // [W][2][GS][hd]: o of each piece
};

// dtype: 0 f32, 1 f16, 2 bf16 (pkv_dtype). Return the launch status (hipGetLastError).
hipError_t launch_write(const WriteParams& p, int32_t dtype, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyParams& p, int32_t dtype, hipStream_t stream);
// Work-groups per block and cache of the copy kernel (grid.y; at most 65535 is launchable).
int32_t copy_blocks_grid_y(int32_t Hkv, int32_t hd, int32_t dtype);
hipError_t launch_stream(const StreamParams& p, int32_t dtype, int32_t kernel,
                         hipStream_t stream);
hipError_t launch_merge(const StreamParams& p, int32_t dtype, int32_t kernel,
                        hipStream_t stream);

// Records the failing step and the HIP error text for pkv_last_error(); returns err.
hipError_t note_error(const char* what, hipError_t err);

// Which kernel the stream pass runs for this shape and request (kVector or kMatrix).
int32_t select_kernel(int32_t dtype, int32_t G, int32_t request);

// Waves that fill the current device once with the chosen stream kernel (0 on a HIP error).
int32_t default_workers(int32_t dtype, int32_t hd, int32_t kernel, int32_t B);

}  // namespace pkv
