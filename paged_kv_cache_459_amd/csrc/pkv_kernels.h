// Internal launcher interface between the C ABI (pkv_api.cpp) and the HIP kernels.
// Not installed; callers use include/pkv.h.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>
#include <vector>

namespace pkv {

constexpr int kBlockSize = 16;  // tokens per block ([P3] §3.2; [P1] §二 example)
constexpr int kWaves = 4;       // waves per work-group of the attention stream kernels
// Block-table entry bit marking a block that several sequences of the batch read (the
// allocator's marked export sets it); the block id is the entry without it.
constexpr int32_t kSharedBit = 0x40000000;

enum AttnKernel : int32_t { kAuto = 0, kVector = 1, kMatrix = 2 };

// Shared-prefix plans (pkv_plan.cpp): packed int32 arrays, layout documented in pkv.h.
constexpr int32_t kPlanMagic = 0x504C4E31;
constexpr int kPlanHeader = 16;
constexpr int kUnitInts = 6;      // ref_seq, b0, b1, member_off, member_cnt, cell_base
constexpr int kRowsPerTile = 16;  // rows of one MFMA tile of the shared pass
constexpr int kPlanChunk = 16;    // blocks per unit of a run
constexpr int kMaxPlannedGroup = 4;  // q heads per kv head up to which batches are planned
constexpr int kMaxUnitBlocks = 64;   // blocks of one unit (one block id per lane)
constexpr int32_t kPrefillMagic = 0x50524631;
constexpr int kPrefillMaxBlocks = 512;  // blocks of one prefill unit (their ids sit in LDS)
constexpr int kPrefillMinChunk = 64;    // shortest unit the planner cuts to fill the device
// Work-groups a prefill launch should have before units are cut shorter: two waves of the
// 512 that MI355X holds at once (256 compute units, two work-groups each). Units are not cut
// below 64 blocks: shorter ones cost more in pieces and merging than they gain.
constexpr int64_t kPrefillMinGroups = 1024;
#ifndef PKV_PREFILL_RT
#define PKV_PREFILL_RT 2
#endif
constexpr int kPrefillRowTiles = PKV_PREFILL_RT;  // 16-row tiles per wave of the prefill kernel

struct PlanView {
  int32_t U = 0, cells = 0;
  bool has_shared = false;
};

// Builds the plan of a batch from host copies of its tables and lengths (table entries may
// carry the shared mark). H / GS: head slots and q heads per slot of the stream kernel.
// share = false gives a plan without runs (every block private). Returns the number of units.
int32_t plan_build(const int32_t* tables, const int32_t* lens, int32_t B, int32_t max_blocks,
                   int32_t max_ctx, int32_t NB, int32_t H, int32_t GS, int32_t G, int32_t chunk,
                   bool share, std::vector<int32_t>* out);
// Validates a packed plan against a launch's shapes; fills v. append: the block of each
// sequence's newest token must not be shared.
bool plan_check(const int32_t* p, size_t n, int32_t B, int32_t max_blocks, int32_t H, int32_t GS,
                int32_t G, bool append, PlanView* v);
// Prefill plan. Rows are the T = query_start[S] new prompt tokens, sequence s's being the last
// q_s = query_start[s+1] - query_start[s] of its context_lens[s] tokens; the row at position
// pos sees vis = pos + 1 tokens. Units cover (sequence, tile of up to tile_rows consecutive
// rows, chunk of the blocks the tile's last row sees); a tile whose blocks fit one chunk has
// one unit, marked direct (cell_base -1: its rows are written straight to the output), the
// others give each row one piece per chunk it sees, merged afterwards. Units are ordered
// longest first (stable), cells handed out in that order. Layout: header (magic
// kPrefillMagic, T, H, GS, U, M, L, cells, chunk, S, tile_rows), skip[T] (1: the row merges),
// vis[T], sh_ptr[T+1], units[U][6], members[M] (rows), sh_list[L].
void prefill_plan_build(const int32_t* query_start, const int32_t* lens, int32_t S, int32_t H,
                        int32_t GS, int32_t tile_rows, int32_t chunk, std::vector<int32_t>* out);
// The unit length (blocks) of a prefill plan: the longest power-of-two fraction of max_chunk
// (down to kPrefillMinChunk) for which the launch still has at least min_groups work-groups
// (units * H). Small batches over long contexts are cut finer: their rows become pieces that
// the merge combines, instead of a launch too small to fill the device.
int32_t prefill_chunk(const int32_t* query_start, const int32_t* lens, int32_t S, int32_t H,
                      int32_t tile_rows, int32_t max_chunk, int64_t min_groups);
bool prefill_plan_check(const int32_t* p, size_t n, int32_t T, int32_t S, int32_t max_blocks,
                        int32_t max_ctx, int32_t H, int32_t GS, int32_t max_tile_rows,
                        int32_t max_chunk, PlanView* v);

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
  float* ws_ml;         // [cells][GS][2]: (m, l) of each piece
  float* ws_o;          // [cells][GS][hd]: o of each piece
  // Shared-prefix plan (all null / 0 without one). Cells of ws_ml / ws_o: [0, 2W) the
  // workers' pieces; [2W, 2W + B*H) the piece of a planned sequence's private segment when one
  // worker holds it whole; from 2W + B*H on, the shared pass's pieces.
  const int32_t* skip;     // [B] leading blocks of each sequence covered by the shared pass
  const int32_t* sh_ptr;   // [B + 1] CSR over sh_list
  const int32_t* sh_list;  // shared-piece cells of each sequence (plus its head slot)
  const int32_t* units;    // [U][kUnitInts]
  const int32_t* members;  // q rows of the units' members (decode: sequences)
  int32_t num_units, shared_cells;
  int32_t shared_base;     // first cell of the shared pieces (decode: 2W + B*H)
  int32_t table_rows;      // rows of block_tables (decode: B; prefill: sequences)
  // Prefill (null for decode): visible tokens of each row (its position + 1); the rows are
  // then new prompt tokens, q and out are [T][Hq][hd], and there is no stream pass (ws_seg
  // null for the merge).
  const int32_t* row_vis;
};

// dtype: 0 f32, 1 f16, 2 bf16 (pkv_dtype). Return the launch status (hipGetLastError).
hipError_t launch_write(const WriteParams& p, int32_t dtype, hipStream_t stream);
// Prefill attention pass (pkv_prefill.hip): units of the prefill plan, f16/bf16.
hipError_t launch_prefill(const StreamParams& p, int32_t dtype, hipStream_t stream);
// Prompt tokens per prefill unit for q-head group size G (a work-group's rows / G).
int32_t prefill_tile_rows(int32_t G);
hipError_t launch_copy_blocks(const CopyParams& p, int32_t dtype, hipStream_t stream);
// A step's staged data, read from a device-visible pinned host buffer (16-byte aligned):
// small_n16 16-byte chunks at src to small_dst; dense_n16 chunks at src + dense_src (bytes)
// to table + dense_dst (ints, a multiple of 4); then npairs (flat index, value) int32 pairs
// at src + pairs_src (bytes) scattered into table (indices outside [0, table_ints) skipped).
struct StageParams {
  const char* src;
  int32_t* small_dst;
  int64_t small_n16;
  int32_t* table;
  int64_t table_ints;
  int64_t dense_src, dense_dst, dense_n16;
  int64_t pairs_src, npairs;
};
hipError_t launch_stage(const StageParams& p, hipStream_t stream);
// The staging and copy-on-write copies (pairs cp.src/cp.dst readable by the device: the pinned
// staging set) in one launch; the copies touch no memory the staging writes.
hipError_t launch_stage_copy(const StageParams& sp, const CopyParams& cp, int32_t dtype,
                             hipStream_t stream);
// Work-groups per block and cache of the copy kernel (grid.y; at most 65535 is launchable).
int32_t copy_blocks_grid_y(int32_t Hkv, int32_t hd, int32_t dtype);
hipError_t launch_stream(const StreamParams& p, int32_t dtype, int32_t kernel,
                         hipStream_t stream);
hipError_t launch_merge(const StreamParams& p, int32_t dtype, int32_t kernel,
                        hipStream_t stream);
// The shared pass of a plan (f16/bf16, G <= 16): p.num_units units on every kv head.
hipError_t launch_shared(const StreamParams& p, int32_t dtype, int32_t kernel,
                         hipStream_t stream);
// The one-launch kernel of the shared and stream passes exists for the vector stream kernel,
// f16/bf16, with num_workers a multiple of 8 work-groups.
bool fused_kernel_exists(int32_t dtype, int32_t kernel, int32_t num_workers);
// Launches (1 or 2) of a validated decode plan's shared and stream passes under the automatic
// choice (pkv_decode_planned_launches without the validation). plan: the packed plan; H is
// read from its header; kernel: the stream kernel; W: the stream pass's workers.
int32_t planned_launches(const int32_t* plan, int32_t B, int32_t Hkv, int32_t dtype,
                         int32_t kernel, int32_t W);
// The shared pass and the stream pass of a plan: one launch where that kernel exists (and
// the plan has units), else the two launches in order. Same results either way.
hipError_t launch_fused(const StreamParams& p, int32_t dtype, int32_t kernel,
                        hipStream_t stream);
// Dynamic LDS of the stream pass for B sequences (their prefix sums).
size_t stream_lds_bytes(int32_t B);

// Read-bandwidth probe (pkv_probe.hip): tiles ids[0..n) of base, max_tile tiles of 4096 bytes.
hipError_t launch_probe_read(const void* base, int32_t max_tile, const int32_t* ids, int32_t n,
                             int32_t num_workers, uint32_t* sink, hipStream_t stream);

}  // namespace pkv

// Host allocator, internal access for the step engine (pkv_alloc.cpp).
struct pkv_allocator;
namespace pkv {
// Entries [from, n) of sequence seq's table row into row (marked as pkv_alloc_tables_marked
// marks them), with n its block count, returned; *len receives its length. -1 if the
// sequence is unknown or has more than max_blocks blocks.
int32_t alloc_row(const pkv_allocator* a, int64_t seq, int32_t from, int32_t max_blocks,
                  int32_t* row, int64_t* len);

// Records the failing step and the HIP error text for pkv_last_error(); returns err.
hipError_t note_error(const char* what, hipError_t err);
// Records a message (no HIP error) for pkv_last_error().
void note_message(const char* what);

// Bytes of the file-scope device scratch array of the allocation-free decode step: enough for
// the stream/merge workspace of every supported shape at the default worker count of a
// 256-compute-unit part (at most 2048 matrix-core waves x 2 cells x 16 q heads x (128 + 2)
// floats, plus 8193 prefix sums: 32.6 MiB).
constexpr size_t kStaticScratchBytes = size_t{40} << 20;
// Device address of that array on the current device (looked up once per device); nullptr on
// a HIP error (recorded for pkv_last_error()).
void* static_scratch();

// Which kernel the stream pass runs for this shape and request (kVector or kMatrix).
int32_t select_kernel(int32_t dtype, int32_t G, int32_t request);

// Waves that fill the current device once with the chosen stream kernel (0 on a HIP error).
int32_t default_workers(int32_t dtype, int32_t hd, int32_t kernel, int32_t B);

}  // namespace pkv
