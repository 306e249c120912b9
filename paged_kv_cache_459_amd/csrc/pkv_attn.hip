// Paged decode attention kernels for gfx950 (CDNA4).
//
// What is computed ([P1] "vLLM 與 PagedAttention：高吞吐推理的關鍵", §三 步驟三 and §五 component
// table; [P2] vLLM overview, "PagedAttention 的核心原理"): for each sequence, attention of its
// query over all of its tokens' K/V, found block by block through the sequence's block table.
// The formula (scaled dot product, max-subtracted softmax, fp32 accumulation) is the library's
// documented contract; the pages give none.
//
// Work decomposition (our design: balanced token streams). A "segment" is the K/V one
// attention row reads: (sequence i, head slot h) with c_i = ceil(n_i/16) blocks, where the
// head slot is a q head (vector kernel) or a kv head with its G q heads (matrix-core kernel).
// All segments of the batch are laid end to end, in head-major order, as one sequence of
// T = H * sum_i c_i (block, head) tiles. A persistent grid of W waves ("workers") cuts that
// sequence into W equal contiguous ranges of per = ceil(T/W) tiles, so every wave streams the
// same number of bytes however ragged the lengths are, and no work-group is launched empty.
// A segment that lies inside one range is finished by its wave (output row written); a
// segment cut by range boundaries leaves one (m, l, o) piece per wave that touched it, and
// merge_kernel combines the pieces in wave order. Every result depends only on the batch's
// lengths and contents, never on timing; placement and sharing of blocks do not change it.
//
// Work-groups are mapped so that each XCD (work-groups go round-robin over the 8 XCDs) owns a
// contiguous eighth of the tile sequence: with head-major order an XCD's L2 sees the tiles of
// a few heads only, so blocks shared between sequences (common prefixes, beams) are re-read
// from that L2 instead of HBM.
//
// Per wave, tiles flow through one register buffer per operand with K and V staggered: the
// next tile's K is requested as soon as this tile's scores are computed, and its V as soon as
// this tile's V has been accumulated, so one tile of loads is always in flight while the
// register footprint stays at one tile. K/V loads are non-temporal (streamed data, no reuse
// inside a launch except through sharing). Scores are kept in base-2 units (scale folded with
// log2 e) so every exponential is one v_exp_f32. Masked tokens (past the end of a sequence's
// last block, or a whole block whose table entry is outside the pool) are *selected* out --
// score -inf, V element 0 -- never multiplied by zero, so NaN in unused slots cannot leak.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>

#include "pkv_kernels.h"

// Device scratch of the allocation-free decode step (pkv_decode_append_attn_noalloc): one copy
// per GPU, held until the process ends. Host code never passes this name to a kernel (on the
// host it is only a stand-in for the symbol); it uses the address static_scratch() obtains
// from the runtime for the current device.
static __device__ __align__(256) char scratch[pkv::kStaticScratchBytes];

namespace pkv {

void* static_scratch() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (note_error("hipGetDevice", hipGetDevice(&dev)) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    (void)note_error("static scratch: device index", hipErrorInvalidDevice);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {  // once per device, with that device current
    void* ptr = nullptr;
    if (note_error("hipGetSymbolAddress(scratch)",
                   hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess ||
        ptr == nullptr)
      return nullptr;
    addr[dev] = ptr;
  }
  return addr[dev];
}

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kThreads = kWaves * 64;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Streaming loads of cache tiles (global_load ... nt).
__device__ __forceinline__ uint4 load_nt16(const char* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_nt8(const char* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
// Tiles of blocks marked shared are read with ordinary (cached) loads instead: other
// sequences of the batch read them too, and the L2 should keep them.
__device__ __forceinline__ uint4 load_tile16(const char* p, bool shared) {
  return shared ? *reinterpret_cast<const uint4*>(p) : load_nt16(p);
}
__device__ __forceinline__ uint2 load_tile8(const char* p, bool shared) {
  return shared ? *reinterpret_cast<const uint2*>(p) : load_nt8(p);
}

// Cross-lane moves inside a row of 16 lanes (DPP): quad permutations and row rotations.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kRowRor4 = 0x124;   // rotate the row of 16 by 4
constexpr int kRowRor8 = 0x128;   // rotate the row of 16 by 8

// All-reduce over the 16 lanes of each row.
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<kQuadSwap1>(v));
  v = fmaxf(v, dpp<kQuadSwap2>(v));
  v = fmaxf(v, dpp<kRowRor4>(v));
  v = fmaxf(v, dpp<kRowRor8>(v));
  return v;
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<kQuadSwap1>(v);
  v += dpp<kQuadSwap2>(v);
  v += dpp<kRowRor4>(v);
  v += dpp<kRowRor8>(v);
  return v;
}

// Orders this wave's LDS accesses (a store before the loads that read other lanes' values).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Makes the loaded value count as used here, so the wait for its load is placed here. Used on
// the rare path that reloads q at a segment start: left pending, that load would make the
// compiler's wait-count merge at the end of the branch wait for every load in flight (the
// next tile's K and V included) before each tile's first multiply.
__device__ __forceinline__ void settle(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// Opaque to the optimiser: the tile registers are "redefined" at the point of use, so no
// computation on them (such as unpacking 16-bit halves) can be hoisted up next to the load
// that fills them, where it would force an early wait for that load and serialise the
// stream of tiles.
__device__ __forceinline__ uint4 pinned(uint4 v) {
  settle(v);
  return v;
}
__device__ __forceinline__ uint2 pinned(uint2 v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y));
  return v;
}

// Element e (lane-dependent) of a 16-byte chunk of EB-byte elements replaced by `bits`.
template <int EB>
__device__ __forceinline__ uint4 set_elem(uint4 v, int e, uint32_t bits) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (EB == 2) {
      if (e >> 1 == i) w[i] = (e & 1) ? ((w[i] & 0x0000FFFFu) | (bits << 16))
                                      : ((w[i] & 0xFFFF0000u) | (bits & 0xFFFFu));
    } else {
      if (e == i) w[i] = bits;
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ uint2 set_elem2(uint2 v, int e, uint32_t bits) {
  uint32_t w[2] = {v.x, v.y};
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (e >> 1 == i) w[i] = (e & 1) ? ((w[i] & 0x0000FFFFu) | (bits << 16))
                                    : ((w[i] & 0xFFFF0000u) | (bits & 0xFFFFu));
  return make_uint2(w[0], w[1]);
}

// Bits of element d of an EB-byte-element row.
template <int EB>
__device__ __forceinline__ uint32_t load_elem(const char* row, int d) {
  if constexpr (EB == 2) return *reinterpret_cast<const uint16_t*>(row + 2 * d);
  else return *reinterpret_cast<const uint32_t*>(row + 4 * d);
}
// Non-temporal element store: the merge pass's new-token stores are partial cache lines that,
// left dirty in the L2, would be written back in the middle of the next step's stream.
template <int EB>
__device__ __forceinline__ void store_elem_nt(char* row, int d, uint32_t bits) {
  if constexpr (EB == 2)
    __builtin_nontemporal_store(static_cast<uint16_t>(bits), reinterpret_cast<uint16_t*>(row + 2 * d));
  else
    __builtin_nontemporal_store(bits, reinterpret_cast<uint32_t*>(row + 4 * d));
}

// Per-dtype element access. DT: 0 = f32, 1 = f16, 2 = bf16.
template <int DT>
struct Elem;

template <>
struct Elem<0> {
  static constexpr int kBytes = 4;
  // acc + sum of the 4 element products of two 16-byte chunks
  __device__ static __forceinline__ float dot(const uint4& a, const uint4& b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = fmaf(__uint_as_float(word(a, i)), __uint_as_float(word(b, i)), acc);
    return acc;
  }
  __device__ static __forceinline__ float get(const uint4& v, int i) {
    return __uint_as_float(word(v, i));
  }
  __device__ static __forceinline__ void put(void* base, size_t idx, float x) {
    static_cast<float*>(base)[idx] = x;
  }
};

template <>
struct Elem<1> {
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float dot(const uint4& a, const uint4& b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, word(a, i)),
                                   __builtin_bit_cast(half2_t, word(b, i)), acc, false);
    return acc;
  }
  __device__ static __forceinline__ float get(const uint4& v, int i) {
    const half2_t h = __builtin_bit_cast(half2_t, word(v, i >> 1));
    return static_cast<float>(h[i & 1]);
  }
  __device__ static __forceinline__ void put(void* base, size_t idx, float x) {
    static_cast<_Float16*>(base)[idx] = static_cast<_Float16>(x);
  }
};

template <>
struct Elem<2> {
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float dot(const uint4& a, const uint4& b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, word(a, i)),
                                            __builtin_bit_cast(bf16x2_t, word(b, i)), acc, false);
    return acc;
  }
  __device__ static __forceinline__ float get(const uint4& v, int i) {
    const uint32_t w = word(v, i >> 1);
    return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
  __device__ static __forceinline__ void put(void* base, size_t idx, float x) {
    static_cast<__bf16*>(base)[idx] = static_cast<__bf16>(x);
  }
};

// Zeroes the tokens of a 16-byte V chunk that are not valid. The chunk holds tokens
// t0 .. t0 + 16/EB - 1 of one dim row; with EB = 2 each 32-bit word holds two tokens.
template <int EB>
__device__ __forceinline__ uint4 mask_tokens(uint4 v, int t0, int valid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (EB == 2) {
      const uint32_t lo = t0 + 2 * i < valid ? 0x0000FFFFu : 0u;
      const uint32_t hi = t0 + 2 * i + 1 < valid ? 0xFFFF0000u : 0u;
      w[i] &= lo | hi;
    } else {
      w[i] &= t0 + i < valid ? 0xFFFFFFFFu : 0u;
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ int clamp_len(const StreamParams& p, int i) {
  return min(max(p.context_lens[i], 0), p.max_ctx);
}

// ---- Stream geometry ----------------------------------------------------------------------

// Exclusive prefix sums of the per-sequence block counts c_i = ceil(n_i/16) - skip_i (the
// blocks after those a shared-prefix plan covers) into pref[0..B]; pref[B] = C, the tiles of
// one head slot. Whole work-group; ends synchronised.
__device__ void scan_block_counts(const StreamParams& p, int* pref) {
  __shared__ int s_wsum[kWaves];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int carry = 0;
  for (int base = 0; base < p.B; base += kThreads) {
    const int i = base + threadIdx.x;
    const int c = i < p.B ? max(0, (clamp_len(p, i) + kBlockSize - 1) / kBlockSize -
                                     (p.skip != nullptr ? p.skip[i] : 0))
                          : 0;
    int x = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wsum[w] = x;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      before += ww < w ? s_wsum[ww] : 0;
      total += s_wsum[ww];
    }
    if (i < p.B) pref[i] = carry + before + x - c;
    carry += total;
    __syncthreads();
  }
  if (threadIdx.x == 0) pref[p.B] = carry;
  __syncthreads();
}

// Largest i in [0, B) with pref[i] <= r, given pref[B] > r (empty segments are skipped).
__device__ __forceinline__ int find_seq(const int* pref, int B, int r) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pref[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// Everything a wave needs about one tile of its range, held one tile per lane.
struct TileInfo {
  int id;   // physical block to read (0 when the table entry is outside the pool)
  int seq;  // sequence i
  int hm;   // head slot << 16 | piece << 11 | shared << 10 | last << 9 | slot << 8 |
            // whole << 7 | end << 6 | start << 5 | valid tokens; last: the sequence's final
            // block (holds its newest token); shared: the table entry carries the shared-block
            // mark; piece: the sequence has shared-pass pieces, so even a whole segment leaves
            // a piece (in its own cell) for the merge
};
constexpr int kStart = 1 << 5, kEnd = 1 << 6, kWhole = 1 << 7, kLast = 1 << 9, kShared = 1 << 10,
              kPiece = 1 << 11;

// Stream position t -> tile of segment (i, h): head-major order, t = h*C + pref[i] + j; table
// index j + skip_i.
__device__ __forceinline__ TileInfo tile_info(const StreamParams& p, const int* pref, int C,
                                              int t, int t0, int t1) {
  const int h = t / C;
  const int r = t - h * C;
  const int i = find_seq(pref, p.B, r);
  const int j = r - pref[i];
  const int c = pref[i + 1] - pref[i];
  const int seg0 = h * C + pref[i];
  const int n = clamp_len(p, i);
  const int sk = p.skip != nullptr ? p.skip[i] : 0;
  int valid = min(kBlockSize, n - kBlockSize * (j + sk));
  const int raw = p.block_tables[static_cast<size_t>(i) * p.max_blocks + j + sk];
  const int shared = raw >= 0 && (raw & kSharedBit) ? 1 : 0;
  int id = raw & ~kSharedBit;
  if (raw < 0 || id >= p.NB) {
    id = 0;  // read (always in bounds) but no token of it counts
    valid = 0;
  }
  const int start = (t == seg0) || (t == t0);
  const int end = (t == seg0 + c - 1) || (t == t1 - 1);
  const int whole = (seg0 >= t0) && (seg0 + c <= t1);
  const int slot = seg0 <= t0 ? 0 : 1;
  const int last = j == c - 1;
  const int piece = sk > 0 ? 1 : 0;
  return TileInfo{id, i, (h << 16) | (piece << 11) | (shared << 10) | (last << 9) | (slot << 8) |
                             (whole << 7) | (end << 6) | (start << 5) | valid};
}

// This wave's worker index and tile range [t0, t1), for work-group b of the stream pass's
// grid work-groups. Work-group b runs on XCD b % 8 (when the stream pass's work-groups start
// a launch, or follow a multiple of 8 others); logical work-group (b % 8) * (grid / 8) + b / 8
// gives each XCD a contiguous share of the workers.
struct Range {
  int worker, t0, t1;
};

__device__ __forceinline__ Range worker_range(const StreamParams& p, int C, int H, int b,
                                              int grid) {
  const int lwg = (grid % 8 == 0) ? (b % 8) * (grid / 8) + b / 8 : b;
  const int worker = lwg * kWaves + uniform(threadIdx.x >> 6);
  const int T = H * C;
  const int per = (T + p.num_workers - 1) / p.num_workers;
  const int t0 = min(T, worker * per);
  const int t1 = min(T, t0 + per);
  return Range{worker, t0, t1};
}

// Work-group 0 publishes the prefix sums for the merge pass and zeroes rows with n = 0 (a
// planned sequence with no private block is finished by the merge).
template <int DT>
__device__ void publish_and_zero(const StreamParams& p, const int* pref, int b) {
  if (b != 0) return;
  for (int i = threadIdx.x; i <= p.B; i += kThreads) p.ws_seg[i] = pref[i];
  const int row = p.Hq * p.hd;
  for (int i = 0; i < p.B; ++i) {
    if (pref[i + 1] != pref[i]) continue;  // has blocks to stream (prefix sums are in LDS)
    // no private block: n = 0 (zero the row), or a planned sequence whose every block is
    // shared (skip > 0 implies n > 0; the merge writes the row)
    if (p.skip != nullptr && p.skip[i] > 0) continue;
    for (int e = threadIdx.x; e < row; e += kThreads)
      Elem<DT>::put(p.out, static_cast<size_t>(i) * row + e, 0.f);
  }
}

// ------------------------------------------------------------------------------------------
// Vector kernel: one q head per segment (G = 1, f32, or G > 16).
//
// Lane layout per (block, kv-head) tile (TILE bytes, NL = TILE/1024 loads of 16 B per lane):
//  K load j: lane l reads bytes 1024 j + 16 l = chunk c = 4 j + l/16 of token l%16, so each
//    lane owns one token (l%16) and a quarter of its dims; the dot product is NL 16-byte
//    chunk dots plus a sum over the 4 rows (lanes l, l^16, l^32, l^48).
//  V load j: lane l reads V dim row d = j*64/LPR + l/LPR, tokens X*(l%LPR) .. +X, where a dim
//    row of 16 tokens spans LPR = element-bytes lanes. The probabilities of those X tokens are
//    broadcast through LDS; the per-lane sums are added over the LPR lanes at the end.
template <int DT, int HD>
__device__ __forceinline__ void vector_pass(const StreamParams& p, int b, int grid) {
  using E = Elem<DT>;
  constexpr int EB = E::kBytes;
  constexpr int X = 16 / EB;
  constexpr int TILE = HD * kBlockSize * EB;
  constexpr int NL = TILE / 1024;
  constexpr int LPR = EB;
  constexpr int VROWS = 64 / LPR;
  static_assert(NL * VROWS == HD, "V lane layout must cover the head");

  extern __shared__ int s_pref[];
  __shared__ float s_p[kWaves][kBlockSize];
  constexpr int NR = HD * EB / 16;  // 16-byte chunks in one token's K (or V) row of one head
  __shared__ uint4 s_new[kWaves][2][NR];  // append mode: the segment's newest K and V rows

  scan_block_counts(p, s_pref);
  publish_and_zero<DT>(p, s_pref, b);
  const int C = s_pref[p.B];
  const Range rg = worker_range(p, C, p.Hq, b, grid);
  if (rg.t0 >= rg.t1) return;

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int G = p.Hq / p.Hkv;
  const int row_id = lane >> 4, tok = lane & 15;
  const int vsub = lane % LPR;
  const uint32_t lane_off = 16u * lane;
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * TILE;

  uint4 qv[NL];
  uint4 nr = make_uint4(0, 0, 0, 0);  // append mode: a chunk of the segment's newest K/V rows
  float m = kNegInf, lsum = 0.f;
  float acc[NL];
  uint4 kr[NL], vr[NL];

  for (int cb = rg.t0; cb < rg.t1; cb += 64) {
    const int cnt = uniform(min(64, rg.t1 - cb));
    TileInfo ti{0, 0, 0};
    if (lane < cnt) ti = tile_info(p, s_pref, C, cb + lane, rg.t0, rg.t1);

    // Tile k of the chunk: block id from lane k, kv head of its q head.
    auto tile_base = [&](const void* cache, int k) {
      const int id = uniform(__builtin_amdgcn_readlane(ti.id, k));
      const int h = uniform(__builtin_amdgcn_readlane(ti.hm, k)) >> 16;
      return static_cast<const char*>(cache) + static_cast<size_t>(id) * blk_stride +
             static_cast<size_t>(h / G) * TILE;
    };
    // K of tile k; when tile k starts a segment, also that segment's q (the previous tile's
    // scores are already computed, so the old q is dead) and, in append mode, its newest K/V
    // rows, so they arrive with the tile instead of stalling the segment's first step.
    auto load_k = [&](int k) {
      const char* kt = tile_base(p.k_cache, k);
      const bool sh = (uniform(__builtin_amdgcn_readlane(ti.hm, k)) & kShared) != 0;
#pragma unroll
      for (int j = 0; j < NL; ++j) kr[j] = load_tile16(kt + (lane_off + 1024u * j), sh);
      const int hmk = uniform(__builtin_amdgcn_readlane(ti.hm, k));
      if (hmk & kStart) {
        const int seq = uniform(__builtin_amdgcn_readlane(ti.seq, k));
        const int h = hmk >> 16;
        const uint4* qp = reinterpret_cast<const uint4*>(
            static_cast<const char*>(p.q) + (static_cast<size_t>(seq) * p.Hq + h) * HD * EB);
#pragma unroll
        for (int j = 0; j < NL; ++j) qv[j] = qp[4 * j + row_id];
        if (p.k_new != nullptr && lane < 2 * NR) {
          const size_t row = (static_cast<size_t>(seq) * p.Hkv + h / G) * HD * EB;
          const char* src = static_cast<const char*>(lane < NR ? p.k_new : p.v_new) + row;
          nr = *reinterpret_cast<const uint4*>(src + 16 * (lane % NR));
        }
      }
    };
    auto load_v = [&](int k) {
      const char* vt = tile_base(p.v_cache, k);
      const bool sh = (uniform(__builtin_amdgcn_readlane(ti.hm, k)) & kShared) != 0;
#pragma unroll
      for (int j = 0; j < NL; ++j) vr[j] = load_tile16(vt + (lane_off + 1024u * j), sh);
    };

    auto step = [&](int k, auto load_next) {
      constexpr bool kLoadNext = decltype(load_next)::value;
      const int seq = uniform(__builtin_amdgcn_readlane(ti.seq, k));
      const int hm = uniform(__builtin_amdgcn_readlane(ti.hm, k));
      const int h = hm >> 16, valid = hm & 31;
      if (hm & kStart) {  // first tile of a segment in this range: fresh state (its q came
                          // with the tile's K)
        m = kNegInf;
        lsum = 0.f;
#pragma unroll
        for (int j = 0; j < NL; ++j) acc[j] = 0.f;
        // Append mode: the sequence's newest K and V rows for this head, staged in LDS for
        // the final block (in whichever tile of this range), after the previous tile's
        // reads of the staging area.
        if (p.k_new != nullptr) {
          if (lane < 2 * NR) s_new[w][lane / NR][lane % NR] = nr;
          wave_lds_sync();
        }
      }
      // Append mode, final block of the sequence: the newest token (offset valid - 1) takes its
      // K/V from the rows staged at the segment start, in place of whatever the tile read from
      // its slot. The merge pass stores those rows into the slot for later steps (stores
      // issued while the tiles stream measurably slow the stream down).
      const bool append = p.k_new != nullptr && (hm & kLast) && valid > 0;
      const int off = valid - 1;
      if (append && tok == off) {  // the lanes holding the newest token's K chunks
#pragma unroll
        for (int j = 0; j < NL; ++j) kr[j] = s_new[w][0][4 * j + row_id];
      }
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < NL; ++j) s = E::dot(qv[j], pinned(kr[j]), s);
      if constexpr (kLoadNext) load_k(k + 1);
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      s *= p.scale_log2;
      if (valid < kBlockSize) s = tok < valid ? s : kNegInf;
      const float m_new = fmaxf(m, row_max16(s));
      float alpha = exp2_fast(m - m_new);
      float pr = exp2_fast(s - m_new);
      if (valid < kBlockSize) {  // partly (or, for a bad table entry, wholly) masked block
        alpha = m_new == kNegInf ? 1.f : alpha;
        pr = tok < valid ? pr : 0.f;
      }
      lsum = fmaf(lsum, alpha, pr);
      m = m_new;
      if (lane < kBlockSize) s_p[w][lane] = pr;
      wave_lds_sync();
      float pv[X];
#pragma unroll
      for (int x = 0; x < X; ++x) pv[x] = s_p[w][X * vsub + x];
      uint4 vt[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) vt[j] = pinned(vr[j]);
      if (append && vsub == off / X) {  // the lanes holding the newest token's V elements
        const char* vn = reinterpret_cast<const char*>(&s_new[w][1][0]);
#pragma unroll
        for (int j = 0; j < NL; ++j)
          vt[j] = set_elem<EB>(vt[j], off % X, load_elem<EB>(vn, VROWS * j + lane / LPR));
      }
      if (valid < kBlockSize) {  // partly filled (or unreadable) block: zero the invalid tokens
#pragma unroll
        for (int j = 0; j < NL; ++j) vt[j] = mask_tokens<EB>(vt[j], X * vsub, valid);
      }
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        float a = acc[j] * alpha;
#pragma unroll
        for (int x = 0; x < X; ++x) a = fmaf(pv[x], E::get(vt[j], x), a);
        acc[j] = a;
      }
      if constexpr (kLoadNext) load_v(k + 1);
      wave_lds_sync();
      if (hm & kEnd) {  // last tile of the segment in this range: emit
        const float l = row_sum16(lsum);
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          float a = acc[j];
          if constexpr (LPR >= 2) a += dpp<kQuadSwap1>(a);
          if constexpr (LPR >= 4) a += dpp<kQuadSwap2>(a);
          acc[j] = a;
        }
        if ((hm & kWhole) && !(hm & kPiece)) {  // the whole segment was ours: final output row
          if (vsub == 0) {
            const size_t row = (static_cast<size_t>(seq) * p.Hq + h) * HD;
#pragma unroll
            for (int j = 0; j < NL; ++j)
              E::put(p.out, row + VROWS * j + lane / LPR, l > 0.f ? acc[j] / l : 0.f);
          }
        } else {  // a piece: of a segment shared with neighbouring workers, or of a planned one
          const size_t cell =
              (hm & kWhole) ? 2 * static_cast<size_t>(p.num_workers) +
                                  static_cast<size_t>(seq) * p.Hq + h
                            : static_cast<size_t>(rg.worker) * 2 + ((hm >> 8) & 1);
          if (vsub == 0) {
#pragma unroll
            for (int j = 0; j < NL; ++j) p.ws_o[cell * HD + VROWS * j + lane / LPR] = acc[j];
          }
          if (lane == 0) {
            p.ws_ml[cell * 2] = m;
            p.ws_ml[cell * 2 + 1] = l;
          }
        }
      }
    };

    load_k(0);
    load_v(0);
    for (int k = 0; k + 1 < cnt; ++k) step(k, std::true_type{});
    step(cnt - 1, std::false_type{});
  }
}

template <int DT, int HD>
__global__ void __launch_bounds__(kThreads)
attn_vector_kernel(const StreamParams p) {
  vector_pass<DT, HD>(p, blockIdx.x, gridDim.x);
}

// ------------------------------------------------------------------------------------------
// Matrix-core kernel: one kv head and its G <= 16 q heads per segment (f16/bf16).
//
// Per tile, S^T = K Q^T on v_mfma_f32_16x16x32 (HD/32 steps; A = the 16 K rows, B = the
// group's q vectors, heads padded to 16 with zeros), then O^T += V^T P^T on
// v_mfma_f32_16x16x16 (HD/16 dim tiles; A = 16 dims x 16 tokens of the dim-major V tile,
// B = P^T). The accumulator layout of the first product (lane l: tokens 4(l/16)+i, head l%16)
// is exactly the B-operand layout the second one needs, so the probabilities never leave the
// lane. Operand loads: K step s, lane l reads bytes 1024 s + 16 l of the tile (one 1 KiB
// contiguous access per instruction); V dim tile j, lane l reads 8 bytes at
// 32 (16 j + l%16) + 8 (l/16) (512 contiguous bytes per instruction).
template <int DT>
struct Mfma;

template <>
struct Mfma<1> {
  __device__ static __forceinline__ float4_t qk(const uint4& a, const uint4& b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ float4_t pv(const uint2& a, const uint2& b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a),
                                                 __builtin_bit_cast(half4_t, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    const half2_t h = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
    return __builtin_bit_cast(uint32_t, h);
  }
};

template <>
struct Mfma<2> {
  __device__ static __forceinline__ float4_t qk(const uint4& a, const uint4& b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ float4_t pv(const uint2& a, const uint2& b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a),
                                                     __builtin_bit_cast(short4_t, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    const bf16x2_t h = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, h);
  }
};

template <int DT, int HD>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(3))) attn_matrix_kernel(const StreamParams p) {
  using M16 = Mfma<DT>;
  constexpr int TILE = HD * kBlockSize * 2;
  constexpr int KS = HD / 32;  // QK steps
  constexpr int VT = HD / 16;  // PV dim tiles

  extern __shared__ int s_pref[];
  constexpr int NR = HD * 2 / 16;  // 16-byte chunks in one token's K (or V) row of one head
  __shared__ uint4 s_new[kWaves][2][NR];  // append mode: the segment's newest K and V rows

  scan_block_counts(p, s_pref);
  publish_and_zero<DT>(p, s_pref, blockIdx.x);
  const int C = s_pref[p.B];
  const Range rg = worker_range(p, C, p.Hkv, blockIdx.x, gridDim.x);
  if (rg.t0 >= rg.t1) return;

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int G = p.Hq / p.Hkv;
  const int hq = lane & 15, g = lane >> 4;
  const uint32_t k_lane = 16u * lane;
  const uint32_t v_lane = 32u * hq + 8u * g;
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * TILE;

  uint4 qb[KS];  // the group's q vectors; lanes of padding heads (hq >= G) keep zeros
#pragma unroll
  for (int s = 0; s < KS; ++s) qb[s] = make_uint4(0, 0, 0, 0);
  uint4 nr = make_uint4(0, 0, 0, 0);  // append mode: a chunk of the segment's newest K/V rows
  float m = kNegInf, lsum = 0.f;
  float4_t o[VT];
  uint4 kr[KS];
  uint2 vr[VT];

  for (int cb = rg.t0; cb < rg.t1; cb += 64) {
    const int cnt = uniform(min(64, rg.t1 - cb));
    TileInfo ti{0, 0, 0};
    if (lane < cnt) ti = tile_info(p, s_pref, C, cb + lane, rg.t0, rg.t1);

    auto tile_base = [&](const void* cache, int k) {
      const int id = uniform(__builtin_amdgcn_readlane(ti.id, k));
      const int h = uniform(__builtin_amdgcn_readlane(ti.hm, k)) >> 16;
      return static_cast<const char*>(cache) + static_cast<size_t>(id) * blk_stride +
             static_cast<size_t>(h) * TILE;
    };
    // K of tile k; when tile k starts a segment, also its q and newest rows (see the vector
    // kernel).
    auto load_k = [&](int k) {
      const char* kt = tile_base(p.k_cache, k);
      const bool sh = (uniform(__builtin_amdgcn_readlane(ti.hm, k)) & kShared) != 0;
#pragma unroll
      for (int s = 0; s < KS; ++s) kr[s] = load_tile16(kt + (k_lane + 1024u * s), sh);
      const int hmk = uniform(__builtin_amdgcn_readlane(ti.hm, k));
      if (hmk & kStart) {
        const int seq = uniform(__builtin_amdgcn_readlane(ti.seq, k));
        const int kvh = hmk >> 16;
        if (hq < G) {
          const uint4* qp = reinterpret_cast<const uint4*>(
              static_cast<const char*>(p.q) +
              (static_cast<size_t>(seq) * p.Hq + kvh * G + hq) * HD * 2);
#pragma unroll
          for (int s = 0; s < KS; ++s) qb[s] = qp[4 * s + g];
        }
        if (p.k_new != nullptr && lane < 2 * NR) {
          const size_t row = (static_cast<size_t>(seq) * p.Hkv + kvh) * HD * 2;
          const char* src = static_cast<const char*>(lane < NR ? p.k_new : p.v_new) + row;
          nr = *reinterpret_cast<const uint4*>(src + 16 * (lane % NR));
        }
      }
    };
    auto load_v = [&](int k) {
      const char* vt = tile_base(p.v_cache, k);
      const bool sh = (uniform(__builtin_amdgcn_readlane(ti.hm, k)) & kShared) != 0;
#pragma unroll
      for (int j = 0; j < VT; ++j) vr[j] = load_tile8(vt + (v_lane + 512u * j), sh);
    };

    auto step = [&](int k, auto load_next) {
      const int seq = uniform(__builtin_amdgcn_readlane(ti.seq, k));
      const int hm = uniform(__builtin_amdgcn_readlane(ti.hm, k));
      const int kvh = hm >> 16, valid = hm & 31;
      if (hm & kStart) {  // first tile of a segment in this range: fresh state (its q came
                          // with the tile's K)
        m = kNegInf;
        lsum = 0.f;
#pragma unroll
        for (int j = 0; j < VT; ++j) o[j] = float4_t{0.f, 0.f, 0.f, 0.f};
        // Append mode: stage the sequence's newest K and V rows of this kv head (see the
        // vector kernel).
        if (p.k_new != nullptr) {
          if (lane < 2 * NR) s_new[w][lane / NR][lane % NR] = nr;
          wave_lds_sync();
        }
      }
      // Append mode, final block of the sequence: see the vector kernel. Here K lane l holds
      // token l%16, chunk 4s + l/16; V lane l holds dim 16j + l%16, tokens 4(l/16) .. +3.
      const bool append = p.k_new != nullptr && (hm & kLast) && valid > 0;
      const int off = valid - 1;
      if (append && hq == off) {  // the lanes holding the newest token's K chunks
#pragma unroll
        for (int s = 0; s < KS; ++s) kr[s] = s_new[w][0][4 * s + g];
      }
      float4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) sacc = M16::qk(pinned(kr[s]), qb[s], sacc);
      if constexpr (decltype(load_next)::value) load_k(k + 1);
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[i] = sacc[i] * p.scale_log2;
        if (valid < kBlockSize) sc[i] = (4 * g + i < valid) ? sc[i] : kNegInf;
      }
      float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float m_new = fmaxf(m, bm);
      float alpha = exp2_fast(m - m_new);
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = exp2_fast(sc[i] - m_new);
      if (valid < kBlockSize) {  // partly (or, for a bad table entry, wholly) masked block
        alpha = m_new == kNegInf ? 1.f : alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = (4 * g + i < valid) ? pr[i] : 0.f;
      }
      lsum = fmaf(lsum, alpha, (pr[0] + pr[1]) + (pr[2] + pr[3]));
      m = m_new;
      const uint2 pb = make_uint2(M16::pack2(pr[0], pr[1]), M16::pack2(pr[2], pr[3]));
      uint2 vt[VT];
#pragma unroll
      for (int j = 0; j < VT; ++j) vt[j] = pinned(vr[j]);
      if (append && g == off / 4) {  // the lanes holding the newest token's V elements
        const char* vn = reinterpret_cast<const char*>(&s_new[w][1][0]);
#pragma unroll
        for (int j = 0; j < VT; ++j) vt[j] = set_elem2(vt[j], off % 4, load_elem<2>(vn, 16 * j + hq));
      }
      if (valid < kBlockSize) {  // partly filled (or unreadable) block: zero the invalid tokens
        const int base = 4 * g;
        const uint32_t mx =
            (base + 0 < valid ? 0x0000FFFFu : 0u) | (base + 1 < valid ? 0xFFFF0000u : 0u);
        const uint32_t my =
            (base + 2 < valid ? 0x0000FFFFu : 0u) | (base + 3 < valid ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int j = 0; j < VT; ++j) vt[j] = make_uint2(vt[j].x & mx, vt[j].y & my);
      }
#pragma unroll
      for (int j = 0; j < VT; ++j) o[j] = M16::pv(vt[j], pb, o[j] * alpha);
      if constexpr (decltype(load_next)::value) load_v(k + 1);
      if (hm & kEnd) {  // last tile of the segment in this range: emit
        float l = lsum + __shfl_xor(lsum, 16);
        l += __shfl_xor(l, 32);
        if ((hm & kWhole) && !(hm & kPiece)) {  // the whole segment was ours: final output rows
          if (hq < G) {
            const size_t row = (static_cast<size_t>(seq) * p.Hq + kvh * G + hq) * HD;
#pragma unroll
            for (int j = 0; j < VT; ++j) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                Elem<DT>::put(p.out, row + 16 * j + 4 * g + e, l > 0.f ? o[j][e] / l : 0.f);
            }
          }
        } else if (hq < G) {  // a piece: of a segment cut between workers, or of a planned one
          const size_t c0 = (hm & kWhole) ? 2 * static_cast<size_t>(p.num_workers) +
                                                static_cast<size_t>(seq) * p.Hkv + kvh
                                          : static_cast<size_t>(rg.worker) * 2 + ((hm >> 8) & 1);
          const size_t cell = c0 * G + hq;
#pragma unroll
          for (int j = 0; j < VT; ++j)
            *reinterpret_cast<float4_t*>(p.ws_o + cell * HD + 16 * j + 4 * g) = o[j];
          if (g == 0) {
            p.ws_ml[cell * 2] = m;
            p.ws_ml[cell * 2 + 1] = l;
          }
        }
      }
    };

    load_k(0);
    load_v(0);
    for (int k = 0; k + 1 < cnt; ++k) step(k, std::true_type{});
    step(cnt - 1, std::false_type{});
  }
}

// ------------------------------------------------------------------------------------------
// Shared pass of a shared-prefix plan (f16/bf16, G <= 16). A unit is (a run's chunk of logical
// blocks [b0, b1), up to 16/G of the run's members); its blocks are the same physical blocks
// in every member's table, so one wave per (unit, kv head) reads each K/V tile once and
// computes the attention piece of all of the unit's rows at once: row r = member r / G, q head
// kvh*G + r % G. The arithmetic is the matrix-core kernel's (S^T = K Q^T, O^T += V^T P^T, P in
// lanes), with one difference: each row masks the tokens at or past its own sequence's length
// (members may end inside a shared, partly filled block). V tokens past every row's length are
// zeroed (unused slots may hold anything). Tiles are read with cached loads: other units of
// the same chunk (the next members, on the next waves) read them too.
//
// Waves map to (kv head, unit) per XCD (below), so that the member tiles of one chunk run side
// by side on one XCD. Each row's (m, l, o) goes to its cell:
// shared_base + cell_base + member*H + head slot, row (q head % GS), in the stream pass's
// layout.
template <int DT, int HD>
__device__ __forceinline__ void shared_pass(const StreamParams& p, int H, int GS, int b,
                                            int grid) {
  using M16 = Mfma<DT>;
  constexpr int TILE = HD * kBlockSize * 2;
  constexpr int KS = HD / 32;  // QK steps
  constexpr int VT = HD / 16;  // PV dim tiles

  // This wave's (kv head, unit). With a multiple of 8 kv heads, XCD x (work-group b runs on
  // XCD b % 8) takes kv heads [x K, (x + 1) K), K = Hkv / 8, unit-major: the plan lists units
  // longest first, so each XCD starts its longest units first and the waves that start late
  // (as earlier ones end) are short ones, while the member tiles of one chunk (adjacent
  // units) still run side by side on one XCD. Otherwise the units of a kv head run
  // side by side, each XCD taking a contiguous share.
  const int U = p.num_units;
  int kvh, u;
  if (p.Hkv % 8 == 0 && grid % 8 == 0) {
    const int K = p.Hkv / 8;
    const int j = (b / 8) * kWaves + uniform(threadIdx.x >> 6);
    if (j >= U * K) return;
    u = j / K;
    kvh = (b % 8) * K + (j - u * K);
  } else {
    const int lwg = (grid % 8 == 0) ? (b % 8) * (grid / 8) + b / 8 : b;
    const int gw = lwg * kWaves + uniform(threadIdx.x >> 6);
    if (gw >= U * p.Hkv) return;
    kvh = gw / U;
    u = gw - kvh * U;
  }
  const int32_t* e = p.units + static_cast<size_t>(u) * kUnitInts;
  const int ref = uniform(e[0]), b0 = uniform(max(e[1], 0)), b1 = uniform(min(e[2], p.max_blocks));
  const int moff = uniform(e[3]), mcnt = uniform(e[4]), cbase = uniform(e[5]);
  if (ref < 0 || ref >= p.B || b0 >= b1) return;

  const int lane = threadIdx.x & 63;
  const int G = p.Hq / p.Hkv;
  const int hq = lane & 15, g = lane >> 4;
  const int mk = hq / G, jq = hq - mk * G;  // this lane's row: member mk, q head kvh*G + jq
  const uint32_t k_lane = 16u * lane;
  const uint32_t v_lane = 32u * hq + 8u * g;
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * TILE;
  const int32_t* table = p.block_tables + static_cast<size_t>(ref) * p.max_blocks;

  // The chunk's block ids, one per lane (read once: a table read inside the loop would make
  // every tile wait for all loads in flight). -1: the entry names no block of the pool (then
  // nothing of the block counts).
  int lane_id = -1;
  if (lane < b1 - b0) {
    const int raw = table[b0 + lane];
    const int id = raw & ~kSharedBit;
    lane_id = (raw < 0 || id >= p.NB) ? -1 : id;
  }
  auto block_id = [&](int t) { return uniform(__builtin_amdgcn_readlane(lane_id, t - b0)); };
  auto load = [&](uint4 (&kr)[KS], uint2 (&vr)[VT], int id) {
    const size_t base = static_cast<size_t>(max(id, 0)) * blk_stride + static_cast<size_t>(kvh) * TILE;
    const char* kt = static_cast<const char*>(p.k_cache) + base;
    const char* vt = static_cast<const char*>(p.v_cache) + base;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) kr[s2] = *reinterpret_cast<const uint4*>(kt + k_lane + 1024u * s2);
#pragma unroll
    for (int j = 0; j < VT; ++j) vr[j] = *reinterpret_cast<const uint2*>(vt + v_lane + 512u * j);
  };
  // Two tiles in flight (buffers a and b, alternating), requested before the rows' lookups
  // below so that their latencies overlap.
  uint4 ka[KS], kb[KS];
  uint2 va[VT], vb[VT];
  int ida = block_id(b0), idb = block_id(min(b0 + 1, b1 - 1));
  load(ka, va, ida);
  load(kb, vb, idb);

  int seq = -1;
  if (hq < mcnt * G) seq = p.members[moff + mk];
  const bool row_ok = seq >= 0 && seq < p.B;
  uint4 qb[KS];
  if (row_ok) {
    const uint4* qp = reinterpret_cast<const uint4*>(
        static_cast<const char*>(p.q) + (static_cast<size_t>(seq) * p.Hq + kvh * G + jq) * HD * 2);
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) qb[s2] = qp[4 * s2 + g];
  } else {
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) qb[s2] = make_uint4(0, 0, 0, 0);
  }
  const int n_row = row_ok ? clamp_len(p, seq) : 0;
  // q settled here: a first use inside the loop would put its wait (for every load issued
  // before it, the tiles included) at the top of each iteration
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) settle(qb[s2]);
  // the rows' shortest and longest lengths: a tile ending at or before the shortest needs no
  // masking; V tokens at or past the longest are read by no row
  int nmin = row_ok ? n_row : 0x7fffffff, nmax = n_row;
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    nmin = min(nmin, __shfl_xor(nmin, off));
    nmax = max(nmax, __shfl_xor(nmax, off));
  }
  nmin = uniform(nmin);
  nmax = uniform(nmax);

  float m = kNegInf, lsum = 0.f;
  float4_t o[VT];
#pragma unroll
  for (int j = 0; j < VT; ++j) o[j] = float4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint4 (&kr)[KS], const uint2 (&vr)[VT], int t, int id) {
    const bool full = id >= 0 && kBlockSize * (t + 1) <= nmin;  // every row sees all 16 tokens
    const int row_valid = id < 0 ? 0 : min(kBlockSize, max(0, n_row - kBlockSize * t));
    float4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) sacc = M16::qk(pinned(kr[s2]), qb[s2], sacc);
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = sacc[i] * p.scale_log2;
      if (!full) sc[i] = (4 * g + i < row_valid) ? sc[i] : kNegInf;
    }
    float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float m_new = fmaxf(m, bm);
    float alpha = exp2_fast(m - m_new);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = exp2_fast(sc[i] - m_new);
    if (!full) {  // partly masked rows (or a row with nothing valid yet)
      alpha = m_new == kNegInf ? 1.f : alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = (4 * g + i < row_valid) ? pr[i] : 0.f;
    }
    lsum = fmaf(lsum, alpha, (pr[0] + pr[1]) + (pr[2] + pr[3]));
    m = m_new;
    const uint2 pb = make_uint2(M16::pack2(pr[0], pr[1]), M16::pack2(pr[2], pr[3]));
    uint2 vt[VT];
#pragma unroll
    for (int j = 0; j < VT; ++j) vt[j] = pinned(vr[j]);
    if (!full) {  // zero the V tokens no row reads
      const int tv = id < 0 ? 0 : min(kBlockSize, max(0, nmax - kBlockSize * t));
      const int base = 4 * g;
      const uint32_t mx = (base + 0 < tv ? 0x0000FFFFu : 0u) | (base + 1 < tv ? 0xFFFF0000u : 0u);
      const uint32_t my = (base + 2 < tv ? 0x0000FFFFu : 0u) | (base + 3 < tv ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int j = 0; j < VT; ++j) vt[j] = make_uint2(vt[j].x & mx, vt[j].y & my);
    }
#pragma unroll
    for (int j = 0; j < VT; ++j) o[j] = M16::pv(vt[j], pb, o[j] * alpha);
  };

  // The reloads are unconditional (past the chunk they re-read its last block): loads issued
  // on every path keep the wait counts exact, so a tile waits only for its own loads.
  for (int t = b0; t < b1; t += 2) {
    compute(ka, va, t, ida);
    ida = block_id(min(t + 2, b1 - 1));
    load(ka, va, ida);
    if (t + 1 < b1) compute(kb, vb, t + 1, idb);
    idb = block_id(min(t + 3, b1 - 1));
    load(kb, vb, idb);
  }
  float l = lsum + __shfl_xor(lsum, 16);
  l += __shfl_xor(l, 32);
  if (!row_ok) return;
  const int qh = kvh * G + jq;
  const int slot = qh / GS, nr = qh - slot * GS;
  const int rel = cbase + mk * H + slot;
  if (rel < 0 || rel >= p.shared_cells) return;
  const size_t cell = (static_cast<size_t>(p.shared_base) + static_cast<size_t>(rel)) * GS + nr;
#pragma unroll
  for (int j = 0; j < VT; ++j)
    *reinterpret_cast<float4_t*>(p.ws_o + cell * HD + 16 * j + 4 * g) = o[j];
  if (g == 0) {
    p.ws_ml[cell * 2] = m;
    p.ws_ml[cell * 2 + 1] = l;
  }
}

template <int DT, int HD>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(3))) attn_shared_kernel(const StreamParams p, int H, int GS) {
  shared_pass<DT, HD>(p, H, GS, blockIdx.x, gridDim.x);
}

// Shared pass and vector stream pass in one launch (G = 1): the first gridDim.x - stream_wgs
// work-groups are the shared pass's (unit, kv head) waves, the last stream_wgs the stream
// pass's workers. The two write disjoint cells and read only what both read when launched
// apart, so every result is bit-identical to the two-launch order. The form is used where the
// shared pass dominates, so its work-groups start first (the dispatcher fills every compute
// unit with them); the stream pass's short ranges then run as shared waves end and fill the
// shared pass's tail. At most 128 VGPRs: four waves per SIMD.
template <int DT, int HD>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(4))) attn_fused_kernel(const StreamParams p, int H, int GS,
                                                         int stream_wgs) {
  const int b = blockIdx.x;
  const int sh = gridDim.x - stream_wgs;  // a multiple of 8: the stream pass's XCD mapping holds
  if (b >= sh) vector_pass<DT, HD>(p, b - sh, stream_wgs);
  else shared_pass<DT, HD>(p, H, GS, b, sh);
}

// ------------------------------------------------------------------------------------------
// Append mode, merge pass: one wave stores sequence i's newest K/V rows of kv head h (k_new,
// v_new), with non-temporal stores, into that token's slot (block_tables[i][(n_i-1)/16], offset (n_i-1)%16): the K row
// as 16-byte chunks (chunk c at 256 c + 16 off in the tile), the V row as one element per dim
// row of the dim-major tile. Nothing is stored for n_i = 0 or a final-block entry outside the
// pool. The stream pass already used these rows in place of the slot's old contents.
template <int DT, int HD>
__device__ void store_new_token(const StreamParams& p, int i, int h) {
  constexpr int EB = Elem<DT>::kBytes;
  constexpr int CH = HD * EB / 16;  // 16-byte chunks per row
  const int n = clamp_len(p, i);
  if (n == 0) return;
  const int raw = p.block_tables[static_cast<size_t>(i) * p.max_blocks + (n - 1) / kBlockSize];
  const int blk = raw & ~kSharedBit;
  if (raw < 0 || blk >= p.NB) return;
  const int off = (n - 1) % kBlockSize;
  const int lane = threadIdx.x & 63;
  const size_t tile = static_cast<size_t>(blk) * p.Hkv + h;
  const size_t row = static_cast<size_t>(i) * p.Hkv + h;
  if (lane < CH) {
    const uint4 kk = reinterpret_cast<const uint4*>(p.k_new)[row * CH + lane];
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(const_cast<void*>(p.k_cache)) +
                   (tile * CH + lane) * kBlockSize + off;
    __builtin_nontemporal_store(u32x4_t{kk.x, kk.y, kk.z, kk.w}, dst);
  }
  const char* vn = static_cast<const char*>(p.v_new) + row * HD * EB;
  char* vtile = static_cast<char*>(const_cast<void*>(p.v_cache)) + tile * HD * kBlockSize * EB;
#pragma unroll
  for (int r = 0; r < HD / 64; ++r) {
    const int d = lane + 64 * r;
    store_elem_nt<EB>(vtile, d * kBlockSize + off, load_elem<EB>(vn, d));
  }
}

// ------------------------------------------------------------------------------------------
// Merge of the pieces of segments cut by worker-range boundaries. One wave per output row
// (sequence i, q head hh of head slot hh / GS). The pieces' (m, l) are read one per lane and
// weighted in parallel; o is accumulated over the pieces in worker order (deterministic).
// The o loads of the first U pieces are issued together with the (m, l) loads, before the
// maximum is known, so a row with up to U pieces costs two dependent memory round trips after
// the prefix sums. Rows of segments inside one range, and rows with n = 0, were finished by
// the stream pass and are left alone.
// With a shared-prefix plan, a planned sequence's row always merges here: its private pieces
// (the workers' cells, or its own cell when one worker held the segment whole; none when all
// of its blocks are shared) come first, then its shared-pass pieces in plan order.
// Append mode: rows H * GS .. H * GS + Hkv - 1 are waves of their own that store each
// sequence's newest K/V rows (one wave per kv head), concurrently with the merge waves.
// A work-group holds kMergeWaves rows of one sequence (fewer, larger work-groups dispatch
// faster than one per row); its waves never synchronise with each other.
constexpr int kMergeWaves = 4;

template <int DT, int HD>
__global__ void __launch_bounds__(64 * kMergeWaves)
merge_kernel(const StreamParams p, int H, int GS, int rows) {
  constexpr int R = HD / 64;
  const int i = blockIdx.x, lane = threadIdx.x & 63;
  const int hh = blockIdx.y * kMergeWaves + uniform(threadIdx.x >> 6);
  if (hh >= rows) return;
  if (hh >= H * GS) {
    store_new_token<DT, HD>(p, i, hh - H * GS);
    return;
  }
  const int h = hh / GS, n = hh - h * GS;
  const bool planned = p.skip != nullptr && p.skip[i] > 0;
  // prefill has no stream pass (ws_seg null): shared-pass pieces only
  const int C = p.ws_seg != nullptr ? p.ws_seg[p.B] : 0;
  const int s0 = p.ws_seg != nullptr ? p.ws_seg[i] : 0;
  const int c = p.ws_seg != nullptr ? p.ws_seg[i + 1] - s0 : 0;
  int np_priv = 0, wf = 0, slot0 = 0;
  bool own_cell = false;
  if (c > 0) {
    const int T = H * C;
    const int per = (T + p.num_workers - 1) / p.num_workers;
    const int tb = h * C + s0, te = tb + c;
    wf = tb / per;
    const int wl = (te - 1) / per;
    if (wf == wl) {
      if (!planned) return;
      np_priv = 1;
      own_cell = true;
    } else {
      np_priv = wl - wf + 1;
      // cell of piece k (worker wf + k): slot 1 only for the first worker if the segment
      // starts inside its range after other segments
      slot0 = wf * per < tb ? 1 : 0;
    }
  } else if (!planned) {
    return;
  }
  int sp0 = 0, nsh = 0;
  if (planned) {
    sp0 = p.sh_ptr[i];
    nsh = p.sh_ptr[i + 1] - sp0;
  }
  const int np = np_priv + nsh;
  const size_t wcells = 2 * static_cast<size_t>(p.num_workers);
  const size_t shared0 = static_cast<size_t>(p.shared_base);
  auto cell = [&](int k) -> size_t {
    size_t c0;
    if (k < np_priv) {
      c0 = own_cell ? wcells + static_cast<size_t>(i) * H + h
                    : static_cast<size_t>(wf + k) * 2 + (k == 0 ? slot0 : 0);
    } else {  // a shared-pass piece (index kept inside the shared cells)
      const int e = min(max(p.sh_list[sp0 + k - np_priv], 0), p.shared_cells - H);
      c0 = shared0 + static_cast<size_t>(e) + h;
    }
    return c0 * GS + n;
  };
  constexpr int U = 16;  // pieces whose o loads are in flight together
  // o of pieces base + k0 .. + U - 1 that exist (cnt is wave-uniform: no load is issued for
  // a missing piece, and the ones issued are all in flight together)
  auto load_o = [&](float (&ov)[U][R], int base, int k0, int cnt) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u < cnt) {
        const float* ok = p.ws_o + cell(base + k0 + u) * HD;
#pragma unroll
        for (int r = 0; r < R; ++r) ov[u][r] = ok[lane + 64 * r];
      }
    }
  };
  auto accumulate = [&](const float (&ov)[U][R], float wt, int k0, int cnt, float (&O)[R]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u < cnt) {
        const float wk = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt), k0 + u));
#pragma unroll
        for (int r = 0; r < R; ++r) O[r] = fmaf(wk, ov[u][r], O[r]);
      }
    }
  };
  // Round trip 1 (after the prefix sums): (m, l) of pieces 0..63 and o of pieces 0..U-1.
  float m0 = kNegInf, l0 = 0.f;
  if (lane < np) {
    const size_t cl = cell(lane);
    m0 = p.ws_ml[cl * 2];
    l0 = p.ws_ml[cl * 2 + 1];
  }
  const int cnt0 = uniform(min(64, np));
  float ov0[U][R];
  load_o(ov0, 0, 0, cnt0);
  float M = m0;
  for (int k = 64 + lane; k < np; k += 64) M = fmaxf(M, p.ws_ml[cell(k) * 2]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  float Lpart = 0.f, O[R];
#pragma unroll
  for (int r = 0; r < R; ++r) O[r] = 0.f;
  for (int base = 0; base < np; base += 64) {
    float wt = 0.f;  // weight of piece base + lane; a piece with no valid token weighs 0
    if (base + lane < np) {
      float mk = m0, lk = l0;
      if (base > 0) {
        const size_t cl = cell(base + lane);
        mk = p.ws_ml[cl * 2];
        lk = p.ws_ml[cl * 2 + 1];
      }
      wt = mk == kNegInf ? 0.f : exp2_fast(mk - M);
      Lpart = fmaf(wt, lk, Lpart);
    }
    const int cnt = uniform(min(64, np - base));
    int k0 = 0;
    if (base == 0) {  // the first U pieces' o is already in registers
      accumulate(ov0, wt, 0, cnt, O);
      k0 = U;
    }
    for (; k0 < cnt; k0 += U) {
      float ov[U][R];
      load_o(ov, base, k0, cnt);
      accumulate(ov, wt, k0, cnt, O);
    }
  }
  float L = Lpart;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) L += __shfl_xor(L, off);
  const size_t orow = (static_cast<size_t>(i) * p.Hq + hh) * HD;
#pragma unroll
  for (int r = 0; r < R; ++r)
    Elem<DT>::put(p.out, orow + lane + 64 * r, L > 0.f ? O[r] / L : 0.f);
}

// ---- host side ------------------------------------------------------------------------------

template <int DT, int HD>
const void* stream_kernel_ptr(int32_t kernel) {
  if constexpr (DT != 0) {
    if (kernel == kMatrix) return reinterpret_cast<const void*>(&attn_matrix_kernel<DT, HD>);
  }
  return reinterpret_cast<const void*>(&attn_vector_kernel<DT, HD>);
}

const void* stream_kernel(int32_t dtype, int32_t hd, int32_t kernel) {
  switch (dtype) {
    case 0: return hd == 64 ? stream_kernel_ptr<0, 64>(kVector) : stream_kernel_ptr<0, 128>(kVector);
    case 1: return hd == 64 ? stream_kernel_ptr<1, 64>(kernel) : stream_kernel_ptr<1, 128>(kernel);
    default: return hd == 64 ? stream_kernel_ptr<2, 64>(kernel) : stream_kernel_ptr<2, 128>(kernel);
  }
}

template <int DT, int HD>
void launch_stream_t(const StreamParams& p, int32_t kernel, dim3 grid, size_t lds,
                     hipStream_t stream) {
  if constexpr (DT != 0) {
    if (kernel == kMatrix) {
      hipLaunchKernelGGL((attn_matrix_kernel<DT, HD>), grid, dim3(kThreads), lds, stream, p);
      return;
    }
  }
  hipLaunchKernelGGL((attn_vector_kernel<DT, HD>), grid, dim3(kThreads), lds, stream, p);
}

int64_t shared_wgs(const StreamParams& p);

template <int DT>
void launch_shared_t(const StreamParams& p, int H, int GS, hipStream_t stream) {
  const int64_t grid = shared_wgs(p);
  if (p.hd == 64)
    hipLaunchKernelGGL((attn_shared_kernel<DT, 64>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, stream, p, H, GS);
  else
    hipLaunchKernelGGL((attn_shared_kernel<DT, 128>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, stream, p, H, GS);
}

// Work-groups of the shared pass: one wave per (unit, kv head), a multiple of 8 work-groups
// for the per-XCD mappings.
int64_t shared_wgs(const StreamParams& p) {
  if (p.Hkv % 8 == 0) {  // each XCD its eighth of the kv heads, for every unit
    const int64_t per_xcd = static_cast<int64_t>(p.num_units) * (p.Hkv / 8);
    return 8 * ((per_xcd + kWaves - 1) / kWaves);
  }
  const int64_t waves = static_cast<int64_t>(p.num_units) * p.Hkv;
  const int64_t grid = (waves + kWaves - 1) / kWaves;
  return (grid + 7) / 8 * 8;
}

template <int DT>
void launch_fused_t(const StreamParams& p, int H, int GS, hipStream_t stream) {
  const int stream_wgs = p.num_workers / kWaves;
  const dim3 grid(static_cast<unsigned>(stream_wgs + shared_wgs(p)));
  const size_t lds = stream_lds_bytes(p.B);
  if (p.hd == 64)
    hipLaunchKernelGGL((attn_fused_kernel<DT, 64>), grid, dim3(kThreads), lds, stream, p, H, GS,
                       stream_wgs);
  else
    hipLaunchKernelGGL((attn_fused_kernel<DT, 128>), grid, dim3(kThreads), lds, stream, p, H,
                       GS, stream_wgs);
}

template <int DT>
void launch_merge_t(const StreamParams& p, int H, int GS, hipStream_t stream) {
  // append mode: one more row per kv head for the newest tokens' stores
  const int rows = H * GS + (p.k_new != nullptr ? p.Hkv : 0);
  const dim3 grid(p.B, (rows + kMergeWaves - 1) / kMergeWaves);
  if (p.hd == 64)
    hipLaunchKernelGGL((merge_kernel<DT, 64>), grid, dim3(64 * kMergeWaves), 0, stream, p, H,
                       GS, rows);
  else
    hipLaunchKernelGGL((merge_kernel<DT, 128>), grid, dim3(64 * kMergeWaves), 0, stream, p, H,
                       GS, rows);
}

}  // namespace

int32_t select_kernel(int32_t dtype, int32_t G, int32_t request) {
  if (dtype == 0 || G > 16 || request == kVector) return kVector;
  if (request == kMatrix) return kMatrix;
  return G >= 2 ? kMatrix : kVector;
}

size_t stream_lds_bytes(int32_t B) { return static_cast<size_t>(B + 1) * sizeof(int32_t); }

int32_t default_workers(int32_t dtype, int32_t hd, int32_t kernel, int32_t B) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int, size_t>, int32_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const size_t lds = stream_lds_bytes(B);
  const auto key = std::make_tuple(dev, static_cast<int>(dtype), static_cast<int>(hd),
                                   static_cast<int>(kernel), lds);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stream_kernel(dtype, hd, kernel),
                                                   kThreads, lds) != hipSuccess ||
      per_cu <= 0)
    return 0;
  // The matrix-core kernel streams fastest at two work-groups per compute unit (measured on
  // the skewed GQA batches: three give more, shorter ranges, and more pieces to merge, for no
  // gain in bandwidth); the vector kernel at what the occupancy allows.
  if (kernel == kMatrix) per_cu = std::min(per_cu, 2);
  int64_t grid = static_cast<int64_t>(cus) * per_cu;
  if (grid >= 8) grid -= grid % 8;  // a whole number of work-groups per XCD
  const int32_t workers = static_cast<int32_t>(grid * kWaves);
  cache.emplace(key, workers);
  return workers;
}

hipError_t launch_stream(const StreamParams& p, int32_t dtype, int32_t kernel,
                         hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale status left by an earlier, unrelated runtime call
  const dim3 grid(p.num_workers / kWaves);
  const size_t lds = stream_lds_bytes(p.B);
  switch (dtype) {
    case 0:
      if (p.hd == 64) launch_stream_t<0, 64>(p, kVector, grid, lds, stream);
      else launch_stream_t<0, 128>(p, kVector, grid, lds, stream);
      break;
    case 1:
      if (p.hd == 64) launch_stream_t<1, 64>(p, kernel, grid, lds, stream);
      else launch_stream_t<1, 128>(p, kernel, grid, lds, stream);
      break;
    default:
      if (p.hd == 64) launch_stream_t<2, 64>(p, kernel, grid, lds, stream);
      else launch_stream_t<2, 128>(p, kernel, grid, lds, stream);
      break;
  }
  return note_error(kernel == kMatrix ? "attn_matrix_kernel launch" : "attn_vector_kernel launch",
                    hipGetLastError());
}

hipError_t launch_shared(const StreamParams& p, int32_t dtype, int32_t kernel,
                         hipStream_t stream) {
  if (p.num_units == 0) return hipSuccess;
  (void)hipGetLastError();
  const int H = kernel == kMatrix ? p.Hkv : p.Hq;
  const int GS = kernel == kMatrix ? p.Hq / p.Hkv : 1;
  switch (dtype) {
    case 1: launch_shared_t<1>(p, H, GS, stream); break;
    case 2: launch_shared_t<2>(p, H, GS, stream); break;
    default: return note_error("attn_shared_kernel (f16/bf16 only)", hipErrorInvalidValue);
  }
  return note_error("attn_shared_kernel launch", hipGetLastError());
}

bool fused_kernel_exists(int32_t dtype, int32_t kernel, int32_t num_workers) {
  return kernel == kVector && (dtype == 1 || dtype == 2) && num_workers > 0 &&
         num_workers % (8 * kWaves) == 0;
}

hipError_t launch_fused(const StreamParams& p, int32_t dtype, int32_t kernel,
                        hipStream_t stream) {
  if (p.num_units == 0 || !fused_kernel_exists(dtype, kernel, p.num_workers)) {
    const hipError_t e = launch_shared(p, dtype, kernel, stream);
    return e != hipSuccess ? e : launch_stream(p, dtype, kernel, stream);
  }
  (void)hipGetLastError();
  if (dtype == 1) launch_fused_t<1>(p, p.Hq, 1, stream);
  else launch_fused_t<2>(p, p.Hq, 1, stream);
  return note_error("attn_fused_kernel launch", hipGetLastError());
}

hipError_t launch_merge(const StreamParams& p, int32_t dtype, int32_t kernel,
                        hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale status left by an earlier, unrelated runtime call
  const int H = kernel == kMatrix ? p.Hkv : p.Hq;
  const int GS = kernel == kMatrix ? p.Hq / p.Hkv : 1;
  switch (dtype) {
    case 0: launch_merge_t<0>(p, H, GS, stream); break;
    case 1: launch_merge_t<1>(p, H, GS, stream); break;
    default: launch_merge_t<2>(p, H, GS, stream); break;
  }
  return note_error("merge_kernel launch", hipGetLastError());
}

}  // namespace pkv
