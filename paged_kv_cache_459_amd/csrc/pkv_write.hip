// Cache write: scatter the K/V of T new tokens into their slots.
//
// [P1] "vLLM 與 PagedAttention：高吞吐推理的關鍵", §三 步驟二/步驟三: each new token's K/V go
// into the current block of its sequence; the allocator has already chosen the slot
// (block * 16 + offset). The copy is bitwise.
//
// Also the copy-on-write block copy (below).
//
// Work-group (g, h) writes rows [16g, 16g + 16) of kv head h. K: one 16-byte store per
// chunk (the K tile keeps 16-byte chunks of dims, token-minor, so the rows of a run of
// consecutive slots land side by side). V: the tile is dim-major ([hd][16 tokens]), so a row
// scatters one element into each dim row; written element by element, a prompt becomes
// millions of 2-byte partial writes. Instead the rows are cut into runs (consecutive rows
// whose slots are consecutive in one block) and each run is written dim row by dim row: the
// span of a dim row that a run covers goes out as a few wide stores, a whole block's span as
// full 32-byte (f16/bf16) rows. The work-group owns the runs that start in its 16 rows; a run
// is at most 16 rows long, so it has those rows' V in LDS (rows 16g .. 16g + 31).

#include <hip/hip_runtime.h>

#include "pkv_kernels.h"

namespace pkv {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int EB, int HD>
__global__ void __launch_bounds__(256)
write_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v, uint4* __restrict__ kc,
             void* __restrict__ vc, const int32_t* __restrict__ slots, int32_t T, int32_t Hkv,
             int32_t NB) {
  constexpr int CH = HD * EB / 16;  // 16-byte chunks in one token-head row
  constexpr int P = 256 / HD;       // threads per V dim row
  constexpr int OP = kBlockSize / P;  // offsets (elements) of a dim row per thread
  constexpr int OB = OP * EB;       // their bytes: 8, 16 or 32
  __shared__ uint4 vrows[32 * CH];  // V of rows 16g .. 16g + 31, head h
  __shared__ int32_t s_slot[33];    // slots of rows 16g - 1 .. 16g + 31; -1: none or invalid
  __shared__ int32_t s_len[16];     // length of the run starting at row 16g + i (0: none)
  const int tid = threadIdx.x, h = blockIdx.y;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t limit = static_cast<int64_t>(NB) * kBlockSize;
  if (tid < 33) {
    const int64_t r = r0 - 1 + tid;
    int32_t sl = -1;
    if (r >= 0 && r < T) {
      sl = slots[r];
      if (sl < 0 || sl >= limit) sl = -1;  // padding, or outside the pool
    }
    s_slot[tid] = sl;
  }
  for (int i = tid; i < 32 * CH; i += 256) {
    const int64_t r = r0 + i / CH;
    if (r < T) vrows[i] = v[(r * Hkv + h) * CH + i % CH];
  }
  __syncthreads();
  // K: rows fastest, so the chunks of a run's rows are contiguous across lanes. Non-temporal
  // stores: partial cache lines left dirty in the L2 would be written back in the middle of
  // the next attention pass's stream of K/V tiles.
  for (int i = tid; i < 16 * CH; i += 256) {
    const int rr = i % 16, c = i / 16;
    const int64_t r = r0 + rr;
    const int32_t sl = s_slot[rr + 1];
    if (r >= T || sl < 0) continue;
    const uint4 kk = k[(r * Hkv + h) * CH + c];
    const size_t tile = static_cast<size_t>(sl / kBlockSize) * Hkv + h;
    __builtin_nontemporal_store(u32x4_t{kk.x, kk.y, kk.z, kk.w},
                                reinterpret_cast<u32x4_t*>(kc) + (tile * CH + c) * kBlockSize +
                                    sl % kBlockSize);
  }
  if (tid < 16) {
    // row j (index j in s_slot) continues the run of row j - 1: same block, next offset
    auto cont = [&](int j) {
      return s_slot[j] >= 0 && s_slot[j - 1] >= 0 && s_slot[j] == s_slot[j - 1] + 1 &&
             s_slot[j] % kBlockSize != 0;
    };
    int len = 0;
    if (s_slot[tid + 1] >= 0 && !cont(tid + 1)) {
      len = 1;
      while (tid + 1 + len < 33 && cont(tid + 1 + len)) ++len;
    }
    s_len[tid] = len;
  }
  __syncthreads();
  const int d = tid / P, lo = (tid % P) * OP;  // this thread: dim row d, offsets [lo, lo + OP)
  const char* vb = reinterpret_cast<const char*>(vrows);
  for (int i = 0; i < 16; ++i) {
    const int len = s_len[i];
    if (len == 0) continue;
    const int32_t sl = s_slot[i + 1];
    const int o0 = sl % kBlockSize;
    const size_t tile = static_cast<size_t>(sl / kBlockSize) * Hkv + h;
    char* row = static_cast<char*>(vc) + ((tile * HD + d) * kBlockSize) * EB;
    // offset o of the block comes from staged row i + (o - o0)
    auto elem = [&](int o) -> const char* { return vb + ((i + o - o0) * CH * 16 + d * EB); };
    if (o0 <= lo && lo + OP <= o0 + len) {  // the whole span: wide stores
      uint32_t w[OB / 4];
#pragma unroll
      for (int x = 0; x < OB / 4; ++x) {
        if constexpr (EB == 4) {
          w[x] = *reinterpret_cast<const uint32_t*>(elem(lo + x));
        } else {
          const uint32_t a = *reinterpret_cast<const uint16_t*>(elem(lo + 2 * x));
          const uint32_t b = *reinterpret_cast<const uint16_t*>(elem(lo + 2 * x + 1));
          w[x] = a | (b << 16);
        }
      }
      if constexpr (OB == 8) {
        typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(u32x2_t{w[0], w[1]},
                                    reinterpret_cast<u32x2_t*>(row + lo * EB));
      } else {
#pragma unroll
        for (int x = 0; x < OB / 16; ++x)
          __builtin_nontemporal_store(u32x4_t{w[4 * x], w[4 * x + 1], w[4 * x + 2], w[4 * x + 3]},
                                      reinterpret_cast<u32x4_t*>(row + lo * EB) + x);
      }
    } else {  // part of the span: element stores
      const int a = max(lo, o0), b = min(lo + OP, o0 + len);
      for (int o = a; o < b; ++o) {
        if constexpr (EB == 4)
          __builtin_nontemporal_store(*reinterpret_cast<const uint32_t*>(elem(o)),
                                      reinterpret_cast<uint32_t*>(row) + o);
        else
          __builtin_nontemporal_store(*reinterpret_cast<const uint16_t*>(elem(o)),
                                      reinterpret_cast<uint16_t*>(row) + o);
      }
    }
  }
}

// Copy-on-write block copy. [P2] vLLM overview, "共享和复用" and the Beam Search item of
// "PagedAttention 的优势": beam candidates share the blocks of their common history; before one
// of them appends into a shared, partly filled block the allocator moves it to a fresh block
// (dst) and this kernel copies the shared block (src) there: every kv head's tile, both
// caches, bitwise, whole.
//
// A block is `chunks` consecutive 16-byte chunks of each cache (the (block, kv head) tiles of
// one block are adjacent). Work-group (pair, y, cache) moves chunks [y*256*U, (y+1)*256*U) of
// pair `pair` in cache `cache` (0 K, 1 V): U loads in flight per lane, then U stores. The
// source is read with ordinary loads (the attention pass reads it next, through the other
// sequences that share it); the destination is written with non-temporal stores.
template <int U>
__device__ __forceinline__ void copy_block_range(u32x4_t* __restrict__ kc,
                                                 u32x4_t* __restrict__ vc,
                                                 const int32_t* __restrict__ src,
                                                 const int32_t* __restrict__ dst, int32_t NB,
                                                 int32_t chunks, int pair, int y, int cache) {
  const int32_t s = src[pair];
  const int32_t d = dst[pair];
  if (s < 0 || s >= NB || d < 0 || d >= NB) return;  // padding, or outside the pool
  u32x4_t* base = cache == 0 ? kc : vc;
  const u32x4_t* from = base + static_cast<size_t>(s) * chunks;
  u32x4_t* to = base + static_cast<size_t>(d) * chunks;
  const int first = y * (256 * U);
  const int i0 = first + static_cast<int>(threadIdx.x);
  if (first + 256 * U <= chunks) {  // whole range inside the block (uniform branch)
    u32x4_t r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = from[i0 + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(r[u], to + i0 + u * 256);
  } else {  // the block's last, partial range
    for (int i = i0; i < chunks; i += 256) __builtin_nontemporal_store(from[i], to + i);
  }
}

template <int U>
__global__ void __launch_bounds__(256)
copy_blocks_kernel(u32x4_t* __restrict__ kc, u32x4_t* __restrict__ vc,
                   const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int32_t NB,
                   int32_t chunks) {
  copy_block_range<U>(kc, vc, src, dst, NB, chunks, blockIdx.x, blockIdx.y, blockIdx.z);
}

constexpr int kCopyUnroll = 4;

}  // namespace

hipError_t launch_copy_blocks(const CopyParams& p, int32_t dtype, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  const int eb = dtype == 0 ? 4 : 2;
  const int32_t chunks = p.Hkv * p.hd * eb;  // 16-byte chunks per block: Hkv*hd*16*eb / 16
  const dim3 grid(static_cast<unsigned>(p.n),
                  static_cast<unsigned>((chunks + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll)),
                  2);
  (void)hipGetLastError();
  hipLaunchKernelGGL(copy_blocks_kernel<kCopyUnroll>, grid, dim3(256), 0, stream,
                     static_cast<u32x4_t*>(p.k_cache), static_cast<u32x4_t*>(p.v_cache), p.src,
                     p.dst, p.NB, chunks);
  return note_error("copy_blocks_kernel launch", hipGetLastError());
}

namespace {

// A step's staged host data (pinned host memory, read over the bus) into device memory, in
// one launch: the small arrays (lengths, copy-on-write pairs, slots, plans) copied whole, a
// dense range of block-table rows, and single changed table entries scattered. A kernel of
// ours rather than a runtime copy: it is ordered in the step's stream like the step's other
// kernels, without the runtime copy's extra synchronization around host memory.
__device__ __forceinline__ void stage_part(const StageParams& p, int b) {
  int64_t i = static_cast<int64_t>(b) * 256 + threadIdx.x;
  if (i < p.small_n16) {
    reinterpret_cast<uint4*>(p.small_dst)[i] = reinterpret_cast<const uint4*>(p.src)[i];
    return;
  }
  i -= p.small_n16;
  if (i < p.dense_n16) {
    if (p.dense_dst + 4 * (i + 1) <= p.table_ints)
      reinterpret_cast<uint4*>(p.table + p.dense_dst)[i] =
          reinterpret_cast<const uint4*>(p.src + p.dense_src)[i];
    return;
  }
  i -= p.dense_n16;
  if (i < p.npairs) {
    const int2 e = reinterpret_cast<const int2*>(p.src + p.pairs_src)[i];
    if (e.x >= 0 && e.x < p.table_ints) p.table[e.x] = e.y;
  }
}

__global__ void __launch_bounds__(256) stage_kernel(const StageParams p) {
  stage_part(p, blockIdx.x);
}

// The staging and a step's copy-on-write copies in one launch, for a step with no other work
// between them: work-groups [0, stage_wgs) stage, the others copy (pair, range, cache) in the
// copy kernel's order. The copies read their pairs from the same pinned host memory the
// staging reads (not from the staged device copy, which may not have landed), and touch only
// cache blocks, which the staging does not.
__global__ void __launch_bounds__(256)
stage_copy_kernel(const StageParams sp, u32x4_t* __restrict__ kc, u32x4_t* __restrict__ vc,
                  const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int32_t NB,
                  int32_t chunks, int32_t stage_wgs, int32_t grid_y) {
  const int b = blockIdx.x;
  if (b < stage_wgs) {
    stage_part(sp, b);
    return;
  }
  const int c = b - stage_wgs;
  const int per_pair = 2 * grid_y;
  copy_block_range<kCopyUnroll>(kc, vc, src, dst, NB, chunks, c / per_pair,
                                (c % per_pair) % grid_y, (c % per_pair) / grid_y);
}

}  // namespace

hipError_t launch_stage_copy(const StageParams& sp, const CopyParams& cp, int32_t dtype,
                             hipStream_t stream) {
  if (cp.n == 0) return launch_stage(sp, stream);
  const int64_t n = sp.small_n16 + sp.dense_n16 + sp.npairs;
  const int32_t stage_wgs = static_cast<int32_t>((n + 255) / 256);
  const int eb = dtype == 0 ? 4 : 2;
  const int32_t chunks = cp.Hkv * cp.hd * eb;
  const int32_t grid_y = (chunks + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll);
  const int64_t grid = stage_wgs + static_cast<int64_t>(cp.n) * 2 * grid_y;
  if (grid * 256 > INT32_MAX) {  // the flat grid would pass 32-bit indexing: launch apart
    const hipError_t e = launch_stage(sp, stream);
    return e != hipSuccess ? e : launch_copy_blocks(cp, dtype, stream);
  }
  (void)hipGetLastError();
  hipLaunchKernelGGL(stage_copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                     sp, static_cast<u32x4_t*>(cp.k_cache), static_cast<u32x4_t*>(cp.v_cache),
                     cp.src, cp.dst, cp.NB, chunks, stage_wgs, grid_y);
  return note_error("stage_copy_kernel launch", hipGetLastError());
}

hipError_t launch_stage(const StageParams& p, hipStream_t stream) {
  const int64_t n = p.small_n16 + p.dense_n16 + p.npairs;
  if (n == 0) return hipSuccess;
  (void)hipGetLastError();
  hipLaunchKernelGGL(stage_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     stream, p);
  return note_error("stage_kernel launch", hipGetLastError());
}

int32_t copy_blocks_grid_y(int32_t Hkv, int32_t hd, int32_t dtype) {
  const int64_t chunks = static_cast<int64_t>(Hkv) * hd * (dtype == 0 ? 4 : 2);
  return static_cast<int32_t>((chunks + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll));
}

hipError_t launch_write(const WriteParams& p, int32_t dtype, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  (void)hipGetLastError();  // drop a stale status left by an earlier, unrelated runtime call
  const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(p.T) + 15) / 16),
                  static_cast<unsigned>(p.Hkv));
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, static_cast<const uint4*>(p.k),
                       static_cast<const uint4*>(p.v), static_cast<uint4*>(p.k_cache), p.v_cache,
                       p.slots, p.T, p.Hkv, p.NB);
  };
  if (dtype == 0) {
    if (p.hd == 64) args(write_kernel<4, 64>);
    else args(write_kernel<4, 128>);
  } else {
    if (p.hd == 64) args(write_kernel<2, 64>);
    else args(write_kernel<2, 128>);
  }
  return note_error("write_kernel launch", hipGetLastError());
}

}  // namespace pkv
