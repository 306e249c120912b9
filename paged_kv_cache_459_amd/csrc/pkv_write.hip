// Cache write: scatter the K/V of T new tokens into their slots.
//
// [P1] "vLLM 與 PagedAttention：高吞吐推理的關鍵", §三 步驟二/步驟三: each new token's K/V go
// into the current block of its sequence; the allocator has already chosen the slot
// (block * 16 + offset). The copy is bitwise.
//
// Also the copy-on-write block copy (below).
//
// One thread moves one 16-byte chunk (X = 16 / element-bytes consecutive dims of one head of
// one token). The K chunk lands as one 16-byte store (the K tile keeps 16-byte chunks of dims,
// token-minor); the V chunk is spread over the X dim rows of the dim-major V tile.

#include <hip/hip_runtime.h>

#include "pkv_kernels.h"

namespace pkv {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int EB>
__global__ void __launch_bounds__(256)
write_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v, uint4* __restrict__ kc,
             void* __restrict__ vc, const int32_t* __restrict__ slots, int32_t T, int32_t Hkv,
             int32_t hd, int32_t NB) {
  constexpr int X = 16 / EB;
  const int chunks = hd / X;  // 16-byte chunks in one token-head row
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = static_cast<int64_t>(T) * Hkv * chunks;
  if (gid >= total) return;
  const int c = static_cast<int>(gid % chunks);
  const int64_t th = gid / chunks;
  const int h = static_cast<int>(th % Hkv);
  const int t = static_cast<int>(th / Hkv);
  const int32_t slot = slots[t];
  if (slot < 0 || slot >= NB * kBlockSize) return;  // padding, or outside the pool
  const int b = slot / kBlockSize;
  const int off = slot % kBlockSize;
  const uint4 kk = k[gid];  // k is [T][Hkv][hd]: chunk (t, h, c) is chunk number gid
  const uint4 vv = v[gid];
  const size_t tile = static_cast<size_t>(b) * Hkv + h;
  // Non-temporal stores: these are partial cache lines which, left dirty in the L2, would be
  // written back in the middle of the next attention pass's stream of K/V tiles.
  __builtin_nontemporal_store(u32x4_t{kk.x, kk.y, kk.z, kk.w},
                              reinterpret_cast<u32x4_t*>(kc) + (tile * chunks + c) * kBlockSize + off);
  const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
  if constexpr (EB == 2) {
    uint16_t* vd = static_cast<uint16_t*>(vc) + (tile * hd + static_cast<size_t>(X) * c) * kBlockSize + off;
#pragma unroll
    for (int x = 0; x < 8; ++x)
      __builtin_nontemporal_store(static_cast<uint16_t>((w[x >> 1] >> ((x & 1) * 16)) & 0xFFFFu),
                                  vd + x * kBlockSize);
  } else {
    uint32_t* vd = static_cast<uint32_t*>(vc) + (tile * hd + static_cast<size_t>(X) * c) * kBlockSize + off;
#pragma unroll
    for (int x = 0; x < 4; ++x) __builtin_nontemporal_store(w[x], vd + x * kBlockSize);
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
__global__ void __launch_bounds__(256)
copy_blocks_kernel(u32x4_t* __restrict__ kc, u32x4_t* __restrict__ vc,
                   const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int32_t NB,
                   int32_t chunks) {
  const int32_t s = src[blockIdx.x];
  const int32_t d = dst[blockIdx.x];
  if (s < 0 || s >= NB || d < 0 || d >= NB) return;  // padding, or outside the pool
  u32x4_t* base = blockIdx.z == 0 ? kc : vc;
  const u32x4_t* from = base + static_cast<size_t>(s) * chunks;
  u32x4_t* to = base + static_cast<size_t>(d) * chunks;
  const int first = static_cast<int>(blockIdx.y) * (256 * U);
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

int32_t copy_blocks_grid_y(int32_t Hkv, int32_t hd, int32_t dtype) {
  const int64_t chunks = static_cast<int64_t>(Hkv) * hd * (dtype == 0 ? 4 : 2);
  return static_cast<int32_t>((chunks + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll));
}

hipError_t launch_write(const WriteParams& p, int32_t dtype, hipStream_t stream) {
  const int eb = dtype == 0 ? 4 : 2;
  const int64_t total = static_cast<int64_t>(p.T) * p.Hkv * (p.hd * eb / 16);
  if (total == 0) return hipSuccess;
  (void)hipGetLastError();  // drop a stale status left by an earlier, unrelated runtime call
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  if (eb == 4)
    hipLaunchKernelGGL(write_kernel<4>, grid, dim3(256), 0, stream,
                       static_cast<const uint4*>(p.k), static_cast<const uint4*>(p.v),
                       static_cast<uint4*>(p.k_cache), p.v_cache, p.slots, p.T, p.Hkv, p.hd, p.NB);
  else
    hipLaunchKernelGGL(write_kernel<2>, grid, dim3(256), 0, stream,
                       static_cast<const uint4*>(p.k), static_cast<const uint4*>(p.v),
                       static_cast<uint4*>(p.k_cache), p.v_cache, p.slots, p.T, p.Hkv, p.hd, p.NB);
  return note_error("write_kernel launch", hipGetLastError());
}

}  // namespace pkv
