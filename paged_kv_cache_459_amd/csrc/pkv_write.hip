// Cache write: scatter the K/V of T new tokens into their slots.
//
// [P1] "vLLM 與 PagedAttention：高吞吐推理的關鍵", §三 步驟二/步驟三: each new token's K/V go
// into the current block of its sequence; the allocator has already chosen the slot
// (block * 16 + offset). The copy is bitwise.
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

}  // namespace

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
