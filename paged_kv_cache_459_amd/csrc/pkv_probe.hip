// Read-bandwidth probe (measurement support; not on the attention path).
//
// How fast this part streams 4 KiB tiles from HBM when nothing is done with them: the access
// pattern of the attention stream pass (whole (block, head) tiles, 16 bytes per lane per load,
// non-temporal), without its arithmetic. Run over consecutive tiles it gives the sequential
// rate, over a random permutation the gather rate the decode path can at best reach.
//
// Wave w reads tiles ids[w*per .. min(n, (w+1)*per)) of `base` (tile t at byte t * 4096; ids
// are clamped into [0, max_tile)), four tiles in flight, and stores the XOR of every 32-bit
// word its lane read to sink[w * 64 + lane], so no load can be dropped.

#include <hip/hip_runtime.h>

#include "pkv_kernels.h"

namespace pkv {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTileBytes = 4096;
constexpr int kInFlight = 4;  // tiles per wave with loads in flight together

__device__ __forceinline__ uint32_t fold(u32x4_t v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ void __launch_bounds__(256)
probe_read_kernel(const char* __restrict__ base, const int32_t* __restrict__ ids, int32_t n,
                  int32_t max_tile, int32_t per, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = min(n, w * per), t1 = min(n, t0 + per);
  uint32_t acc = 0;
  for (int t = t0; t < t1; t += kInFlight) {
    u32x4_t v[kInFlight][4];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      if (t + k < t1) {
        const int id = min(max(ids[t + k], 0), max_tile - 1);
        const u32x4_t* p = reinterpret_cast<const u32x4_t*>(
                               base + static_cast<size_t>(id) * kTileBytes) + lane;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[k][j] = __builtin_nontemporal_load(p + 64 * j);
      }
    }
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      if (t + k < t1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc ^= fold(v[k][j]);
      }
    }
  }
  sink[static_cast<size_t>(w) * 64 + lane] = acc;
}

}  // namespace

hipError_t launch_probe_read(const void* base, int32_t max_tile, const int32_t* ids, int32_t n,
                             int32_t num_workers, uint32_t* sink, hipStream_t stream) {
  (void)hipGetLastError();
  const int32_t per = (n + num_workers - 1) / num_workers;
  hipLaunchKernelGGL(probe_read_kernel, dim3(num_workers / kWaves), dim3(256), 0, stream,
                     static_cast<const char*>(base), ids, n, max_tile, per, sink);
  return note_error("probe_read_kernel launch", hipGetLastError());
}

}  // namespace pkv
