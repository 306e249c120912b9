// Paged decode attention kernels for gfx950 (CDNA4).
//
// What is computed ([P1] "vLLM 與 PagedAttention：高吞吐推理的關鍵", §三 步驟三 and §五 component
// table; [P2] vLLM overview, "PagedAttention 的核心原理"): for each sequence, attention of its
// query over all of its tokens' K/V, found block by block through the sequence's block table.
// The formula (scaled dot product, max-subtracted softmax, fp32 accumulation) is the library's
// documented contract; the pages give none.
//
// Work decomposition (our design). A work-group of NW waves owns one (sequence, head,
// partition): the partition's P tokens are P/16 blocks, dealt round-robin to the waves. Each
// wave streams whole (block, kv-head) tiles from HBM with coalesced 16-byte (8-byte for the
// matrix-core V operand) loads, the next tile in flight while the current one is consumed,
// and keeps an online-softmax state. The waves' states are merged through LDS in a fixed
// order, so results never depend on timing or on physical placement. A sequence that fits in
// one partition is finished here; longer ones leave (m, l, o) partials for merge_kernel.
//
// Scores are kept in base-2 units (scale folded with log2 e) so that every exponential is one
// v_exp_f32. Masked tokens (past the sequence end inside its last block) are *selected* out:
// score -inf and V element 0, never multiplied by zero, so NaN in unused slots cannot leak.

#include <hip/hip_runtime.h>

#include "pkv_kernels.h"

namespace pkv {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

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

// Opaque to the optimiser: the value is "redefined" here, so no use of it (such as unpacking
// 16-bit halves) can be hoisted above this point, e.g. next to a prefetch load, where it would
// force an early wait for that load.
__device__ __forceinline__ uint4 pinned(uint4 v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
  return v;
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
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

// Shared prologue: clamp the length and locate the partition (all values wave-uniform).
struct PartInfo {
  int n, nparts, t0, t1, nblk;
};

__device__ __forceinline__ bool part_setup(const AttnParams& p, int seq, int part,
                                           PartInfo* info) {
  int n = p.context_lens[seq];
  n = min(max(n, 0), p.max_ctx);
  const int P = p.part_tokens;
  const int nparts = (n + P - 1) / P;
  if (part > 0 && part >= nparts) return false;  // partition 0 always runs: n = 0 gives zeros
  const int t0 = part * P;
  const int t1 = min(n, t0 + P);
  const int nblk = t1 > t0 ? (t1 - t0 + kBlockSize - 1) / kBlockSize : 0;
  *info = PartInfo{n, nparts, t0, t1, nblk};
  return true;
}

// Block-table staging: wave w of NW owns the partition's blocks w, w+NW, w+2NW, ...; lane k
// of the wave holds the physical id of the wave's k-th block (one coalesced load of at most
// 64 ids per wave). The block loop reads them with v_readlane, so an id lookup never waits on
// memory. Ids outside [0, NB) become -1.
template <int NW>
__device__ __forceinline__ int stage_block_ids(const AttnParams& p, int seq, const PartInfo& pi,
                                               int w, int lane) {
  const int i = w + NW * lane;
  if (i >= pi.nblk) return -1;
  const int id = p.block_tables[static_cast<size_t>(seq) * p.max_blocks + pi.t0 / kBlockSize + i];
  return (id >= 0 && id < p.NB) ? id : -1;
}

// k-th block of this wave: (physical id to read, valid tokens in it). An id outside the pool
// reads block 0 (always in bounds) with no valid token, so it contributes nothing.
template <int NW>
__device__ __forceinline__ void wave_block(int ids, int k, int w, const PartInfo& pi, int* id,
                                           int* valid) {
  const int raw = __builtin_amdgcn_readlane(ids, k);
  const int i = w + NW * k;
  const int v = min(kBlockSize, pi.t1 - (pi.t0 + kBlockSize * i));
  *id = raw >= 0 ? raw : 0;
  *valid = raw >= 0 ? v : 0;
}

// The partition bounds are the same in every lane; saying so keeps the block loop on scalar
// branches (the staging loop above would otherwise make them look lane-dependent).
__device__ __forceinline__ void make_uniform(PartInfo* pi) {
  pi->n = __builtin_amdgcn_readfirstlane(pi->n);
  pi->nparts = __builtin_amdgcn_readfirstlane(pi->nparts);
  pi->t0 = __builtin_amdgcn_readfirstlane(pi->t0);
  pi->t1 = __builtin_amdgcn_readfirstlane(pi->t1);
  pi->nblk = __builtin_amdgcn_readfirstlane(pi->nblk);
}

// Final combine of the NW waves' (m, l, o) for one head and one dim, in wave order.
// m values are base-2 maxima; waves that saw no token have m = -inf and are skipped.
template <int NW>
__device__ __forceinline__ void combine_waves(const float* ms, const float* ls, const float* os,
                                              int ostride, float* M_out, float* L_out,
                                              float* O_out) {
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, ms[w]);
  float L = 0.f, O = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (ms[w] != kNegInf) {
      const float wt = exp2_fast(ms[w] - M);
      L = fmaf(wt, ls[w], L);
      O = fmaf(wt, os[w * ostride], O);
    }
  }
  *M_out = M;
  *L_out = L;
  *O_out = O;
}

template <int DT>
__device__ __forceinline__ void emit(const AttnParams& p, const PartInfo& pi, int seq, int h,
                                     int part, int d, int hd, float M, float L, float O) {
  const size_t row = static_cast<size_t>(seq) * p.Hq + h;
  if (pi.nparts <= 1) {
    Elem<DT>::put(p.out, row * hd + d, L > 0.f ? O / L : 0.f);
  } else {
    const size_t idx = row * p.max_parts + part;
    if (d == 0) {
      p.ws_m[idx] = M == kNegInf ? kNegInf : M * kLn2;
      p.ws_l[idx] = L;
    }
    p.ws_o[idx * hd + d] = O;
  }
}

// ------------------------------------------------------------------------------------------
// Vector kernel: one q head per work-group (G = 1, or f32, or G > 16).
//
// Lane layout per (block, kv-head) tile (TILE bytes, NL = TILE/1024 loads of 16 B per lane):
//  K load j: lane l reads bytes 1024 j + 16 l = chunk c = 4 j + l/16 of token l%16, so each
//    lane owns one token (l%16) and a quarter of its dims; the dot product is NL 16-byte
//    chunk dots plus a sum over the 4 rows (lanes l, l^16, l^32, l^48).
//  V load j: lane l reads V dim row d = j*64/LPR + l/LPR, tokens X*(l%LPR) .. +X, where a dim
//    row of 16 tokens spans LPR = element-bytes lanes. The probabilities of those X tokens are
//    broadcast through LDS; the per-lane accumulators are summed over the LPR lanes at the end.
template <int DT, int HD, int NW>
__global__ void __launch_bounds__(NW * 64)
attn_vector_kernel(const AttnParams p) {
  using E = Elem<DT>;
  constexpr int EB = E::kBytes;
  constexpr int X = 16 / EB;
  constexpr int TILE = HD * kBlockSize * EB;
  constexpr int NL = TILE / 1024;
  constexpr int LPR = EB;
  constexpr int VROWS = 64 / LPR;
  static_assert(NL * VROWS == HD, "V lane layout must cover the head");

  __shared__ float s_p[NW][kBlockSize];
  __shared__ float s_o[NW][HD];
  __shared__ float s_m[NW], s_l[NW];

  const int seq = blockIdx.x, h = blockIdx.y, part = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  PartInfo pi;
  if (!part_setup(p, seq, part, &pi)) return;
  make_uniform(&pi);
  const int ids = stage_block_ids<NW>(p, seq, pi, w, lane);
  const int nmine = pi.nblk > w ? (pi.nblk - w + NW - 1) / NW : 0;  // blocks of this wave

  const int G = p.Hq / p.Hkv;
  const int kvh = h / G;
  const int row_id = lane >> 4, tok = lane & 15;
  const int vsub = lane % LPR;

  uint4 qv[NL];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const char*>(p.q) +
                                                     (static_cast<size_t>(seq) * p.Hq + h) * HD * EB);
#pragma unroll
    for (int j = 0; j < NL; ++j) qv[j] = qp[4 * j + row_id];
  }
  const size_t head_off = static_cast<size_t>(kvh) * TILE;
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * TILE;
  const char* kbase = static_cast<const char*>(p.k_cache) + head_off;
  const char* vbase = static_cast<const char*>(p.v_cache) + head_off;
  const uint32_t lane_off = 16u * lane;

  float m = kNegInf, lsum = 0.f;
  float acc[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) acc[j] = 0.f;

  struct Regs {
    uint4 k[NL], v[NL];
  };
  auto load = [&](Regs& r, int id) {
    const char* kt = kbase + static_cast<size_t>(id) * blk_stride;  // scalar tile base
    const char* vt = vbase + static_cast<size_t>(id) * blk_stride;
#pragma unroll
    for (int j = 0; j < NL; ++j)
      r.k[j] = *reinterpret_cast<const uint4*>(kt + (lane_off + 1024u * j));
#pragma unroll
    for (int j = 0; j < NL; ++j)
      r.v[j] = *reinterpret_cast<const uint4*>(vt + (lane_off + 1024u * j));
  };
  auto consume = [&](const Regs& r, int valid) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NL; ++j) s = E::dot(qv[j], r.k[j], s);
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
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const uint4 vj = pinned(r.v[j]);
      float a = acc[j] * alpha;
#pragma unroll
      for (int x = 0; x < X; ++x) {
        float vx = E::get(vj, x);
        if (valid < kBlockSize) vx = (X * vsub + x < valid) ? vx : 0.f;
        a = fmaf(pv[x], vx, a);
      }
      acc[j] = a;
    }
    wave_lds_sync();
  };
  // Double-buffered stream over this wave's blocks: tile k+1 is in flight while tile k is
  // consumed. Every load is unconditional inside its branch, so the wait counters stay exact.
  Regs ra, rb;
  int k = 0;
  if (nmine > 0) {
    int id, valid;
    wave_block<NW>(ids, 0, w, pi, &id, &valid);
    load(ra, id);
    int va = valid;
    while (true) {
      if (k + 1 >= nmine) {
        consume(ra, va);
        break;
      }
      wave_block<NW>(ids, k + 1, w, pi, &id, &valid);
      load(rb, id);
      consume(ra, va);
      const int vb = valid;
      ++k;
      if (k + 1 >= nmine) {
        consume(rb, vb);
        break;
      }
      wave_block<NW>(ids, k + 1, w, pi, &id, &valid);
      load(ra, id);
      consume(rb, vb);
      va = valid;
      ++k;
    }
  }

  const float l = row_sum16(lsum);
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    float a = acc[j];
    if constexpr (LPR >= 2) a += dpp<kQuadSwap1>(a);
    if constexpr (LPR >= 4) a += dpp<kQuadSwap2>(a);
    acc[j] = a;
  }
  if (vsub == 0) {
#pragma unroll
    for (int j = 0; j < NL; ++j) s_o[w][VROWS * j + lane / LPR] = acc[j];
  }
  if (lane == 0) {
    s_m[w] = m;
    s_l[w] = l;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < HD; d += NW * 64) {
    float M, L, O;
    combine_waves<NW>(s_m, s_l, &s_o[0][d], HD, &M, &L, &O);
    emit<DT>(p, pi, seq, h, part, d, HD, M, L, O);
  }
}

// ------------------------------------------------------------------------------------------
// Matrix-core kernel: one kv head and its G <= 16 q heads per work-group (f16/bf16).
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

template <int DT, int HD, int NW>
__global__ void __launch_bounds__(NW * 64)
attn_matrix_kernel(const AttnParams p) {
  using M16 = Mfma<DT>;
  constexpr int TILE = HD * kBlockSize * 2;
  constexpr int KS = HD / 32;  // QK steps
  constexpr int VT = HD / 16;  // PV dim tiles
  constexpr int OSTR = HD + 4;  // padded LDS row (heads map to different banks)

  __shared__ float s_o[NW][16][OSTR];
  __shared__ float s_m[NW][16], s_l[NW][16];

  const int seq = blockIdx.x, kvh = blockIdx.y, part = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  PartInfo pi;
  if (!part_setup(p, seq, part, &pi)) return;
  make_uniform(&pi);
  const int ids = stage_block_ids<NW>(p, seq, pi, w, lane);
  const int nmine = pi.nblk > w ? (pi.nblk - w + NW - 1) / NW : 0;  // blocks of this wave

  const int G = p.Hq / p.Hkv;
  const int hq = lane & 15, g = lane >> 4;

  uint4 qb[KS];
  if (hq < G) {
    const uint4* qp = reinterpret_cast<const uint4*>(
        static_cast<const char*>(p.q) + (static_cast<size_t>(seq) * p.Hq + kvh * G + hq) * HD * 2);
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[s] = qp[4 * s + g];
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[s] = make_uint4(0, 0, 0, 0);
  }
  const size_t head_off = static_cast<size_t>(kvh) * TILE;
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * TILE;
  const char* kbase = static_cast<const char*>(p.k_cache) + head_off;
  const char* vbase = static_cast<const char*>(p.v_cache) + head_off;
  const uint32_t k_lane = 16u * lane;
  const uint32_t v_lane = 32u * hq + 8u * g;

  float m = kNegInf, lsum = 0.f;
  float4_t o[VT];
#pragma unroll
  for (int j = 0; j < VT; ++j) o[j] = float4_t{0.f, 0.f, 0.f, 0.f};

  struct Regs {
    uint4 k[KS];
    uint2 v[VT];
  };
  auto load = [&](Regs& r, int id) {
    const char* kt = kbase + static_cast<size_t>(id) * blk_stride;  // scalar tile base
    const char* vt = vbase + static_cast<size_t>(id) * blk_stride;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      r.k[s] = *reinterpret_cast<const uint4*>(kt + (k_lane + 1024u * s));
#pragma unroll
    for (int j = 0; j < VT; ++j) r.v[j] = *reinterpret_cast<const uint2*>(vt + (v_lane + 512u * j));
  };
  auto consume = [&](const Regs& r, int valid) {
    float4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) sacc = M16::qk(r.k[s], qb[s], sacc);
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
    uint2 vmask = make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu);
    if (valid < kBlockSize) {
      const int base = 4 * g;
      vmask.x = (base + 0 < valid ? 0x0000FFFFu : 0u) | (base + 1 < valid ? 0xFFFF0000u : 0u);
      vmask.y = (base + 2 < valid ? 0x0000FFFFu : 0u) | (base + 3 < valid ? 0xFFFF0000u : 0u);
    }
#pragma unroll
    for (int j = 0; j < VT; ++j) {
      const uint2 va = make_uint2(r.v[j].x & vmask.x, r.v[j].y & vmask.y);
      o[j] = M16::pv(va, pb, o[j] * alpha);
    }
  };
  // Double-buffered stream over this wave's blocks: tile k+1 is in flight while tile k is
  // consumed. Every load is unconditional inside its branch, so the wait counters stay exact.
  Regs ra, rb;
  int k = 0;
  if (nmine > 0) {
    int id, valid;
    wave_block<NW>(ids, 0, w, pi, &id, &valid);
    load(ra, id);
    int va = valid;
    while (true) {
      if (k + 1 >= nmine) {
        consume(ra, va);
        break;
      }
      wave_block<NW>(ids, k + 1, w, pi, &id, &valid);
      load(rb, id);
      consume(ra, va);
      const int vb = valid;
      ++k;
      if (k + 1 >= nmine) {
        consume(rb, vb);
        break;
      }
      wave_block<NW>(ids, k + 1, w, pi, &id, &valid);
      load(ra, id);
      consume(rb, vb);
      va = valid;
      ++k;
    }
  }

  float l = lsum + __shfl_xor(lsum, 16);
  l += __shfl_xor(l, 32);
#pragma unroll
  for (int j = 0; j < VT; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) s_o[w][hq][16 * j + 4 * g + e] = o[j][e];
  }
  if (g == 0) {
    s_m[w][hq] = m;
    s_l[w][hq] = l;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * HD; e += NW * 64) {
    const int hh = e / HD, d = e % HD;
    float ms[NW], ls[NW];
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      ms[ww] = s_m[ww][hh];
      ls[ww] = s_l[ww][hh];
    }
    float M, L, O;
    combine_waves<NW>(ms, ls, &s_o[0][hh][d], 16 * OSTR, &M, &L, &O);
    emit<DT>(p, pi, seq, kvh * G + hh, part, d, HD, M, L, O);
  }
}

// ------------------------------------------------------------------------------------------
// Log-sum-exp merge of the partitions of sequences longer than one partition. One wave per
// (sequence, q head); partitions are combined in index order (deterministic).
template <int DT, int HD>
__global__ void __launch_bounds__(64)
merge_kernel(const AttnParams p) {
  constexpr int R = HD / 64;
  const int seq = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  int n = p.context_lens[seq];
  n = min(max(n, 0), p.max_ctx);
  const int nparts = (n + p.part_tokens - 1) / p.part_tokens;
  if (nparts <= 1) return;  // finished by the partition pass
  const size_t base = (static_cast<size_t>(seq) * p.Hq + h) * p.max_parts;
  float M = kNegInf;
  for (int j = lane; j < nparts; j += 64) M = fmaxf(M, p.ws_m[base + j]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  float L = 0.f, O[R];
#pragma unroll
  for (int r = 0; r < R; ++r) O[r] = 0.f;
  for (int j = 0; j < nparts; ++j) {
    const float mj = p.ws_m[base + j];
    if (mj == kNegInf) continue;
    const float wt = exp2_fast((mj - M) * kLog2e);
    L = fmaf(wt, p.ws_l[base + j], L);
    const float* oj = p.ws_o + (base + j) * HD;
#pragma unroll
    for (int r = 0; r < R; ++r) O[r] = fmaf(wt, oj[lane + 64 * r], O[r]);
  }
  const size_t orow = (static_cast<size_t>(seq) * p.Hq + h) * HD;
#pragma unroll
  for (int r = 0; r < R; ++r) Elem<DT>::put(p.out, orow + lane + 64 * r, L > 0.f ? O[r] / L : 0.f);
}

constexpr int kWaves = 4;

template <int DT, int HD>
hipError_t launch_partition_t(const AttnParams& p, int32_t kernel, hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale status left by an earlier, unrelated runtime call
  const dim3 block(kWaves * 64);
  if constexpr (DT != 0) {
    if (kernel == kMatrix) {
      const dim3 grid(p.B, p.Hkv, p.max_parts);
      hipLaunchKernelGGL((attn_matrix_kernel<DT, HD, kWaves>), grid, block, 0, stream, p);
      return note_error("attn_matrix_kernel launch", hipGetLastError());
    }
  }
  const dim3 grid(p.B, p.Hq, p.max_parts);
  hipLaunchKernelGGL((attn_vector_kernel<DT, HD, kWaves>), grid, block, 0, stream, p);
  return note_error("attn_vector_kernel launch", hipGetLastError());
}

template <int DT>
hipError_t launch_partition_d(const AttnParams& p, int32_t kernel, hipStream_t stream) {
  return p.hd == 64 ? launch_partition_t<DT, 64>(p, kernel, stream)
                    : launch_partition_t<DT, 128>(p, kernel, stream);
}

template <int DT>
hipError_t launch_merge_d(const AttnParams& p, hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale status left by an earlier, unrelated runtime call
  const dim3 grid(p.B, p.Hq);
  if (p.hd == 64)
    hipLaunchKernelGGL((merge_kernel<DT, 64>), grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((merge_kernel<DT, 128>), grid, dim3(64), 0, stream, p);
  return note_error("merge_kernel launch", hipGetLastError());
}

}  // namespace

int32_t select_kernel(int32_t dtype, int32_t G, int32_t request) {
  if (dtype == 0 || G > 16 || request == kVector) return kVector;
  if (request == kMatrix) return kMatrix;
  return G >= 2 ? kMatrix : kVector;
}

hipError_t launch_partition(const AttnParams& p, int32_t dtype, int32_t kernel,
                            hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_partition_d<0>(p, kVector, stream);
    case 1: return launch_partition_d<1>(p, kernel, stream);
    default: return launch_partition_d<2>(p, kernel, stream);
  }
}

hipError_t launch_merge(const AttnParams& p, int32_t dtype, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_merge_d<0>(p, stream);
    case 1: return launch_merge_d<1>(p, stream);
    default: return launch_merge_d<2>(p, stream);
  }
}

}  // namespace pkv
