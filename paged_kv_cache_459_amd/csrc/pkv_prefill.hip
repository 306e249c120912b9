// Paged prefill attention for gfx950 (CDNA4).
//
// What is computed ([P1] "vLLM 與 PagedAttention：高吞吐推理的關鍵", §三 步驟二 (預填充): the
// prompt's K/V go into the sequence's blocks, then the prompt is attended; the pages give no
// formula, ours is the textbook causal rule): the new token at position pos of a sequence
// attends over that sequence's tokens 0..pos, K/V found block by block through its block
// table, scaled dot products, max-subtracted softmax, fp32 accumulation.
//
// Work decomposition (our design). The host plan cuts each sequence's new tokens into tiles
// of up to 64*RT/G consecutive tokens; a unit is (sequence, tile, blocks [b0, b1)). One
// work-group of four waves takes one unit and one kv head: its 64*RT rows are (token, q head
// of the kv head's group), 16*RT per wave as RT row tiles of 16. The unit's blocks stream
// through LDS two at a time (double-buffered): each K/V tile is read from memory once per
// work-group and from LDS once per wave, and every fragment read from LDS feeds the RT row
// tiles' contractions; loads run three stages ahead, and each wave issues the next stage's
// q . k before the current stage's softmax. Both contractions run on 16x16x32 matrix-core
// instructions:
//   S^T (16 tokens x 16 rows) = K (16 x hd) . Q^T, per block;
//   O^T (16 dims x 16 rows) += V^T (16 dims x 32 tokens) . P^T, over the stage's two blocks,
// with the contraction index k = 8g + i standing for token 4g + i of the first block (i < 4)
// and token 4g + i - 4 of the second: exactly the tokens whose scores the lane already holds
// from the S^T tiles, so P needs no shuffle. Online softmax per row, in base-2 units.
//
// Masking: a row sees tokens < its position + 1 (row_vis); other tokens get probability 0
// (selected, not multiplied). K and V slots at or past the work-group's last visible token,
// and blocks whose table entry names no block of the pool, are zeroed in LDS once staged
// (unused slots may hold anything; a zero probability times NaN would still be NaN), so every
// score is finite and the row max may include tokens a row does not see.
//
// A unit holding all of its rows' blocks writes their outputs directly; a unit that is one
// chunk of a longer range (more than kPrefillMaxBlocks blocks) leaves (m, l, o) pieces that
// merge_kernel combines, as in decode.

#include <hip/hip_runtime.h>

#include "pkv_kernels.h"

namespace pkv {
namespace {

constexpr int kPW = 4;  // waves per work-group
constexpr int kPThreads = kPW * 64;
constexpr int kSB = 2;  // blocks per stage: one 32-token contraction
constexpr int kNBuf = 4;  // LDS stage buffers (loads run kNBuf - 1 stages ahead)
constexpr float kNegInf = -__builtin_inff();
// Running max before any visible token: finite, so 2^(x - m) needs no guard for rows that
// have seen nothing yet (x = -inf gives 0, and the first visible scores always rescale).
constexpr float kMaxInit = -3.0e38f;
// Lazy rescaling: a row's running max (base-2 units) is raised, and its sums rescaled, only
// when a stage's scores exceed it by more than this, so most stages skip the rescale.
// Probabilities then stay <= 2^8 (exact range for f16/bf16, far from fp32 overflow in the
// sums); the row sum adds the probabilities as rounded for the p.v contraction, so numerator
// and denominator weigh every token alike whatever the running max.
constexpr float kLazy = 8.f;

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <int DT>
struct Mma;

template <>
struct Mma<1> {
  __device__ static __forceinline__ float4_t mul(const uint4& a, const uint4& b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    const half2_t h = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
    return __builtin_bit_cast(uint32_t, h);
  }
  __device__ static __forceinline__ void put(void* base, size_t idx, float x) {
    static_cast<_Float16*>(base)[idx] = static_cast<_Float16>(x);
  }
  // acc + the sum of the 8 packed probabilities, as rounded for the p.v contraction
  __device__ static __forceinline__ float sum8(const uint4& pb, float acc) {
    const half2_t one = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pb.x), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pb.y), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pb.z), one, acc, false);
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pb.w), one, acc, false);
  }
};

template <>
struct Mma<2> {
  __device__ static __forceinline__ float4_t mul(const uint4& a, const uint4& b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    const bf16x2_t h = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, h);
  }
  __device__ static __forceinline__ void put(void* base, size_t idx, float x) {
    static_cast<__bf16*>(base)[idx] = static_cast<__bf16>(x);
  }
  __device__ static __forceinline__ float sum8(const uint4& pb, float acc) {
    const bf16x2_t one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pb.x), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pb.y), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pb.z), one, acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pb.w), one, acc, false);
  }
};

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Max of scores (no NaN reaches it: masked scores are replaced by -inf first). The
// NaN-propagating maximum maps to gfx950's v_maximum3_f32 and needs no quieting of its inputs,
// which fmaxf does in IEEE mode (two extra instructions per comparison).
__device__ __forceinline__ float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes holding one row's scores),
// with the gfx950 half-swaps: each returns the pair (own half copied, other half copied), so
// the max of the pair is the max over the two halves.
__device__ __forceinline__ float row_max4(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float m1 = smax(__builtin_bit_cast(float, a[0]), __builtin_bit_cast(float, a[1]));
  const unsigned u1 = __builtin_bit_cast(unsigned, m1);
  const auto b = __builtin_amdgcn_permlane16_swap(u1, u1, false, false);
  return smax(__builtin_bit_cast(float, b[0]), __builtin_bit_cast(float, b[1]));
}

// Zeroes the 16-bit tokens t0 + j (j < 8) of a V chunk with t0 + j >= valid.
__device__ __forceinline__ uint4 keep_tokens(uint4 v, int t0, int valid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = t0 + 2 * i < valid ? 0x0000FFFFu : 0u;
    const uint32_t hi = t0 + 2 * i + 1 < valid ? 0xFFFF0000u : 0u;
    w[i] &= lo | hi;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// One lane's 16 bytes from global memory straight into LDS (gfx950 global_load_lds_dwordx4):
// the wave's 64 lanes fill the 1 KB at LDS byte address `lds` (wave-uniform, through M0) in
// lane order. The source is a wave-uniform base address in scalar registers plus the lane's
// 32-bit byte offset, so a load needs no per-lane 64-bit address arithmetic. Issued as inline
// assembly so that the compiler neither tracks it nor adds its own (conservative: every later
// LDS read) waits; the kernel waits on vmcnt itself. M0 is an input operand bound to that
// register ("{m0}"), so the compiler sets it and knows its value; the statement only reads it.
// The s_nop is the one wait state an LDS DMA needs after an SALU write of M0, which the
// compiler cannot see through the statement.
__device__ __forceinline__ void load_lds16(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "{m0}"(lds)
               : "memory");
}

// Barrier of the stage loop: orders LDS only (a full __syncthreads would also wait for every
// load to LDS still in flight, the later stages' included). Each wave's reads of the previous
// stage have completed (lgkmcnt) before it passes, so that stage's buffer may be reloaded.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS placement swizzles (see the staging comment in the kernel).
__device__ __forceinline__ int kpos(int t, int blk) { return t ^ (((t >> 3) & 1) << 2) ^ (blk << 3); }
// the token at slot position pos (inverse of kpos: bit 3 of pos is bit 3 of t ^ blk)
__device__ __forceinline__ int ktok(int pos, int blk) {
  return pos ^ (blk << 3) ^ ((((pos >> 3) & 1) ^ blk) << 2);
}
__device__ __forceinline__ int vswz(int d) { return ((d >> 2) ^ (d >> 3)) & 1; }

// Waits until at most n of this wave's vector-memory operations are outstanding (they
// complete in order), n a multiple of the per-stage count; only the values used here.
template <int NCH>
__device__ __forceinline__ void wait_stages(int ahead) {
  // s_waitcnt: vmcnt in bits [3:0] (and [15:14]), expcnt [6:4] and lgkmcnt [11:8] left at max
  if (ahead >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * NCH));
  else if (ahead == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | NCH);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <int DT, int HD, int RT>
__global__ void __launch_bounds__(kPThreads)
__attribute__((amdgpu_waves_per_eu(RT >= 4 ? 1 : 2, RT >= 4 ? 1 : 2)))
attn_prefill_kernel(const StreamParams p) {
  using MM = Mma<DT>;
  constexpr int TILE = HD * kBlockSize * 2;  // bytes of one (block, kv head) K or V tile
  constexpr int PPT = TILE / 1024;           // 1 KB pieces per tile (one wave-wide load each)
  constexpr int KS = HD / 32;                // contraction steps of q . k
  constexpr int VT = HD / 16;                // 16-dim tiles of the output
  constexpr int STAGE = 2 * kSB * TILE;      // bytes of one stage: K, then V, of its blocks
  constexpr int NCH = STAGE / 1024 / kPW;    // loads per thread per stage
  static_assert(NCH * kPW * 1024 == STAGE && 2 * NCH <= 15, "stage size");
  static_assert(kSB == 2, "one 32-token contraction per stage");
  __shared__ __attribute__((aligned(1024))) char s_kv[kNBuf][STAGE];
  // the unit's block ids (-1: no block of the pool), then -1 past its end, so that a stage's
  // pair of ids is one aligned 8-byte read at an even index
  __shared__ __attribute__((aligned(16))) int32_t s_ids[kPrefillMaxBlocks + 4];
  __shared__ int32_t s_vmax[kPW];

  const int grid = gridDim.x, wg = blockIdx.x;
  const int lwg = (grid % 8 == 0) ? (wg % 8) * (grid / 8) + wg / 8 : wg;
  const int U = p.num_units;
  if (lwg >= U * p.Hkv) return;  // the whole work-group: before any barrier
  const int kvh = lwg / U, u = lwg - kvh * U;  // units fastest: a sequence's tiles share an XCD
  const int32_t* e = p.units + static_cast<size_t>(u) * kUnitInts;
  const int ref = uniform(e[0]), b0 = uniform(max(e[1], 0));
  const int b1 = uniform(min(min(e[2], p.max_blocks), b0 + kPrefillMaxBlocks));
  const int moff = uniform(e[3]), mcnt = uniform(e[4]), cbase = uniform(e[5]);
  if (ref < 0 || ref >= p.table_rows || b0 >= b1) return;

  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int hq = lane & 15, g = lane >> 4;
  const int G = p.Hq / p.Hkv;
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * TILE;
  const int nblk = b1 - b0;
  // Scores are kept unscaled; c > 0 scales them to base-2 units inside the exponentials (a
  // negative scale is carried by q's sign bits, flipped exactly on load).
  const float c = fabsf(p.scale_log2);
  const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;

  const int32_t* table = p.block_tables + static_cast<size_t>(ref) * p.max_blocks;
  const int nblk_even = (nblk + 1) & ~1;
  for (int i = tid; i < nblk_even + 2; i += kPThreads) {
    int v = -1;
    if (i < nblk) {
      const int raw = table[b0 + i];
      const int id = raw & ~kSharedBit;
      v = (raw < 0 || id >= p.NB) ? -1 : id;
    }
    s_ids[i] = v;
  }

  // This lane's rows: row tile k holds local rows (w*RT + k)*16 + hq.
  int seq[RT], jq[RT], mk[RT], n_row[RT];
  uint4 qb[RT][KS];
  int wmax = 0, wmin = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    const int r = (w * RT + k) * 16 + hq;
    mk[k] = r / G;
    jq[k] = r - mk[k] * G;
    int sq = -1;
    if (mk[k] < mcnt) sq = p.members[moff + mk[k]];
    seq[k] = (sq >= 0 && sq < p.B) ? sq : -1;
    n_row[k] = seq[k] < 0 ? 0 : min(max(p.row_vis[seq[k]], 0), p.max_ctx);
    if (seq[k] >= 0) {
      const uint4* qp = reinterpret_cast<const uint4*>(
          static_cast<const char*>(p.q) +
          (static_cast<size_t>(seq[k]) * p.Hq + kvh * G + jq[k]) * HD * 2);
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) {
        const uint4 v = qp[4 * s2 + g];
        qb[k][s2] = make_uint4(v.x ^ qsign, v.y ^ qsign, v.z ^ qsign, v.w ^ qsign);
      }
    } else {
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) qb[k][s2] = make_uint4(0, 0, 0, 0);
    }
    wmin = min(wmin, seq[k] >= 0 ? n_row[k] : 0x7fffffff);
    wmax = max(wmax, n_row[k]);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    wmin = min(wmin, __shfl_xor(wmin, off));
    wmax = max(wmax, __shfl_xor(wmax, off));
  }
  wmin = uniform(wmin);  // the wave's shortest and longest visible lengths
  wmax = uniform(wmax);
  if (lane == 0) s_vmax[w] = wmax;
  __syncthreads();  // s_ids, s_vmax
  int vmax = s_vmax[0];
#pragma unroll
  for (int i = 1; i < kPW; ++i) vmax = max(vmax, s_vmax[i]);
  vmax = uniform(vmax);

  // Staging: the stage's blocks a (t) and b (t + 1) go straight from memory to LDS, each
  // wave-wide load moving one 1 KB piece of a tile; the lanes' source addresses place the
  // 16-byte chunks (bank-swizzled for the reads below):
  //   K tile: slot 16c + pos holds chunk c (dims 8c .. 8c+7) of token t,
  //           pos = t ^ (4 * bit 3 of t) ^ (8 * block), block 0 for a, 1 for b;
  //   V tile: slot 2d + (h ^ bit 2 of d ^ bit 3 of d) holds tokens 8h .. 8h+7 of dim d.
  // Each group of 8 (and of 16) lanes of the reads below then covers distinct 16-byte columns
  // of the LDS banks.
  // An entry naming no block of the pool (or a block past the unit) is read from block 0 and
  // zeroed by the fix-up below.
  // each lane's source offset inside its tile, per piece (the same for every stage)
  int src_off[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int piece = w + kPW * i;
    const int tile = piece / PPT, sigma = (piece % PPT) * 64 + lane;
    const int kv = tile / kSB, sb = tile % kSB;
    if (kv == 0) {
      src_off[i] = 256 * (sigma >> 4) + 16 * ktok(sigma & 15, sb);
    } else {
      const int d = sigma >> 1;
      src_off[i] = 32 * d + 16 * ((sigma & 1) ^ vswz(d));
    }
  }
  const char* k_head = static_cast<const char*>(p.k_cache) + static_cast<size_t>(kvh) * TILE;
  const char* v_head = static_cast<const char*>(p.v_cache) + static_cast<size_t>(kvh) * TILE;
  // The two block ids of stage s (blocks b0 + 2s and b0 + 2s + 1; -1 for no block of the
  // pool or past the unit), read from LDS as one pair. The loop keeps the ids of the stages
  // in flight in registers: each stage's pair is read once, a step before it is needed, so
  // that no LDS read in the loop waits on its own.
  auto stage_ids = [&](int s) {
    return *reinterpret_cast<const int2*>(&s_ids[min(2 * s, nblk_even)]);
  };
  auto issue = [&](int2 ids, int buf) {
    const int id0 = uniform(max(ids.x, 0));
    const int id1 = uniform(max(ids.y, 0));
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int piece = w + kPW * i;  // wave-uniform
      const int tile = piece / PPT;
      const int kv = tile / kSB, sb = tile % kSB;
      const uintptr_t addr = reinterpret_cast<uintptr_t>(kv ? v_head : k_head) +
                             static_cast<uintptr_t>(sb == 0 ? id0 : id1) * blk_stride;
      const uint32_t lo = static_cast<uint32_t>(uniform(static_cast<int>(addr & 0xffffffffu)));
      const uint32_t hi = static_cast<uint32_t>(uniform(static_cast<int>(addr >> 32)));
      const char* base = reinterpret_cast<const char*>((static_cast<uintptr_t>(hi) << 32) | lo);
      const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
          (__attribute__((address_space(3))) char*)(&s_kv[buf][piece * 1024])));
      load_lds16(base, static_cast<uint32_t>(src_off[i]),
                 static_cast<uint32_t>(uniform(static_cast<int>(lds))));
    }
  };

  // Zeroes, in the staged copy of stage t, the K and V slots of tokens at or past vmax and of
  // entries naming no block (-1).
  auto fixup = [&](int buf, int t, int ida, int idb) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int piece = w + kPW * i;
      const int tile = piece / PPT, sigma = (piece % PPT) * 64 + lane;
      const int kv = tile / kSB, sb = tile % kSB;
      const int lim = (sb == 0 ? ida : idb) < 0 ? 0 : vmax - kBlockSize * (t + sb);
      if (lim >= kBlockSize) continue;
      uint4* slot = reinterpret_cast<uint4*>(&s_kv[buf][piece * 1024 + 16 * lane]);
      if (kv == 0) {
        if (ktok(sigma & 15, sb) >= lim) *slot = make_uint4(0, 0, 0, 0);
      } else {
        const int d = sigma >> 1;
        *slot = keep_tokens(*slot, 8 * ((sigma & 1) ^ vswz(d)), lim);
      }
    }
  };

  float m[RT], lsum[RT];
  float4_t o[RT][VT];
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    m[k] = kMaxInit;
    lsum[k] = 0.f;
#pragma unroll
    for (int j = 0; j < VT; ++j) o[k][j] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  // q . k runs as two 16-token contractions whose K rows are permuted so that lane (hq, g)
  // ends with the scores of 8 consecutive tokens of one block: block g >> 1, tokens
  // 8 (g & 1) .. +7 (the first four from contraction 1, the rest from contraction 2). Row m
  // of contraction 1 is token (m & 3) + 8 ((m >> 2) & 1) of block m >> 3; contraction 2 adds 4.
  const int rm = lane & 15, kg = lane >> 4;
  const int rblk = rm >> 3, rt1 = (rm & 3) + 8 * ((rm >> 2) & 1), rt2 = rt1 + 4;
  const int k_off1 = rblk * TILE + 256 * kg + 16 * kpos(rt1, rblk);
  const int k_off2 = rblk * TILE + 256 * kg + 16 * kpos(rt2, rblk);
  // p.v: lane (dim 16j + hq, g) takes tokens 8 (g & 1) .. +7 of block g >> 1 in one read
  const int v_off = kSB * TILE + (g >> 1) * TILE + 32 * hq + 16 * ((g & 1) ^ vswz(hq));
  const int tok_lane = kBlockSize * (g >> 1) + 8 * (g & 1);  // first token of this lane's 8

  // q . k of one stage (both blocks, every row tile) into (sa, sbv)
  auto qk = [&](int buf, float4_t (&sa)[RT], float4_t (&sbv)[RT]) {
    const char* st = s_kv[buf];
    uint4 kf1[KS], kf2[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      kf1[s2] = *reinterpret_cast<const uint4*>(st + k_off1 + 1024 * s2);
      kf2[s2] = *reinterpret_cast<const uint4*>(st + k_off2 + 1024 * s2);
    }
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      sa[k] = float4_t{0.f, 0.f, 0.f, 0.f};
      sbv[k] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        sa[k] = MM::mul(kf1[s2], qb[k][s2], sa[k]);
        sbv[k] = MM::mul(kf2[s2], qb[k][s2], sbv[k]);
      }
    // every K fragment read issued before the first contraction waits on one
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * KS * RT, 0);
  };

  // Softmax and p . v of stage t (block ids ida, idb) from its scores (sa, sbv).
  auto finish = [&](int buf, int t, int ida, int idb, const float4_t (&sa)[RT],
                    const float4_t (&sbv)[RT]) {
    if (kBlockSize * t >= wmax) return;  // nothing of the stage is visible to this wave
    const char* st = s_kv[buf];
    uint4 vf[VT];
#pragma unroll
    for (int j = 0; j < VT; ++j) vf[j] = *reinterpret_cast<const uint4*>(st + v_off + 512 * j);
    // The softmax runs at raised wave priority, up to the last row tile's contraction: the
    // other wave of the SIMD (another work-group, in its own stage) then issues its matrix-core
    // instructions in the gaps of this wave's VALU chain rather than in turn with it.
    __builtin_amdgcn_s_setprio(3);
    // this lane's 8 tokens: valid (a block of the pool) and their first logical index
    const bool lane_blk_ok = (g >> 1) == 0 ? ida >= 0 : idb >= 0;
    const int tok0 = kBlockSize * t + tok_lane;
    float x[RT][8];
#pragma unroll
    for (int k = 0; k < RT; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[k][i] = sa[k][i];
        x[k][4 + i] = sbv[k][i];
      }
    // Every score is finite here (slots past the work-group's last visible token, and blocks
    // outside the pool, were zeroed in LDS), so the row max may include tokens a row does not
    // see: it only keeps the exponentials in range. Invisible tokens get probability 0 below.
    const bool full = ida >= 0 && idb >= 0 && kBlockSize * (t + 2) <= wmin;
    // The lazy test needs no row maximum: a row's scores exceed its running max by more than
    // kLazy exactly when one of its four lanes' own maxima does (c >= 0 keeps the order). The
    // row maximum (across the lanes) is taken only on the rare stage that raises it.
    float lm[RT];
    bool grow = false;
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      lm[k] = smax(smax(smax(x[k][0], x[k][1]), smax(x[k][2], x[k][3])),
                   smax(smax(x[k][4], x[k][5]), smax(x[k][6], x[k][7])));
      grow = grow || lm[k] * c > m[k] + kLazy;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // wave-uniform
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        const float bm = row_max4(lm[k]) * c;  // base-2 units
        const float mn = fmaxf(m[k], bm);
        const float alpha = __builtin_amdgcn_exp2f(m[k] - mn);
        m[k] = mn;
        lsum[k] *= alpha;
#pragma unroll
        for (int j = 0; j < VT; ++j) o[k][j] *= alpha;
      }
    }
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      float pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(x[k][i], c, -m[k]));
      if (!full) {  // tokens past the row's position (or of no block): probability 0
        const int nr = lane_blk_ok ? min(8, max(0, n_row[k] - tok0)) : 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) pr[i] = i < nr ? pr[i] : 0.f;
      }
      const uint4 pb = make_uint4(MM::pack2(pr[0], pr[1]), MM::pack2(pr[2], pr[3]),
                                  MM::pack2(pr[4], pr[5]), MM::pack2(pr[6], pr[7]));
      // the row sum takes the probabilities as rounded for the contraction: numerator and
      // denominator then weigh every token alike
      lsum[k] = MM::sum8(pb, lsum[k]);
      if (k == RT - 1) __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int j = 0; j < VT; ++j) o[k][j] = MM::mul(vf[j], pb, o[k][j]);
    }
  };

  // Stage s lands: this wave's loads of it are done (at most `ahead` later stages in flight),
  // the barrier publishes every wave's, and a stage holding slots at or past the work-group's
  // last visible token (its last), a block outside the pool or no second block has those K
  // and V slots zeroed in LDS once, for every wave (unused slots may hold anything, NaN too).
  auto land = [&](int s, int ahead, int ida, int idb) {
    const int t = b0 + kSB * s;
    wait_stages<NCH>(ahead);
    lds_barrier();
    if (!(ida >= 0 && idb >= 0 && kBlockSize * (t + 2) <= vmax)) {
      fixup(s % kNBuf, t, ida, idb);
      lds_barrier();
    }
  };

  // Pipeline. Loads run kNBuf - 1 stages ahead into kNBuf LDS buffers. Within a wave, the
  // q . k contractions of stage s + 1 are issued before the softmax of stage s, so the matrix
  // cores work while the VALU does; stage s + 1 therefore lands (and the loads of stage
  // s + kNBuf - 1 go into the buffer of stage s - 1, which every wave finished before that
  // landing's barrier) before stage s is finished.
  const int nst = (nblk + kSB - 1) / kSB;
  constexpr int PD = kNBuf - 1;
  static_assert(PD >= 2, "the loop lands stage s + 1 while stage s + PD loads");
  // block ids of stages s .. s + PD - 1 (wave-uniform), and the pair of stage s + PD read
  // ahead
  int r0[PD], r1[PD];
#pragma unroll
  for (int q = 0; q < PD; ++q) {
    const int2 iq = stage_ids(q);
    r0[q] = uniform(iq.x);
    r1[q] = uniform(iq.y);
  }
  int2 ahead_ids = stage_ids(PD);
#pragma unroll
  for (int q = 0; q < PD; ++q)
    if (q < nst) issue(make_int2(r0[q], r1[q]), q);
  land(0, min(PD - 1, nst - 1), r0[0], r1[0]);
  float4_t sa0[RT], sb0[RT], sa1[RT], sb1[RT];
  if (kBlockSize * b0 < wmax) qk(0, sa0, sb0);
  auto step = [&](int s, const float4_t (&ca)[RT], const float4_t (&cb)[RT], float4_t (&na)[RT],
                  float4_t (&nb)[RT]) {
    const int t = b0 + kSB * s;
    // the ids of stage s + PD (read a step ago), and the read of the next step's
    const int e0 = uniform(ahead_ids.x), e1 = uniform(ahead_ids.y);
    ahead_ids = stage_ids(s + PD + 1);
    if (s + 1 < nst) {
      land(s + 1, min(PD - 2, nst - 2 - s), r0[1], r1[1]);
      if (s + PD < nst) issue(make_int2(e0, e1), (s + PD) % kNBuf);
      if (kBlockSize * (t + kSB) < wmax) qk((s + 1) % kNBuf, na, nb);
      __builtin_amdgcn_sched_barrier(0);  // keep those contractions ahead of the softmax
    }
    finish(s % kNBuf, t, r0[0], r1[0], ca, cb);
#pragma unroll
    for (int q = 0; q + 1 < PD; ++q) {
      r0[q] = r0[q + 1];
      r1[q] = r1[q + 1];
    }
    r0[PD - 1] = e0;
    r1[PD - 1] = e1;
  };
  for (int s = 0; s < nst; s += 2) {
    step(s, sa0, sb0, sa1, sb1);
    if (s + 1 >= nst) break;
    step(s + 1, sa1, sb1, sa0, sb0);
  }

#pragma unroll
  for (int k = 0; k < RT; ++k) {
    float l = lsum[k] + __shfl_xor(lsum[k], 16);
    l += __shfl_xor(l, 32);
    if (seq[k] < 0) continue;
    const int qh = kvh * G + jq[k];
    if (cbase < 0) {  // the unit saw every token of its rows
      const size_t orow = (static_cast<size_t>(seq[k]) * p.Hq + qh) * HD;
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int j = 0; j < VT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) MM::put(p.out, orow + 16 * j + 4 * g + i, o[k][j][i] * inv);
    } else {  // a piece: cell (shared_base + cell_base + member*Hkv + kvh), row jq
      const int rel = cbase + mk[k] * p.Hkv + kvh;
      if (rel >= p.shared_cells) continue;
      const size_t cell = (static_cast<size_t>(p.shared_base) + rel) * G + jq[k];
#pragma unroll
      for (int j = 0; j < VT; ++j)
        *reinterpret_cast<float4_t*>(p.ws_o + cell * HD + 16 * j + 4 * g) = o[k][j];
      if (g == 0) {
        p.ws_ml[cell * 2] = l > 0.f ? m[k] : kNegInf;  // no visible token: an empty piece
        p.ws_ml[cell * 2 + 1] = l;
      }
    }
  }
}

template <int DT, int HD>
void launch_prefill_t(const StreamParams& p, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_prefill_kernel<DT, HD, kPrefillRowTiles>), dim3(grid),
                     dim3(kPThreads), 0, stream, p);
}

}  // namespace

int32_t prefill_tile_rows(int32_t G) { return G > 0 ? kPW * 16 * kPrefillRowTiles / G : 0; }

hipError_t launch_prefill(const StreamParams& p, int32_t dtype, hipStream_t stream) {
  if (p.num_units == 0) return hipSuccess;
  (void)hipGetLastError();  // drop a stale status left by an earlier, unrelated runtime call
  int64_t grid = static_cast<int64_t>(p.num_units) * p.Hkv;
  grid = (grid + 7) / 8 * 8;  // a multiple of 8 for the XCD-contiguous mapping
  const unsigned g = static_cast<unsigned>(grid);
  switch (dtype) {
    case 1:
      if (p.hd == 64) launch_prefill_t<1, 64>(p, g, stream);
      else launch_prefill_t<1, 128>(p, g, stream);
      break;
    case 2:
      if (p.hd == 64) launch_prefill_t<2, 64>(p, g, stream);
      else launch_prefill_t<2, 128>(p, g, stream);
      break;
    default: return note_error("attn_prefill_kernel (f16/bf16 only)", hipErrorInvalidValue);
  }
  return note_error("attn_prefill_kernel launch", hipGetLastError());
}

}  // namespace pkv
