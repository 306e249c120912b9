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
// tiles' contractions. Both contractions run on 16x16x32 matrix-core instructions:
//   S^T (16 tokens x 16 rows) = K (16 x hd) . Q^T, per block;
//   O^T (16 dims x 16 rows) += V^T (16 dims x 32 tokens) . P^T, over the stage's two blocks,
// with the contraction index k = 8g + i standing for token 4g + i of the first block (i < 4)
// and token 4g + i - 4 of the second: exactly the tokens whose scores the lane already holds
// from the S^T tiles, so P needs no shuffle. Online softmax per row, in base-2 units.
//
// Masking: a row sees tokens < its position + 1 (row_vis); scores of other tokens are
// selected to -inf. V slots at or past the work-group's last visible token are zeroed when
// staged (unused slots may hold anything; a zero probability times NaN would still be NaN),
// and blocks whose table entry names no block of the pool are staged as zeros and masked.
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
constexpr float kNegInf = -__builtin_inff();
// Running max before any visible token: finite, so 2^(x - m) needs no guard for rows that
// have seen nothing yet (x = -inf gives 0, and the first visible scores always rescale).
constexpr float kMaxInit = -3.0e38f;

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

// Max over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes holding one row's scores),
// with the gfx950 half-swaps: each returns the pair (own half copied, other half copied), so
// the max of the pair is the max over the two halves.
__device__ __forceinline__ float row_max4(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float m1 = fmaxf(__builtin_bit_cast(float, a[0]), __builtin_bit_cast(float, a[1]));
  const unsigned u1 = __builtin_bit_cast(unsigned, m1);
  const auto b = __builtin_amdgcn_permlane16_swap(u1, u1, false, false);
  return fmaxf(__builtin_bit_cast(float, b[0]), __builtin_bit_cast(float, b[1]));
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

template <int DT, int HD, int RT>
__global__ void __launch_bounds__(kPThreads)
__attribute__((amdgpu_waves_per_eu(RT >= 4 ? 1 : 2, RT >= 4 ? 1 : 2)))
attn_prefill_kernel(const StreamParams p) {
  using MM = Mma<DT>;
  constexpr int TILE = HD * kBlockSize * 2;  // bytes of one (block, kv head) K or V tile
  constexpr int CHT = TILE / 16;             // 16-byte chunks per tile
  constexpr int KS = HD / 32;                // contraction steps of q . k
  constexpr int VT = HD / 16;                // 16-dim tiles of the output
  constexpr int NCH = 2 * kSB * CHT / kPThreads;  // staged chunks per thread per stage
  static_assert(NCH * kPThreads == 2 * kSB * CHT, "stage size");
  static_assert(kSB == 2, "one 32-token contraction per stage");
  // Per buffer: the stage's K tiles as in the cache, then its V as one [HD][64 B] array: for
  // dim d, 16-byte slot g ^ ((d & 15) >> 2) holds tokens 4g .. 4g+3 of the first block, then
  // of the second. A lane's p.v operand is then one 16-byte read, and the 16 lanes reading a
  // slot of dims 16j .. 16j+15 together touch all 64 banks once.
  __shared__ __attribute__((aligned(16))) char s_kv[2][2 * kSB * TILE];
  __shared__ int32_t s_ids[kPrefillMaxBlocks];
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
  for (int i = tid; i < nblk; i += kPThreads) {
    const int raw = table[b0 + i];
    const int id = raw & ~kSharedBit;
    s_ids[i] = (raw < 0 || id >= p.NB) ? -1 : id;
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

  // Staging: chunk c of a stage is chunk c % CHT of tile c / CHT, tiles ordered K of the
  // stage's blocks, then V of them.
  auto stage_load = [&](uint4 (&r)[NCH], int t) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = tid + kPThreads * i;
      const int tile = ch / CHT, ci = ch - tile * CHT;
      const int kv = tile / kSB, sb = tile - kv * kSB;
      const int blk = t + sb;
      const int id = blk < b1 ? s_ids[blk - b0] : -1;
      r[i] = make_uint4(0, 0, 0, 0);
      if (id >= 0) {
        const char* src = static_cast<const char*>(kv ? p.v_cache : p.k_cache) +
                          static_cast<size_t>(id) * blk_stride + static_cast<size_t>(kvh) * TILE;
        r[i] = *reinterpret_cast<const uint4*>(src + 16 * ci);
      }
    }
  };
  auto stage_store = [&](const uint4 (&r)[NCH], int buf, int t) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = tid + kPThreads * i;
      const int tile = ch / CHT, ci = ch - tile * CHT;
      const int kv = tile / kSB, sb = tile - kv * kSB;
      uint4 v = r[i];
      if (kv == 0) {
        *reinterpret_cast<uint4*>(&s_kv[buf][sb * TILE + 16 * ci]) = v;
      } else {
        // a V chunk: dim d = ci / 2, tokens 8h .. 8h+7 (h = ci & 1) of block sb: groups 2h, 2h+1
        const int tok0 = kBlockSize * (t + sb), d = ci >> 1, h = ci & 1;
        // slots at or past every row's last visible token: zero
        if (tok0 + kBlockSize > vmax) v = keep_tokens(v, 8 * h, vmax - tok0);
        char* row = &s_kv[buf][kSB * TILE + 64 * d + 8 * sb];
        const int sw = (d & 15) >> 2;
        *reinterpret_cast<uint2*>(row + 16 * ((2 * h) ^ sw)) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2*>(row + 16 * ((2 * h + 1) ^ sw)) = make_uint2(v.z, v.w);
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
  const int v_lane = 64 * hq + 16 * (g ^ (hq >> 2));

  auto compute = [&](int buf, int t) {
    if (kBlockSize * t >= wmax) return;  // nothing of the stage is visible to this wave
    const int ida = s_ids[t - b0];
    const int idb = t + 1 < b1 ? s_ids[t + 1 - b0] : -1;
    const char* kt = s_kv[buf];
    const char* vt = s_kv[buf] + kSB * TILE;
    uint4 kfa[KS], kfb[KS], vf[VT];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      kfa[s2] = *reinterpret_cast<const uint4*>(kt + 1024 * s2 + 16 * lane);
      kfb[s2] = *reinterpret_cast<const uint4*>(kt + TILE + 1024 * s2 + 16 * lane);
    }
#pragma unroll
    for (int j = 0; j < VT; ++j) vf[j] = *reinterpret_cast<const uint4*>(vt + 1024 * j + v_lane);
    // S^T of every row tile (independent accumulation chains, interleaved)
    float4_t sa[RT], sbv[RT];
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      sa[k] = float4_t{0.f, 0.f, 0.f, 0.f};
      sbv[k] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        sa[k] = MM::mul(kfa[s2], qb[k][s2], sa[k]);
        sbv[k] = MM::mul(kfb[s2], qb[k][s2], sbv[k]);
      }
    float x[RT][8];
#pragma unroll
    for (int k = 0; k < RT; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[k][i] = sa[k][i];
        x[k][4 + i] = sbv[k][i];
      }
    // every row of the wave sees all 32 tokens: no masking
    const bool full = ida >= 0 && idb >= 0 && kBlockSize * (t + 2) <= wmin;
    if (!full) {
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        const int ra = ida < 0 ? 0 : min(kBlockSize, max(0, n_row[k] - kBlockSize * t));
        const int rb = idb < 0 ? 0 : min(kBlockSize, max(0, n_row[k] - kBlockSize * (t + 1)));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[k][i] = 4 * g + i < ra ? x[k][i] : kNegInf;
          x[k][4 + i] = 4 * g + i < rb ? x[k][4 + i] : kNegInf;
        }
      }
    }
    float bm[RT];
    bool grow = false;
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      const float v = fmaxf(fmaxf(fmaxf(x[k][0], x[k][1]), fmaxf(x[k][2], x[k][3])),
                            fmaxf(fmaxf(x[k][4], x[k][5]), fmaxf(x[k][6], x[k][7])));
      bm[k] = row_max4(v) * c;  // base-2 units (c > 0 keeps the order)
      grow = grow || bm[k] > m[k];
    }
    // Exact running max (the largest probability of a row is exactly 1, so its token's weight
    // carries no rounding in the 16-bit p.v operand); the rescale is skipped, wave-uniformly,
    // when no row's max rose.
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        const float mn = fmaxf(m[k], bm[k]);
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
      if (!full) {  // masked tokens: probability 0 whatever the scale (-inf * 0 would be NaN)
#pragma unroll
        for (int i = 0; i < 8; ++i) pr[i] = x[k][i] == kNegInf ? 0.f : pr[i];
      }
      const uint4 pb = make_uint4(MM::pack2(pr[0], pr[1]), MM::pack2(pr[2], pr[3]),
                                  MM::pack2(pr[4], pr[5]), MM::pack2(pr[6], pr[7]));
      // the row sum takes the probabilities as rounded for the contraction: numerator and
      // denominator then weigh every token alike
      lsum[k] = MM::sum8(pb, lsum[k]);
#pragma unroll
      for (int j = 0; j < VT; ++j) o[k][j] = MM::mul(vf[j], pb, o[k][j]);
    }
  };

  uint4 stg[NCH];
  const int nst = (nblk + kSB - 1) / kSB;
  stage_load(stg, b0);
  stage_store(stg, 0, b0);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int t = b0 + kSB * s;
    const bool more = s + 1 < nst;
    if (more) stage_load(stg, t + kSB);  // in flight while this stage is computed
    compute(s & 1, t);
    if (more) stage_store(stg, (s + 1) & 1, t + kSB);
    __syncthreads();
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
