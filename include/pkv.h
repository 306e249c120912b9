/*
 * pkv.h -- C ABI of libpkv: PagedAttention decode on AMD Instinct MI355X (gfx950).
 *
 * Sources. The method is the one described on three web pages:
 *   [P1] "vLLM 與 PagedAttention：高吞吐推理的關鍵" (blog-7wy.pages.dev)
 *   [P2] vLLM overview, section "PagedAttention 的核心原理" (xiexianbin.cn)
 *   [P3] "vLLM 与 PagedAttention：大模型高性能推理服务实战" (zhengtianqi.github.io)
 * The pages describe the KV cache as fixed-size blocks of 16 tokens that sit anywhere in a
 * shared pool, reached through a per-sequence block table, allocated on demand, freed when a
 * request finishes, and shared between sequences with a common prefix or beam history.
 * They give no attention formula, no memory layout and no kernel; where this header fixes one
 * it says so ("our reading").
 *
 * Conventions shared by every call
 *   - Every call returns a pkv_status (int32). No C++ exception crosses this boundary.
 *   - Device calls take plain device pointers and a hipStream_t passed as `void* stream`
 *     (NULL = the default stream). They only enqueue work: the status covers host-side argument
 *     checks and launch errors, not the kernels' completion. They allocate no device memory:
 *     the caller owns every device buffer (inputs, outputs, caches, tables, workspace).
 *   - Arguments are validated on the host before any HIP call; on an error nothing is launched.
 *   - Device-resident indices (slot mappings, block tables, context lengths) are not read by the
 *     host on the fast path. Kernels treat them defensively so that no value can make them
 *     access memory out of bounds: see each call. Setting the environment variable PKV_CHECK=1
 *     makes the device calls copy those indices to the host (synchronously), validate them
 *     against the contract and return PKV_ERR_INDEX before launching if they break it.
 *   - All device pointers must be 16-byte aligned (PKV_ERR_INVALID_ARG otherwise).
 *   - Token positions, logical blocks and slots are 0-based (our reading: [P1] numbers tokens
 *     from 1 in one figure and logical blocks from 0 in the block-table example).
 *
 * Cache layout (our reading; the pages fix only the 16-token block, [P1] §二 "具體運作方式",
 * [P3] §3.2). Let E = element bytes (4 for f32, 2 for f16/bf16), X = 16 / E (elements in one
 * 16-byte chunk), bs = 16 tokens per block, hd = head_dim, Hkv = number of KV heads, NB =
 * number of physical blocks in the pool. One (block, kv-head) pair owns one contiguous "tile"
 * of bs*hd elements in each cache:
 *   k_cache: [NB][Hkv][hd/X][bs][X]   element (b, h, token t, dim d) at
 *            ((b*Hkv + h)*(hd/X) + d/X)*bs*X + t*X + d%X
 *   v_cache: [NB][Hkv][hd][bs]        element (b, h, token t, dim d) at
 *            ((b*Hkv + h)*hd + d)*bs + t
 * i.e. K is stored as 16-byte chunks of consecutive dims, token-minor, and V is stored
 * dim-major with the 16 tokens of a block contiguous. Both choices make every per-lane load of
 * the attention kernels a single contiguous 8- or 16-byte access. Token t of a sequence lives
 * in its logical block t/bs, at offset t%bs inside the physical block the table names.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, negative size, bad combination      */
  PKV_ERR_UNSUPPORTED = 2,   /* head_dim not in {64,128}, block size != 16, unknown dtype     */
  PKV_ERR_OUT_OF_BLOCKS = 3, /* allocator: pool exhausted; the allocator state is unchanged   */
  PKV_ERR_UNKNOWN_SEQ = 4,   /* allocator: sequence id not present                           */
  PKV_ERR_SEQ_EXISTS = 5,    /* allocator: sequence id already present                       */
  PKV_ERR_WORKSPACE = 6,     /* workspace pointer null or smaller than required               */
  PKV_ERR_INDEX = 7,         /* PKV_CHECK=1 found a device index outside the contract         */
  PKV_ERR_HIP = 8            /* a HIP runtime call or a kernel launch failed                  */
};

typedef int32_t pkv_dtype;
enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 };

/* Human-readable name of a status code (static storage; never NULL). */
const char* pkv_status_string(pkv_status status);

/* Detail of the most recent PKV_ERR_HIP returned on the calling thread: which launch or runtime
 * call failed and the HIP error text (also set with the PKV_ERR_WORKSPACE of
 * pkv_decode_append_attn_noalloc). Thread-local storage owned by the library, valid until the
 * thread's next failing call; "" if none. */
const char* pkv_last_error(void);

/* Bytes of ONE cache tensor (k_cache or v_cache) for a pool of NB blocks; 0 on bad arguments. */
size_t pkv_cache_bytes(int32_t NB, int32_t Hkv, int32_t hd, int32_t bs, pkv_dtype dtype);

/* ------------------------------------------------------------------------------------------ */
/* Cache write.                                                                              */
/* [P1] §三 步驟二/步驟三: the new tokens' K/V are computed and written into the current block */
/* (a fresh block is taken when it is full). The slot of token i, slot = block*bs + offset,  */
/* is chosen by the allocator (pkv_alloc_append); this call only scatters.                   */
/*   k, v          device, [T][Hkv][hd] contiguous, dtype `dtype` (read)                     */
/*   k_cache, v_cache  device, cache layout above, NB blocks (written at the given slots only) */
/*   slot_mapping  device int32 [T]; token i goes to block slot/bs, offset slot%bs.          */
/*                 slot < 0 (padding) and slot >= NB*bs are skipped, so no value can write   */
/*                 outside the caches. Two tokens with the same slot in one call is a caller */
/*                 error: which one lands is undefined.                                       */
/* The copy is bitwise. T == 0 is a no-op. Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED  */
/* (also Hkv > 65535), PKV_ERR_INDEX (PKV_CHECK=1: slot >= NB*bs or duplicate non-negative    */
/* slots), PKV_ERR_HIP.                                                                        */
pkv_status pkv_write(const void* k, const void* v, void* k_cache, void* v_cache,
                     const int32_t* slot_mapping, int32_t T, int32_t Hkv, int32_t hd, int32_t bs,
                     int32_t NB, pkv_dtype dtype, void* stream);

/* Copy-on-write block copy.                                                                 */
/* [P2] vLLM overview, "共享和复用" and the Beam Search item of "PagedAttention 的优势": beam  */
/* candidates share the blocks of their common history. The pages leave open what happens    */
/* when one of them appends into a shared, partly filled block; here pkv_alloc_append moves   */
/* the appender to a fresh block and reports the pair (src, dst), and this call copies the    */
/* data: for every pair i, every kv head's tile of block src[i] in both caches is copied      */
/* bitwise into block dst[i] (the whole block, slots past the filled ones included). Run it   */
/* before the write or attention that uses the new block, on the same stream.                 */
/*   k_cache, v_cache  device, cache layout above, NB blocks (written at blocks dst[i] only)  */
/*   src, dst      device int32 [n]. A pair with either entry outside [0, NB) is skipped      */
/*                 (negative entries: padding). Caller contract: the non-skipped dst are      */
/*                 distinct and none of them is also a src of the call (pkv_alloc_append's    */
/*                 pairs satisfy both); otherwise the result is undefined, but every access   */
/*                 stays inside the caches.                                                   */
/* n == 0 is a no-op. Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED (also when one block    */
/* of one cache exceeds 1 GiB), PKV_ERR_INDEX (PKV_CHECK=1: an entry >= NB, a repeated dst or */
/* a dst that is also a src), PKV_ERR_HIP.                                                    */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                           int32_t n, int32_t Hkv, int32_t hd, int32_t bs, int32_t NB,
                           pkv_dtype dtype, void* stream);

/* ------------------------------------------------------------------------------------------ */
/* Decode attention.                                                                         */
/* [P1] §三 步驟三 (last step) and §五 (the attention-kernel row of the component table);     */
/* [P2] "PagedAttention 的核心原理": each sequence's KV is logically contiguous but physically */
/* scattered; attention is computed by finding all previous KV through the block table. The  */
/* pages give no formula; ours is scaled dot-product attention over the n = context_lens[i]   */
/* tokens of sequence i (the token just written included):                                    */
/*   out[i,h,:] = sum_t softmax_t(scale * q[i,h,:] . K_i[t,g(h),:]) * V_i[t,g(h),:]           */
/* with g(h) = h / (Hq/Hkv) (grouped-query heads: contiguous groups of G = Hq/Hkv q heads     */
/* share one kv head; G = 1 is multi-head attention). A row with n = 0 gives out = 0.          */
/* Arithmetic: products and sums in fp32, softmax with max subtraction, output rounded to     */
/* `dtype` to nearest-even. Results are deterministic: the same inputs give the same bits,    */
/* and they do not change with which physical blocks hold the K/V or whether blocks are       */
/* shared. The order of the fp32 sums of a row follows the batch's lengths (see the stream    */
/* pass below), so a sequence's result can differ in rounding between batches of different   */
/* lengths; it never depends on other sequences' values.                                      */
/*   out, q        device, [B][Hq][hd] contiguous, dtype `dtype` (out written, q read)         */
/*   block_tables  device int32 [B][max_blocks]; entry j of row i names the physical block of */
/*                 tokens [j*bs, (j+1)*bs) of sequence i. Only entries j < ceil(n_i/bs) are   */
/*                 read. An entry may carry PKV_BLOCK_SHARED (see pkv_alloc_tables_marked):   */
/*                 the block is the entry without it. An entry naming a block outside [0, NB) */
/*                 is never dereferenced for data: its tokens are skipped (the output is then */
/*                 undefined but no memory fault can occur).                                  */
/*   context_lens  device int32 [B]; values are clamped to [0, max_context_len] on the device.*/
/*   max_context_len  host bound on every n_i; must satisfy max_context_len <= max_blocks*bs. */
/*   scale         the softmax scale (1/sqrt(hd) in the usual model).                          */
/*   workspace     device scratch of at least pkv_decode_workspace_bytes(...) bytes, caller    */
/*                 owned; contents on entry are ignored. May be NULL only when that size is 0. */
/* Supported: hd in {64,128}, bs == 16, Hq % Hkv == 0, Hq <= 32767, dtype f32/f16/bf16.       */
/* Batches of more than 8192 sequences (or of more tiles than int32 positions allow) run as */
/* several stream+merge launches over consecutive row ranges, reusing the workspace in order.*/
/* The launch size comes from the calling thread's current HIP device.                        */
/* Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_INDEX          */
/* (PKV_CHECK=1: an entry j < ceil(n_i/bs) outside [0,NB), or n_i outside [0,max_context_len]),*/
/* PKV_ERR_HIP.                                                                                */
pkv_status pkv_decode_attn(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                           int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs, int32_t NB,
                           int32_t max_blocks, int32_t max_context_len, float scale,
                           pkv_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Decode step with the cache write fused in ([P1] §三 步驟三: the new token's K/V go into the */
/* current block, then attention runs over all of the sequence's tokens through the table).  */
/* For every sequence i with n_i >= 1 whose table entry b = block_tables[i][(n_i-1)/bs] lies  */
/* in [0, NB): the token at position n_i - 1 takes its K/V from k_new[i], v_new[i]; they are   */
/* stored bitwise into slot (b, (n_i-1) % bs) of the caches -- the slot pkv_alloc_append gave */
/* that token -- and the output is exactly that of pkv_decode_attn on the updated caches.     */
/* The call therefore equals pkv_write(k_new, v_new, those slots) followed by pkv_decode_attn, */
/* bit for bit, in one launch fewer (the stores ride in the merge pass). Caller contract: that slot is in a block no other        */
/* sequence of the batch reads (an appending sequence owns its last block: pkv_alloc_append   */
/* reports a copy-on-write pair otherwise).                                                   */
/*   k_new, v_new  device, [B][Hkv][hd] contiguous, dtype `dtype` (read); row i is ignored     */
/*                 when n_i = 0 or the entry is outside the pool (nothing is written then).    */
/*   k_cache, v_cache  written at those slots only. Other arguments as pkv_decode_attn, which  */
/*                 also gives the workspace size.                                              */
pkv_status pkv_decode_append_attn(void* out, const void* q, const void* k_new,
                                  const void* v_new, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs,
                                  int32_t NB, int32_t max_blocks, int32_t max_context_len,
                                  float scale, pkv_dtype dtype, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* pkv_decode_append_attn for callers that cannot allocate device memory (code under HIP graph */
/* capture, tight serving loops, harnesses that forbid allocation): the same arguments without */
/* the workspace, the same kernels and the same results, bit for bit. The stream/merge scratch */
/* is a file-scope device array of the library, 40 MiB on each GPU the library runs on, held   */
/* until the process ends; its address is looked up once per device on the first call there.  */
/* The call allocates nothing (no hipMalloc, no host-side allocation either). Every call on a  */
/* GPU shares that GPU's array: calls that overlap on one GPU (on different streams, or from   */
/* different threads without ordering) race and give undefined results; calls ordered on one  */
/* stream are safe (the scratch's contents on entry are ignored). PKV_CHECK index validation,  */
/* which needs host buffers and a synchronization, is not performed by this call.              */
/* Errors: as pkv_decode_append_attn; PKV_ERR_WORKSPACE when the shape needs more scratch than */
/* the array holds (pkv_decode_workspace_bytes > 40 MiB; pkv_last_error() says how much);      */
/* PKV_ERR_HIP if the array's address cannot be obtained.                                      */
pkv_status pkv_decode_append_attn_noalloc(void* out, const void* q, const void* k_new,
                                          const void* v_new, void* k_cache, void* v_cache,
                                          const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t B, int32_t Hq,
                                          int32_t Hkv, int32_t hd, int32_t bs, int32_t NB,
                                          int32_t max_blocks, int32_t max_context_len,
                                          float scale, pkv_dtype dtype, void* stream);

/* ---- Shared-prefix plans ([P1] §二 "解決三大問題" and [P2] "共享和复用": sequences with a   */
/* ---- common prefix, such as a system prompt or beam candidates, point at the same physical  */
/* ---- blocks). Attention over such blocks reads the same K/V for every sequence that shares */
/* ---- them; a plan lets the decode step read it once for all of them.                       */
/* A run is (members, logical blocks [j0, j1)): every member's table names the same block of  */
/* the pool at each index of the range. pkv_decode_plan finds the batch's runs from host      */
/* copies of its tables and lengths (entries may carry PKV_BLOCK_SHARED): sequences grouped by */
/* their first block, each group of two or more extended while all of its members agree,     */
/* then split where they part. A sequence's shared blocks are thus the first skip_s blocks of  */
/* its table. The decode step then runs three kernels (pkv_decode_planned):                   */
/*  1. shared pass: per unit (a chunk of up to 16 blocks of a run, up to 16/G of its members) */
/*     and kv head, one read of each K/V tile and an MFMA contraction over all of the unit's  */
/*     (member, q head) rows, each row masked at its own sequence's length -> one (m, l, o)   */
/*     piece per row;                                                                          */
/*  2. the stream pass over each sequence's remaining blocks (those after skip_s);            */
/*  3. the merge: for planned sequences, their private pieces and shared pieces, in order.    */
/* Results equal pkv_decode_attn's within rounding: the sums run in another order (the plan's), */
/* deterministic for a given plan. pkv_decode_plan puts runs in a plan only for f16/bf16 and  */
/* G = Hq/Hkv <= max_group (0: the default, 4 -- at least four sequences share each 16-row    */
/* tile; with fewer, the plain matrix-core pass, which re-reads shared blocks from the L2, is  */
/* faster; at most 16); for other shapes it returns a plan without runs (the planned call then */
/* does what the plain one does). Batches above 8192 sequences are not planned                */
/* (PKV_ERR_UNSUPPORTED).                                                                     */
/*                                                                                            */
/* Plan layout (int32, built by pkv_decode_plan, read by the kernels): header[16] = {magic,    */
/* B, H, GS, U, M, L, cells, chunk, 0...}, skip[B], blocks[B] (ceil(n/16) when planned),       */
/* sh_ptr[B+1], units[U][6] = {ref_seq, b0, b1, member_off, member_cnt, cell_base},             */
/* members[M], sh_list[L]. H / GS are the stream kernel's head slots and q heads per slot     */
/* (pkv_decode_kernel: matrix-core -> Hkv, G; vector -> Hq, 1); a plan is tied to them and to  */
/* B, so build it after choosing the kernel.                                                   */

/* Upper bound on the int32 entries of a plan for B sequences of up to max_blocks blocks.     */
size_t pkv_decode_plan_max_ints(int32_t B, int32_t max_blocks);

/* Host only (no GPU). block_tables/context_lens: host int32 [B][max_blocks] / [B] (the same   */
/* contents the device copies will hold). plan: host buffer of capacity ints; *plan_ints      */
/* receives the plan's size (also when capacity is too small: PKV_ERR_WORKSPACE). Errors:      */
/* PKV_ERR_INVALID_ARG (also max_group outside [0, 16]), PKV_ERR_UNSUPPORTED (dtype),           */
/* PKV_ERR_WORKSPACE.                                                                          */
pkv_status pkv_decode_plan(const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                           int32_t max_blocks, int32_t max_context_len, int32_t Hq, int32_t Hkv,
                           int32_t NB, pkv_dtype dtype, int32_t max_group, int32_t* plan,
                           size_t capacity, size_t* plan_ints);

/* Launches (1 or 2) of the shared and stream passes that pkv_decode_planned's passes 0 and 4   */
/* use for this plan: one where the one-launch kernel exists and the plan's shared pass reads  */
/* at least as many (block, head) tiles as its stream pass (the shared pass's work-groups     */
/* start first, the stream pass's short ranges fill its tail; where the stream pass dominates */
/* the one launch is no faster), else two; one for a plan without units. Host only; plan as   */
/* for pkv_decode_planned (the same B, heads, dtype,                                          */
/* max_blocks and num_workers). 0 on bad arguments or a plan that fails validation.            */
int32_t pkv_decode_planned_launches(const int32_t* plan, size_t plan_ints, int32_t B,
                                    int32_t Hq, int32_t Hkv, int32_t max_blocks,
                                    pkv_dtype dtype, int32_t num_workers);

/* Workspace bytes of pkv_decode_planned (stream cells plus B*H private and the plan's shared   */
/* cells); 0 on bad arguments or a plan built for another shape.                              */
size_t pkv_decode_planned_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t hd,
                                          pkv_dtype dtype, int32_t num_workers,
                                          const int32_t* plan, size_t plan_ints);

/* The planned decode step. pass: 0 the whole step (passes 4 and 3), 1 the shared pass, 2 the  */
/* stream pass, 3 the merge, 4 the shared and stream passes as pkv_decode_planned_launches    */
/* chooses (one launch or passes 1 and 2), 5 those two passes in one launch where it exists   */
/* (exported to time them: run 1, 2, 3 or 4, 3 or 5, 3 in that order on one stream). The one  */
/* launch exists for the vector stream kernel (G = 1, or pkv_set_attn_kernel(1)) with         */
/* num_workers a multiple of 32; elsewhere pass 5 is passes 1 and 2. Every pass order gives    */
/* bit-identical results.                                                                     */
/* k_new/v_new NULL: attention as pkv_decode_attn; non-NULL: the fused step of                 */
/* pkv_decode_append_attn (same contract; additionally no sequence's newest-token block may be */
/* in a run, which the plan check enforces through blocks[] and skip[]). plan_host and        */
/* plan_dev hold the same plan_ints entries (host, validated here; device, read by the        */
/* kernels); context_lens and the tables must be those the plan was built from.                */
/* num_workers as pkv_decode_stream. Errors: as pkv_decode_append_attn, plus                   */
/* PKV_ERR_INVALID_ARG for a plan that fails the check or does not match the shapes, and      */
/* PKV_ERR_UNSUPPORTED for f32 or G > 16 with units, or when (units * Hkv + num_workers) * 64  */
/* work-items would pass 2^31 - 1.                                                            */
pkv_status pkv_decode_planned(int32_t pass, void* out, const void* q, const void* k_new,
                              const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                              int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs, int32_t NB,
                              int32_t max_blocks, int32_t max_context_len, float scale,
                              pkv_dtype dtype, const int32_t* plan_host, const int32_t* plan_dev,
                              size_t plan_ints, int32_t num_workers, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------ */
/* Paged prefill attention. [P1] §三 步驟二 (預填充): a prompt's tokens are written to the      */
/* cache and attended; with a cached prefix ([P2] "共享和复用", automatic prefix caching) or in     */
/* chunks, only the last q_s of a sequence's n_s tokens are new. Causal rule: the new token at */
/* position pos = n_s - q_s + k (k = 0..q_s-1) attends to its own sequence's tokens 0..pos,   */
/* all read from the paged cache through the block table (pkv_write them first):             */
/*   out[t][h] = softmax_j(scale * q[t][h] . K[s][h/G][j], j <= pos) . V[s][h/G][j]            */
/* with t = query_start[s] + k the row of the new token. f16/bf16 only (matrix cores), G <= 16. */
/*                                                                                            */
/* The work is planned on the host (pkv_prefill_plan, from host copies of query_start and    */
/* context_lens): tiles of consecutive rows of one sequence, each split into chunks of at most */
/* `chunk` blocks when its last row sees more (then every row's chunks give (m, l, o) pieces   */
/* that a merge combines in chunk order, as pkv_decode_merge does). chunk is 512, halved      */
/* (down to 64) while the launch would have fewer than 1024 (unit, kv head) work-groups.      */
/* Plan layout (int32):                                                                        */
/* header[16] = {magic 0x50524631, T, H, GS, U, M, L, cells, chunk, S, tile_rows, 0...},       */
/* skip[T] (1: the row is merged), vis[T] (pos + 1), ptr[T+1], units[U][6] = {sequence, b0,   */
/* b1, member_off, member_cnt, cell_base (-1: written directly)}, members[M] (rows),           */
/* list[L] (each merged row's piece cells, in chunk order); H = Hkv, GS = G.                  */

/* Host only. query_start: [S+1] with query_start[0] = 0, non-decreasing; T = query_start[S].  */
/* context_lens: [S], q_s <= n_s <= max_context_len <= 16*max_blocks. plan: host buffer of    */
/* capacity ints; *plan_ints receives the plan's size (also with PKV_ERR_WORKSPACE when the   */
/* capacity is too small). Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED (f32, G > 16),    */
/* PKV_ERR_WORKSPACE.                                                                          */
pkv_status pkv_prefill_plan(const int32_t* query_start, const int32_t* context_lens, int32_t S,
                            int32_t max_blocks, int32_t max_context_len, int32_t Hq, int32_t Hkv,
                            pkv_dtype dtype, int32_t* plan, size_t capacity, size_t* plan_ints);

/* Workspace bytes of pkv_prefill_attn for this plan: cells*G*(2 + hd)*4 rounded up ((m, l)    */
/* at 0, then o at round_up(cells*G*8, 256)); may be 0 (every tile direct). (size_t)-1 on bad   */
/* arguments or a plan that is not a prefill plan.                                            */
size_t pkv_prefill_workspace_bytes(int32_t Hq, int32_t Hkv, int32_t hd, const int32_t* plan,
                                   size_t plan_ints);

/* out, q: device [T][Hq][hd] in dtype (16-byte aligned). k_cache, v_cache, block_tables       */
/* ([S][max_blocks] device int32) as pkv_decode_attn; the cache already holds every token     */
/* attended. plan_host and plan_dev hold the same plan_ints entries, built for these           */
/* query_start/context_lens and shapes. Writes only out (and the workspace). Errors:          */
/* PKV_ERR_INVALID_ARG (shapes, pointers, a plan that fails the check), PKV_ERR_UNSUPPORTED   */
/* (also when units * Hkv * 256 work-items would pass 2^31 - 1), PKV_ERR_WORKSPACE,           */
/* PKV_ERR_HIP. Stream-ordered, asynchronous. pass: 0 both kernels, 1 the                     */
/* attention pass (direct rows finished, pieces of split rows written), 2 the merge of the    */
/* split rows (run 1 then 2 on one stream; exported to time them).                            */
pkv_status pkv_prefill_attn(int32_t pass, void* out, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables, int32_t S,
                            int32_t T, int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs,
                            int32_t NB, int32_t max_blocks, int32_t max_context_len, float scale,
                            pkv_dtype dtype, const int32_t* plan_host, const int32_t* plan_dev,
                            size_t plan_ints, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Workspace bytes pkv_decode_attn needs for this shape on the current device (0 if B == 0 or */
/* the arguments are invalid).                                                                 */
size_t pkv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t hd,
                                  int32_t max_context_len, pkv_dtype dtype);

/* ---- The two passes pkv_decode_attn is made of, exported so they can be run, timed and     */
/* ---- checked on their own: pkv_decode_attn(...) == pkv_decode_stream(W) then               */
/* ---- pkv_decode_merge(W) with W = pkv_decode_num_workers(...), per sub-batch.             */
/*                                                                                            */
/* Stream layout (our design; the pages do not discuss kernels). Let c_i = ceil(n_i/16) (n_i   */
/* clamped as above), S_i = c_0 + ... + c_{i-1}, C = S_B. Each sequence has H "head slots":    */
/* H = Hq with GS = 1 q head per slot for the vector kernel, H = Hkv with GS = G q heads per   */
/* slot (q heads s*G .. s*G+G-1) for the matrix-core kernel (pkv_decode_kernel says which).   */
/* Segment (i, s) is the sequence's c_i blocks for slot s, placed at stream positions          */
/* [s*C + S_i, s*C + S_i + c_i) of a stream of T = H*C positions (one 16-token block each).    */
/* Worker w (a wave; w in [0, W)) takes positions [w*per, min(T, (w+1)*per)), per =            */
/* ceil(T/W). A segment inside one worker's range is finished by the stream pass (its out     */
/* rows written). Every worker holding part of a segment that crosses a range boundary writes */
/* a "piece" for each of the GS q heads into cell (w, slot): slot = 1 if the segment starts   */
/* after w*per, else 0. Over the piece's tokens t (those of the segment's positions in w's    */
/* range that are < n_i), with s2_t = scale * log2(e) * (q . k_t) (base-2 units):             */
/*   m = max_t s2_t,   l = sum_t 2^(s2_t - m),   o[:] = sum_t 2^(s2_t - m) v_t[:].             */
/* Workspace, bytes (A = round_up(x, 256)):                                                    */
/*   seg  int32 [B+1]           S_0..S_B                 at 0                                  */
/*   ml   float [W][2][GS][2]   (m, l) of cell (w,slot)   at A(4*(B+1))                         */
/*   o    float [W][2][GS][hd]  o of cell (w, slot)      after ml, at + A(W*2*GS*2*4)          */
/* pkv_decode_stream_workspace_bytes gives the total. Cells of workers that hold no cut       */
/* segment are not written.                                                                   */

/* Which kernel the stream pass uses for this shape under the current setting: 1 = vector,    */
/* 2 = matrix core; 0 on bad arguments.                                                       */
int32_t pkv_decode_kernel(int32_t Hq, int32_t Hkv, pkv_dtype dtype);

/* W that fills the current device once with that kernel (a multiple of 4); 0 on error.       */
int32_t pkv_decode_num_workers(int32_t Hq, int32_t Hkv, int32_t hd, pkv_dtype dtype);

/* Workspace bytes of the stream layout for W = num_workers (a positive multiple of 4).       */
size_t pkv_decode_stream_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t hd,
                                         pkv_dtype dtype, int32_t num_workers);

/* Pass 1: writes seg, the out rows of every segment inside one worker's range and of every  */
/* sequence with n_i = 0, and the pieces of cut segments. B <= 8192 and B*max_blocks*H + W    */
/* < 2^31 (else PKV_ERR_UNSUPPORTED). Other arguments and errors as pkv_decode_attn.          */
pkv_status pkv_decode_stream(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs,
                             int32_t NB, int32_t max_blocks, int32_t max_context_len,
                             float scale, pkv_dtype dtype, int32_t num_workers, void* workspace,
                             size_t workspace_bytes, void* stream);

/* The two passes of pkv_decode_append_attn. Pass 1 is pkv_decode_stream with each sequence's */
/* newest token taken from k_new/v_new instead of its slot (same arguments as                  */
/* pkv_decode_stream plus k_new, v_new as in pkv_decode_append_attn); it writes no cache.      */
/* Pass 2, pkv_decode_append_merge, is pkv_decode_merge plus the stores of those rows into     */
/* their slots (the caches are written only here: stores issued while the K/V tiles stream    */
/* slow the stream down on this hardware). The caches and the output are complete after pass */
/* 2; between the passes the caches still hold the old slot contents.                          */
pkv_status pkv_decode_append_stream(void* out, const void* q, const void* k_new,
                                    const void* v_new, void* k_cache, void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    int32_t B, int32_t Hq, int32_t Hkv, int32_t hd, int32_t bs,
                                    int32_t NB, int32_t max_blocks, int32_t max_context_len,
                                    float scale, pkv_dtype dtype, int32_t num_workers,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Pass 2: for every cut segment and each of its GS q heads, combines the pieces of workers   */
/* w_first..w_last in worker order (log-sum-exp): M = max m_w, a_w = 2^(m_w - M),             */
/* out = sum_w a_w o_w / sum_w a_w l_w (a piece with m = -inf has weight 0), rounded to        */
/* `dtype`. Reads seg and the pieces from the workspace the stream pass filled (same B, heads, */
/* dtype, num_workers and kernel setting); writes only the rows of cut segments.              */
pkv_status pkv_decode_merge(void* out, const void* workspace, size_t workspace_bytes, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t hd, pkv_dtype dtype,
                            int32_t num_workers, void* stream);

pkv_status pkv_decode_append_merge(void* out, const void* k_new, const void* v_new,
                                   void* k_cache, void* v_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, int32_t NB, int32_t max_blocks,
                                   int32_t max_context_len, const void* workspace,
                                   size_t workspace_bytes, int32_t B, int32_t Hq, int32_t Hkv,
                                   int32_t hd, pkv_dtype dtype, int32_t num_workers,
                                   void* stream);

/* Test and measurement hook, not part of the product path (no serving code needs it).      */
/* Attention-kernel selection, process-wide: 0 = automatic (matrix-core kernel for f16/bf16   */
/* with 2 <= G <= 16, vector kernel otherwise), 1 = always the vector kernel, 2 = matrix-core  */
/* kernel where supported (f16/bf16, G <= 16). Both give results within the same tolerance;   */
/* exists so the two can be measured on the same shape. Returns the previous value (-1 and no */
/* change for an unknown value).                                                              */
int32_t pkv_set_attn_kernel(int32_t which);

/* ------------------------------------------------------------------------------------------ */
/* Host block allocator (no GPU). [P1] §三 步驟一..四 and §二 "解決三大問題"; [P2] "按需分配",  */
/* "共享和复用". Opaque handle, not thread-safe (one per scheduler thread).                    */
/* Conventions (our reading where the pages are silent):                                       */
/*  - The free list is a FIFO queue. It starts as free_order[0..NB-1] (NULL = 0,1,...,NB-1).    */
/*    Allocation pops from the front; a block whose refcount drops to 0 is pushed to the back. */
/*  - A sequence has a length n and a list of ceil(n/bs) blocks. Appending one token at length */
/*    n takes a new block iff n % bs == 0 ([P1] §三 步驟三: write into the current block if it  */
/*    has room, otherwise allocate a new one and update the table).                            */
/*  - Sharing: pkv_alloc_fork makes the child point at all of the parent's blocks and adds one */
/*    to each block's refcount ([P1] §二, three tables pointing at the same physical blocks).  */
/*  - Copy-on-write: appending into a partially filled last block whose refcount is > 1 first  */
/*    moves the appending sequence to a fresh block and reports the pair (src, dst); the      */
/*    caller copies the tile contents (both caches) from src to dst before writing. A token   */
/*    written by one sequence is therefore never visible to another.                          */
/*  - Free ([P1] §三 步驟四): the sequence's blocks are visited in logical order, each refcount */
/*    is decremented, and each block reaching 0 is pushed to the back of the free list.       */
/*  - Every operation is atomic: on any error the allocator is unchanged.                     */
typedef struct pkv_allocator pkv_allocator;

/* NB > 0, bs > 0. free_order: NULL or a permutation of 0..NB-1 (else PKV_ERR_INVALID_ARG). */
pkv_status pkv_alloc_create(int32_t NB, int32_t bs, const int32_t* free_order,
                            pkv_allocator** out);
void pkv_alloc_destroy(pkv_allocator* a);

/* New sequence with an empty block table ([P1] §三 步驟一). seq must not exist. */
pkv_status pkv_alloc_add_seq(pkv_allocator* a, int64_t seq);

/* Append ntok[k] >= 0 tokens to sequence seqs[k], k = 0..n-1 (distinct ids), in that order.   */
/* slots_out (host, sum(ntok) entries, may be NULL) receives the slot of every new token, in   */
/* argument order. cow_src/cow_dst (host, capacity n, may be NULL together with n_cow) receive */
/* the copy-on-write pairs, *n_cow their count. PKV_ERR_OUT_OF_BLOCKS if the pool cannot hold  */
/* the whole batch (checked before anything changes).                                          */
pkv_status pkv_alloc_append(pkv_allocator* a, int32_t n, const int64_t* seqs, const int32_t* ntok,
                            int32_t* slots_out, int32_t* cow_src, int32_t* cow_dst,
                            int32_t* n_cow);

/* child becomes a new sequence sharing every block (and the length) of parent. */
pkv_status pkv_alloc_fork(pkv_allocator* a, int64_t parent, int64_t child);

/* Release the sequence and its blocks ([P1] §三 步驟四). */
pkv_status pkv_alloc_free(pkv_allocator* a, int64_t seq);

/* Batched forms for a beam-search re-selection ([P2] "PagedAttention 的优势", Beam Search:  */
/* candidates share their common history): the same as pkv_alloc_fork(parents[k],          */
/* children[k]) for k = 0..n-1, in order, resp. pkv_alloc_free(seqs[k]) in order (so blocks  */
/* reach the free list in the same order), in one call. All-or-nothing: fork_many needs every */
/* parent present before the call and every child absent and distinct (PKV_ERR_UNKNOWN_SEQ,  */
/* PKV_ERR_SEQ_EXISTS); free_many needs distinct ids (PKV_ERR_INVALID_ARG), all present       */
/* (PKV_ERR_UNKNOWN_SEQ). A failing call changes nothing.                                      */
pkv_status pkv_alloc_fork_many(pkv_allocator* a, int32_t n, const int64_t* parents,
                               const int64_t* children);
pkv_status pkv_alloc_free_many(pkv_allocator* a, int32_t n, const int64_t* seqs);

/* A beam re-selection in one call: exactly pkv_alloc_fork_many(n, parents, children) followed */
/* by pkv_alloc_free_many(n, old) (the same state afterwards, the same free-list order, the    */
/* same checks, all before any change), without their copies: the old sequences' storage is    */
/* reused for the children. Errors as those two calls.                                          */
pkv_status pkv_alloc_replace_many(pkv_allocator* a, int32_t n, const int64_t* parents,
                                  const int64_t* old, const int64_t* children);

/* Export block tables for seqs[0..n-1]: block_tables_out [n][max_blocks] (host int32, entries */
/* past a sequence's block count set to -1) and context_lens_out [n] (host int32). A sequence  */
/* with more than max_blocks blocks gives PKV_ERR_INVALID_ARG.                                 */
pkv_status pkv_alloc_tables(const pkv_allocator* a, int32_t n, const int64_t* seqs,
                            int32_t max_blocks, int32_t* block_tables_out,
                            int32_t* context_lens_out);

/* Block-table entry mark: set on entries of blocks that several sequences share. The block  */
/* is entry & ~PKV_BLOCK_SHARED; valid block ids stay below 2^27, so the mark never collides. */
#define PKV_BLOCK_SHARED 0x40000000

/* As pkv_alloc_tables, but the entry of every block whose reference count is above 1 carries */
/* PKV_BLOCK_SHARED. The decode calls accept marked tables; the mark never changes a result,   */
/* only the cache policy of the block's loads: marked blocks are read with ordinary (cached)  */
/* loads so that the L2 keeps them for the other sequences that read them ([P1] §二: common    */
/* prefixes point at the same physical blocks), unmarked blocks with streaming (non-temporal) */
/* loads. An unmarked table is always correct; a mark on an unshared block only costs speed. */
pkv_status pkv_alloc_tables_marked(const pkv_allocator* a, int32_t n, const int64_t* seqs,
                                   int32_t max_blocks, int32_t* block_tables_out,
                                   int32_t* context_lens_out);

int32_t pkv_alloc_num_free(const pkv_allocator* a);            /* free blocks                */
int32_t pkv_alloc_refcount(const pkv_allocator* a, int32_t block); /* -1 if out of range      */
/* Length of a sequence in tokens, or -1 if unknown. */
int64_t pkv_alloc_seq_len(const pkv_allocator* a, int64_t seq);
/* ---- Automatic prefix caching ([P1] §五 "前綴共享" and §八 "前綴快取": requests that begin  */
/* ---- with the same tokens share that prefix's KV cache without being forked; [P3] §4.2:     */
/* ---- a 2000-token system prompt reused by later requests). Our reading, full blocks only:   */
/*  - a full block of a sequence whose token ids are all known is indexed by (the index entry */
/*    of the block before it, or the empty prefix; its bs token ids), so two blocks match only */
/*    when their whole prefixes match (ids are compared, not only hashed);                     */
/*  - pkv_alloc_add_seq_tokens starts a sequence from its prompt's ids: it shares the longest  */
/*    chain of indexed full blocks the prompt begins with (refcount + 1 each), takes fresh     */
/*    blocks for the rest and indexes the prompt's new full blocks. The caller writes the K/V */
/*    of tokens [*cached_out, n) only;                                                         */
/*  - pkv_alloc_append_tokens is pkv_alloc_append plus the new tokens' ids (sum(ntok), in      */
/*    argument order): blocks of indexed sequences that become full are indexed. A sequence   */
/*    created by pkv_alloc_add_seq, or grown by pkv_alloc_append, is not indexed from then on; */
/*    forks inherit the parent's state;                                                        */
/*  - a freed indexed block keeps its entry and its FIFO place in the free list: a later hit  */
/*    takes it back out (refcount 1); a fresh allocation that pops it drops the entry.         */
/* Content equal to an indexed block's but in another block is not indexed twice.             */
/* add_seq_tokens: slots_out (host, n entries, may be NULL) receives every prompt token's     */
/* slot; *cached_out (may be NULL) the tokens found in the cache, a multiple of bs. Errors:    */
/* PKV_ERR_INVALID_ARG, PKV_ERR_SEQ_EXISTS, PKV_ERR_OUT_OF_BLOCKS (nothing changes).           */
pkv_status pkv_alloc_add_seq_tokens(pkv_allocator* a, int64_t seq, int32_t n,
                                    const int32_t* token_ids, int32_t* slots_out,
                                    int32_t* cached_out);
pkv_status pkv_alloc_append_tokens(pkv_allocator* a, int32_t n, const int64_t* seqs,
                                   const int32_t* ntok, const int32_t* token_ids,
                                   int32_t* slots_out, int32_t* cow_src, int32_t* cow_dst,
                                   int32_t* n_cow);
/* Blocks whose content is indexed, in use or free (-1 for a null handle). */
int32_t pkv_alloc_cached_blocks(const pkv_allocator* a);

/* Memory accounting ([P1] §一 and §二 "內部碎片": a contiguous reservation wastes what a      */
/* request does not use; with blocks only a sequence's last block can be partly empty).       */
/* out (host, 4 entries) receives: live sequences; logical tokens (sum of their lengths);     */
/* blocks in use (NB - free blocks); filled slots (over the blocks in use, the most tokens    */
/* any owner keeps in the block, so a shared block counts once). Utilisation of the blocks in */
/* use = filled / (blocks in use * bs). Errors: PKV_ERR_INVALID_ARG (null argument).          */
pkv_status pkv_alloc_usage(const pkv_allocator* a, int64_t* out);
/* Copies up to cap entries of the free list, front first, into out; returns the list length. */
int32_t pkv_alloc_free_list(const pkv_allocator* a, int32_t* out, int32_t cap);

/* ------------------------------------------------------------------------------------------ */
/* Serving step engine: one call per decode step of a continuous batch or a beam search.      */
/* [P1] §四 (連續批次) and §十一: finished requests leave the batch and new ones join at any     */
/* step, so the GPU is not left waiting for a whole batch; §三 步驟一..四 for each request's     */
/* blocks (allocated on demand, written, attended through the table, freed). [P2]             */
/* "PagedAttention 的优势", Beam Search: candidates fork from the beams they extend and share  */
/* their history's blocks. The engine drives a caller-owned pkv_allocator (borrowed: it must   */
/* outlive the engine, and the caller must not change it between create and destroy except   */
/* through the engine or while no step is in flight) and keeps the request queue, the running */
/* set (admission order), two sets of pinned host + device staging buffers for the step's     */
/* block tables, lengths, slots, copy-on-write pairs and plans, and its decode and prefill     */
/* workspaces. A step is one host call that enqueues the upload of its staging set and all of */
/* the step's kernels on the caller's stream and returns without waiting for them: the host   */
/* prepares step k+1 while the kernels of step k run (a staging set is reused only after the  */
/* step that last read it has finished; that wait is on the host). Every step of an engine    */
/* must use the same stream. The engine allocates device and pinned memory at                 */
/* create and grows it inside a step only when a step needs more than any before (a growth of */
/* a workspace first drains the caller's stream). Not thread-safe; use it from one thread, on  */
/* the HIP device current at create (PKV_ERR_INVALID_ARG otherwise).                           */
/* Errors: the steps check their arguments and the running sequences' lengths before changing */
/* anything; an error from the allocator or a launch after that (PKV_ERR_OUT_OF_BLOCKS cannot  */
/* occur for admitted work, whose blocks admission reserved) leaves the engine's bookkeeping   */
/* unspecified: destroy it.                                                                   */
typedef struct pkv_engine pkv_engine;

/* Shared-prefix plans (pkv_decode_plan, default max_group) for every decode step. */
#define PKV_ENGINE_PLAN 1
/* With PKV_ENGINE_PLAN: run the shared pass and the stream pass as two launches (passes 1 and */
/* 2 of pkv_decode_planned), or as one (pass 5), rather than as pkv_decode_planned_launches    */
/* chooses per step (pass 4). Same results; for measuring the forms. Not both.                */
#define PKV_ENGINE_SPLIT_SHARED 2
#define PKV_ENGINE_ONE_LAUNCH 4

/* alloc: the allocator of the NB-block pool the caches hold (the caller keeps ownership).    */
/* k_cache, v_cache: device caches in the layout above. max_batch: most running sequences     */
/* (<= 8192); max_context_len: longest sequence, which fixes the tables' width                 */
/* ceil(max_context_len/16). flags: 0, PKV_ENGINE_PLAN, or PKV_ENGINE_PLAN with one of         */
/* PKV_ENGINE_SPLIT_SHARED and PKV_ENGINE_ONE_LAUNCH. Errors: PKV_ERR_INVALID_ARG,               */
/* PKV_ERR_UNSUPPORTED, PKV_ERR_HIP.                                                            */
pkv_status pkv_engine_create(pkv_allocator* alloc, void* k_cache, void* v_cache, int32_t NB,
                             int32_t Hq, int32_t Hkv, int32_t hd, pkv_dtype dtype,
                             int32_t max_batch, int32_t max_context_len, int32_t flags,
                             pkv_engine** out);
/* Waits for the engine's steps in flight, then releases what the engine holds (not the        */
/* allocator or the caches).                                                                  */
void pkv_engine_destroy(pkv_engine* e);

/* Queue a request (first come, first served). prompt_len >= 1, max_new_tokens >= 1, their sum */
/* <= max_context_len and its blocks <= NB; arrival_step: the first step that may admit it.   */
/* token_ids: NULL, or its prompt_len token ids (host, copied): admission then starts the      */
/* sequence with pkv_alloc_add_seq_tokens (automatic prefix caching), else pkv_alloc_add_seq +  */
/* pkv_alloc_append. rid: the sequence id it gets in the allocator (must then be free).        */
pkv_status pkv_engine_submit(pkv_engine* e, int64_t rid, int32_t prompt_len,
                             int32_t max_new_tokens, int32_t arrival_step,
                             const int32_t* token_ids);

/* Append existing allocator sequences to the running set (after the running ones, in order); */
/* they never retire (beam search, or a decode loop the caller ends). PKV_ERR_UNKNOWN_SEQ,     */
/* PKV_ERR_SEQ_EXISTS (already running or repeated), PKV_ERR_INVALID_ARG (more than max_batch).*/
pkv_status pkv_engine_adopt(pkv_engine* e, int32_t n, const int64_t* seqs);

/* Running sequence ids in row order into seqs (up to cap); returns their number (-1: NULL e). */
int32_t pkv_engine_running(const pkv_engine* e, int64_t* seqs, int32_t cap);
/* Requests waiting in the queue (-1: NULL e). */
int32_t pkv_engine_queued(const pkv_engine* e);

/* One continuous-batching step (step number k = the number of steps taken before):            */
/*  1. retire: running requests that produced max_new_tokens tokens are freed                 */
/*     (pkv_alloc_free_many, in row order) and leave the running set;                          */
/*  2. admit: while the queue head has arrived (arrival_step <= k), fewer than max_batch run,  */
/*     its whole prompt fits in the prompt rows not yet used this step (prompt_rows), and the   */
/*     free blocks minus the blocks the running requests may still take cover                  */
/*     ceil((prompt + max new) / 16), the head is started and its prompt slots taken; it joins */
/*     the running set (our admission rule: the pages give none; no preemption is ever needed);*/
/*  3. append one token to every running sequence (admitted ones included), with new_ids[i]   */
/*     as its id when new_ids is given (pkv_alloc_append_tokens), and export the marked tables */
/*     and lengths (plus a shared-prefix plan with PKV_ENGINE_PLAN);                           */
/*  4. launch, on `stream`: pkv_write of the admitted prompts' uncached tokens                  */
/*     (k_prompt/v_prompt rows 0..T-1, admission order); the copy-on-write copies, if any; the */
/*     causal prefill attention of those tokens when q_prompt is given (pkv_prefill_attn,      */
/*     q_prompt rows 0..T-1, prefill_out written; f16/bf16, G <= 16); the fused decode step of */
/*     the B running rows (pkv_decode_planned with PKV_ENGINE_PLAN, else                       */
/*     pkv_decode_append_stream + pkv_decode_append_merge): row i of q/k_new/v_new is running  */
/*     sequence i's, out row i is written.                                                     */
/* Buffers (device, dtype of the caches, 16-byte aligned): q, out [max_batch][Hq][hd]; k_new,  */
/* v_new [max_batch][Hkv][hd]; k_prompt, v_prompt [prompt_rows][Hkv][hd]; q_prompt,            */
/* prefill_out [prompt_rows][Hq][hd] or both NULL. Only the first B (resp. T) rows are read or */
/* written. new_ids: host int32 [max_batch] or NULL. scale: softmax scale of both attentions.  */
/* events: NULL or 8 hipEvent_t (each may be NULL) recorded on the stream: [0] before the      */
/* upload of the step's staged tables, lengths, slots and plans (a small copy kernel that      */
/* reads the pinned set), [1] after it, [2] after the prompt write, [3] after the copies (a    */
/* step with copies and no prompt write stages and copies in one launch: [1], [2] and [3]     */
/* after it), [4] after the prefill, [5] after the shared pass (before the one launch of the  */
/* shared and stream passes, when they are one), [6] after the stream pass (or that launch),  */
/* [7] after the merge.                                                                        */
/* info: NULL or host                                                                          */
/* int64 [8] = {B, T, retired, admitted, plan units (-1: unplanned), copy-on-write pairs,      */
/* queued after the step, k}.                                                                  */
pkv_status pkv_engine_step(pkv_engine* e, const void* q, const void* k_new, const void* v_new,
                           const int32_t* new_ids, void* out, const void* k_prompt,
                           const void* v_prompt, int32_t prompt_rows, const void* q_prompt,
                           void* prefill_out, float scale, void* const* events, int64_t* info,
                           void* stream);

/* One beam-search step over the running set (B beams): with parents (host int32 [B], each in */
/* [0, B)) and children (host int64 [B], new distinct ids), new beam i forks from running beam */
/* parents[i] as children[i] (pkv_alloc_fork_many), the old beams are freed (free_many, in row */
/* order) and the children become the running set; with both NULL the running set stays. Then */
/* steps 3 and 4 of pkv_engine_step without prompts: one token appended per beam, the         */
/* copy-on-write pairs this reports copied (pkv_copy_blocks), the decode step launched. q,    */
/* k_new, v_new, out, events, info as pkv_engine_step.                                         */
pkv_status pkv_engine_beam_step(pkv_engine* e, const int32_t* parents, const int64_t* children,
                                const void* q, const void* k_new, const void* v_new, void* out,
                                float scale, void* const* events, int64_t* info, void* stream);

/* What the last step did, into host buffers (each may be NULL; sizes from its info): retired */
/* ids [retired], admitted (id, prompt_len, cached tokens) triples [3*admitted], prompt slots */
/* [T], lengths [B] and marked tables [B][ceil(max_context_len/16)] as uploaded. Valid until  */
/* the next step. The block ids are exact; a mark (PKV_BLOCK_SHARED, a cache hint only) is     */
/* refreshed where the engine re-reads an entry (a row's last blocks each step, a whole row   */
/* when its sequence changes; a forked beam takes its parent's earlier entries as they were), */
/* so it can lag a change in sharing: a shared block left unmarked, or the reverse.            */
pkv_status pkv_engine_last(const pkv_engine* e, int64_t* retired, int64_t* admitted,
                           int32_t* prompt_slots, int32_t* lens, int32_t* tables);

/* Waits (on the host) for every step in flight. */
pkv_status pkv_engine_sync(pkv_engine* e);

/* ------------------------------------------------------------------------------------------ */
/* Measurement hook, not part of the product path.                                           */
/* Read-bandwidth probe (measurement support; not part of the attention path). The pages give */
/* no hardware figures; the decode path's roofline is quoted against the published HBM peak   */
/* and, beside it, against what this probe reaches on the same part with the stream pass's    */
/* access pattern and none of its arithmetic.                                                 */
/* Wave w of num_workers reads the 4096-byte tiles tile_ids[w*per .. min(n, (w+1)*per)) of    */
/* base (per = ceil(n / num_workers); tile t at byte 4096*t; ids clamped into                 */
/* [0, base_bytes / 4096)), 16 bytes per lane per non-temporal load, and stores the XOR of the */
/* 32-bit words each lane read to sink[w*64 + lane].                                          */
/*   base        device, at least 4096 bytes, 16-byte aligned (read only)                     */
/*   tile_ids    device int32 [n]                                                              */
/*   sink        device uint32 [num_workers * 64] (written)                                    */
/*   num_workers a positive multiple of 4                                                      */
/* n == 0 is a no-op. Errors: PKV_ERR_INVALID_ARG, PKV_ERR_HIP.                               */
pkv_status pkv_probe_read(const void* base, size_t base_bytes, const int32_t* tile_ids,
                          int32_t n, int32_t num_workers, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
