// Serving step engine: one host call per continuous-batching or beam-search decode step.
//
// [P1] §四 (連續批次) and §十一: a request leaves the batch as soon as it is done and a new one
// joins at any step, so the GPU never waits for a whole batch; §三 步驟一..四: blocks are taken
// on demand, written, attended through the table and released per request. [P2]
// "PagedAttention 的优势", Beam Search: beam candidates share their history's blocks and fork
// at every step. The engine keeps the request queue, the running set and the step's staging
// on the host side of the library, so that a step is one call: retire, admit (with the
// prompts' slots), append one token per running sequence, bring the device block table up to
// date, plan, and launch the step's kernels on the caller's stream.
//
// Device state: one block table [max_batch][mb] and one region of small per-step arrays
// (lengths, copy-on-write pairs, prompt slots, plans), both written by the step's first
// kernel from a pinned host set; stream order keeps that write after the previous step's
// kernels. The host keeps a mirror of the device table and sends only the entries that
// changed (a decode step changes one or two entries of a row: the block it opened, or the
// last block a copy-on-write replaced), or a dense range of rows when that is smaller. The
// pinned sets are double-buffered: the host fills set k % 2 for step k while step k - 1 runs,
// and reuses a set only after the step that last read it finished.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <limits>
#include <unordered_set>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_kernels.h"

namespace {

constexpr int kSets = 2;
constexpr int64_t kNoLimit = std::numeric_limits<int64_t>::max();

int64_t blocks_for(int64_t n) { return (n + pkv::kBlockSize - 1) / pkv::kBlockSize; }
size_t up4(size_t n) { return (n + 3) & ~size_t{3}; }  // ints, to 16-byte offsets

struct Request {
  int64_t rid;
  int32_t prompt, max_new, arrival;
  std::vector<int32_t> ids;  // prompt token ids (prefix caching), else empty
};

struct Running {
  int64_t rid;
  int64_t final_len;  // prompt + max new tokens (kNoLimit for adopted sequences)
  int64_t max_new;    // kNoLimit: never retires
  int64_t done;       // tokens produced so far
  uint64_t serial;    // unique per sequence the engine ever ran (ids may be reused)
};

// Offsets (ints) of one step's arrays inside its pinned set. [0, small) is copied whole to
// the device's small region (same offsets); then the dense table rows; then the entry pairs.
struct Layout {
  size_t lens = 0, cow_src = 0, cow_dst = 0, pf_lens = 0, pf_qs = 0, slots = 0, plan = 0,
         pf_plan = 0, small = 0, dense = 0, pairs = 0, end = 0;
};

hipError_t fail(const char* what, hipError_t e) { return pkv::note_error(what, e); }

}  // namespace

struct pkv_engine {
  pkv_allocator* alloc = nullptr;
  void* k_cache = nullptr;
  void* v_cache = nullptr;
  int32_t NB = 0, Hq = 0, Hkv = 0, hd = 0;
  pkv_dtype dtype = PKV_BF16;
  int32_t max_batch = 0, max_ctx = 0, mb = 0, flags = 0, W = 0;
  int device = -1;

  std::deque<Request> queue;
  std::vector<Running> run;
  int64_t step_no = 0;
  uint64_t next_serial = 1;

  // pinned host sets (and their device-side addresses), the device table and small region
  int32_t* host[kSets] = {nullptr, nullptr};
  void* host_dev[kSets] = {nullptr, nullptr};
  size_t cap_ints[kSets] = {0, 0};
  hipEvent_t done[kSets] = {nullptr, nullptr};
  bool launched[kSets] = {false, false};  // done[s] recorded and not yet waited for
  int cur = 0;
  int32_t* dtab = nullptr;
  size_t tab_ints = 0;
  int32_t* dsmall = nullptr;
  size_t small_ints = 0;
  bool device_used = false;  // a step was launched (a buffer growth must drain the stream)

  // host mirror of the device table, and which sequence (serial, 0: none) and how many blocks
  // each row holds
  std::vector<int32_t> mirror;
  std::vector<uint64_t> row_serial;
  std::vector<int32_t> row_nblk;
  int32_t rows_tracked = 0;  // rows whose serial is set
  std::vector<int32_t> rowbuf;
  std::vector<int32_t> pairs;  // (flat index, value) pairs of this step
  std::vector<int32_t> snap, snap_nblk;  // the rows before a beam re-selection

  void* ws = nullptr;
  size_t ws_bytes = 0;
  void* pf_ws = nullptr;
  size_t pf_ws_bytes = 0;

  // host scratch reused across steps
  std::vector<int64_t> ids, retired, admitted;  // admitted: (rid, prompt_len, cached) triples
  std::vector<int32_t> ones, tmp_slots, plan, pf_plan;

  // the last step, for pkv_engine_last
  int last_set = -1;
  Layout last;
  int32_t last_B = 0, last_T = 0;

  ~pkv_engine() {
    if (device >= 0) (void)hipSetDevice(device);
    for (int s = 0; s < kSets; ++s)
      if (done[s]) (void)hipEventSynchronize(done[s]);
    for (int s = 0; s < kSets; ++s) {
      if (host[s]) (void)hipHostFree(host[s]);
      if (done[s]) (void)hipEventDestroy(done[s]);
    }
    if (dtab) (void)hipFree(dtab);
    if (dsmall) (void)hipFree(dsmall);
    if (ws) (void)hipFree(ws);
    if (pf_ws) (void)hipFree(pf_ws);
  }

  // Pinned set s may be refilled: the step that last used it has finished (its stage kernel,
  // which read the set, ran first).
  hipError_t acquire(int s) {
    if (!launched[s]) return hipSuccess;
    launched[s] = false;
    return fail("engine: wait for the step two back", hipEventSynchronize(done[s]));
  }

  // Capacity of pinned set s (ints, a multiple of 4), keeping its contents up to `keep`.
  hipError_t reserve(int s, size_t ints, size_t keep) {
    if (ints <= cap_ints[s]) return hipSuccess;
    const size_t cap = up4(std::max(ints, cap_ints[s] + cap_ints[s] / 2));
    int32_t* h = nullptr;
    void* hd = nullptr;
    hipError_t e = fail("engine: staging (pinned)",
                        hipHostMalloc(reinterpret_cast<void**>(&h), cap * 4, hipHostMallocDefault));
    if (e != hipSuccess) return e;
    e = fail("engine: staging (device address)", hipHostGetDevicePointer(&hd, h, 0));
    if (e != hipSuccess) {
      (void)hipHostFree(h);
      return e;
    }
    if (host[s] && keep) std::memcpy(h, host[s], std::min(keep, cap_ints[s]) * 4);
    if (host[s]) (void)hipHostFree(host[s]);  // set s is acquired: nothing reads it
    host[s] = h;
    host_dev[s] = hd;
    cap_ints[s] = cap;
    return hipSuccess;
  }

  // Device buffer of at least `bytes`; the old one may still be read by the step before, so
  // the stream is drained before it is released.
  hipError_t grow(void** buf, size_t* have, size_t bytes, hipStream_t stream) {
    if (bytes <= *have) return hipSuccess;
    const size_t want = std::max(bytes, *have + *have / 2);
    if (device_used) {
      hipError_t e = fail("engine: drain before growth", hipStreamSynchronize(stream));
      if (e != hipSuccess) return e;
    }
    if (*buf) (void)hipFree(*buf);
    *buf = nullptr;
    *have = 0;
    hipError_t e = fail("engine: device buffer", hipMalloc(buf, want));
    if (e == hipSuccess) *have = want;
    return e;
  }
};

namespace {

void record(void* const* events, int k, hipStream_t stream) {
  if (events && events[k]) (void)hipEventRecord(static_cast<hipEvent_t>(events[k]), stream);
}

// Brings rows [0, B) of the mirror up to date with the allocator and collects the entries
// that changed (as pairs) and the range of rows they lie in. A row that still holds the same
// sequence is re-read from its old last block on (a copy-on-write may have replaced it, an
// append may have opened the next). A row whose sequence was forked this step from the
// sequence of row src[i] (beam re-selection; the rows as they were are in e->snap) takes that
// row's blocks up to the parent's last and re-reads the rest; any other row is re-read whole.
// Entries past a row's blocks are reset to -1. Lengths go to lens.
pkv_status update_rows(pkv_engine* e, int32_t B, int32_t* lens, int32_t* r0, int32_t* r1,
                       const int32_t* src) {
  const int32_t mb = e->mb;
  e->pairs.clear();
  *r0 = B;
  *r1 = 0;
  for (int32_t i = 0; i < B; ++i) {
    const int64_t seq = e->run[i].rid;
    const bool same = e->row_serial[i] == e->run[i].serial;
    int32_t from = same ? std::max(0, e->row_nblk[i] - 1) : 0;
    if (!same && src) {  // the parent's blocks before its last are the child's
      const int32_t p = src[i];
      from = std::max(0, e->snap_nblk[p] - 1);
      std::memcpy(e->rowbuf.data(), e->snap.data() + static_cast<size_t>(p) * mb,
                  static_cast<size_t>(from) * 4);
    }
    int64_t len = 0;
    const int32_t n = pkv::alloc_row(e->alloc, seq, from, mb, e->rowbuf.data(), &len);
    if (n < 0) return PKV_ERR_INVALID_ARG;
    int32_t* m = e->mirror.data() + static_cast<size_t>(i) * mb;
    const int32_t upto = std::max(n, e->row_nblk[i]);
    bool changed = false;
    for (int32_t j = same ? from : 0; j < upto; ++j) {
      const int32_t v = j < n ? e->rowbuf[j] : -1;
      if (m[j] != v) {
        m[j] = v;
        e->pairs.push_back(i * mb + j);
        e->pairs.push_back(v);
        changed = true;
      }
    }
    if (changed) {
      *r0 = std::min(*r0, i);
      *r1 = i + 1;
    }
    e->row_serial[i] = e->run[i].serial;
    e->row_nblk[i] = n;
    lens[i] = static_cast<int32_t>(len);
  }
  // rows past the batch are not kept up to date: forget who held them (their entries stay,
  // and are reset when a row is next used)
  for (int32_t i = B; i < e->rows_tracked; ++i) e->row_serial[i] = 0;
  e->rows_tracked = B;
  return PKV_OK;
}

// The common tail of both steps: append one token to every running sequence (with its id
// when new_ids is given), update the table, plan, stage, launch. Prompt slots (T) and the
// admitted rows' prefill data are already staged in set s at lay.slots / lay.pf_*.
pkv_status decode_tail(pkv_engine* e, int s, Layout& lay, int32_t T, int32_t A,
                       const int32_t* src_rows, const int32_t* new_ids, const void* q,
                       const void* k_new,
                       const void* v_new, void* out, const void* k_prompt, const void* v_prompt,
                       const void* q_prompt, void* prefill_out, float scale,
                       void* const* events, int64_t* info, hipStream_t stream) {
  const int32_t B = static_cast<int32_t>(e->run.size());
  const int32_t mb = e->mb;
  int32_t ncow = 0;
  e->ids.resize(B);
  for (int32_t i = 0; i < B; ++i) e->ids[i] = e->run[i].rid;
  if (static_cast<int32_t>(e->ones.size()) < B) e->ones.assign(B, 1);
  int32_t* H = e->host[s];
  int32_t r0 = 0, r1 = 0;
  if (B > 0) {  // copy-on-write pairs land directly in the staged set (capacity B each)
    pkv_status st;
    if (new_ids)
      st = pkv_alloc_append_tokens(e->alloc, B, e->ids.data(), e->ones.data(), new_ids, nullptr,
                                   H + lay.cow_src, H + lay.cow_dst, &ncow);
    else
      st = pkv_alloc_append(e->alloc, B, e->ids.data(), e->ones.data(), nullptr, H + lay.cow_src,
                            H + lay.cow_dst, &ncow);
    if (st != PKV_OK) return st;
    for (auto& r : e->run) r.done += 1;
    st = update_rows(e, B, H + lay.lens, &r0, &r1, src_rows);
    if (st != PKV_OK) return st;
  }
  // shared-prefix plan of the updated rows (runs only where the shape gains from them)
  size_t plan_ints = 0;
  const bool planned = B > 0 && (e->flags & PKV_ENGINE_PLAN);
  lay.plan = lay.slots + up4(T);
  if (planned) {
    size_t need = 0;
    pkv_status st = pkv_decode_plan(e->mirror.data(), H + lay.lens, B, mb, e->max_ctx, e->Hq,
                                    e->Hkv, e->NB, e->dtype, 0, e->plan.data(), e->plan.size(),
                                    &need);
    if (st == PKV_ERR_WORKSPACE) {
      e->plan.resize(need);
      st = pkv_decode_plan(e->mirror.data(), H + lay.lens, B, mb, e->max_ctx, e->Hq, e->Hkv,
                           e->NB, e->dtype, 0, e->plan.data(), e->plan.size(), &need);
    }
    if (st != PKV_OK) return st;
    plan_ints = need;
  }
  lay.pf_plan = lay.plan + up4(plan_ints);
  // prefill plan of the admitted prompts' written tokens
  size_t pf_ints = 0;
  const bool prefill = q_prompt && T > 0;
  if (prefill) {
    size_t need = 0;
    pkv_status st = pkv_prefill_plan(H + lay.pf_qs, H + lay.pf_lens, A, mb, e->max_ctx, e->Hq,
                                     e->Hkv, e->dtype, e->pf_plan.data(), e->pf_plan.size(),
                                     &need);
    if (st == PKV_ERR_WORKSPACE) {
      e->pf_plan.resize(need);
      st = pkv_prefill_plan(H + lay.pf_qs, H + lay.pf_lens, A, mb, e->max_ctx, e->Hq, e->Hkv,
                            e->dtype, e->pf_plan.data(), e->pf_plan.size(), &need);
    }
    if (st != PKV_OK) return st;
    pf_ints = need;
  }
  lay.small = lay.pf_plan + up4(pf_ints);
  // table changes: the pairs, or the rows they lie in when those are fewer bytes (a dense
  // range starts and ends on 16-byte boundaries of the table)
  const size_t npairs = e->pairs.size() / 2;
  size_t d0 = 0, d1 = 0;
  if (npairs) {
    d0 = (static_cast<size_t>(r0) * mb) & ~size_t{3};
    d1 = up4(static_cast<size_t>(r1) * mb);
  }
  const bool dense = npairs && (d1 - d0) <= 2 * npairs;
  lay.dense = lay.small;
  lay.pairs = lay.dense + (dense ? d1 - d0 : 0);
  lay.end = lay.pairs + (dense ? 0 : 2 * npairs);
  if (e->reserve(s, lay.end, lay.small) != hipSuccess) return PKV_ERR_HIP;
  H = e->host[s];
  if (plan_ints) std::memcpy(H + lay.plan, e->plan.data(), plan_ints * 4);
  if (pf_ints) std::memcpy(H + lay.pf_plan, e->pf_plan.data(), pf_ints * 4);
  if (dense)
    std::memcpy(H + lay.dense, e->mirror.data() + d0, (d1 - d0) * 4);
  else if (npairs)
    std::memcpy(H + lay.pairs, e->pairs.data(), npairs * 8);

  // device buffers for this step's shapes
  size_t ws_need = 0;
  if (B > 0) {
    ws_need = planned ? pkv_decode_planned_workspace_bytes(B, e->Hq, e->Hkv, e->hd, e->dtype,
                                                           e->W, e->plan.data(), plan_ints)
                      : pkv_decode_stream_workspace_bytes(B, e->Hq, e->Hkv, e->hd, e->dtype,
                                                          e->W);
    if (ws_need == 0) return PKV_ERR_INVALID_ARG;
  }
  size_t pf_need = 0;
  if (prefill) {
    pf_need = pkv_prefill_workspace_bytes(e->Hq, e->Hkv, e->hd, e->pf_plan.data(), pf_ints);
    if (pf_need == static_cast<size_t>(-1)) return PKV_ERR_INVALID_ARG;
  }
  size_t small_bytes = e->small_ints * 4;
  if (e->grow(&e->ws, &e->ws_bytes, ws_need, stream) != hipSuccess ||
      e->grow(&e->pf_ws, &e->pf_ws_bytes, pf_need, stream) != hipSuccess ||
      e->grow(reinterpret_cast<void**>(&e->dsmall), &small_bytes, lay.small * 4, stream) !=
          hipSuccess)
    return PKV_ERR_HIP;
  e->small_ints = small_bytes / 4;
  e->device_used = true;

  // The stage kernel writes the step's arrays and table changes, then the step's kernels run.
  // The host does not wait for any of them: it prepares the next step meanwhile.
  record(events, 0, stream);
  pkv::StageParams sp{};
  sp.src = static_cast<const char*>(e->host_dev[s]);
  sp.small_dst = e->dsmall;
  sp.small_n16 = static_cast<int64_t>(lay.small / 4);
  sp.table = e->dtab;
  sp.table_ints = static_cast<int64_t>(e->tab_ints);
  sp.dense_src = static_cast<int64_t>(lay.dense * 4);
  sp.dense_dst = static_cast<int64_t>(d0);
  sp.dense_n16 = dense ? static_cast<int64_t>((d1 - d0) / 4) : 0;
  sp.pairs_src = static_cast<int64_t>(lay.pairs * 4);
  sp.npairs = dense ? 0 : static_cast<int64_t>(npairs);
  const int32_t* D = e->dsmall;
  const int32_t NB = e->NB, Hq = e->Hq, Hkv = e->Hkv, hd = e->hd;
  // With copy-on-write copies and no prompt write between them (a beam step), the staging and
  // the copies are one launch, the copies reading their pairs from the pinned set.
  if (T == 0 && ncow > 0 && pkv::copy_blocks_grid_y(Hkv, hd, e->dtype) <= 65535) {
    const int32_t* Hp = static_cast<const int32_t*>(e->host_dev[s]);
    pkv::CopyParams cp{e->k_cache, e->v_cache, Hp + lay.cow_src, Hp + lay.cow_dst, ncow, Hkv,
                       hd, NB};
    if (pkv::launch_stage_copy(sp, cp, e->dtype, stream) != hipSuccess) return PKV_ERR_HIP;
    for (int k = 1; k <= 3; ++k) record(events, k, stream);
  } else {
    if (pkv::launch_stage(sp, stream) != hipSuccess) return PKV_ERR_HIP;
    record(events, 1, stream);
    if (T > 0) {
      pkv_status st = pkv_write(k_prompt, v_prompt, e->k_cache, e->v_cache, D + lay.slots, T,
                                Hkv, hd, pkv::kBlockSize, NB, e->dtype, stream);
      if (st != PKV_OK) return st;
    }
    record(events, 2, stream);
    if (ncow > 0) {
      pkv_status st = pkv_copy_blocks(e->k_cache, e->v_cache, D + lay.cow_src, D + lay.cow_dst,
                                      ncow, Hkv, hd, pkv::kBlockSize, NB, e->dtype, stream);
      if (st != PKV_OK) return st;
    }
    record(events, 3, stream);
  }
  if (prefill) {
    // the admitted sequences are the last A rows; their rows (one decode token longer now)
    // hold every prompt block, and the plan's lengths are the prompt lengths
    pkv_status st = pkv_prefill_attn(0, prefill_out, q_prompt, e->k_cache, e->v_cache,
                                     e->dtab + static_cast<size_t>(B - A) * mb, A, T, Hq, Hkv,
                                     hd, pkv::kBlockSize, NB, mb, e->max_ctx, scale, e->dtype,
                                     H + lay.pf_plan, D + lay.pf_plan, pf_ints, e->pf_ws,
                                     e->pf_ws_bytes, stream);
    if (st != PKV_OK) return st;
  }
  record(events, 4, stream);
  if (B > 0) {
    if (planned) {
      // The shared pass and the stream pass as one launch (PKV_ENGINE_ONE_LAUNCH, pass 5), as
      // two (PKV_ENGINE_SPLIT_SHARED, passes 1 and 2), or as the library chooses for the plan
      // (pass 0); then the merge (pass 3). With events the passes are separate calls, so that
      // the events fall between the kernels (the automatic choice taken here); event 5 marks
      // the start of the one launch.
      bool split = (e->flags & PKV_ENGINE_SPLIT_SHARED) != 0;
      bool one = (e->flags & PKV_ENGINE_ONE_LAUNCH) != 0;
      if (events && !split && !one) {
        const int32_t kernel = pkv_decode_kernel(Hq, Hkv, e->dtype);
        (pkv::planned_launches(H + lay.plan, B, Hkv, e->dtype, kernel, e->W) == 1 ? one : split) =
            true;
      }
      static const int32_t kWhole[] = {0}, kOne[] = {5, 3}, kSplit[] = {1, 2, 3};
      const int32_t* passes = split ? kSplit : one ? kOne : kWhole;
      const int np = split ? 3 : one ? 2 : 1;
      if (events && one) record(events, 5, stream);
      for (int k = 0; k < np; ++k) {
        const int32_t pass = passes[k];
        pkv_status st = pkv_decode_planned(pass, out, q, k_new, v_new, e->k_cache, e->v_cache,
                                           e->dtab, D + lay.lens, B, Hq, Hkv, hd,
                                           pkv::kBlockSize, NB, mb, e->max_ctx, scale, e->dtype,
                                           H + lay.plan, D + lay.plan, plan_ints, e->W, e->ws,
                                           e->ws_bytes, stream);
        if (st != PKV_OK) return st;
        if (events) record(events, pass == 5 ? 6 : 4 + pass, stream);
      }
    } else {
      record(events, 5, stream);
      pkv_status st = pkv_decode_append_stream(out, q, k_new, v_new, e->k_cache, e->v_cache,
                                               e->dtab, D + lay.lens, B, Hq, Hkv, hd,
                                               pkv::kBlockSize, NB, mb, e->max_ctx, scale,
                                               e->dtype, e->W, e->ws, e->ws_bytes, stream);
      if (st != PKV_OK) return st;
      record(events, 6, stream);
      st = pkv_decode_append_merge(out, k_new, v_new, e->k_cache, e->v_cache, e->dtab,
                                   D + lay.lens, NB, mb, e->max_ctx, e->ws, e->ws_bytes, B, Hq,
                                   Hkv, hd, e->dtype, e->W, stream);
      if (st != PKV_OK) return st;
      record(events, 7, stream);
    }
  } else {
    for (int k = 5; k <= 7; ++k) record(events, k, stream);
  }
  if (fail("engine: step event", hipEventRecord(e->done[s], stream)) != hipSuccess)
    return PKV_ERR_HIP;
  e->launched[s] = true;
  e->last_set = s;
  e->last = lay;
  e->last_B = B;
  e->last_T = T;
  if (info) {
    info[0] = B;
    info[1] = T;
    info[2] = static_cast<int64_t>(e->retired.size());
    info[3] = A;
    info[4] = planned ? e->plan[4] : -1;
    info[5] = ncow;
    info[6] = static_cast<int64_t>(e->queue.size());
    info[7] = e->step_no;
  }
  e->cur ^= 1;
  e->step_no += 1;
  return PKV_OK;
}

// The engine is used on the device it was created on.
bool engine_ok(const pkv_engine* e) {
  int d = -1;
  return e && hipGetDevice(&d) == hipSuccess && d == e->device;
}

// Offsets of the arrays staged before the append, for up to Bmax rows.
Layout small_layout(int32_t Bmax) {
  Layout lay;
  lay.lens = 0;
  lay.cow_src = up4(Bmax);
  lay.cow_dst = lay.cow_src + up4(Bmax);
  lay.pf_lens = lay.cow_dst + up4(Bmax);
  lay.pf_qs = lay.pf_lens + up4(Bmax);
  lay.slots = lay.pf_qs + up4(static_cast<size_t>(Bmax) + 1);
  return lay;
}

}  // namespace

extern "C" {

pkv_status pkv_engine_create(pkv_allocator* alloc, void* k_cache, void* v_cache, int32_t NB,
                             int32_t Hq, int32_t Hkv, int32_t hd, pkv_dtype dtype,
                             int32_t max_batch, int32_t max_context_len, int32_t flags,
                             pkv_engine** out) {
  if (!out) return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  if (dtype != PKV_F32 && dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (hd != 64 && hd != 128) return PKV_ERR_UNSUPPORTED;
  if (!alloc || !k_cache || !v_cache || NB <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 ||
      Hq > 32767 || max_batch <= 0 || max_batch > 8192 || max_context_len <= 0 ||
      (flags & ~(PKV_ENGINE_PLAN | PKV_ENGINE_SPLIT_SHARED | PKV_ENGINE_ONE_LAUNCH)) != 0 ||
      ((flags & PKV_ENGINE_SPLIT_SHARED) && (flags & PKV_ENGINE_ONE_LAUNCH)) ||
      (reinterpret_cast<uintptr_t>(k_cache) & 15u) || (reinterpret_cast<uintptr_t>(v_cache) & 15u))
    return PKV_ERR_INVALID_ARG;
  const int64_t mb = blocks_for(max_context_len);
  if (static_cast<int64_t>(max_batch) * mb >= (int64_t{1} << 31)) return PKV_ERR_UNSUPPORTED;
  const int32_t W = pkv_decode_num_workers(Hq, Hkv, hd, dtype);
  if (W <= 0) return PKV_ERR_HIP;
  auto* e = new (std::nothrow) pkv_engine();
  if (!e) return PKV_ERR_HIP;
  e->alloc = alloc;
  e->k_cache = k_cache;
  e->v_cache = v_cache;
  e->NB = NB;
  e->Hq = Hq;
  e->Hkv = Hkv;
  e->hd = hd;
  e->dtype = dtype;
  e->max_batch = max_batch;
  e->max_ctx = max_context_len;
  e->mb = static_cast<int32_t>(mb);
  e->flags = flags;
  e->W = W;
  e->tab_ints = up4(static_cast<size_t>(max_batch) * e->mb);
  e->mirror.assign(e->tab_ints, -1);
  e->row_serial.assign(max_batch, 0);
  e->row_nblk.assign(max_batch, 0);
  e->rowbuf.assign(e->mb, -1);
  hipError_t he = fail("engine: device", hipGetDevice(&e->device));
  for (int s = 0; s < kSets && he == hipSuccess; ++s)
    he = fail("engine: event", hipEventCreateWithFlags(&e->done[s], hipEventDisableTiming |
                                                                    hipEventDisableSystemFence));
  if (he == hipSuccess)
    he = fail("engine: table", hipMalloc(reinterpret_cast<void**>(&e->dtab), e->tab_ints * 4));
  if (he == hipSuccess)  // the device table starts as the mirror does: all -1
    he = fail("engine: table init", hipMemcpy(e->dtab, e->mirror.data(), e->tab_ints * 4,
                                              hipMemcpyHostToDevice));
  const size_t base = small_layout(max_batch).slots + 64;
  for (int s = 0; s < kSets && he == hipSuccess; ++s) he = e->reserve(s, base, 0);
  if (he != hipSuccess) {
    delete e;
    return PKV_ERR_HIP;
  }
  e->plan.resize(pkv_decode_plan_max_ints(max_batch, e->mb));
  e->pf_plan.resize(4096);
  *out = e;
  return PKV_OK;
}

void pkv_engine_destroy(pkv_engine* e) { delete e; }

pkv_status pkv_engine_submit(pkv_engine* e, int64_t rid, int32_t prompt_len,
                             int32_t max_new_tokens, int32_t arrival_step,
                             const int32_t* token_ids) {
  if (!e || prompt_len < 1 || max_new_tokens < 1 || arrival_step < 0)
    return PKV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(prompt_len) + max_new_tokens > e->max_ctx) return PKV_ERR_INVALID_ARG;
  if (blocks_for(static_cast<int64_t>(prompt_len) + max_new_tokens) > e->NB)
    return PKV_ERR_INVALID_ARG;
  Request r{rid, prompt_len, max_new_tokens, arrival_step, {}};
  if (token_ids) r.ids.assign(token_ids, token_ids + prompt_len);
  e->queue.push_back(std::move(r));
  return PKV_OK;
}

pkv_status pkv_engine_adopt(pkv_engine* e, int32_t n, const int64_t* seqs) {
  if (!e || n < 0 || (n > 0 && !seqs)) return PKV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(e->run.size()) + n > e->max_batch) return PKV_ERR_INVALID_ARG;
  std::unordered_set<int64_t> seen;
  for (const auto& r : e->run) seen.insert(r.rid);
  for (int32_t i = 0; i < n; ++i) {
    if (pkv_alloc_seq_len(e->alloc, seqs[i]) < 0) return PKV_ERR_UNKNOWN_SEQ;
    if (!seen.insert(seqs[i]).second) return PKV_ERR_SEQ_EXISTS;
  }
  for (int32_t i = 0; i < n; ++i)
    e->run.push_back({seqs[i], kNoLimit, kNoLimit, 0, e->next_serial++});
  return PKV_OK;
}

int32_t pkv_engine_running(const pkv_engine* e, int64_t* seqs, int32_t cap) {
  if (!e) return -1;
  const int32_t n = static_cast<int32_t>(e->run.size());
  if (seqs)
    for (int32_t i = 0; i < std::min(n, cap); ++i) seqs[i] = e->run[i].rid;
  return n;
}

int32_t pkv_engine_queued(const pkv_engine* e) {
  return e ? static_cast<int32_t>(e->queue.size()) : -1;
}

pkv_status pkv_engine_step(pkv_engine* e, const void* q, const void* k_new, const void* v_new,
                           const int32_t* new_ids, void* out, const void* k_prompt,
                           const void* v_prompt, int32_t prompt_rows, const void* q_prompt,
                           void* prefill_out, float scale, void* const* events, int64_t* info,
                           void* stream) {
  if (!engine_ok(e) || prompt_rows < 0 || !(scale == scale)) return PKV_ERR_INVALID_ARG;
  if ((q_prompt == nullptr) != (prefill_out == nullptr)) return PKV_ERR_INVALID_ARG;
  if (q_prompt && (e->dtype == PKV_F32 || e->Hq / e->Hkv > pkv::kRowsPerTile))
    return PKV_ERR_UNSUPPORTED;
  auto hs = static_cast<hipStream_t>(stream);
  for (const auto& r : e->run)  // the continuing sequences' next token must fit
    if (r.done < r.max_new && pkv_alloc_seq_len(e->alloc, r.rid) + 1 > e->max_ctx)
      return PKV_ERR_INVALID_ARG;
  const int s = e->cur;
  if (e->acquire(s) != hipSuccess) return PKV_ERR_HIP;

  // 1. retire the requests that produced all their tokens
  e->retired.clear();
  for (const auto& r : e->run)
    if (r.done >= r.max_new) e->retired.push_back(r.rid);
  if (!e->retired.empty()) {
    pkv_status st = pkv_alloc_free_many(e->alloc, static_cast<int32_t>(e->retired.size()),
                                        e->retired.data());
    if (st != PKV_OK) return st;
    e->run.erase(std::remove_if(e->run.begin(), e->run.end(),
                                [](const Running& r) { return r.done >= r.max_new; }),
                 e->run.end());
  }
  // 2. admit queue heads, first come first served: while the batch has room, the head has
  // arrived, its whole prompt fits in the prompt rows left, and the free blocks cover its
  // final size on top of what the running requests may still take
  int64_t reserve = 0;
  for (const auto& r : e->run)
    if (r.max_new != kNoLimit)
      reserve += blocks_for(r.final_len) - blocks_for(r.final_len - r.max_new + r.done);
  const int32_t B0 = static_cast<int32_t>(e->run.size());
  e->admitted.clear();
  int32_t T = 0, A = 0;
  const int32_t Bmax = static_cast<int32_t>(std::min<size_t>(
      e->max_batch, static_cast<size_t>(B0) + e->queue.size()));
  Layout lay = small_layout(Bmax);
  if (e->reserve(s, lay.slots + up4(prompt_rows) + 64, 0) != hipSuccess) return PKV_ERR_HIP;
  int32_t* H = e->host[s];
  H[lay.pf_qs] = 0;
  while (!e->queue.empty()) {
    const Request& r = e->queue.front();
    if (r.arrival > e->step_no || B0 + A >= e->max_batch) break;
    const int64_t need = blocks_for(static_cast<int64_t>(r.prompt) + r.max_new);
    if (pkv_alloc_num_free(e->alloc) - reserve < need) break;
    if (T + static_cast<int64_t>(r.prompt) > prompt_rows) break;
    int32_t cached = 0;
    if (!r.ids.empty()) {
      e->tmp_slots.resize(r.prompt);
      pkv_status st = pkv_alloc_add_seq_tokens(e->alloc, r.rid, r.prompt, r.ids.data(),
                                               e->tmp_slots.data(), &cached);
      if (st != PKV_OK) return st;
      std::memcpy(H + lay.slots + T, e->tmp_slots.data() + cached,
                  static_cast<size_t>(r.prompt - cached) * 4);
    } else {
      pkv_status st = pkv_alloc_add_seq(e->alloc, r.rid);
      if (st != PKV_OK) return st;
      const int32_t p = r.prompt;
      st = pkv_alloc_append(e->alloc, 1, &r.rid, &p, H + lay.slots + T, nullptr, nullptr,
                            nullptr);
      if (st != PKV_OK) {
        (void)pkv_alloc_free(e->alloc, r.rid);
        return st;
      }
    }
    T += r.prompt - cached;
    reserve += need - blocks_for(r.prompt);
    H[lay.pf_lens + A] = r.prompt;
    H[lay.pf_qs + A + 1] = T;
    e->admitted.push_back(r.rid);
    e->admitted.push_back(r.prompt);
    e->admitted.push_back(cached);
    e->run.push_back(
        {r.rid, static_cast<int64_t>(r.prompt) + r.max_new, r.max_new, 0, e->next_serial++});
    e->queue.pop_front();
    ++A;
  }
  return decode_tail(e, s, lay, T, A, nullptr, new_ids, q, k_new, v_new, out, k_prompt,
                     v_prompt, q_prompt, prefill_out, scale, events, info, hs);
}

pkv_status pkv_engine_beam_step(pkv_engine* e, const int32_t* parents, const int64_t* children,
                                const void* q, const void* k_new, const void* v_new, void* out,
                                float scale, void* const* events, int64_t* info, void* stream) {
  if (!engine_ok(e) || !(scale == scale)) return PKV_ERR_INVALID_ARG;
  if ((parents == nullptr) != (children == nullptr)) return PKV_ERR_INVALID_ARG;
  auto hs = static_cast<hipStream_t>(stream);
  const int32_t B = static_cast<int32_t>(e->run.size());
  for (int32_t i = 0; i < B; ++i) {  // arguments and lengths checked before any change
    const int32_t src = parents ? parents[i] : i;
    if (src < 0 || src >= B) return PKV_ERR_INVALID_ARG;
    if (pkv_alloc_seq_len(e->alloc, e->run[src].rid) + 1 > e->max_ctx) return PKV_ERR_INVALID_ARG;
  }
  const int s = e->cur;
  if (e->acquire(s) != hipSuccess) return PKV_ERR_HIP;
  e->retired.clear();
  e->admitted.clear();
  if (parents && B > 0) {
    // every new beam i forks from running beam parents[i]; then the old beams are freed (one
    // allocator call); the rows as they were serve the children's rows
    std::vector<int64_t> par(B), old(B);
    for (int32_t i = 0; i < B; ++i) {
      par[i] = e->run[parents[i]].rid;
      old[i] = e->run[i].rid;
    }
    pkv_status st = pkv_alloc_replace_many(e->alloc, B, par.data(), old.data(), children);
    if (st != PKV_OK) return st;
    const size_t rows = static_cast<size_t>(B) * e->mb;
    if (e->snap.size() < rows) e->snap.resize(rows);
    std::memcpy(e->snap.data(), e->mirror.data(), rows * 4);
    e->snap_nblk.assign(e->row_nblk.begin(), e->row_nblk.begin() + B);
    for (int32_t i = 0; i < B; ++i)  // rows whose content the mirror does not track
      if (e->row_serial[i] != e->run[i].serial) e->snap_nblk[i] = 0;
    std::vector<Running> next(B);
    for (int32_t i = 0; i < B; ++i) {
      next[i] = e->run[parents[i]];
      next[i].rid = children[i];
      next[i].serial = e->next_serial++;
    }
    e->run.swap(next);
  }
  Layout lay = small_layout(B);
  if (e->reserve(s, lay.slots + 64, 0) != hipSuccess) return PKV_ERR_HIP;
  return decode_tail(e, s, lay, 0, 0, parents, nullptr, q, k_new, v_new, out, nullptr, nullptr,
                     nullptr, nullptr, scale, events, info, hs);
}

pkv_status pkv_engine_last(const pkv_engine* e, int64_t* retired, int64_t* admitted,
                           int32_t* prompt_slots, int32_t* lens, int32_t* tables) {
  if (!e) return PKV_ERR_INVALID_ARG;
  if (e->last_set < 0) return PKV_OK;
  const int32_t* H = e->host[e->last_set];
  if (retired) std::copy(e->retired.begin(), e->retired.end(), retired);
  if (admitted) std::copy(e->admitted.begin(), e->admitted.end(), admitted);
  if (prompt_slots) std::memcpy(prompt_slots, H + e->last.slots, e->last_T * 4);
  if (lens) std::memcpy(lens, H + e->last.lens, e->last_B * 4);
  if (tables)
    std::memcpy(tables, e->mirror.data(), static_cast<size_t>(e->last_B) * e->mb * 4);
  return PKV_OK;
}

pkv_status pkv_engine_sync(pkv_engine* e) {
  if (!e) return PKV_ERR_INVALID_ARG;
  for (int s = 0; s < kSets; ++s)
    if (e->acquire(s) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

}  // extern "C"
