// Host block allocator of libpkv: allocate on demand, share (fork), copy-on-write, free.
//
// [P1] "vLLM 與 PagedAttention：高吞吐推理的關鍵", §三 steps 一..四: a request starts with an
// empty block table, takes a new block only when its current block is full, and gives every
// block back when it finishes; §二 "解決三大問題": several tables may point at one physical
// block. [P2] vLLM overview, "PagedAttention 的核心原理": on-demand allocation, sharing of
// prefix and beam-search blocks.
//
// Conventions the pages leave open (documented in pkv.h): FIFO free list seeded with a caller
// order; per-block reference counts; copy-on-write of a shared, partly filled last block;
// blocks released in logical order; every call all-or-nothing.

#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pkv.h"

namespace {

struct Seq {
  std::vector<int32_t> blocks;  // physical blocks, logical order
  int64_t len = 0;              // tokens
  uint64_t mark = 0;            // last append call that named this sequence (duplicate check)
};

}  // namespace

struct pkv_allocator {
  int32_t nb = 0;
  int32_t bs = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  uint64_t calls = 0;             // append calls so far (stamps Seq::mark)
  std::vector<Seq*> batch;        // reused per append call

  // Blocks needed to append ntok tokens to s: a copy-on-write block when the last block is
  // partly filled and shared, plus the new blocks the extra tokens spill into.
  void needs(const Seq& s, int32_t ntok, bool* cow, int64_t* fresh) const {
    *cow = ntok > 0 && (s.len % bs) != 0 && ref[s.blocks.back()] > 1;
    const int64_t have = (s.len + bs - 1) / bs;
    const int64_t want = (s.len + ntok + bs - 1) / bs;
    *fresh = want - have;
  }

  int32_t pop() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    ref[b] = 1;
    return b;
  }
};

extern "C" {

pkv_status pkv_alloc_create(int32_t NB, int32_t bs, const int32_t* free_order,
                            pkv_allocator** out) {
  if (!out || NB <= 0 || bs <= 0 || static_cast<int64_t>(NB) * bs >= (int64_t{1} << 31))
    return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  if (free_order) {
    std::vector<char> seen(NB, 0);
    for (int32_t i = 0; i < NB; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= NB || seen[b]) return PKV_ERR_INVALID_ARG;
      seen[b] = 1;
    }
  }
  auto* a = new (std::nothrow) pkv_allocator();
  if (!a) return PKV_ERR_INVALID_ARG;
  a->nb = NB;
  a->bs = bs;
  a->ref.assign(NB, 0);
  for (int32_t i = 0; i < NB; ++i) a->free_list.push_back(free_order ? free_order[i] : i);
  *out = a;
  return PKV_OK;
}

void pkv_alloc_destroy(pkv_allocator* a) { delete a; }

pkv_status pkv_alloc_add_seq(pkv_allocator* a, int64_t seq) {
  if (!a) return PKV_ERR_INVALID_ARG;
  if (a->seqs.count(seq)) return PKV_ERR_SEQ_EXISTS;
  a->seqs.emplace(seq, Seq{});
  return PKV_OK;
}

pkv_status pkv_alloc_append(pkv_allocator* a, int32_t n, const int64_t* seqs, const int32_t* ntok,
                            int32_t* slots_out, int32_t* cow_src, int32_t* cow_dst,
                            int32_t* n_cow) {
  if (!a || n < 0 || (n > 0 && (!seqs || !ntok))) return PKV_ERR_INVALID_ARG;
  if ((cow_src == nullptr) != (cow_dst == nullptr) || ((cow_src != nullptr) != (n_cow != nullptr)))
    return PKV_ERR_INVALID_ARG;
  // Validate everything and count the blocks the whole batch needs before changing anything.
  // Duplicate ids are found by stamping each named sequence with this call's number; an id
  // that is not present sends the check to a set, so that a repeated unknown id still reads
  // as a duplicate (PKV_ERR_INVALID_ARG) before it reads as unknown.
  for (int32_t k = 0; k < n; ++k)
    if (ntok[k] < 0) return PKV_ERR_INVALID_ARG;
  std::vector<Seq*>& ptr = a->batch;
  ptr.assign(n, nullptr);
  const uint64_t call = ++a->calls;
  bool unknown = false, dup = false;
  for (int32_t k = 0; k < n; ++k) {
    auto it = a->seqs.find(seqs[k]);
    if (it == a->seqs.end()) {
      unknown = true;
      continue;
    }
    if (it->second.mark == call) dup = true;
    it->second.mark = call;
    ptr[k] = &it->second;
  }
  if (unknown && !dup) {
    std::unordered_set<int64_t> distinct;
    for (int32_t k = 0; k < n; ++k)
      if (!distinct.insert(seqs[k]).second) dup = true;
  }
  if (dup) return PKV_ERR_INVALID_ARG;
  if (unknown) return PKV_ERR_UNKNOWN_SEQ;
  int64_t total = 0;
  for (int32_t k = 0; k < n; ++k) {
    bool cow;
    int64_t fresh;
    a->needs(*ptr[k], ntok[k], &cow, &fresh);
    total += (cow ? 1 : 0) + fresh;
  }
  if (total > static_cast<int64_t>(a->free_list.size())) return PKV_ERR_OUT_OF_BLOCKS;

  int32_t ncow = 0;
  int64_t out_pos = 0;
  for (int32_t k = 0; k < n; ++k) {
    Seq& s = *ptr[k];
    bool cow;
    int64_t fresh;
    a->needs(s, ntok[k], &cow, &fresh);
    if (cow) {  // move off the shared, partly filled block before writing into it
      const int32_t src = s.blocks.back();
      const int32_t dst = a->pop();
      a->ref[src] -= 1;
      s.blocks.back() = dst;
      if (cow_src) {
        cow_src[ncow] = src;
        cow_dst[ncow] = dst;
      }
      ++ncow;
    }
    for (int32_t t = 0; t < ntok[k]; ++t) {
      if (s.len % a->bs == 0) s.blocks.push_back(a->pop());  // current block full: a new one
      const int32_t blk = s.blocks[s.len / a->bs];
      if (slots_out) slots_out[out_pos] = blk * a->bs + static_cast<int32_t>(s.len % a->bs);
      ++out_pos;
      ++s.len;
    }
  }
  if (n_cow) *n_cow = ncow;
  return PKV_OK;
}

pkv_status pkv_alloc_fork(pkv_allocator* a, int64_t parent, int64_t child) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  if (a->seqs.count(child)) return PKV_ERR_SEQ_EXISTS;
  Seq copy = it->second;
  for (int32_t b : copy.blocks) a->ref[b] += 1;
  a->seqs.emplace(child, std::move(copy));
  return PKV_OK;
}

pkv_status pkv_alloc_free(pkv_allocator* a, int64_t seq) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  for (int32_t b : it->second.blocks) {
    if (--a->ref[b] == 0) a->free_list.push_back(b);
  }
  a->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_alloc_fork_many(pkv_allocator* a, int32_t n, const int64_t* parents,
                               const int64_t* children) {
  if (!a || n < 0 || (n > 0 && (!parents || !children))) return PKV_ERR_INVALID_ARG;
  // All-or-nothing: every parent present before the call, every child absent and named once.
  std::vector<const Seq*> from(n);
  for (int32_t k = 0; k < n; ++k) {
    auto it = a->seqs.find(parents[k]);
    if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    from[k] = &it->second;
  }
  std::unordered_set<int64_t> kids;
  kids.reserve(static_cast<size_t>(n));
  for (int32_t k = 0; k < n; ++k)
    if (a->seqs.count(children[k]) || !kids.insert(children[k]).second) return PKV_ERR_SEQ_EXISTS;
  std::vector<Seq> copies(n);  // copied before any insertion can move the parents
  for (int32_t k = 0; k < n; ++k) {
    copies[k].blocks = from[k]->blocks;
    copies[k].len = from[k]->len;
  }
  a->seqs.reserve(a->seqs.size() + static_cast<size_t>(n));
  for (int32_t k = 0; k < n; ++k) {
    for (int32_t b : copies[k].blocks) a->ref[b] += 1;
    a->seqs.emplace(children[k], std::move(copies[k]));
  }
  return PKV_OK;
}

pkv_status pkv_alloc_free_many(pkv_allocator* a, int32_t n, const int64_t* seqs) {
  if (!a || n < 0 || (n > 0 && !seqs)) return PKV_ERR_INVALID_ARG;
  // All-or-nothing: every id present and named once (stamped like pkv_alloc_append's check).
  const uint64_t call = ++a->calls;
  bool unknown = false, dup = false;
  for (int32_t k = 0; k < n; ++k) {
    auto it = a->seqs.find(seqs[k]);
    if (it == a->seqs.end()) {
      unknown = true;
      continue;
    }
    if (it->second.mark == call) dup = true;
    it->second.mark = call;
  }
  if (unknown && !dup) {
    std::unordered_set<int64_t> distinct;
    for (int32_t k = 0; k < n; ++k)
      if (!distinct.insert(seqs[k]).second) dup = true;
  }
  if (dup) return PKV_ERR_INVALID_ARG;
  if (unknown) return PKV_ERR_UNKNOWN_SEQ;
  for (int32_t k = 0; k < n; ++k) pkv_alloc_free(a, seqs[k]);
  return PKV_OK;
}

}  // extern "C"

namespace {

pkv_status export_tables(const pkv_allocator* a, int32_t n, const int64_t* seqs,
                         int32_t max_blocks, int32_t* block_tables_out, int32_t* context_lens_out,
                         bool mark_shared) {
  if (!a || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !block_tables_out || !context_lens_out)))
    return PKV_ERR_INVALID_ARG;
  std::vector<const Seq*> ptr(n);
  for (int32_t k = 0; k < n; ++k) {
    auto it = a->seqs.find(seqs[k]);
    if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    if (static_cast<int64_t>(it->second.blocks.size()) > max_blocks ||
        it->second.len > INT32_MAX)
      return PKV_ERR_INVALID_ARG;
    ptr[k] = &it->second;
  }
  for (int32_t k = 0; k < n; ++k) {
    int32_t* row = block_tables_out + static_cast<int64_t>(k) * max_blocks;
    const auto& b = ptr[k]->blocks;
    int32_t j = 0;
    if (mark_shared) {
      for (; j < static_cast<int32_t>(b.size()); ++j)
        row[j] = a->ref[b[j]] > 1 ? (b[j] | PKV_BLOCK_SHARED) : b[j];
    } else {
      for (; j < static_cast<int32_t>(b.size()); ++j) row[j] = b[j];
    }
    for (; j < max_blocks; ++j) row[j] = -1;
    context_lens_out[k] = static_cast<int32_t>(ptr[k]->len);
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_alloc_tables(const pkv_allocator* a, int32_t n, const int64_t* seqs,
                            int32_t max_blocks, int32_t* block_tables_out,
                            int32_t* context_lens_out) {
  return export_tables(a, n, seqs, max_blocks, block_tables_out, context_lens_out, false);
}

pkv_status pkv_alloc_tables_marked(const pkv_allocator* a, int32_t n, const int64_t* seqs,
                                   int32_t max_blocks, int32_t* block_tables_out,
                                   int32_t* context_lens_out) {
  return export_tables(a, n, seqs, max_blocks, block_tables_out, context_lens_out, true);
}

int32_t pkv_alloc_num_free(const pkv_allocator* a) {
  return a ? static_cast<int32_t>(a->free_list.size()) : -1;
}

int32_t pkv_alloc_refcount(const pkv_allocator* a, int32_t block) {
  if (!a || block < 0 || block >= a->nb) return -1;
  return a->ref[block];
}

int64_t pkv_alloc_seq_len(const pkv_allocator* a, int64_t seq) {
  if (!a) return -1;
  auto it = a->seqs.find(seq);
  return it == a->seqs.end() ? -1 : it->second.len;
}

pkv_status pkv_alloc_usage(const pkv_allocator* a, int64_t* out) {
  if (!a || !out) return PKV_ERR_INVALID_ARG;
  // filled slots of a block: the most tokens any owner keeps in it (owners of a shared block
  // hold the same tokens there)
  std::vector<int32_t> fill(static_cast<size_t>(a->nb), 0);
  int64_t logical = 0;
  for (const auto& kv : a->seqs) {
    const Seq& s = kv.second;
    logical += s.len;
    for (size_t j = 0; j < s.blocks.size(); ++j) {
      const int64_t f = std::min<int64_t>(a->bs, s.len - static_cast<int64_t>(j) * a->bs);
      int32_t& cell = fill[static_cast<size_t>(s.blocks[j])];
      if (f > cell) cell = static_cast<int32_t>(f);
    }
  }
  int64_t filled = 0;
  for (int32_t f : fill) filled += f;
  out[0] = static_cast<int64_t>(a->seqs.size());
  out[1] = logical;
  out[2] = static_cast<int64_t>(a->nb) - static_cast<int64_t>(a->free_list.size());
  out[3] = filled;
  return PKV_OK;
}

int32_t pkv_alloc_free_list(const pkv_allocator* a, int32_t* out, int32_t cap) {
  if (!a) return -1;
  int32_t i = 0;
  if (out) {
    for (auto it = a->free_list.begin(); it != a->free_list.end() && i < cap; ++it) out[i++] = *it;
  }
  return static_cast<int32_t>(a->free_list.size());
}

}  // extern "C"
