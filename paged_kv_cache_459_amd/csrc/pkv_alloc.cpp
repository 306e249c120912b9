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
//
// Automatic prefix caching ([P1] §五 "前綴共享", §八 "前綴快取"; [P3] §4.2): full blocks of
// sequences whose token ids are known are indexed by (node of the block before them, their
// ids); a new sequence given its prompt's ids shares the longest indexed chain it begins
// with. Freed indexed blocks stay in the free list (FIFO) and keep their entry until a fresh
// allocation pops them; a hit takes a free one back out of the list, so the list is an
// intrusive doubly linked list over block ids.

#include <algorithm>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_kernels.h"

namespace {

struct Seq {
  std::vector<int32_t> blocks;  // physical blocks, logical order
  int64_t len = 0;              // tokens
  uint64_t mark = 0;            // last append call that named this sequence (duplicate check)
  // prefix-cache tracking: only sequences whose every token id is known are indexed
  bool tracked = false;
  int64_t last_node = 0;         // node of the last indexed full block (0: the empty prefix)
  std::vector<int32_t> pending;  // ids of the tokens in the partly filled last block
};

// An indexed full block: its content is (parent node, ids).
struct Node {
  int64_t parent;
  int32_t block;
  uint64_t hash;
  std::vector<int32_t> ids;
};

uint64_t content_hash(int64_t parent, const int32_t* ids, int32_t n) {
  uint64_t h = 0x9E3779B97F4A7C15ull ^ static_cast<uint64_t>(parent);
  for (int32_t i = 0; i < n; ++i) {
    h ^= static_cast<uint32_t>(ids[i]);
    h *= 0x100000001B3ull;
    h ^= h >> 29;
  }
  return h;
}

}  // namespace

struct pkv_allocator {
  int32_t nb = 0;
  int32_t bs = 0;
  // free list: FIFO, intrusive doubly linked over block ids (-1 ends)
  std::vector<int32_t> next, prev;
  int32_t head = -1, tail = -1, nfree = 0;
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  uint64_t calls = 0;             // append calls so far (stamps Seq::mark)
  std::vector<Seq*> batch;        // reused per append call
  std::vector<Seq> staged;        // reused per replace_many call (the children's contents)
  std::unordered_map<int32_t, int32_t> moved;  // reused per append call (copy-on-write count)
  // prefix cache
  std::unordered_multimap<uint64_t, int64_t> index;  // content hash -> node
  std::unordered_map<int64_t, Node> nodes;
  std::vector<int64_t> block_node;  // node indexing each block, 0 if none
  int64_t next_node = 1;
  int32_t cached = 0;               // blocks with an entry

  void push_back(int32_t b) {
    next[b] = -1;
    prev[b] = tail;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    ++nfree;
  }

  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    --nfree;
  }

  void drop_entry(int32_t b) {
    const int64_t id = block_node[b];
    if (id == 0) return;
    auto it = nodes.find(id);
    auto range = index.equal_range(it->second.hash);
    for (auto r = range.first; r != range.second; ++r)
      if (r->second == id) {
        index.erase(r);
        break;
      }
    nodes.erase(it);
    block_node[b] = 0;
    --cached;
  }

  // Node naming the content (parent, ids[0..bs)), or 0.
  int64_t find(int64_t parent, const int32_t* ids) const {
    const uint64_t h = content_hash(parent, ids, bs);
    auto range = index.equal_range(h);
    for (auto r = range.first; r != range.second; ++r) {
      const Node& nd = nodes.at(r->second);
      if (nd.parent == parent && std::equal(nd.ids.begin(), nd.ids.end(), ids)) return r->second;
    }
    return 0;
  }

  // Index full block `block` under (parent, ids); returns the node now naming that content
  // (an existing one when the same content is indexed already).
  int64_t enter(int64_t parent, const int32_t* ids, int32_t block) {
    const int64_t have = find(parent, ids);
    if (have) return have;
    const int64_t id = next_node++;
    const uint64_t h = content_hash(parent, ids, bs);
    nodes.emplace(id, Node{parent, block, h, std::vector<int32_t>(ids, ids + bs)});
    index.emplace(h, id);
    block_node[block] = id;
    ++cached;
    return id;
  }

  // Blocks needed to append ntok tokens to s: a copy-on-write block when the last block is
  // partly filled and shared, plus the new blocks the extra tokens spill into.
  void needs(const Seq& s, int32_t ntok, bool* cow, int64_t* fresh) const {
    *cow = ntok > 0 && (s.len % bs) != 0 && ref[s.blocks.back()] > 1;
    const int64_t have = (s.len + bs - 1) / bs;
    const int64_t want = (s.len + ntok + bs - 1) / bs;
    *fresh = want - have;
  }

  // Fresh allocation: the free list's front, its index entry dropped (eviction).
  int32_t pop() {
    const int32_t b = head;
    unlink(b);
    drop_entry(b);
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
  a->next.assign(NB, -1);
  a->prev.assign(NB, -1);
  a->block_node.assign(NB, 0);
  for (int32_t i = 0; i < NB; ++i) a->push_back(free_order ? free_order[i] : i);
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

}  // extern "C"

namespace {

pkv_status append_impl(pkv_allocator* a, int32_t n, const int64_t* seqs, const int32_t* ntok,
                       const int32_t* token_ids, int32_t* slots_out, int32_t* cow_src,
                       int32_t* cow_dst, int32_t* n_cow) {
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
  // The count follows the loop below: sharers of a partly filled block that append in this
  // call move off it one by one, so the last of them (refcount back to 1 by then) writes in
  // place and takes no copy. `moved` holds, per such block, the sharers already counted off.
  int64_t total = 0;
  std::unordered_map<int32_t, int32_t>& moved = a->moved;
  moved.clear();
  for (int32_t k = 0; k < n; ++k) {
    bool cow;
    int64_t fresh;
    a->needs(*ptr[k], ntok[k], &cow, &fresh);
    if (cow) {
      int32_t& gone = moved[ptr[k]->blocks.back()];
      cow = a->ref[ptr[k]->blocks.back()] - gone > 1;
      gone += cow ? 1 : 0;
    }
    total += (cow ? 1 : 0) + fresh;
  }
  if (total > a->nfree) return PKV_ERR_OUT_OF_BLOCKS;

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
      if (s.tracked && token_ids) {
        s.pending.push_back(token_ids[out_pos]);
        if (static_cast<int32_t>(s.pending.size()) == a->bs) {  // the block just filled
          s.last_node = a->enter(s.last_node, s.pending.data(), blk);
          s.pending.clear();
        }
      }
      ++out_pos;
      ++s.len;
    }
    if (ntok[k] > 0 && !token_ids) {  // tokens of unknown content: no longer indexed
      s.tracked = false;
      s.pending.clear();
    }
  }
  if (n_cow) *n_cow = ncow;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_alloc_append(pkv_allocator* a, int32_t n, const int64_t* seqs, const int32_t* ntok,
                            int32_t* slots_out, int32_t* cow_src, int32_t* cow_dst,
                            int32_t* n_cow) {
  return append_impl(a, n, seqs, ntok, nullptr, slots_out, cow_src, cow_dst, n_cow);
}

pkv_status pkv_alloc_append_tokens(pkv_allocator* a, int32_t n, const int64_t* seqs,
                                   const int32_t* ntok, const int32_t* token_ids,
                                   int32_t* slots_out, int32_t* cow_src, int32_t* cow_dst,
                                   int32_t* n_cow) {
  if (n > 0 && !token_ids) return PKV_ERR_INVALID_ARG;
  return append_impl(a, n, seqs, ntok, token_ids, slots_out, cow_src, cow_dst, n_cow);
}

pkv_status pkv_alloc_add_seq_tokens(pkv_allocator* a, int64_t seq, int32_t n,
                                    const int32_t* token_ids, int32_t* slots_out,
                                    int32_t* cached_out) {
  if (!a || n < 0 || (n > 0 && !token_ids)) return PKV_ERR_INVALID_ARG;
  if (a->seqs.count(seq)) return PKV_ERR_SEQ_EXISTS;
  const int32_t bs = a->bs;
  // the longest indexed chain of full blocks the prompt begins with
  std::vector<int32_t> hits;
  int64_t parent = 0;
  for (int32_t j = 0; j < n / bs; ++j) {
    const int64_t node = a->find(parent, token_ids + static_cast<int64_t>(j) * bs);
    if (!node) break;
    hits.push_back(a->nodes.at(node).block);
    parent = node;
  }
  int32_t revived = 0;
  for (int32_t b : hits) revived += a->ref[b] == 0 ? 1 : 0;
  const int64_t fresh = (static_cast<int64_t>(n) + bs - 1) / bs - static_cast<int64_t>(hits.size());
  if (fresh > a->nfree - revived) return PKV_ERR_OUT_OF_BLOCKS;
  Seq s;
  s.blocks.reserve(hits.size() + static_cast<size_t>(fresh));
  for (int32_t b : hits) {
    if (a->ref[b] == 0) a->unlink(b);  // a free indexed block, revived
    a->ref[b] += 1;
    s.blocks.push_back(b);
  }
  for (int64_t i = 0; i < fresh; ++i) s.blocks.push_back(a->pop());
  int64_t last = parent;
  for (int32_t j = static_cast<int32_t>(hits.size()); j < n / bs; ++j)
    last = a->enter(last, token_ids + static_cast<int64_t>(j) * bs, s.blocks[j]);
  s.len = n;
  s.tracked = true;
  s.last_node = last;
  s.pending.assign(token_ids + (n / bs) * bs, token_ids + n);
  if (slots_out)
    for (int32_t t = 0; t < n; ++t) slots_out[t] = s.blocks[t / bs] * bs + t % bs;
  if (cached_out) *cached_out = static_cast<int32_t>(hits.size()) * bs;
  a->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

int32_t pkv_alloc_cached_blocks(const pkv_allocator* a) { return a ? a->cached : -1; }

pkv_status pkv_alloc_fork(pkv_allocator* a, int64_t parent, int64_t child) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  if (a->seqs.count(child)) return PKV_ERR_SEQ_EXISTS;
  Seq copy = it->second;
  copy.mark = 0;
  for (int32_t b : copy.blocks) a->ref[b] += 1;
  a->seqs.emplace(child, std::move(copy));
  return PKV_OK;
}

pkv_status pkv_alloc_free(pkv_allocator* a, int64_t seq) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  for (int32_t b : it->second.blocks) {
    if (--a->ref[b] == 0) a->push_back(b);
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
    copies[k] = *from[k];
    copies[k].mark = 0;
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

pkv_status pkv_alloc_replace_many(pkv_allocator* a, int32_t n, const int64_t* parents,
                                  const int64_t* old, const int64_t* children) {
  if (!a || n < 0 || (n > 0 && (!parents || !old || !children))) return PKV_ERR_INVALID_ARG;
  if (n == 0) return PKV_OK;
  // The checks of fork_many(parents, children) then free_many(old), all before any change:
  // parents present, children absent and distinct, old present (the children cannot be among
  // them) and distinct.
  std::vector<const Seq*> from(n);
  for (int32_t k = 0; k < n; ++k) {
    auto it = a->seqs.find(parents[k]);
    if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    from[k] = &it->second;
  }
  {
    std::unordered_set<int64_t> kids;
    kids.reserve(static_cast<size_t>(n));
    for (int32_t k = 0; k < n; ++k)
      if (a->seqs.count(children[k]) || !kids.insert(children[k]).second) return PKV_ERR_SEQ_EXISTS;
  }
  const uint64_t call = ++a->calls;
  std::vector<Seq*> gone(n, nullptr);
  bool unknown = false, dup = false;
  for (int32_t k = 0; k < n; ++k) {
    auto it = a->seqs.find(old[k]);
    if (it == a->seqs.end()) {
      unknown = true;
      continue;
    }
    if (it->second.mark == call) dup = true;
    it->second.mark = call;
    gone[k] = &it->second;
  }
  if (unknown && !dup) {
    std::unordered_set<int64_t> distinct;
    for (int32_t k = 0; k < n; ++k)
      if (!distinct.insert(old[k]).second) dup = true;
  }
  if (dup) return PKV_ERR_INVALID_ARG;
  if (unknown) return PKV_ERR_UNKNOWN_SEQ;
  // References. The two calls add one per child for each of its parent's blocks, then take
  // one per freed sequence for each of its blocks, pushing a block on the free list when it
  // reaches zero. Here each freed sequence's blocks change once, by its number of children
  // minus one, in the same order: a block still reaches zero only at its last freed holder
  // (before that, the holders not yet visited keep it above zero), so the free list receives
  // the same blocks in the same order. Children of parents that are not freed add their one
  // reference per block directly.
  std::vector<const Seq*> by_ptr(from);
  std::sort(by_ptr.begin(), by_ptr.end());
  std::vector<const Seq*> freed(gone.begin(), gone.end());
  std::sort(freed.begin(), freed.end());
  for (int32_t k = 0; k < n; ++k)
    if (!std::binary_search(freed.begin(), freed.end(), from[k]))
      for (int32_t b : from[k]->blocks) a->ref[b] += 1;
  if (a->staged.size() < static_cast<size_t>(n)) a->staged.resize(n);
  for (int32_t k = 0; k < n; ++k) {  // the children's contents, before any parent goes
    a->staged[k] = *from[k];
    a->staged[k].mark = 0;
  }
  for (int32_t k = 0; k < n; ++k) {
    const auto range = std::equal_range(by_ptr.begin(), by_ptr.end(), gone[k]);
    const int32_t delta = static_cast<int32_t>(range.second - range.first) - 1;
    if (delta == 0) continue;
    for (int32_t b : gone[k]->blocks) {
      a->ref[b] += delta;
      if (a->ref[b] == 0) a->push_back(b);
    }
  }
  // each old entry becomes a child's (its node and storage reused)
  for (int32_t k = 0; k < n; ++k) {
    auto node = a->seqs.extract(old[k]);
    node.key() = children[k];
    std::swap(node.mapped(), a->staged[k]);
    a->seqs.insert(std::move(node));
  }
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

int32_t pkv::alloc_row(const pkv_allocator* a, int64_t seq, int32_t from, int32_t max_blocks,
                      int32_t* row, int64_t* len) {
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return -1;
  const auto& b = it->second.blocks;
  const int32_t n = static_cast<int32_t>(b.size());
  if (n > max_blocks) return -1;
  for (int32_t j = std::max(from, 0); j < n; ++j)
    row[j] = a->ref[b[j]] > 1 ? (b[j] | PKV_BLOCK_SHARED) : b[j];
  *len = it->second.len;
  return n;
}

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

int32_t pkv_alloc_num_free(const pkv_allocator* a) { return a ? a->nfree : -1; }

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
  out[2] = static_cast<int64_t>(a->nb) - a->nfree;
  out[3] = filled;
  return PKV_OK;
}

int32_t pkv_alloc_free_list(const pkv_allocator* a, int32_t* out, int32_t cap) {
  if (!a) return -1;
  int32_t i = 0;
  if (out) {
    for (int32_t b = a->head; b >= 0 && i < cap; b = a->next[b]) out[i++] = b;
  }
  return a->nfree;
}

}  // extern "C"
