// Shared-prefix plan of a decode batch (host side).
//
// [P1] §二 "解決三大問題" and [P2] "共享和复用": sequences with a common prefix (a system prompt,
// beam candidates) point at the same physical blocks. Attention over such blocks is the same
// K/V for every sequence that shares them, so it can be read once for all of them: the shared
// pass (attn_shared_kernel) computes, per run of shared blocks, every member's (m, l, o) piece
// over the run in one MFMA contraction (rows = members' q heads), the stream pass streams only
// each sequence's private remainder, and the merge folds the pieces together.
//
// A run is (members, logical blocks [j0, j1)): every member's table names the same physical
// block at each index of the range. Runs are found top-down: the batch's sequences grouped by
// their first block; a group of two or more extends its run while all members have a block at
// the next index and it is the same block; where they part (or some end) the group is split by
// the block id at that index and each part of two or more continues. A sequence's shared
// blocks are therefore a prefix of its table, skip_s blocks long. The work is one integer
// compare per shared table entry, each member's row scanned contiguously.
//
// Packed int32 layout (see pkv.h): a 16-int header, then skip[B], blocks[B], sh_ptr[B+1],
// units[U][6] = {ref_seq, b0, b1, member_off, member_cnt, cell_base}, members[], sh_list[].

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_kernels.h"

namespace pkv {

namespace {

struct Run {
  std::vector<int32_t> members;
  int32_t j0, j1;
};

}  // namespace

int32_t plan_build(const int32_t* tables, const int32_t* lens, int32_t B, int32_t max_blocks,
                   int32_t max_ctx, int32_t NB, int32_t H, int32_t GS, int32_t G, int32_t chunk,
                   bool share, std::vector<int32_t>* out) {
  // a table entry's block, or -1 when it names no block of the pool (never shared)
  auto entry = [&](int32_t s, int32_t j) {
    const int32_t raw = tables[static_cast<int64_t>(s) * max_blocks + j];
    const int32_t id = raw & ~kSharedBit;
    return raw < 0 || id >= NB ? -1 : id;
  };
  std::vector<int32_t> c(B);
  for (int32_t s = 0; s < B; ++s) {
    const int32_t n = std::min(std::max(lens[s], 0), max_ctx);
    c[s] = std::min((n + kBlockSize - 1) / kBlockSize, max_blocks);
  }
  std::vector<int32_t> skip(B, 0);
  std::vector<Run> runs;
  // groups of >= 2 members that hold the same block at index j (sorted by block id, then
  // member: deterministic)
  std::vector<std::pair<int32_t, int32_t>> keyed;
  auto split = [&](const std::vector<int32_t>& from, int32_t j, std::vector<Run>* todo) {
    keyed.clear();
    for (int32_t s : from)
      if (c[s] > j && entry(s, j) >= 0) keyed.emplace_back(entry(s, j), s);
    std::sort(keyed.begin(), keyed.end());
    for (size_t a = 0; a < keyed.size();) {
      size_t z = a + 1;
      while (z < keyed.size() && keyed[z].first == keyed[a].first) ++z;
      if (z - a >= 2) {
        Run r{{}, j, j};
        r.members.reserve(z - a);
        for (size_t k = a; k < z; ++k) r.members.push_back(keyed[k].second);
        todo->push_back(std::move(r));
      }
      a = z;
    }
  };
  std::vector<Run> todo;
  if (share) {
    std::vector<int32_t> all(B);
    for (int32_t s = 0; s < B; ++s) all[s] = s;
    split(all, 0, &todo);
  }
  while (!todo.empty()) {
    Run r = std::move(todo.back());
    todo.pop_back();
    // the run ends where any member's row first differs from the first member's (rows are
    // scanned contiguously), or ends
    const int32_t first = r.members[0];
    const int32_t* ref = tables + static_cast<int64_t>(first) * max_blocks;
    int32_t e = r.j0;  // the first member's valid entries bound the run
    while (e < c[first] && entry(first, e) >= 0) ++e;
    for (int32_t s : r.members) {  // entries equal to a valid one are valid
      const int32_t* row = tables + static_cast<int64_t>(s) * max_blocks;
      const int32_t lim = std::min(e, c[s]);
      int32_t k = r.j0;
      while (k + 16 <= lim && std::memcmp(row + k, ref + k, 64) == 0) k += 16;  // fast path
      while (k < lim && ((row[k] ^ ref[k]) & ~kSharedBit) == 0) ++k;
      e = k;
    }
    r.j1 = e;
    for (int32_t s : r.members) skip[s] = e;
    std::vector<int32_t> members = r.members;
    runs.push_back(std::move(r));
    split(members, e, &todo);
  }
  // deterministic order: by first member, then start block
  std::sort(runs.begin(), runs.end(), [](const Run& a, const Run& b) {
    return a.members[0] != b.members[0] ? a.members[0] < b.members[0] : a.j0 < b.j0;
  });
  const int32_t per_tile = std::max(1, kRowsPerTile / G);
  // Units: (run, chunk of its blocks, up to per_tile of its members). Listed longest first
  // (stable, so the member tiles of one chunk stay adjacent): the shared pass starts them in
  // this order, so the units that start late, as earlier ones end, are short ones.
  struct Unit {
    const Run* run;
    int32_t b0, b1;
    size_t t;  // first member (index into the run's members)
  };
  std::vector<Unit> order;
  for (const Run& r : runs)
    for (int32_t b0 = r.j0; b0 < r.j1; b0 += chunk)
      for (size_t t = 0; t < r.members.size(); t += per_tile)
        order.push_back(Unit{&r, b0, std::min(r.j1, b0 + chunk), t});
  std::stable_sort(order.begin(), order.end(), [](const Unit& a, const Unit& b) {
    return a.b1 - a.b0 > b.b1 - b.b0;
  });
  std::vector<int32_t> units, members;
  std::vector<int32_t> count(B, 0);  // shared pieces per sequence
  int32_t cells = 0;
  for (const Unit& x : order) {
    const Run& r = *x.run;
    const int32_t cnt = static_cast<int32_t>(std::min<size_t>(per_tile, r.members.size() - x.t));
    units.insert(units.end(), {r.members[0], x.b0, x.b1, static_cast<int32_t>(members.size()), cnt,
                               cells});
    for (int32_t k = 0; k < cnt; ++k) {
      members.push_back(r.members[x.t + k]);
      ++count[r.members[x.t + k]];
    }
    cells += cnt * H;
  }
  // each sequence's piece cells, in unit order (CSR)
  std::vector<int32_t> ptr(B + 1, 0);
  for (int32_t s = 0; s < B; ++s) ptr[s + 1] = ptr[s] + count[s];
  std::vector<int32_t> list(ptr[B]);
  {
    std::vector<int32_t> fill(ptr.begin(), ptr.end() - 1);
    for (size_t u = 0; u < units.size(); u += kUnitInts) {
      const int32_t off = units[u + 3], cnt = units[u + 4], base = units[u + 5];
      for (int32_t k = 0; k < cnt; ++k) list[fill[members[off + k]]++] = base + k * H;
    }
  }
  const int32_t U = static_cast<int32_t>(units.size() / kUnitInts);
  std::vector<int32_t>& p = *out;
  p.assign(kPlanHeader, 0);
  p[0] = kPlanMagic;
  p[1] = B;
  p[2] = H;
  p[3] = GS;
  p[4] = U;
  p[5] = static_cast<int32_t>(members.size());
  p[6] = ptr[B];
  p[7] = cells;
  p[8] = chunk;
  p.insert(p.end(), skip.begin(), skip.end());
  p.insert(p.end(), c.begin(), c.end());
  p.insert(p.end(), ptr.begin(), ptr.end());
  p.insert(p.end(), units.begin(), units.end());
  p.insert(p.end(), members.begin(), members.end());
  p.insert(p.end(), list.begin(), list.end());
  return U;
}

bool plan_check(const int32_t* p, size_t n, int32_t B, int32_t max_blocks, int32_t H, int32_t GS,
                int32_t G, bool append, PlanView* v) {
  if (n < static_cast<size_t>(kPlanHeader) || p[0] != kPlanMagic || p[1] != B || p[2] != H ||
      p[3] != GS)
    return false;
  const int64_t U = p[4], M = p[5], L = p[6], cells = p[7];
  if (U < 0 || M < 0 || L < 0 || cells < 0 || p[8] <= 0 || p[8] > kMaxUnitBlocks) return false;
  const int64_t need = kPlanHeader + 3 * static_cast<int64_t>(B) + 1 + U * kUnitInts + M + L;
  if (static_cast<int64_t>(n) != need || cells > (int64_t{1} << 30)) return false;
  const int32_t* skip = p + kPlanHeader;
  const int32_t* blocks = skip + B;
  const int32_t* ptr = blocks + B;
  const int32_t* units = ptr + B + 1;
  const int32_t* members = units + U * kUnitInts;
  const int32_t* list = members + M;
  for (int32_t s = 0; s < B; ++s) {
    if (skip[s] < 0 || blocks[s] < 0 || blocks[s] > max_blocks || skip[s] > blocks[s])
      return false;
    // the block of a sequence's newest token must stay private in append mode
    if (append && blocks[s] > 0 && skip[s] >= blocks[s]) return false;
    if (ptr[s + 1] < ptr[s]) return false;
  }
  if (ptr[0] != 0 || ptr[B] != L) return false;
  const int32_t per_tile = std::max(1, kRowsPerTile / G);
  for (int64_t u = 0; u < U; ++u) {
    const int32_t* e = units + u * kUnitInts;
    if (e[0] < 0 || e[0] >= B || e[1] < 0 || e[1] >= e[2] || e[2] > max_blocks ||
        e[2] - e[1] > p[8])
      return false;
    if (e[3] < 0 || e[4] < 1 || e[4] > per_tile || static_cast<int64_t>(e[3]) + e[4] > M)
      return false;
    if (e[5] < 0 || static_cast<int64_t>(e[5]) + static_cast<int64_t>(e[4]) * H > cells)
      return false;
  }
  for (int64_t k = 0; k < M; ++k)
    if (members[k] < 0 || members[k] >= B) return false;
  for (int64_t k = 0; k < L; ++k)
    if (list[k] < 0 || static_cast<int64_t>(list[k]) + H > cells) return false;
  v->U = static_cast<int32_t>(U);
  v->cells = static_cast<int32_t>(cells);
  v->has_shared = L > 0;
  return true;
}

// ---- prefill ----------------------------------------------------------------------------
//
// [P1] §三 (the prompt's tokens are written to the cache, then attended) and the causal rule
// of attention: the prompt token at position pos attends to positions 0..pos of its own
// sequence, the cached prefix included. The same (m, l, o) pieces and merge as decode serve a
// row whose visible blocks are split over several chunks.

int32_t prefill_chunk(const int32_t* qs, const int32_t* lens, int32_t S, int32_t H,
                      int32_t tile_rows, int32_t max_chunk, int64_t min_groups) {
  // the tiles' block counts, as prefill_plan_build cuts them
  std::vector<int32_t> nbs;
  for (int32_t s = 0; s < S; ++s) {
    const int32_t q = qs[s + 1] - qs[s], n = lens[s];
    for (int32_t a = 0; a < q; a += tile_rows) {
      const int32_t last = std::min(q, a + tile_rows) - 1;  // the tile's last row
      nbs.push_back((n - q + last + 1 + kBlockSize - 1) / kBlockSize);
    }
  }
  int32_t chunk = max_chunk;
  for (; chunk > kPrefillMinChunk; chunk /= 2) {
    int64_t units = 0;
    for (int32_t nb : nbs) units += (nb + chunk - 1) / chunk;
    if (units * H >= min_groups) break;
  }
  return chunk;
}

void prefill_plan_build(const int32_t* qs, const int32_t* lens, int32_t S, int32_t H, int32_t GS,
                        int32_t tile_rows, int32_t chunk, std::vector<int32_t>* out) {
  const int32_t T = qs[S];
  std::vector<int32_t> skip(T, 0), vis(T, 0), count(T, 0);
  std::vector<int32_t> units, members;
  int32_t cells = 0;
  for (int32_t s = 0; s < S; ++s) {
    const int32_t q0 = qs[s], q = qs[s + 1] - q0, n = lens[s];
    for (int32_t t = 0; t < q; ++t) vis[q0 + t] = n - q + t + 1;
    for (int32_t a = 0; a < q; a += tile_rows) {
      const int32_t cnt = std::min(tile_rows, q - a);
      // the tile's last row sees the most blocks
      const int32_t nb = (vis[q0 + a + cnt - 1] + kBlockSize - 1) / kBlockSize;
      const bool direct = nb <= chunk;
      for (int32_t b0 = 0; b0 < nb; b0 += chunk) {
        const int32_t b1 = std::min(nb, b0 + chunk);
        units.insert(units.end(), {s, b0, b1, static_cast<int32_t>(members.size()), cnt,
                                   direct ? -1 : cells});
        for (int32_t k = 0; k < cnt; ++k) {
          const int32_t r = q0 + a + k;
          members.push_back(r);
          if (!direct && vis[r] > kBlockSize * b0) ++count[r];
        }
        if (!direct) cells += cnt * H;
      }
      if (!direct)
        for (int32_t k = 0; k < cnt; ++k) skip[q0 + a + k] = 1;
    }
  }
  // Longest units first (stable: a row's chunks keep their order): work-groups are dispatched
  // in unit order, so the last ones to start, which set the launch's tail, are the short
  // ones. Cells are then handed out in that order.
  {
    const size_t U = units.size() / kUnitInts;
    std::vector<int32_t> order(U);
    for (size_t u = 0; u < U; ++u) order[u] = static_cast<int32_t>(u);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
      return units[a * kUnitInts + 2] - units[a * kUnitInts + 1] >
             units[b * kUnitInts + 2] - units[b * kUnitInts + 1];
    });
    std::vector<int32_t> sorted;
    sorted.reserve(units.size());
    int32_t next = 0;
    for (int32_t u : order) {
      const int32_t* e = &units[static_cast<size_t>(u) * kUnitInts];
      sorted.insert(sorted.end(), {e[0], e[1], e[2], e[3], e[4], e[5] < 0 ? -1 : next});
      if (e[5] >= 0) next += e[4] * H;
    }
    units.swap(sorted);
  }
  // each merged row's piece cells, in unit order (CSR); a chunk wholly past a row's position
  // gives it no piece
  std::vector<int32_t> ptr(T + 1, 0);
  for (int32_t r = 0; r < T; ++r) ptr[r + 1] = ptr[r] + count[r];
  std::vector<int32_t> list(ptr[T]);
  {
    std::vector<int32_t> fill(ptr.begin(), ptr.end() - 1);
    for (size_t u = 0; u < units.size(); u += kUnitInts) {
      const int32_t b0 = units[u + 1], off = units[u + 3], cnt = units[u + 4], base = units[u + 5];
      if (base < 0) continue;
      for (int32_t k = 0; k < cnt; ++k) {
        const int32_t r = members[off + k];
        if (vis[r] > kBlockSize * b0) list[fill[r]++] = base + k * H;
      }
    }
  }
  std::vector<int32_t>& p = *out;
  p.assign(kPlanHeader, 0);
  p[0] = kPrefillMagic;
  p[1] = T;
  p[2] = H;
  p[3] = GS;
  p[4] = static_cast<int32_t>(units.size() / kUnitInts);
  p[5] = static_cast<int32_t>(members.size());
  p[6] = ptr[T];
  p[7] = cells;
  p[8] = chunk;
  p[9] = S;
  p[10] = tile_rows;
  p.insert(p.end(), skip.begin(), skip.end());
  p.insert(p.end(), vis.begin(), vis.end());
  p.insert(p.end(), ptr.begin(), ptr.end());
  p.insert(p.end(), units.begin(), units.end());
  p.insert(p.end(), members.begin(), members.end());
  p.insert(p.end(), list.begin(), list.end());
}

bool prefill_plan_check(const int32_t* p, size_t n, int32_t T, int32_t S, int32_t max_blocks,
                        int32_t max_ctx, int32_t H, int32_t GS, int32_t max_tile_rows,
                        int32_t max_chunk, PlanView* v) {
  if (n < static_cast<size_t>(kPlanHeader) || p[0] != kPrefillMagic || p[1] != T || p[2] != H ||
      p[3] != GS || p[9] != S)
    return false;
  const int64_t U = p[4], M = p[5], L = p[6], cells = p[7], chunk = p[8], rows = p[10];
  if (U < 0 || M < 0 || L < 0 || cells < 0 || chunk <= 0 || chunk > max_chunk || rows <= 0 ||
      rows > max_tile_rows)
    return false;
  const int64_t need = kPlanHeader + 3 * static_cast<int64_t>(T) + 1 + U * kUnitInts + M + L;
  if (static_cast<int64_t>(n) != need || cells > (int64_t{1} << 30)) return false;
  const int32_t* skip = p + kPlanHeader;
  const int32_t* vis = skip + T;
  const int32_t* ptr = vis + T;
  const int32_t* units = ptr + T + 1;
  const int32_t* members = units + U * kUnitInts;
  const int32_t* list = members + M;
  for (int32_t r = 0; r < T; ++r) {
    if (skip[r] < 0 || skip[r] > 1 || vis[r] < 1 || vis[r] > max_ctx || ptr[r + 1] < ptr[r])
      return false;
  }
  if (ptr[0] != 0 || ptr[T] != L) return false;
  for (int64_t u = 0; u < U; ++u) {
    const int32_t* e = units + u * kUnitInts;
    if (e[0] < 0 || e[0] >= S || e[1] < 0 || e[1] >= e[2] || e[2] > max_blocks ||
        e[2] - e[1] > chunk)
      return false;
    if (e[3] < 0 || e[4] < 1 || e[4] > rows || static_cast<int64_t>(e[3]) + e[4] > M) return false;
    if (e[5] < -1 || (e[5] >= 0 && static_cast<int64_t>(e[5]) + static_cast<int64_t>(e[4]) * H > cells))
      return false;
  }
  for (int64_t k = 0; k < M; ++k)
    if (members[k] < 0 || members[k] >= T) return false;
  for (int64_t k = 0; k < L; ++k)
    if (list[k] < 0 || static_cast<int64_t>(list[k]) + H > cells) return false;
  v->U = static_cast<int32_t>(U);
  v->cells = static_cast<int32_t>(cells);
  v->has_shared = L > 0;
  return true;
}

}  // namespace pkv
