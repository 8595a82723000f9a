// Host block allocator of libpa: lazy block allocation, fork, copy-on-write,
// prefix sharing and release over a FIFO free pool with per-block refcounts.
//
// What it implements (each rule as the pages state it):
//  * lazy allocation -- a physical block is taken only when a position first
//    enters a logical block ("Lazy Allocation 与 Copy-on-Write 在 LLM 推理系统
//    中的应用", section 3.3; "放下账簿，打开源码", section "PagedAttention：
//    虚实分离，按需取用");
//  * fork copies the block table and raises refcounts ("vLLM：把 KV 缓存当成
//    虚拟内存", section "碎片从哪里来");
//  * copy-on-write of a shared block on its first write, the last holder
//    writing in place ("Lazy Allocation 与 Copy-on-Write ...", section 4.4;
//    "放下账簿，打开源码", section "写时复制与前缀缓存");
//  * prefix sharing and release to the free pool at refcount zero ("第 6 章
//    缓存管理：把显存当操作系统来管", section "块表长什么样").
//
// Policy choices the pages leave open: FIFO free pool (pop front, push back in
// logical order on release); all-or-nothing appends; at most one CoW copy per
// append (only the first written position can fall in an existing block).
#include <algorithm>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

struct pa_alloc {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_pool;
  std::vector<int32_t> refcount;
  struct Seq {
    std::vector<int32_t> table;
    int32_t len = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;
  int64_t next_id = 0;
  int64_t lazy_allocs = 0;
  int64_t cow_copies = 0;
};

namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Blocks an append of n tokens to `s` needs: fresh blocks for the positions
// that start a logical block, plus one if the first position lands in a
// shared block.
struct AppendPlan {
  int64_t new_blocks;
  bool cow;
};

AppendPlan plan_append(const pa_alloc* a, const pa_alloc::Seq& s, int32_t n) {
  AppendPlan p{0, false};
  if (n <= 0) return p;
  const int64_t bs = a->block_size;
  const int64_t start = s.len, end = start + n;
  p.cow = (start % bs != 0) && a->refcount[s.table[start / bs]] > 1;
  p.new_blocks = ceil_div(end, bs) - ceil_div(start, bs);
  return p;
}

// Carries out a planned append (the caller checked the free pool).
void do_append(pa_alloc* a, pa_alloc::Seq& s, int32_t n, int64_t* slots, int32_t* pair,
               int32_t* num_pair) {
  const int32_t bs = a->block_size;
  const int64_t start = s.len, end = start + n;
  *num_pair = 0;
  if (n <= 0) return;
  if (start % bs != 0) {
    int32_t& last = s.table[start / bs];
    if (a->refcount[last] > 1) {
      const int32_t dst = a->free_pool.front();
      a->free_pool.pop_front();
      pair[0] = last;
      pair[1] = dst;
      *num_pair = 1;
      a->refcount[last] -= 1;
      a->refcount[dst] = 1;
      last = dst;
      a->cow_copies += 1;
    }
  }
  for (int64_t pos = start; pos < end; ++pos) {
    if (pos % bs == 0) {
      const int32_t b = a->free_pool.front();
      a->free_pool.pop_front();
      a->refcount[b] = 1;
      s.table.push_back(b);
      a->lazy_allocs += 1;
    }
    slots[pos - start] = (int64_t)s.table[pos / bs] * bs + pos % bs;
  }
  s.len = (int32_t)end;
}

}  // namespace

extern "C" {

pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size,
                          const int32_t* initial_free_order, pa_alloc** out) {
  if (!out || num_blocks <= 0 || block_size <= 0) return PA_ERR_ARG;
  *out = nullptr;
  pa_alloc* a = new (std::nothrow) pa_alloc();
  if (!a) return PA_ERR_OOM;
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->refcount.assign(num_blocks, 0);
  if (initial_free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return PA_ERR_ARG;
      }
      seen[b] = 1;
      a->free_pool.push_back(b);
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->free_pool.push_back(i);
  }
  *out = a;
  return PA_OK;
}

void pa_alloc_destroy(pa_alloc* a) { delete a; }

pa_status pa_seq_create(pa_alloc* a, int64_t* seq_out) {
  if (!a || !seq_out) return PA_ERR_ARG;
  const int64_t id = a->next_id++;
  a->seqs.emplace(id, pa_alloc::Seq{});
  *seq_out = id;
  return PA_OK;
}

pa_status pa_seq_append(pa_alloc* a, int64_t seq, int32_t n_tokens, int64_t* slots_out,
                        int32_t* cow_pair_out, int32_t* num_cow_out) {
  if (!a || n_tokens < 0 || (n_tokens > 0 && !slots_out) || !cow_pair_out || !num_cow_out)
    return PA_ERR_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
  if ((int64_t)it->second.len + n_tokens > INT32_MAX) return PA_ERR_ARG;
  const AppendPlan p = plan_append(a, it->second, n_tokens);
  if (p.new_blocks + (p.cow ? 1 : 0) > (int64_t)a->free_pool.size()) return PA_ERR_OOM;
  do_append(a, it->second, n_tokens, slots_out, cow_pair_out, num_cow_out);
  return PA_OK;
}

pa_status pa_seq_append_batch(pa_alloc* a, const int64_t* seqs, int32_t n, int32_t n_tokens,
                              int64_t* slots_out, int32_t* pairs_out, int32_t* num_pairs_out) {
  if (!a || n < 0 || n_tokens < 0 || (n > 0 && (!seqs || !pairs_out)) || !num_pairs_out ||
      (n > 0 && n_tokens > 0 && !slots_out))
    return PA_ERR_ARG;
  *num_pairs_out = 0;
  // Plan first so a failure changes nothing.  Appends to distinct sequences
  // are independent except through refcounts of blocks they share: a later
  // writer of a block an earlier writer already copied may find it unshared.
  // Simulate refcount drops of the copies to count exactly.
  std::vector<pa_alloc::Seq*> ptrs(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seqs[i]);
    if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
    for (int32_t j = 0; j < i; ++j)
      if (seqs[j] == seqs[i]) return PA_ERR_ARG;  // one append per sequence per step
    if ((int64_t)it->second.len + n_tokens > INT32_MAX) return PA_ERR_ARG;
    ptrs[i] = &it->second;
  }
  int64_t need = 0;
  std::unordered_map<int32_t, int32_t> drops;  // block -> refcount drops so far
  const int64_t bs = a->block_size;
  for (int32_t i = 0; i < n && n_tokens > 0; ++i) {
    const pa_alloc::Seq& s = *ptrs[i];
    const int64_t start = s.len, end = start + n_tokens;
    need += ceil_div(end, bs) - ceil_div(start, bs);
    if (start % bs != 0) {
      const int32_t last = s.table[start / bs];
      const int32_t rc = a->refcount[last] - drops[last];
      if (rc > 1) {
        need += 1;
        drops[last] += 1;
      }
    }
  }
  if (need > (int64_t)a->free_pool.size()) return PA_ERR_OOM;
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t one = 0;
    do_append(a, *ptrs[i], n_tokens, slots_out + (int64_t)i * n_tokens, pairs_out + 2 * np, &one);
    np += one;
  }
  *num_pairs_out = np;
  return PA_OK;
}

pa_status pa_seq_fork(pa_alloc* a, int64_t parent, int64_t* child_out) {
  if (!a || !child_out) return PA_ERR_ARG;
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
  pa_alloc::Seq child = it->second;  // copy before emplace (rehash)
  for (int32_t b : child.table) a->refcount[b] += 1;
  const int64_t id = a->next_id++;
  a->seqs.emplace(id, std::move(child));
  *child_out = id;
  return PA_OK;
}

pa_status pa_seq_share_prefix(pa_alloc* a, int64_t src, int32_t n_tokens, int64_t* seq_out) {
  if (!a || !seq_out) return PA_ERR_ARG;
  auto it = a->seqs.find(src);
  if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
  if (n_tokens < 0 || n_tokens > it->second.len) return PA_ERR_ARG;
  pa_alloc::Seq s;
  const int64_t k = ceil_div(n_tokens, a->block_size);
  s.table.assign(it->second.table.begin(), it->second.table.begin() + k);
  s.len = n_tokens;
  for (int32_t b : s.table) a->refcount[b] += 1;
  const int64_t id = a->next_id++;
  a->seqs.emplace(id, std::move(s));
  *seq_out = id;
  return PA_OK;
}

pa_status pa_seq_free(pa_alloc* a, int64_t seq) {
  if (!a) return PA_ERR_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
  for (int32_t b : it->second.table)
    if (a->refcount[b] <= 0) return PA_ERR_REFCOUNT;
  for (int32_t b : it->second.table) {
    if (--a->refcount[b] == 0) a->free_pool.push_back(b);
  }
  a->seqs.erase(it);
  return PA_OK;
}

pa_status pa_seq_info(const pa_alloc* a, int64_t seq, int32_t* len_out, int32_t* table_out,
                      int32_t capacity, int32_t* num_blocks_out) {
  if (!a) return PA_ERR_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
  const auto& t = it->second.table;
  if (len_out) *len_out = it->second.len;
  if (num_blocks_out) *num_blocks_out = (int32_t)t.size();
  if (table_out) {
    if ((int64_t)t.size() > capacity) return PA_ERR_ARG;
    std::copy(t.begin(), t.end(), table_out);
  }
  return PA_OK;
}

pa_status pa_build_tables(const pa_alloc* a, const int64_t* seqs, int32_t n, int32_t max_blocks,
                          int32_t* tables_out, int32_t* lens_out) {
  if (!a || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !lens_out)) ||
      (n > 0 && max_blocks > 0 && !tables_out))
    return PA_ERR_ARG;
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seqs[i]);
    if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
    if ((int64_t)it->second.table.size() > max_blocks) return PA_ERR_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& s = a->seqs.find(seqs[i])->second;
    int32_t* row = tables_out + (int64_t)i * max_blocks;
    std::copy(s.table.begin(), s.table.end(), row);
    std::fill(row + s.table.size(), row + max_blocks, -1);
    lens_out[i] = s.len;
  }
  return PA_OK;
}

pa_status pa_alloc_query(const pa_alloc* a, int32_t* num_free, int32_t* free_list_out,
                         int32_t* refcounts_out) {
  if (!a) return PA_ERR_ARG;
  if (num_free) *num_free = (int32_t)a->free_pool.size();
  if (free_list_out) std::copy(a->free_pool.begin(), a->free_pool.end(), free_list_out);
  if (refcounts_out) std::copy(a->refcount.begin(), a->refcount.end(), refcounts_out);
  return PA_OK;
}

pa_status pa_alloc_stats(const pa_alloc* a, int64_t* lazy_allocs, int64_t* cow_copies,
                         int32_t* live_seqs, int32_t* shared_blocks) {
  if (!a) return PA_ERR_ARG;
  if (lazy_allocs) *lazy_allocs = a->lazy_allocs;
  if (cow_copies) *cow_copies = a->cow_copies;
  if (live_seqs) *live_seqs = (int32_t)a->seqs.size();
  if (shared_blocks) {
    int32_t c = 0;
    for (int32_t r : a->refcount) c += r > 1;
    *shared_blocks = c;
  }
  return PA_OK;
}

pa_status pa_alloc_check_invariants(const pa_alloc* a) {
  if (!a) return PA_ERR_ARG;
  std::vector<int32_t> indeg(a->num_blocks, 0);
  for (const auto& kv : a->seqs) {
    const auto& s = kv.second;
    if ((int64_t)s.table.size() != ceil_div(s.len, a->block_size)) return PA_ERR_REFCOUNT;
    for (int32_t b : s.table) {
      if (b < 0 || b >= a->num_blocks) return PA_ERR_REFCOUNT;
      indeg[b] += 1;
    }
  }
  if (indeg != a->refcount) return PA_ERR_REFCOUNT;
  std::vector<char> in_free(a->num_blocks, 0);
  for (int32_t b : a->free_pool) {
    if (b < 0 || b >= a->num_blocks || in_free[b]) return PA_ERR_REFCOUNT;
    in_free[b] = 1;
  }
  for (int32_t b = 0; b < a->num_blocks; ++b)
    if ((bool)in_free[b] != (a->refcount[b] == 0)) return PA_ERR_REFCOUNT;
  return PA_OK;
}

}  // extern "C"
