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
//  * the prefix cache: full blocks of a common prompt prefix stay cached, kept
//    out of the free pool, and later requests with that prefix take them
//    instead of computing it ("vLLM：把 KV 缓存当成虚拟内存", sections
//    "碎片从哪里来" and "KV 的体积从哪来，页表如何把它切开"; "放下账簿，打开源码",
//    section "写时复制与前缀缓存"); when memory runs out cached blocks are dropped
//    least recently used first ("第 6 章 缓存管理", section "缓存放不下的时候").
//
// Policy choices the pages leave open: FIFO free pool (pop front, push back in
// logical order on release); all-or-nothing appends; at most one CoW copy per
// append (only the first written position can fall in an existing block).
// Prefix cache: only full blocks whose token ids are known are cached, keyed
// by the whole token prefix up to the block's end (a chained 64-bit hash, with
// the block's own tokens and its parent's hash kept and compared on a hit);
// the first registration of a prefix stays; a lookup takes cached blocks from
// the start of the prompt up to the first miss and leaves at least one token;
// released cached blocks enter a least-recently-used list from the sequence's
// last block to its first; new blocks come from the free pool, else by
// evicting the least recently used cached block; a cached block is never
// written (an append into one copies it first).
//
//  * swapping: a preempted sequence's KV moves to host memory and back block
//    by block, not as one contiguous buffer ("vLLM：把 KV 缓存当成虚拟内存",
//    section "碎片从哪里来"; "第 6 章 缓存管理", section "缓存放不下的时候").
//    Choices: a host pool of its own with a FIFO free list; swap-out moves the
//    blocks only this sequence holds (refcount 1) and releases them, keeping
//    its references to shared blocks on the device; swap-in takes device
//    blocks the way an append does; both are all or nothing; a swapped-out
//    sequence can only be swapped in or freed.
//
//  * sliding window: with a window of W positions the newest token and every
//    later one attend only positions >= len - W, so blocks wholly below that
//    are released and leave a hole (PA_NO_BLOCK) in the table, which keeps
//    its length ("vLLM：把 KV 缓存当成虚拟内存": sliding windows change how long
//    K/V live).  Holes are skipped everywhere; a fork copies them; a prefix
//    that includes one cannot be shared.
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
    std::vector<int32_t> tokens;  // known token ids of positions 0 .. tokens.size()-1
    std::vector<uint64_t> hashes;  // chain hash of each leading full known block
    bool swapped = false;          // table entries < 0 are host blocks -(h + 1)
  };
  std::unordered_map<int64_t, Seq> seqs;
  int64_t next_id = 0;
  int64_t lazy_allocs = 0;
  int64_t cow_copies = 0;

  // prefix cache
  bool caching = false;
  std::unordered_map<uint64_t, int32_t> index;  // prefix hash -> cached block
  std::vector<char> cached;                     // per block
  std::vector<uint64_t> key_of, parent_of;      // per cached block
  std::vector<std::vector<int32_t>> tokens_of;  // per cached block
  std::vector<int32_t> lru_prev, lru_next;      // evictable blocks, head = least recent
  std::vector<char> in_lru;
  int32_t lru_head = -1, lru_tail = -1, lru_size = 0;
  int64_t lookup_tokens = 0, hit_tokens = 0, evictions = 0;
  // swapping
  int32_t num_host_blocks = 0;  // 0: swap off
  std::deque<int32_t> host_free;
  int64_t swap_outs = 0, swap_ins = 0, blocks_out = 0, blocks_in = 0;
  int32_t swapped_seqs = 0;
};

namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- prefix cache
constexpr uint64_t kRootHash = 0x9E3779B97F4A7C15ull;

inline uint64_t mix64(uint64_t x) {  // splitmix64 finaliser
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

// Hash of a block's prefix: its parent's hash and the block's token ids.
uint64_t chain_hash(uint64_t parent, const int32_t* tok, int32_t bs) {
  uint64_t h = mix64(parent);
  for (int32_t i = 0; i < bs; ++i) h = mix64(h ^ (uint64_t)(uint32_t)tok[i]);
  return h;
}

void lru_push_back(pa_alloc* a, int32_t b) {
  a->lru_prev[b] = a->lru_tail;
  a->lru_next[b] = -1;
  if (a->lru_tail >= 0) a->lru_next[a->lru_tail] = b; else a->lru_head = b;
  a->lru_tail = b;
  a->in_lru[b] = 1;
  a->lru_size += 1;
}

void lru_remove(pa_alloc* a, int32_t b) {
  const int32_t p = a->lru_prev[b], n = a->lru_next[b];
  if (p >= 0) a->lru_next[p] = n; else a->lru_head = n;
  if (n >= 0) a->lru_prev[n] = p; else a->lru_tail = p;
  a->in_lru[b] = 0;
  a->lru_size -= 1;
}

inline int64_t available(const pa_alloc* a) {
  return (int64_t)a->free_pool.size() + a->lru_size;
}

// A block for new data: free pool front, else evict the least recently used
// cached block (its registration goes).  The caller checked available().
int32_t take_block(pa_alloc* a) {
  if (!a->free_pool.empty()) {
    const int32_t b = a->free_pool.front();
    a->free_pool.pop_front();
    return b;
  }
  const int32_t b = a->lru_head;
  lru_remove(a, b);
  a->index.erase(a->key_of[b]);
  a->cached[b] = 0;
  a->tokens_of[b].clear();
  a->tokens_of[b].shrink_to_fit();
  a->evictions += 1;
  return b;
}

// Cache every full block of `s` whose token ids are all known.
void register_blocks(pa_alloc* a, pa_alloc::Seq& s) {
  if (!a->caching) return;
  const int32_t bs = a->block_size;
  const int64_t full = std::min<int64_t>(s.len, (int64_t)s.tokens.size()) / bs;
  for (int64_t j = (int64_t)s.hashes.size(); j < full; ++j) {
    const uint64_t parent = j ? s.hashes[j - 1] : kRootHash;
    const int32_t* tok = s.tokens.data() + j * bs;
    const uint64_t h = chain_hash(parent, tok, bs);
    s.hashes.push_back(h);
    const int32_t b = s.table[j];
    if (b == PA_NO_BLOCK || a->cached[b] || a->index.count(h)) continue;
    a->index.emplace(h, b);
    a->cached[b] = 1;
    a->key_of[b] = h;
    a->parent_of[b] = parent;
    a->tokens_of[b].assign(tok, tok + bs);
  }
}

// Drops one reference from each block of a released table.  Blocks that
// reach zero go to the back of the free pool in logical order if uncached;
// cached ones enter the LRU list from the table's last block to its first, so
// a sequence's first blocks are its most recently used.
void release_blocks(pa_alloc* a, const std::vector<int32_t>& released) {
  for (int32_t b : released)
    if (!a->cached[b]) a->free_pool.push_back(b);
  for (auto it = released.rbegin(); it != released.rend(); ++it)
    if (a->cached[*it]) lru_push_back(a, *it);
}

void release_table(pa_alloc* a, const std::vector<int32_t>& table) {
  std::vector<int32_t> released;
  for (int32_t b : table)
    if (b != PA_NO_BLOCK && --a->refcount[b] == 0) released.push_back(b);
  release_blocks(a, released);
}

// A resident sequence, or the status that says why not.
pa_status find_resident(pa_alloc* a, int64_t seq, pa_alloc::Seq** out) {
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
  if (it->second.swapped) return PA_ERR_SWAPPED;
  *out = &it->second;
  return PA_OK;
}

// Blocks an append of n tokens to `s` needs: fresh blocks for the positions
// that start a logical block, plus one if the first position lands in a
// shared block.
struct AppendPlan {
  int64_t new_blocks;
  bool cow;
};

// The first written position falls in an existing block that must not be
// written in place: shared (refcount > 1) or cached.
inline bool must_copy(const pa_alloc* a, int32_t b, int32_t refcount) {
  return refcount > 1 || a->cached[b];
}

AppendPlan plan_append(const pa_alloc* a, const pa_alloc::Seq& s, int32_t n) {
  AppendPlan p{0, false};
  if (n <= 0) return p;
  const int64_t bs = a->block_size;
  const int64_t start = s.len, end = start + n;
  if (start % bs != 0) {
    const int32_t last = s.table[start / bs];
    p.cow = must_copy(a, last, a->refcount[last]);
  }
  p.new_blocks = ceil_div(end, bs) - ceil_div(start, bs);
  return p;
}

// Carries out a planned append (the caller checked the free pool).  A copied
// cached block whose last holder this was becomes evictable, or, with `held`,
// is put aside for the caller to make evictable later.
void do_append(pa_alloc* a, pa_alloc::Seq& s, int32_t n, int64_t* slots, int32_t* pair,
               int32_t* num_pair, std::vector<int32_t>* held = nullptr) {
  const int32_t bs = a->block_size;
  const int64_t start = s.len, end = start + n;
  *num_pair = 0;
  if (n <= 0) return;
  if (start % bs != 0) {
    int32_t& last = s.table[start / bs];
    if (must_copy(a, last, a->refcount[last])) {
      const int32_t src = last;
      const int32_t dst = take_block(a);
      pair[0] = src;
      pair[1] = dst;
      *num_pair = 1;
      if (--a->refcount[src] == 0) {  // a cached block's last holder
        if (held) held->push_back(src); else lru_push_back(a, src);
      }
      a->refcount[dst] = 1;
      last = dst;
      a->cow_copies += 1;
    }
  }
  for (int64_t pos = start; pos < end; ++pos) {
    if (pos % bs == 0) {
      const int32_t b = take_block(a);
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
  a->cached.assign(num_blocks, 0);
  a->key_of.assign(num_blocks, 0);
  a->parent_of.assign(num_blocks, 0);
  a->tokens_of.resize(num_blocks);
  a->lru_prev.assign(num_blocks, -1);
  a->lru_next.assign(num_blocks, -1);
  a->in_lru.assign(num_blocks, 0);
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
  if (it->second.swapped) return PA_ERR_SWAPPED;
  if ((int64_t)it->second.len + n_tokens > INT32_MAX) return PA_ERR_ARG;
  const AppendPlan p = plan_append(a, it->second, n_tokens);
  if (p.new_blocks + (p.cow ? 1 : 0) > available(a)) return PA_ERR_OOM;
  do_append(a, it->second, n_tokens, slots_out, cow_pair_out, num_cow_out);
  return PA_OK;
}

pa_status pa_seq_append_tokens(pa_alloc* a, int64_t seq, const int32_t* tokens, int32_t n_tokens,
                               int64_t* slots_out, int32_t* cow_pair_out, int32_t* num_cow_out) {
  if (!a || n_tokens < 0 || (n_tokens > 0 && !tokens)) return PA_ERR_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
  if (it->second.swapped) return PA_ERR_SWAPPED;
  const int32_t before = it->second.len;
  const pa_status st = pa_seq_append(a, seq, n_tokens, slots_out, cow_pair_out, num_cow_out);
  if (st != PA_OK) return st;
  pa_alloc::Seq& s = a->seqs.find(seq)->second;
  if ((int64_t)s.tokens.size() == before) s.tokens.insert(s.tokens.end(), tokens, tokens + n_tokens);
  register_blocks(a, s);
  return PA_OK;
}

pa_status pa_alloc_enable_prefix_cache(pa_alloc* a) {
  if (!a || !a->seqs.empty()) return PA_ERR_ARG;
  a->caching = true;
  return PA_OK;
}

pa_status pa_seq_create_prefix(pa_alloc* a, const int32_t* tokens, int32_t n_tokens,
                               int64_t* seq_out, int32_t* hit_tokens_out) {
  if (!a || !seq_out || !hit_tokens_out || n_tokens < 0 || (n_tokens > 0 && !tokens) ||
      !a->caching)
    return PA_ERR_ARG;
  const int32_t bs = a->block_size;
  pa_alloc::Seq s;
  uint64_t parent = kRootHash;
  const int64_t max_blocks = n_tokens > 0 ? (int64_t)(n_tokens - 1) / bs : 0;
  for (int64_t j = 0; j < max_blocks; ++j) {
    const int32_t* tok = tokens + j * bs;
    const uint64_t h = chain_hash(parent, tok, bs);
    auto hit = a->index.find(h);
    if (hit == a->index.end()) break;
    const int32_t b = hit->second;
    if (a->parent_of[b] != parent || !std::equal(tok, tok + bs, a->tokens_of[b].begin())) break;
    if (a->refcount[b] == 0) lru_remove(a, b);
    a->refcount[b] += 1;
    s.table.push_back(b);
    s.hashes.push_back(h);
    parent = h;
  }
  s.len = (int32_t)(s.table.size() * bs);
  s.tokens.assign(tokens, tokens + s.len);
  a->lookup_tokens += n_tokens;
  a->hit_tokens += s.len;
  const int64_t id = a->next_id++;
  *hit_tokens_out = s.len;
  a->seqs.emplace(id, std::move(s));
  *seq_out = id;
  return PA_OK;
}

pa_status pa_prefix_cache_stats(const pa_alloc* a, pa_prefix_stats* out) {
  if (!a || !out) return PA_ERR_ARG;
  out->lookup_tokens = a->lookup_tokens;
  out->hit_tokens = a->hit_tokens;
  out->evictions = a->evictions;
  int32_t cached = 0, pinned = 0;
  for (int32_t b = 0; b < a->num_blocks; ++b) {
    cached += a->cached[b];
    pinned += a->cached[b] && a->refcount[b] > 0;
  }
  out->cached_blocks = cached;
  out->evictable_blocks = a->lru_size;
  out->pinned_blocks = pinned;
  return PA_OK;
}

pa_status pa_prefix_cache_query(const pa_alloc* a, int32_t* evictable_out, int32_t* num_out) {
  if (!a) return PA_ERR_ARG;
  if (num_out) *num_out = a->lru_size;
  if (evictable_out)
    for (int32_t b = a->lru_head, k = 0; b >= 0; b = a->lru_next[b]) evictable_out[k++] = b;
  return PA_OK;
}

pa_status pa_alloc_enable_swap(pa_alloc* a, int32_t num_host_blocks) {
  if (!a || num_host_blocks <= 0 || a->num_host_blocks > 0) return PA_ERR_ARG;
  a->num_host_blocks = num_host_blocks;
  for (int32_t h = 0; h < num_host_blocks; ++h) a->host_free.push_back(h);
  return PA_OK;
}

pa_status pa_seq_swap_out(pa_alloc* a, int64_t seq, int32_t* pairs_out, int32_t capacity,
                          int32_t* num_pairs_out) {
  if (!a || !num_pairs_out || capacity < 0 || (capacity > 0 && !pairs_out) ||
      a->num_host_blocks == 0)
    return PA_ERR_ARG;
  pa_alloc::Seq* s = nullptr;
  const pa_status st = find_resident(a, seq, &s);
  if (st != PA_OK) return st;
  int64_t own = 0;
  for (int32_t b : s->table) own += b != PA_NO_BLOCK && a->refcount[b] == 1;
  if (own > capacity) return PA_ERR_ARG;
  if (own > (int64_t)a->host_free.size()) return PA_ERR_OOM;
  std::vector<int32_t> released;
  int32_t np = 0;
  for (int32_t& b : s->table) {
    if (b == PA_NO_BLOCK || a->refcount[b] != 1) continue;  // shared: stays on the device
    const int32_t h = a->host_free.front();
    a->host_free.pop_front();
    pairs_out[2 * np] = b;
    pairs_out[2 * np + 1] = h;
    ++np;
    a->refcount[b] = 0;
    released.push_back(b);
    b = -h - 1;
  }
  release_blocks(a, released);
  s->swapped = true;
  a->swapped_seqs += 1;
  a->swap_outs += 1;
  a->blocks_out += np;
  *num_pairs_out = np;
  return PA_OK;
}

pa_status pa_seq_swap_in(pa_alloc* a, int64_t seq, int32_t* pairs_out, int32_t capacity,
                         int32_t* num_pairs_out) {
  if (!a || !num_pairs_out || capacity < 0 || (capacity > 0 && !pairs_out)) return PA_ERR_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
  pa_alloc::Seq& s = it->second;
  if (!s.swapped) return PA_ERR_ARG;
  int64_t on_host = 0;
  for (int32_t b : s.table) on_host += b < 0 && b != PA_NO_BLOCK;
  if (on_host > capacity) return PA_ERR_ARG;
  if (on_host > available(a)) return PA_ERR_OOM;
  std::vector<int32_t> hosts;
  int32_t np = 0;
  for (int32_t& b : s.table) {
    if (b >= 0 || b == PA_NO_BLOCK) continue;
    const int32_t h = -b - 1;
    const int32_t d = take_block(a);
    a->refcount[d] = 1;
    pairs_out[2 * np] = h;
    pairs_out[2 * np + 1] = d;
    ++np;
    hosts.push_back(h);
    b = d;
  }
  for (int32_t h : hosts) a->host_free.push_back(h);
  s.swapped = false;
  a->swapped_seqs -= 1;
  a->swap_ins += 1;
  a->blocks_in += np;
  *num_pairs_out = np;
  return PA_OK;
}

pa_status pa_swap_query(const pa_alloc* a, pa_swap_stats* stats, int32_t* host_free_out) {
  if (!a) return PA_ERR_ARG;
  if (stats) {
    stats->swap_outs = a->swap_outs;
    stats->swap_ins = a->swap_ins;
    stats->blocks_out = a->blocks_out;
    stats->blocks_in = a->blocks_in;
    stats->swapped_seqs = a->swapped_seqs;
    stats->host_free = (int32_t)a->host_free.size();
  }
  if (host_free_out) std::copy(a->host_free.begin(), a->host_free.end(), host_free_out);
  return PA_OK;
}

pa_status pa_seq_append_batch(pa_alloc* a, const int64_t* seqs, int32_t n, int32_t n_tokens,
                              int64_t* slots_out, int32_t* pairs_out, int32_t* num_pairs_out,
                              int32_t* lens_out) {
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
    if (it->second.swapped) return PA_ERR_SWAPPED;
    for (int32_t j = 0; j < i; ++j)
      if (seqs[j] == seqs[i]) return PA_ERR_ARG;  // one append per sequence per step
    if ((int64_t)it->second.len + n_tokens > INT32_MAX) return PA_ERR_ARG;
    ptrs[i] = &it->second;
  }
  // Each append must fit what is available when it runs, as if the appends
  // were made one by one.  The step's copies run together in one launch, so
  // a copied cached block whose last holder wrote is held back until the
  // step's last append (it must not become a later copy's destination while
  // its own copy reads it) and does not count as available meanwhile.
  int64_t avail = available(a);
  std::unordered_map<int32_t, int32_t> drops;  // block -> refcount drops so far
  const int64_t bs = a->block_size;
  for (int32_t i = 0; i < n && n_tokens > 0; ++i) {
    const pa_alloc::Seq& s = *ptrs[i];
    const int64_t start = s.len, end = start + n_tokens;
    int64_t need = ceil_div(end, bs) - ceil_div(start, bs);
    if (start % bs != 0) {
      const int32_t last = s.table[start / bs];
      const int32_t rc = a->refcount[last] - drops[last];
      if (must_copy(a, last, rc)) {
        need += 1;
        drops[last] += 1;
      }
    }
    if (need > avail) return PA_ERR_OOM;
    avail -= need;
  }
  int32_t np = 0;
  std::vector<int32_t> held;
  for (int32_t i = 0; i < n; ++i) {
    int32_t one = 0;
    do_append(a, *ptrs[i], n_tokens, slots_out + (int64_t)i * n_tokens, pairs_out + 2 * np, &one,
              &held);
    np += one;
  }
  for (int32_t b : held) lru_push_back(a, b);
  *num_pairs_out = np;
  if (lens_out)
    for (int32_t i = 0; i < n; ++i) lens_out[i] = ptrs[i]->len;
  return PA_OK;
}

pa_status pa_seq_fork(pa_alloc* a, int64_t parent, int64_t* child_out) {
  if (!a || !child_out) return PA_ERR_ARG;
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
  if (it->second.swapped) return PA_ERR_SWAPPED;
  pa_alloc::Seq child = it->second;  // copy before emplace (rehash)
  for (int32_t b : child.table)
    if (b != PA_NO_BLOCK) a->refcount[b] += 1;
  const int64_t id = a->next_id++;
  a->seqs.emplace(id, std::move(child));
  *child_out = id;
  return PA_OK;
}

pa_status pa_seq_share_prefix(pa_alloc* a, int64_t src, int32_t n_tokens, int64_t* seq_out) {
  if (!a || !seq_out) return PA_ERR_ARG;
  auto it = a->seqs.find(src);
  if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
  if (it->second.swapped) return PA_ERR_SWAPPED;
  if (n_tokens < 0 || n_tokens > it->second.len) return PA_ERR_ARG;
  pa_alloc::Seq s;
  const pa_alloc::Seq& src_seq = it->second;
  const int64_t k = ceil_div(n_tokens, a->block_size);
  if (std::find(src_seq.table.begin(), src_seq.table.begin() + k, PA_NO_BLOCK) !=
      src_seq.table.begin() + k)
    return PA_ERR_ARG;  // part of the prefix was released by a sliding window
  s.table.assign(src_seq.table.begin(), src_seq.table.begin() + k);
  s.len = n_tokens;
  s.tokens.assign(src_seq.tokens.begin(),
                  src_seq.tokens.begin() + std::min<int64_t>(n_tokens, src_seq.tokens.size()));
  s.hashes.assign(src_seq.hashes.begin(),
                  src_seq.hashes.begin() +
                      std::min<int64_t>(n_tokens / a->block_size, src_seq.hashes.size()));
  for (int32_t b : s.table) a->refcount[b] += 1;
  const int64_t id = a->next_id++;
  a->seqs.emplace(id, std::move(s));
  *seq_out = id;
  return PA_OK;
}

pa_status pa_seq_trim_window(pa_alloc* a, int64_t seq, int32_t window, int32_t* released_out) {
  if (!a || window <= 0) return PA_ERR_ARG;
  pa_alloc::Seq* s = nullptr;
  const pa_status st = find_resident(a, seq, &s);
  if (st != PA_OK) return st;
  const int64_t dead = std::max<int64_t>((int64_t)s->len - window, 0) / a->block_size;
  std::vector<int32_t> released;
  int32_t n = 0;
  for (int64_t j = 0; j < dead; ++j) {
    int32_t& b = s->table[j];
    if (b == PA_NO_BLOCK) continue;
    if (--a->refcount[b] == 0) released.push_back(b);
    b = PA_NO_BLOCK;
    ++n;
  }
  release_blocks(a, released);
  if (released_out) *released_out = n;
  return PA_OK;
}

pa_status pa_seq_free(pa_alloc* a, int64_t seq) {
  if (!a) return PA_ERR_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
  for (int32_t b : it->second.table)
    if (b >= 0 && a->refcount[b] <= 0) return PA_ERR_REFCOUNT;  // holes and host entries are < 0
  if (it->second.swapped) {
    // host blocks back to the host list, device references dropped
    std::vector<int32_t> released;
    for (int32_t b : it->second.table) {
      if (b == PA_NO_BLOCK) continue;
      if (b < 0)
        a->host_free.push_back(-b - 1);
      else if (--a->refcount[b] == 0)
        released.push_back(b);
    }
    release_blocks(a, released);
    a->swapped_seqs -= 1;
  } else {
    release_table(a, it->second.table);
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
    if (it->second.swapped) return PA_ERR_SWAPPED;
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
  std::vector<char> host_seen(a->num_host_blocks, 0);
  for (const auto& kv : a->seqs) {
    const auto& s = kv.second;
    if ((int64_t)s.table.size() != ceil_div(s.len, a->block_size)) return PA_ERR_REFCOUNT;
    for (int32_t b : s.table) {
      if (b == PA_NO_BLOCK) continue;
      if (b < 0 && s.swapped) {
        const int32_t h = -b - 1;
        if (h >= a->num_host_blocks || host_seen[h]) return PA_ERR_REFCOUNT;
        host_seen[h] = 1;
        continue;
      }
      if (b < 0 || b >= a->num_blocks) return PA_ERR_REFCOUNT;
      indeg[b] += 1;
    }
  }
  if (indeg != a->refcount) return PA_ERR_REFCOUNT;
  for (int32_t h : a->host_free) {
    if (h < 0 || h >= a->num_host_blocks || host_seen[h]) return PA_ERR_REFCOUNT;
    host_seen[h] = 1;
  }
  for (char c : host_seen)
    if (!c) return PA_ERR_REFCOUNT;
  std::vector<char> in_free(a->num_blocks, 0);
  for (int32_t b : a->free_pool) {
    if (b < 0 || b >= a->num_blocks || in_free[b]) return PA_ERR_REFCOUNT;
    in_free[b] = 1;
  }
  int32_t lru = 0;
  for (int32_t b = a->lru_head, prev = -1; b >= 0; prev = b, b = a->lru_next[b]) {
    if (!a->in_lru[b] || a->lru_prev[b] != prev || ++lru > a->num_blocks) return PA_ERR_REFCOUNT;
  }
  if (lru != a->lru_size) return PA_ERR_REFCOUNT;
  int32_t cached = 0;
  for (int32_t b = 0; b < a->num_blocks; ++b) {
    const bool idle = a->refcount[b] == 0;
    if ((bool)in_free[b] != (idle && !a->cached[b])) return PA_ERR_REFCOUNT;
    if ((bool)a->in_lru[b] != (idle && a->cached[b])) return PA_ERR_REFCOUNT;
    if (a->cached[b]) {
      auto hit = a->index.find(a->key_of[b]);
      if (hit == a->index.end() || hit->second != b) return PA_ERR_REFCOUNT;
      cached += 1;
    }
  }
  if (cached != (int32_t)a->index.size()) return PA_ERR_REFCOUNT;
  return PA_OK;
}

}  // extern "C"
