// pkv_host.cpp — host half of libpkv: status strings, sizing, and the block
// pool with per-sequence block tables.
//
// The pool follows the paging scheme of "LLM Primer VI, Capítulo 8 — Gestión
// de caché KV de nueva generación" §8.1 (fixed blocks in one flat pool, a
// table per sequence from logical to physical block, refcounted sharing for
// branching), the on-demand growth and copy-on-write of "KV Cache y
// PagedAttention: por qué se reduce la velocidad de tu servidor LLM", and the
// release-on-cancel rule of "PagedAttention y Gestión de KV-Cache" §4.02.
// No HIP here: this file is plain C++17 and runs without a GPU.
#include <algorithm>
#include <atomic>
#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

#include "pkv.h"

extern "C" const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported layout or shape";
    case PKV_ERR_NO_FREE_BLOCKS: return "no free cache blocks";
    case PKV_ERR_HIP: return "HIP launch failed";
    case PKV_ERR_WORKSPACE: return "workspace too small";
    case PKV_ERR_BAD_HANDLE: return "unknown pool or sequence";
    case PKV_ERR_REFCOUNT: return "block reference count underflow";
    default: return "unknown status";
  }
}

// ------------------------------------------------------------------ sizing

// 2 (K and V) x layers x KV heads x head dim x element bytes: the formula of
// "Optimización de KV Cache con PagedAttention y Cuantización FP8 ...", §2.
extern "C" uint64_t pkv_bytes_per_token(int32_t n_layers, int32_t n_kv_heads, int32_t d_head,
                                        int32_t elem_bytes) {
  if (n_layers <= 0 || n_kv_heads <= 0 || d_head <= 0 || elem_bytes <= 0) return 0;
  return 2ull * (uint64_t)n_layers * (uint64_t)n_kv_heads * (uint64_t)d_head *
         (uint64_t)elem_bytes;
}

extern "C" uint64_t pkv_pool_bytes(const pkv_cache_layout* l) {
  if (!l || l->num_blocks <= 0 || l->block_size <= 0 || l->num_kv_heads <= 0 ||
      l->head_dim <= 0)
    return 0;
  uint64_t e;
  if (l->dtype == PKV_F16)
    e = 2;
  else if (l->dtype == PKV_FP8_E4M3FN)
    e = 1;
  else
    return 0;
  return (uint64_t)l->num_blocks * (uint64_t)l->num_kv_heads * (uint64_t)l->block_size *
         (uint64_t)l->head_dim * e;
}

// ----------------------------------------------------- table checks (debug)
//
// The decode kernel takes the block table as an extra input ("LLM Primer VI
// ...", §8.1); a table entry names a physical block of the pool and a length
// may not run past the table.  The kernels clamp lengths and skip ids outside
// the pool; these checks turn such contents into an error instead.

extern "C" pkv_status pkv_validate_tables(const int32_t* block_tables,
                                          int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t max_context_len, int32_t num_blocks,
                                          int32_t* bad_seq_out) {
  if (bad_seq_out) *bad_seq_out = -1;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || num_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!block_tables || !context_lens)) return PKV_ERR_INVALID_ARG;
  const int64_t cap =
      std::min<int64_t>(max_context_len, (int64_t)max_blocks_per_seq * 16);
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t L = context_lens[b];
    bool ok = L >= 0 && L <= cap;
    const int32_t* row = block_tables + (int64_t)b * max_blocks_per_seq;
    for (int64_t j = 0; ok && j < (L + 15) / 16; ++j)
      ok = row[j] >= 0 && row[j] < num_blocks;
    if (!ok) {
      if (bad_seq_out) *bad_seq_out = b;
      return PKV_ERR_INVALID_ARG;
    }
  }
  return PKV_OK;
}

namespace {
std::atomic<int32_t>& debug_checks_flag() {
  static std::atomic<int32_t> flag([] {
    const char* e = std::getenv("PKV_DEBUG_CHECKS");
    return (int32_t)(e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0);
  }());
  return flag;
}
}  // namespace

extern "C" int32_t pkv_set_debug_checks(int32_t on) {
  return debug_checks_flag().exchange(on != 0 ? 1 : 0);
}

extern "C" int32_t pkv_get_debug_checks(void) { return debug_checks_flag().load(); }

// ------------------------------------------------------------- block pool
//
// Reference counts count the sequences whose table holds a block.  Besides
// the sequences, the prefix cache ("LLM Primer VI ...", §8.3: prompts hashed in
// block-sized chunks; a hit points the new table at the cached block and its
// prefill is skipped; a miss is prefilled and then registered) can hold a full
// block.  A block is
//   free       when no sequence holds it and it is not cached,
//   evictable  when no sequence holds it but it is cached,
//   in use     otherwise.
// A new block comes from the free list first, else the least recently used
// evictable block is dropped from the cache and reused.

namespace {

// A sequence's logical blocks: a device block id (>= 0), or a block swapped
// out to host slot k, stored as -(k + 2).
struct Seq {
  std::vector<int32_t> blocks;
  int64_t len = 0;
  int32_t swapped = 0;  // blocks now in host slots
};

inline int32_t host_code(int32_t slot) { return -slot - 2; }
inline int32_t host_slot(int32_t code) { return -code - 2; }

struct CacheEntry {
  int32_t block;
  uint64_t parent;              // key of the previous chunk (0 for the first)
  std::vector<int32_t> tokens;  // the chunk, to verify a key match
  uint64_t tick;                // last hit or registration
};

uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Key of a chunk of block_size token ids chained onto its parent's key.
uint64_t chunk_key(uint64_t parent, const int32_t* tokens, int32_t n) {
  uint64_t h = parent ^ 0x243F6A8885A308D3ull;
  for (int32_t i = 0; i < n; ++i) {
    uint64_t x = h ^ (uint64_t)(uint32_t)tokens[i];
    h = splitmix64(x);
  }
  return h == 0 ? 1 : h;  // 0 is reserved for "no parent"
}

}  // namespace

struct pkv_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;  // popped at the front, returned at the back
  std::vector<int32_t> ref;       // sequences holding each block
  std::unordered_map<int32_t, Seq> seqs;
  int32_t next_id = 0;
  // prefix cache
  std::unordered_map<uint64_t, CacheEntry> cache;
  std::vector<uint64_t> cache_key;                  // per block, 0 = not cached
  std::set<std::pair<uint64_t, int32_t>> evictable;  // (tick, block), LRU first
  uint64_t tick = 0;
  int64_t hit_blocks = 0, miss_blocks = 0;
  // swap space: host slots for swapped-out blocks
  int32_t num_host = 0;
  std::deque<int32_t> host_free;

  int64_t available() const { return (int64_t)free_list.size() + (int64_t)evictable.size(); }

  // A block for a sequence (the caller has checked available()).
  int32_t take() {
    int32_t b;
    if (!free_list.empty()) {
      b = free_list.front();
      free_list.pop_front();
    } else {
      auto it = evictable.begin();
      b = it->second;
      evictable.erase(it);
      cache.erase(cache_key[(size_t)b]);
      cache_key[(size_t)b] = 0;
    }
    ref[(size_t)b] += 1;
    return b;
  }

  void acquire(int32_t b) {  // one more sequence holds b
    if (ref[(size_t)b] == 0 && cache_key[(size_t)b] != 0)
      evictable.erase({cache.at(cache_key[(size_t)b]).tick, b});
    ref[(size_t)b] += 1;
  }

  void release(int32_t b) {  // one sequence fewer holds b
    if (--ref[(size_t)b] > 0) return;
    if (cache_key[(size_t)b] != 0)
      evictable.insert({cache.at(cache_key[(size_t)b]).tick, b});
    else
      free_list.push_back(b);
  }
};

extern "C" pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size,
                                      uint64_t shuffle_seed, pkv_pool** out) {
  if (!out || num_blocks <= 0 || block_size <= 0) return PKV_ERR_INVALID_ARG;
  pkv_pool* p = new (std::nothrow) pkv_pool();
  if (!p) return PKV_ERR_INVALID_ARG;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->ref.assign((size_t)num_blocks, 0);
  p->cache_key.assign((size_t)num_blocks, 0);
  std::vector<int32_t> order((size_t)num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) order[(size_t)i] = i;
  if (shuffle_seed != 0) {  // Fisher-Yates with a splitmix64 stream
    uint64_t s = shuffle_seed;
    for (int32_t i = num_blocks - 1; i > 0; --i) {
      int32_t j = (int32_t)(splitmix64(s) % (uint64_t)(i + 1));
      std::swap(order[(size_t)i], order[(size_t)j]);
    }
  }
  p->free_list.assign(order.begin(), order.end());
  *out = p;
  return PKV_OK;
}

extern "C" void pkv_pool_destroy(pkv_pool* p) { delete p; }

extern "C" int32_t pkv_pool_num_blocks(const pkv_pool* p) { return p ? p->num_blocks : -1; }

extern "C" int32_t pkv_pool_num_free(const pkv_pool* p) {
  return p ? (int32_t)p->free_list.size() : -1;
}

extern "C" double pkv_pool_usage(const pkv_pool* p) {
  if (!p || p->num_blocks == 0) return 0.0;
  return (double)(p->num_blocks - p->available()) / (double)p->num_blocks;
}

extern "C" int32_t pkv_pool_refcount(const pkv_pool* p, int32_t block) {
  if (!p || block < 0 || block >= p->num_blocks) return -1;
  return p->ref[(size_t)block];
}

extern "C" int32_t pkv_pool_num_seqs(const pkv_pool* p) {
  return p ? (int32_t)p->seqs.size() : -1;
}

extern "C" pkv_status pkv_seq_create(pkv_pool* p, int32_t* seq_out) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  if (!seq_out) return PKV_ERR_INVALID_ARG;
  int32_t id = p->next_id++;
  p->seqs.emplace(id, Seq());
  *seq_out = id;
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_fork(pkv_pool* p, int32_t parent, int32_t* child_out) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  if (!child_out) return PKV_ERR_INVALID_ARG;
  auto it = p->seqs.find(parent);
  if (it == p->seqs.end()) return PKV_ERR_BAD_HANDLE;
  if (it->second.swapped) return PKV_ERR_INVALID_ARG;  // swap it in first
  Seq child = it->second;  // same blocks, same length
  for (int32_t b : child.blocks) p->acquire(b);
  int32_t id = p->next_id++;
  p->seqs.emplace(id, std::move(child));
  *child_out = id;
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_append(pkv_pool* p, int32_t seq, int32_t n_tokens,
                                     int64_t* slots_out, int32_t* cow_pairs_out,
                                     int32_t* n_cow_out) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  if (n_tokens < 0 || (n_tokens > 0 && !slots_out)) return PKV_ERR_INVALID_ARG;
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return PKV_ERR_BAD_HANDLE;
  Seq& s = it->second;
  const int64_t bs = p->block_size;
  if (n_cow_out) *n_cow_out = 0;
  if (n_tokens == 0) return PKV_OK;
  if (s.swapped) return PKV_ERR_INVALID_ARG;  // swap it in first
  // Writing into a partially filled last block that another sequence also
  // holds would change that sequence's tokens: copy the block first.
  const bool cow = (s.len % bs) != 0 && p->ref[(size_t)s.blocks.back()] > 1;
  if (cow && !cow_pairs_out) return PKV_ERR_INVALID_ARG;
  const int64_t have = (s.len + bs - 1) / bs;
  const int64_t want = (s.len + n_tokens + bs - 1) / bs;
  const int64_t need = want - have + (cow ? 1 : 0);
  if (need > p->available()) return PKV_ERR_NO_FREE_BLOCKS;  // nothing changed
  if (cow) {
    const int32_t fresh = p->take();
    const int32_t old = s.blocks.back();
    p->release(old);
    s.blocks.back() = fresh;
    cow_pairs_out[0] = old;
    cow_pairs_out[1] = fresh;
    if (n_cow_out) *n_cow_out = 1;
  }
  for (int64_t i = 0; i < n_tokens; ++i) {
    const int64_t pos = s.len + i;
    if (pos / bs >= (int64_t)s.blocks.size()) s.blocks.push_back(p->take());  // a new block
    slots_out[i] = (int64_t)s.blocks[(size_t)(pos / bs)] * bs + pos % bs;
  }
  s.len += n_tokens;
  return PKV_OK;
}

// One token for each listed sequence (a decode step's slots), in order.
extern "C" pkv_status pkv_seq_append_each(pkv_pool* p, const int32_t* seqs, int32_t n,
                                          int64_t* slots_out, int32_t* cow_pairs_out,
                                          int32_t* n_cow_out, int32_t* n_done_out) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  if (n < 0 || (n > 0 && (!seqs || !slots_out || !cow_pairs_out)) || !n_cow_out || !n_done_out)
    return PKV_ERR_INVALID_ARG;
  *n_cow_out = 0;
  *n_done_out = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t nc = 0;
    const pkv_status st = pkv_seq_append(p, seqs[i], 1, slots_out + i,
                                         cow_pairs_out + 2 * (size_t)*n_cow_out, &nc);
    if (st != PKV_OK) return st;  // sequences before i are appended, i is unchanged
    *n_cow_out += nc;
    *n_done_out = i + 1;
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_free(pkv_pool* p, int32_t seq) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return PKV_ERR_BAD_HANDLE;
  for (int32_t b : it->second.blocks)
    if (b >= 0 && p->ref[(size_t)b] <= 0) return PKV_ERR_REFCOUNT;  // checked before any change
  for (int32_t b : it->second.blocks) {
    if (b >= 0)
      p->release(b);
    else
      p->host_free.push_back(host_slot(b));
  }
  p->seqs.erase(it);
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_block_table(const pkv_pool* p, int32_t seq, int32_t* out,
                                          int32_t cap, int32_t* n_out) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return PKV_ERR_BAD_HANDLE;
  const int32_t n = (int32_t)it->second.blocks.size();
  if (n_out) *n_out = n;
  if (cap < n || (n > 0 && !out)) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = it->second.blocks[(size_t)i];
    out[i] = b >= 0 ? b : -1;  // swapped out: no device block
  }
  return PKV_OK;
}

extern "C" int64_t pkv_seq_len(const pkv_pool* p, int32_t seq) {
  if (!p) return -1;
  auto it = p->seqs.find(seq);
  return it == p->seqs.end() ? -1 : it->second.len;
}

extern "C" pkv_status pkv_pool_cascade_tail_units(const pkv_pool* p, const int32_t* seqs,
                                                  int32_t n, const int32_t* prefix_blocks,
                                                  int32_t max_prefix_blocks,
                                                  int32_t partition_size, int64_t* units_out) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  if (n < 0 || !units_out || (n > 0 && !seqs) || partition_size <= 0 ||
      partition_size % 16 != 0 || max_prefix_blocks < 0)
    return PKV_ERR_INVALID_ARG;
  const int64_t pb = partition_size / 16;
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = p->seqs.find(seqs[i]);
    if (it == p->seqs.end()) return PKV_ERR_BAD_HANDLE;
    const int64_t L = it->second.len;
    int64_t S = prefix_blocks ? prefix_blocks[i] : 0;
    if (!(S > 0 && S <= max_prefix_blocks && 16 * S < L)) S = 0;
    const int64_t tail = (L + 15) / 16 - S;
    total += std::max<int64_t>(1, (tail + pb - 1) / pb);
  }
  *units_out = total;
  return PKV_OK;
}

extern "C" pkv_status pkv_pool_cascade_tail_map(const pkv_pool* p, const int32_t* seqs,
                                                int32_t n, const int32_t* prefix_blocks,
                                                int32_t max_prefix_blocks,
                                                int32_t partition_size, const int32_t* order,
                                                int32_t* map_out, int64_t map_cap,
                                                int64_t* units_out) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  if (n < 0 || !units_out || (n > 0 && !seqs) || partition_size <= 0 ||
      partition_size % 16 != 0 || max_prefix_blocks < 0 || map_cap < 0 ||
      (map_cap > 0 && !map_out))
    return PKV_ERR_INVALID_ARG;
  const int64_t pb = partition_size / 16;
  int64_t k = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = order ? order[i] : i;
    if (b < 0 || b >= n) return PKV_ERR_INVALID_ARG;
    auto it = p->seqs.find(seqs[b]);
    if (it == p->seqs.end()) return PKV_ERR_BAD_HANDLE;
    const int64_t L = it->second.len;
    int64_t S = prefix_blocks ? prefix_blocks[b] : 0;
    if (!(S > 0 && S <= max_prefix_blocks && 16 * S < L)) S = 0;
    const int64_t tail = (L + 15) / 16 - S;
    const int64_t units = std::max<int64_t>(1, (tail + pb - 1) / pb);
    if (k + units > map_cap) return PKV_ERR_INVALID_ARG;
    for (int64_t u = 0; u < units; ++u, ++k) {
      map_out[2 * k] = b;
      map_out[2 * k + 1] = (int32_t)u;
    }
  }
  *units_out = k;
  return PKV_OK;
}

extern "C" int32_t pkv_seq_shared_prefix_blocks(const pkv_pool* p, int32_t seq) {
  if (!p) return -1;
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return -1;
  int32_t n = 0;
  for (int32_t b : it->second.blocks) {
    if (b < 0 || p->ref[(size_t)b] <= 1) break;
    ++n;
  }
  return n;
}

// Groups for the cascade decode: batch entries whose first block is one
// shared physical block ([PRIMER-8] §8.1: forks of one prompt hold the same
// pages), each group's prefix being the leading table entries all its members
// hold, cut so that every member keeps at least one token after it.
extern "C" pkv_status pkv_pool_prefix_groups(const pkv_pool* p, const int32_t* seqs, int32_t n,
                                             int32_t group_cap, int32_t cap_groups,
                                             int32_t* prefix_blocks_out, int32_t* groups_out,
                                             int32_t* n_groups_out, int32_t* max_prefix_out,
                                             int32_t* order_out) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  if (n < 0 || group_cap <= 0 || cap_groups < 0 || !n_groups_out || !max_prefix_out ||
      (n > 0 && (!seqs || !prefix_blocks_out)) || (cap_groups > 0 && !groups_out))
    return PKV_ERR_INVALID_ARG;
  std::vector<const Seq*> sq((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = p->seqs.find(seqs[i]);
    if (it == p->seqs.end()) return PKV_ERR_BAD_HANDLE;
    sq[(size_t)i] = &it->second;
  }
  // batch entries by first block, groups in order of first appearance
  std::unordered_map<int32_t, size_t> by_first;
  std::vector<std::vector<int32_t>> cand;
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = *sq[(size_t)i];
    if (s.blocks.empty() || s.blocks[0] < 0 || p->ref[(size_t)s.blocks[0]] <= 1) continue;
    auto ins = by_first.emplace(s.blocks[0], cand.size());
    if (ins.second) cand.emplace_back();
    cand[ins.first->second].push_back(i);
  }
  std::vector<int32_t> prefix((size_t)n, 0);
  std::vector<std::vector<int32_t>> groups;
  int32_t max_prefix = 0;
  for (const auto& mem : cand) {
    if (mem.size() < 2) continue;
    // longest run of leading entries every member holds, on the device
    const std::vector<int32_t>& lead = sq[(size_t)mem[0]]->blocks;
    int64_t S = (int64_t)lead.size();
    for (int32_t i : mem) {
      const Seq& s = *sq[(size_t)i];
      int64_t k = 0;
      while (k < S && k < (int64_t)s.blocks.size() && s.blocks[(size_t)k] >= 0 &&
             s.blocks[(size_t)k] == lead[(size_t)k])
        ++k;
      S = std::min<int64_t>(k, (s.len - 1) / p->block_size);  // a token after it
    }
    if (S <= 0) continue;
    for (size_t c = 0; c < mem.size(); c += (size_t)group_cap) {
      std::vector<int32_t> g(mem.begin() + (std::ptrdiff_t)c,
                             mem.begin() + (std::ptrdiff_t)std::min(mem.size(), c + group_cap));
      for (int32_t i : g) prefix[(size_t)i] = (int32_t)S;
      groups.push_back(std::move(g));
    }
    max_prefix = std::max<int32_t>(max_prefix, (int32_t)S);
  }
  *n_groups_out = (int32_t)groups.size();
  *max_prefix_out = max_prefix;
  if ((int32_t)groups.size() > cap_groups) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) prefix_blocks_out[i] = prefix[(size_t)i];
  if (order_out) {  // longest tail first, ties in batch order
    std::vector<int32_t> ord((size_t)n);
    for (int32_t i = 0; i < n; ++i) ord[(size_t)i] = i;
    auto tail = [&](int32_t i) {
      return sq[(size_t)i]->len - (int64_t)prefix[(size_t)i] * p->block_size;
    };
    std::stable_sort(ord.begin(), ord.end(),
                     [&](int32_t x, int32_t y) { return tail(x) > tail(y); });
    for (int32_t i = 0; i < n; ++i) order_out[i] = ord[(size_t)i];
  }
  for (size_t gi = 0; gi < groups.size(); ++gi)
    for (int32_t k = 0; k < group_cap; ++k)
      groups_out[gi * (size_t)group_cap + (size_t)k] =
          k < (int32_t)groups[gi].size() ? groups[gi][(size_t)k] : -1;
  return PKV_OK;
}

// ------------------------------------------------------------ prefix cache

extern "C" pkv_status pkv_seq_create_cached(pkv_pool* p, const int32_t* tokens,
                                            int32_t n_tokens, int32_t* seq_out,
                                            int32_t* n_cached_out) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  if (!seq_out || n_tokens < 0 || (n_tokens > 0 && !tokens)) return PKV_ERR_INVALID_ARG;
  const int32_t bs = p->block_size;
  const int32_t chunks = n_tokens / bs;
  Seq s;
  uint64_t key = 0;
  int32_t hits = 0;
  for (int32_t i = 0; i < chunks; ++i) {
    const int32_t* chunk = tokens + (int64_t)i * bs;
    const uint64_t k = chunk_key(key, chunk, bs);
    auto it = p->cache.find(k);
    if (it == p->cache.end() || it->second.parent != key ||
        !std::equal(it->second.tokens.begin(), it->second.tokens.end(), chunk))
      break;  // miss: this chunk and every later one must be prefilled
    const int32_t b = it->second.block;
    p->acquire(b);  // leaves the evictable set if nobody held it
    it->second.tick = ++p->tick;
    s.blocks.push_back(b);
    key = k;
    ++hits;
  }
  s.len = (int64_t)hits * bs;
  p->hit_blocks += hits;
  p->miss_blocks += chunks - hits;
  const int32_t id = p->next_id++;
  p->seqs.emplace(id, std::move(s));
  *seq_out = id;
  if (n_cached_out) *n_cached_out = hits * bs;
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_cache_prefix(pkv_pool* p, int32_t seq, const int32_t* tokens,
                                           int32_t n_tokens) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  if (n_tokens < 0 || (n_tokens > 0 && !tokens)) return PKV_ERR_INVALID_ARG;
  auto sit = p->seqs.find(seq);
  if (sit == p->seqs.end()) return PKV_ERR_BAD_HANDLE;
  const Seq& s = sit->second;
  if (s.swapped) return PKV_ERR_INVALID_ARG;
  const int32_t bs = p->block_size;
  const int64_t chunks = std::min<int64_t>(n_tokens, s.len) / bs;
  uint64_t key = 0;
  for (int64_t i = 0; i < chunks; ++i) {
    const int32_t* chunk = tokens + i * bs;
    const uint64_t k = chunk_key(key, chunk, bs);
    auto it = p->cache.find(k);
    if (it != p->cache.end()) {
      if (it->second.parent != key ||
          !std::equal(it->second.tokens.begin(), it->second.tokens.end(), chunk))
        break;  // a different prefix owns this key: stop registering
    } else {
      const int32_t b = s.blocks[(size_t)i];
      if (p->cache_key[(size_t)b] != 0) break;  // the block is cached for another chunk
      CacheEntry e{b, key, std::vector<int32_t>(chunk, chunk + bs), ++p->tick};
      p->cache.emplace(k, std::move(e));
      p->cache_key[(size_t)b] = k;
    }
    key = k;
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_prefix_cache_stats(const pkv_pool* p, int64_t* hit_blocks,
                                             int64_t* miss_blocks, int32_t* cached_blocks,
                                             int32_t* evictable_blocks) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  if (hit_blocks) *hit_blocks = p->hit_blocks;
  if (miss_blocks) *miss_blocks = p->miss_blocks;
  if (cached_blocks) *cached_blocks = (int32_t)p->cache.size();
  if (evictable_blocks) *evictable_blocks = (int32_t)p->evictable.size();
  return PKV_OK;
}

extern "C" void pkv_prefix_cache_clear(pkv_pool* p) {
  if (!p) return;
  for (const auto& e : p->evictable) p->free_list.push_back(e.second);  // LRU first
  p->evictable.clear();
  for (const auto& kv : p->cache) p->cache_key[(size_t)kv.second.block] = 0;
  p->cache.clear();
}

// ------------------------------------------------------------------- swap

extern "C" pkv_status pkv_pool_set_swap_space(pkv_pool* p, int32_t num_host_blocks) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  if (num_host_blocks < 0) return PKV_ERR_INVALID_ARG;
  if ((int32_t)p->host_free.size() != p->num_host) return PKV_ERR_INVALID_ARG;  // slots in use
  p->num_host = num_host_blocks;
  p->host_free.clear();
  for (int32_t i = 0; i < num_host_blocks; ++i) p->host_free.push_back(i);
  return PKV_OK;
}

extern "C" int32_t pkv_pool_num_free_host(const pkv_pool* p) {
  return p ? (int32_t)p->host_free.size() : -1;
}

extern "C" int32_t pkv_seq_num_swapped(const pkv_pool* p, int32_t seq) {
  if (!p) return -1;
  auto it = p->seqs.find(seq);
  return it == p->seqs.end() ? -1 : it->second.swapped;
}

extern "C" pkv_status pkv_seq_swap_out(pkv_pool* p, int32_t seq, int32_t first_block,
                                       int32_t n_blocks, int32_t* pairs_out) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return PKV_ERR_BAD_HANDLE;
  Seq& s = it->second;
  if (n_blocks < 0 || first_block < 0 || (n_blocks > 0 && !pairs_out) ||
      (int64_t)first_block + n_blocks > (int64_t)s.blocks.size())
    return PKV_ERR_INVALID_ARG;
  for (int32_t i = first_block; i < first_block + n_blocks; ++i) {  // all checked first
    const int32_t b = s.blocks[(size_t)i];
    if (b < 0) return PKV_ERR_INVALID_ARG;             // already swapped out
    if (p->ref[(size_t)b] != 1) return PKV_ERR_REFCOUNT;  // shared: not this sequence's alone
  }
  if (n_blocks > (int32_t)p->host_free.size()) return PKV_ERR_NO_FREE_BLOCKS;
  for (int32_t i = 0; i < n_blocks; ++i) {
    int32_t& e = s.blocks[(size_t)(first_block + i)];
    const int32_t b = e;
    const int32_t slot = p->host_free.front();
    p->host_free.pop_front();
    if (p->cache_key[(size_t)b] != 0) {  // its prefix-cache entry leaves with it
      p->cache.erase(p->cache_key[(size_t)b]);
      p->cache_key[(size_t)b] = 0;
    }
    p->release(b);
    e = host_code(slot);
    pairs_out[2 * i] = b;
    pairs_out[2 * i + 1] = slot;
  }
  s.swapped += n_blocks;
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_swap_in(pkv_pool* p, int32_t seq, int32_t* pairs_out, int32_t cap,
                                      int32_t* n_out) {
  if (!p) return PKV_ERR_BAD_HANDLE;
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return PKV_ERR_BAD_HANDLE;
  Seq& s = it->second;
  if (n_out) *n_out = s.swapped;
  if (s.swapped == 0) return PKV_OK;
  if (cap < s.swapped || !pairs_out) return PKV_ERR_INVALID_ARG;
  if (s.swapped > p->available()) return PKV_ERR_NO_FREE_BLOCKS;  // nothing changed
  int32_t k = 0;
  for (int32_t& e : s.blocks) {
    if (e >= 0) continue;
    const int32_t slot = host_slot(e);
    const int32_t b = p->take();
    p->host_free.push_back(slot);
    e = b;
    pairs_out[2 * k] = slot;
    pairs_out[2 * k + 1] = b;
    ++k;
  }
  s.swapped = 0;
  return PKV_OK;
}
