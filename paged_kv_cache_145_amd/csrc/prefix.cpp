// Prefix-aware block reuse for the paged KV cache: a chained block key over
// token ids, a prefix index with token-level verification, copy-on-write of
// shared blocks and eviction of blocks only the index still holds.  Plain
// C++17, no HIP; the device copy that completes a copy-on-write lives in
// write_kernels.hip.
//
// What the pages fix ("Ollama的内存管理策略…" (xdnf.cn/news/5086), sections
// "三、KV Cache内存管理的工程实现" and "四、内存管理策略的边界"; the resident
// system-prompt blocks of "端侧 SLM 显存保活术…" (sheratonhq.com/news/141880),
// section "共享前缀块"): a 64-bit FNV-1a style key over the token ids of a
// block, one id folded per step; a key hit confirmed on the ids themselves;
// one more reference per reuse; read-only shared blocks copied before a
// write; least-recently-used eviction of unshared blocks; a warmed-up prefix
// that is never evicted.
//
// Where that page's code leaves a step open or gets it wrong, this file
// takes the following course:
//   - block i's key continues the fold from block i-1's key, so it covers
//     every token up to the block's end (the page restarts at each block);
//   - verification compares the ids and requires the entry to hang off the
//     entry matched for the previous block, so a key collision never joins
//     two different prefixes;
//   - the index holds one reference per listed block; eviction frees only
//     blocks whose one remaining reference is the index's, and only leaf
//     entries, least recent use first (ties: oldest entry), never resident
//     ones; each match / insert call is one tick of the use clock;
//   - a partial last block ("tail") is listed under its parent and matches
//     when its ids are a prefix of the remaining request, longest first.
#include <algorithm>
#include <new>
#include <set>
#include <utility>

#include "pool_internal.h"

namespace pa {
namespace {

constexpr uint64_t kFnvBasis = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

uint64_t fold(uint64_t h, const uint32_t *t, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    h ^= t[i];
    h *= kFnvPrime;
  }
  return h;
}

bool same_tokens(const PrefixEntry &e, const uint32_t *t, int64_t n) {
  return (int64_t)e.tokens.size() == n && std::equal(e.tokens.begin(), e.tokens.end(), t);
}

int32_t find_full(const PrefixIndex &ix, int32_t parent, uint64_t key, const uint32_t *t,
                  int64_t n) {
  auto range = ix.by_key.equal_range(key);
  for (auto it = range.first; it != range.second; ++it) {
    const PrefixEntry &e = ix.entries[(size_t)it->second];
    if (e.parent == parent && same_tokens(e, t, n)) return it->second;
  }
  return -1;
}

int32_t find_tail(const PrefixIndex &ix, int32_t parent, const uint32_t *t, int64_t n) {
  auto range = ix.tails.equal_range(parent);
  for (auto it = range.first; it != range.second; ++it)
    if (same_tokens(ix.entries[(size_t)it->second], t, n)) return it->second;
  return -1;
}

// Longest tail under `parent` whose ids are a prefix of t[0, n).
int32_t longest_tail(const PrefixIndex &ix, int32_t parent, const uint32_t *t, int64_t n) {
  int32_t best = -1;
  size_t best_len = 0;
  auto range = ix.tails.equal_range(parent);
  for (auto it = range.first; it != range.second; ++it) {
    const PrefixEntry &e = ix.entries[(size_t)it->second];
    const size_t m = e.tokens.size();
    if ((int64_t)m <= n && m > best_len && std::equal(e.tokens.begin(), e.tokens.end(), t)) {
      best = it->second;
      best_len = m;
    }
  }
  return best;
}

template <class Map, class K>
void erase_pair(Map &m, const K &k, int32_t slot) {
  auto range = m.equal_range(k);
  for (auto it = range.first; it != range.second; ++it)
    if (it->second == slot) {
      m.erase(it);
      return;
    }
}

// Remove a leaf entry and drop the index's reference on its block.
void drop_entry(pa_pool *pool, int32_t slot) {
  PrefixIndex &ix = pool->prefix;
  PrefixEntry &e = ix.entries[(size_t)slot];
  if (e.full)
    erase_pair(ix.by_key, e.key, slot);
  else {
    erase_pair(ix.tails, e.parent, slot);
    ix.tail_entries -= 1;
  }
  if (e.parent >= 0) ix.entries[(size_t)e.parent].children -= 1;
  if (e.resident) ix.resident -= 1;
  ix.block_entry[(size_t)e.block] = -1;
  drop_ref_locked(pool, e.block);
  e = PrefixEntry();
  ix.free_slots.push_back(slot);
  ix.live -= 1;
}

bool evictable(const pa_pool *pool, const PrefixEntry &e) {
  return e.live && !e.resident && e.children == 0 && pool->refcount[(size_t)e.block] == 1;
}

// Planned step of an insert: an existing entry, or a new one for blocks[i].
struct Step {
  int32_t existing;  // slot, or -1 for a new entry
  int32_t block;
  bool full;
  uint64_t key;
  int64_t first;  // index of the block's first token
  int64_t count;
};

}  // namespace
}  // namespace pa

extern "C" {

int pa_block_hashes(const uint32_t *tokens, int64_t num_tokens, int32_t block_size,
                    uint64_t *out) {
  if (num_tokens < 0 || block_size <= 0) return PA_ERR_INVAL;
  const int64_t nfull = num_tokens / block_size;
  if (nfull == 0) return PA_OK;
  if (tokens == nullptr || out == nullptr) return PA_ERR_INVAL;
  uint64_t h = pa::kFnvBasis;
  for (int64_t i = 0; i < nfull; ++i) {
    h = pa::fold(h, tokens + i * block_size, block_size);
    out[i] = h;
  }
  return PA_OK;
}

int pa_prefix_match(pa_pool *pool, const uint32_t *tokens, int64_t num_tokens,
                    int32_t *blocks_out, int32_t max_blocks, int32_t *num_blocks_out,
                    int64_t *num_tokens_matched) {
  if (pool == nullptr || num_tokens < 0 || max_blocks < 0 || num_blocks_out == nullptr ||
      num_tokens_matched == nullptr)
    return PA_ERR_INVAL;
  if ((num_tokens > 0 && tokens == nullptr) || (max_blocks > 0 && blocks_out == nullptr))
    return PA_ERR_INVAL;
  std::lock_guard<std::mutex> lock(pool->mu);
  pa::PrefixIndex &ix = pool->prefix;
  ix.clock += 1;
  const int64_t bs = pool->block_size;
  int32_t parent = -1, got = 0;
  uint64_t h = pa::kFnvBasis;
  int64_t p = 0;
  while (got < max_blocks && num_tokens - p >= bs) {
    const uint64_t key = pa::fold(h, tokens + p, bs);
    const int32_t slot = pa::find_full(ix, parent, key, tokens + p, bs);
    if (slot < 0) break;
    pa::PrefixEntry &e = ix.entries[(size_t)slot];
    if (pool->refcount[(size_t)e.block] == INT32_MAX) break;
    e.last_use = ix.clock;
    pa::add_ref_locked(pool, e.block);
    blocks_out[got++] = e.block;
    parent = slot;
    h = key;
    p += bs;
  }
  if (got < max_blocks) {
    const int32_t slot = pa::longest_tail(ix, parent, tokens + p, num_tokens - p);
    if (slot >= 0 && pool->refcount[(size_t)ix.entries[(size_t)slot].block] < INT32_MAX) {
      pa::PrefixEntry &e = ix.entries[(size_t)slot];
      e.last_use = ix.clock;
      pa::add_ref_locked(pool, e.block);
      blocks_out[got++] = e.block;
      p += (int64_t)e.tokens.size();
    }
  }
  *num_blocks_out = got;
  *num_tokens_matched = p;
  return PA_OK;
}

int pa_prefix_insert(pa_pool *pool, const uint32_t *tokens, int64_t num_tokens,
                     const int32_t *blocks, int32_t num_blocks, uint32_t flags, int32_t *num_new) {
  if (pool == nullptr || num_tokens < 0 || num_blocks < 0) return PA_ERR_INVAL;
  if ((flags & ~(uint32_t)(PA_PREFIX_TAIL | PA_PREFIX_RESIDENT)) != 0) return PA_ERR_INVAL;
  const int64_t bs = pool->block_size;
  const int64_t nfull = num_tokens / bs;
  const bool has_tail = (flags & PA_PREFIX_TAIL) && num_tokens % bs != 0;
  const int64_t need = nfull + (has_tail ? 1 : 0);
  if (num_blocks < need) return PA_ERR_INVAL;
  if ((num_tokens > 0 && tokens == nullptr) || (need > 0 && blocks == nullptr)) return PA_ERR_INVAL;
  const bool resident = (flags & PA_PREFIX_RESIDENT) != 0;

  std::lock_guard<std::mutex> lock(pool->mu);
  pa::PrefixIndex &ix = pool->prefix;
  std::vector<pa::Step> plan;
  try {
    plan.reserve((size_t)need);
  } catch (...) {
    return PA_ERR_NOMEM;
  }
  // walk: known entries first, then (once one is missing) new ones only
  int32_t parent = -1;
  bool fresh = false;
  uint64_t h = pa::kFnvBasis;
  for (int64_t i = 0; i < need; ++i) {
    const bool full = i < nfull;
    const int64_t first = i * bs;
    const int64_t count = full ? bs : num_tokens - first;
    pa::Step st{-1, blocks[i], full, 0, first, count};
    if (full) {
      h = pa::fold(h, tokens + first, bs);
      st.key = h;
    }
    if (!fresh) {
      st.existing = full ? pa::find_full(ix, parent, h, tokens + first, bs)
                         : pa::find_tail(ix, parent, tokens + first, count);
      if (st.existing >= 0)
        parent = st.existing;
      else
        fresh = true;
    }
    plan.push_back(st);
  }
  // validate every new entry's block before changing anything
  for (const pa::Step &st : plan) {
    if (st.existing >= 0) continue;
    if (st.block < 0 || st.block >= pool->num_blocks) return PA_ERR_INVAL;
    if (pool->refcount[(size_t)st.block] == 0) return PA_ERR_STATE;
    if (pool->refcount[(size_t)st.block] == INT32_MAX) return PA_ERR_STATE;
    if (ix.block_entry[(size_t)st.block] >= 0) return PA_ERR_STATE;
  }
  for (size_t a = 0; a < plan.size(); ++a) {
    if (plan[a].existing >= 0) continue;
    for (size_t b = a + 1; b < plan.size(); ++b)
      if (plan[b].existing < 0 && plan[b].block == plan[a].block) return PA_ERR_STATE;
  }
  // Phase 1: every allocation the insert may need except the map nodes.
  size_t new_count = 0;
  for (const pa::Step &st : plan) new_count += st.existing < 0 ? 1 : 0;
  std::vector<std::vector<uint32_t>> toks;
  std::vector<int32_t> made, path;
  try {
    toks.resize(new_count);
    size_t k = 0;
    for (const pa::Step &st : plan)
      if (st.existing < 0) toks[k++].assign(tokens + st.first, tokens + st.first + st.count);
    made.reserve(new_count);
    path.reserve(plan.size());
    ix.entries.reserve(ix.entries.size() + new_count);
    ix.free_slots.reserve(ix.free_slots.size() + new_count);  // room to give slots back
    ix.by_key.reserve(ix.by_key.size() + new_count);
    ix.tails.reserve(ix.tails.size() + new_count);
  } catch (...) {
    return PA_ERR_NOMEM;  // nothing changed
  }
  // Phase 2: the new entries and their map nodes; a failed node allocation
  // takes every new entry back out.
  try {
    parent = -1;
    size_t k = 0;
    for (const pa::Step &st : plan) {
      int32_t slot = st.existing;
      if (slot < 0) {
        if (!ix.free_slots.empty()) {
          slot = ix.free_slots.back();
          ix.free_slots.pop_back();
        } else {
          slot = (int32_t)ix.entries.size();
          ix.entries.emplace_back();  // within the reserved capacity
        }
        made.push_back(slot);
        pa::PrefixEntry &e = ix.entries[(size_t)slot];
        e.full = st.full;
        e.block = st.block;
        e.parent = parent;
        e.children = 0;
        e.key = st.key;
        e.tokens = std::move(toks[k++]);
        if (st.full)
          ix.by_key.emplace(st.key, slot);
        else
          ix.tails.emplace(parent, slot);
        e.live = true;
      }
      path.push_back(slot);
      parent = slot;
    }
  } catch (...) {
    for (auto it = made.rbegin(); it != made.rend(); ++it) {
      pa::PrefixEntry &e = ix.entries[(size_t)*it];
      if (e.live) {
        if (e.full)
          pa::erase_pair(ix.by_key, e.key, *it);
        else
          pa::erase_pair(ix.tails, e.parent, *it);
      }
      e = pa::PrefixEntry();
      ix.free_slots.push_back(*it);  // within the reserved capacity
    }
    return PA_ERR_NOMEM;
  }
  // Phase 3: counts, references and use stamps (nothing allocates).
  for (int32_t slot : made) {
    pa::PrefixEntry &e = ix.entries[(size_t)slot];
    e.serial = ix.next_serial++;
    if (!e.full) ix.tail_entries += 1;
    if (e.parent >= 0) ix.entries[(size_t)e.parent].children += 1;
    ix.block_entry[(size_t)e.block] = slot;
    pa::add_ref_locked(pool, e.block);
    ix.live += 1;
  }
  ix.clock += 1;
  for (int32_t slot : path) {
    pa::PrefixEntry &e = ix.entries[(size_t)slot];
    e.last_use = ix.clock;
    if (resident && !e.resident) {
      e.resident = true;
      ix.resident += 1;
    }
  }
  if (num_new != nullptr) *num_new = (int32_t)made.size();
  return PA_OK;
}

int pa_prefix_evict(pa_pool *pool, int32_t max_blocks, int32_t *freed, int32_t *num_freed) {
  if (pool == nullptr || max_blocks < 0 || num_freed == nullptr) return PA_ERR_INVAL;
  std::lock_guard<std::mutex> lock(pool->mu);
  pa::PrefixIndex &ix = pool->prefix;
  int32_t n = 0;
  if (max_blocks > 0) {
    using Rank = std::pair<std::pair<uint64_t, uint64_t>, int32_t>;  // ((last use, serial), slot)
    std::set<Rank> cand;
    try {
      for (size_t s = 0; s < ix.entries.size(); ++s) {
        const pa::PrefixEntry &e = ix.entries[s];
        if (pa::evictable(pool, e)) cand.insert({{e.last_use, e.serial}, (int32_t)s});
      }
      while (n < max_blocks && !cand.empty()) {
        const int32_t slot = cand.begin()->second;
        cand.erase(cand.begin());
        const int32_t block = ix.entries[(size_t)slot].block;
        const int32_t parent = ix.entries[(size_t)slot].parent;
        pa::drop_entry(pool, slot);
        if (freed != nullptr) freed[n] = block;
        n += 1;
        if (parent >= 0 && pa::evictable(pool, ix.entries[(size_t)parent])) {
          const pa::PrefixEntry &pe = ix.entries[(size_t)parent];
          cand.insert({{pe.last_use, pe.serial}, parent});
        }
      }
    } catch (...) {
      *num_freed = n;
      return PA_ERR_NOMEM;
    }
  }
  *num_freed = n;
  return PA_OK;
}

int pa_prefix_clear(pa_pool *pool) {
  if (pool == nullptr) return PA_ERR_INVAL;
  std::lock_guard<std::mutex> lock(pool->mu);
  pa::PrefixIndex &ix = pool->prefix;
  for (const pa::PrefixEntry &e : ix.entries)
    if (e.live) {
      ix.block_entry[(size_t)e.block] = -1;
      pa::drop_ref_locked(pool, e.block);
    }
  ix.entries.clear();
  ix.free_slots.clear();
  ix.by_key.clear();
  ix.tails.clear();
  ix.live = ix.tail_entries = ix.resident = 0;
  return PA_OK;
}

int pa_prefix_get_stats(const pa_pool *pool, pa_prefix_stats *out) {
  if (pool == nullptr || out == nullptr) return PA_ERR_INVAL;
  std::lock_guard<std::mutex> lock(pool->mu);
  const pa::PrefixIndex &ix = pool->prefix;
  out->entries = ix.live;
  out->tail_entries = ix.tail_entries;
  out->resident = ix.resident;
  int32_t alone = 0;
  for (const pa::PrefixEntry &e : ix.entries)
    if (e.live && pool->refcount[(size_t)e.block] == 1) alone += 1;
  out->index_only = alone;
  return PA_OK;
}

int pa_cow_block(pa_pool *pool, int32_t block_id, int32_t *out_block) {
  if (pool == nullptr || out_block == nullptr) return PA_ERR_INVAL;
  *out_block = -1;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (block_id < 0 || block_id >= pool->num_blocks) return PA_ERR_INVAL;
  const int32_t rc = pool->refcount[(size_t)block_id];
  if (rc == 0) return PA_ERR_STATE;
  // a block whose one reference is the index's has no caller to write it
  if (rc == 1 && pool->prefix.block_entry[(size_t)block_id] >= 0) return PA_ERR_STATE;
  if (rc == 1) {
    *out_block = block_id;
    return PA_OK;
  }
  const int32_t fresh = pa::alloc_block_locked(pool);
  if (fresh < 0) return PA_ERR_NOMEM;
  pa::drop_ref_locked(pool, block_id);  // rc >= 2: never frees
  *out_block = fresh;
  return PA_OK;
}

}  // extern "C"
