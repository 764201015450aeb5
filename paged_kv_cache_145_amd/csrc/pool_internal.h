// Host-side pool state shared by the allocator (pool.cpp, plain C++) and the
// HIP entry points (api.hip).  No HIP types here, so pool.cpp builds with g++.
#ifndef PA_POOL_INTERNAL_H_
#define PA_POOL_INTERNAL_H_

#include <cstdint>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace pa {

// One listed block of the prefix index.  A full entry covers block_size
// token ids and is found by its chained key; a tail entry covers fewer and
// is found under its parent.  Entries form a forest: `parent` is the slot of
// the entry for the previous block (-1 for the first block).
struct PrefixEntry {
  bool live = false;
  bool full = false;
  bool resident = false;
  int32_t block = -1;
  int32_t parent = -1;
  int32_t children = 0;
  uint64_t key = 0;
  uint64_t serial = 0;    // creation order
  uint64_t last_use = 0;  // use clock of the last match / insert that walked it
  std::vector<uint32_t> tokens;
};

struct PrefixIndex {
  std::vector<PrefixEntry> entries;  // slots; dead slots are reused
  std::vector<int32_t> free_slots;
  std::unordered_multimap<uint64_t, int32_t> by_key;  // chained key -> full entry slot
  std::unordered_multimap<int32_t, int32_t> tails;    // parent slot -> tail entry slot
  std::vector<int32_t> block_entry;                   // block id -> slot, or -1
  uint64_t clock = 0;
  uint64_t next_serial = 0;
  int32_t live = 0;
  int32_t tail_entries = 0;
  int32_t resident = 0;
};

}  // namespace pa

struct pa_pool {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  pa_dtype dtype;  // element type of K/V rows, or the activation type of an 8-bit pool
  bool kv_fp8;     // pools hold 8-bit codes scaled per KV head
  pa_dtype kv_dtype;  // storage type of K/V rows: dtype, or PA_FP8_E4M3 / PA_FP8_E5M2
  std::vector<float> k_scale, v_scale;  // 8-bit pools: per-head scales
  std::vector<float> k_inv, v_inv;      // fp32(1 / scale)
  void *k_cache;
  void *v_cache;

  // Allocator: one bit per block (1 = free), scanned lowest word first with a
  // count-trailing-zeros step, plus a reference count per block.
  mutable std::mutex mu;
  std::vector<uint64_t> free_bits;     // bit b % 64 of word b / 64: block b is free
  std::vector<uint64_t> free_summary;  // bit w % 64 of word w / 64: free_bits[w] != 0
  std::vector<int32_t> refcount;
  int32_t used;
  int32_t shared;
  // Blocks listed by the prefix index, each holding one reference.
  pa::PrefixIndex prefix;
};

namespace pa {

inline int dtype_bytes(pa_dtype t) { return t == PA_F32 ? 4 : 2; }
constexpr int kMaxFp8Heads = 64;  // per-head scales travel in kernel arguments
inline bool valid_dtype(int t) { return t == PA_F32 || t == PA_F16 || t == PA_BF16; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Effective number of cached keys a decode can read for a context bound.
inline int64_t effective_context(int64_t max_context_len, const pa_ring *ring) {
  if (ring == nullptr) return max_context_len;
  int64_t cap = (int64_t)ring->sink + ring->window;
  return max_context_len < cap ? max_context_len : cap;
}

bool ring_valid(const pa_ring *ring);

// Allocator steps with pool->mu held (pool.cpp).
int32_t alloc_block_locked(pa_pool *pool);
void add_ref_locked(pa_pool *pool, int32_t block_id);   // refcount >= 1
void drop_ref_locked(pa_pool *pool, int32_t block_id);  // refcount >= 1

}  // namespace pa

#endif  // PA_POOL_INTERNAL_H_
