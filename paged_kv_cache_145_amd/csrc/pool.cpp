// Host side of the paged KV cache: pool description, block allocator with
// reference counts, ring slot equation and slot mapping.  Plain C++17, no HIP.
//
// Allocation order is that of "端侧 SLM 显存保活术…" (sheratonhq.com/news/141880),
// section "嵌入式轻量 Block 分配器设计": a new block is the lowest free id, and
// -1 reports an exhausted pool.  The free set is kept as a two-level bitmap:
// leaf word w has bit i set when block 64 w + i is free, and bit w of the
// summary words is set when leaf word w has any free block, so the lowest
// free id is found by reading one summary word per 4,096 blocks.
// Reference counts and release at the last reference follow
// "Ollama的内存管理策略…" (xdnf.cn/news/5086), section
// "三、KV Cache内存管理的工程实现"; misuse that page leaves unchecked (release
// of a free block) is an error here.
#include <cstring>
#include <new>

#include <cmath>

#include "pool_internal.h"

namespace pa {

int32_t alloc_block_locked(pa_pool *pool) {
  // lowest leaf word with a free block, then its lowest free block
  size_t s = 0;
  while (s < pool->free_summary.size() && pool->free_summary[s] == 0) ++s;
  if (s == pool->free_summary.size()) return -1;
  const size_t w = s * 64 + (size_t)__builtin_ctzll(pool->free_summary[s]);
  uint64_t &leaf = pool->free_bits[w];
  const int32_t id = (int32_t)(w * 64 + (size_t)__builtin_ctzll(leaf));
  leaf &= leaf - 1;  // that block is taken
  if (leaf == 0) pool->free_summary[s] &= ~(1ull << (w % 64));
  pool->refcount[(size_t)id] = 1;
  pool->used += 1;
  return id;
}

void add_ref_locked(pa_pool *pool, int32_t block_id) {
  int32_t &rc = pool->refcount[(size_t)block_id];
  rc += 1;
  if (rc == 2) pool->shared += 1;
}

void drop_ref_locked(pa_pool *pool, int32_t block_id) {
  int32_t &rc = pool->refcount[(size_t)block_id];
  rc -= 1;
  if (rc == 1) pool->shared -= 1;
  if (rc == 0) {
    const size_t w = (size_t)block_id / 64;
    pool->free_bits[w] |= 1ull << (block_id % 64);
    pool->free_summary[w / 64] |= 1ull << (w % 64);
    pool->used -= 1;
  }
}

bool ring_valid(const pa_ring *ring) {
  if (ring == nullptr) return true;
  if (ring->sink < 0 || ring->window < 1) return false;
  if ((int64_t)ring->sink + ring->window > INT32_MAX) return false;
  if (ring->rope_style != 0) return false;
  if (!(ring->rope_base > 0.0f)) return false;
  return true;
}

}  // namespace pa

extern "C" {

int pa_create_pool(pa_pool **out, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, pa_dtype dtype, void *k_cache, void *v_cache) {
  if (out == nullptr) return PA_ERR_INVAL;
  *out = nullptr;
  if (num_blocks <= 0 || num_kv_heads <= 0) return PA_ERR_INVAL;
  if (block_size != 16 && block_size != 64) return PA_ERR_INVAL;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_INVAL;
  if (!pa::valid_dtype((int)dtype)) return PA_ERR_INVAL;
  if (k_cache == nullptr || v_cache == nullptr) return PA_ERR_INVAL;
  if ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15u)
    return PA_ERR_INVAL;
  pa_pool *p = new (std::nothrow) pa_pool();
  if (p == nullptr) return PA_ERR_NOMEM;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->num_kv_heads = num_kv_heads;
  p->head_dim = head_dim;
  p->dtype = dtype;
  p->kv_fp8 = false;
  p->kv_dtype = dtype;
  p->k_cache = k_cache;
  p->v_cache = v_cache;
  try {
    // every block starts free
    const size_t words = (size_t)pa::ceil_div(num_blocks, 64);
    p->free_bits.assign(words, 0ull);
    for (int32_t b = 0; b < num_blocks; ++b) p->free_bits[(size_t)b / 64] |= 1ull << (b % 64);
    p->free_summary.assign((size_t)pa::ceil_div((int64_t)words, 64), 0ull);
    for (size_t w = 0; w < words; ++w) p->free_summary[w / 64] |= 1ull << (w % 64);
    p->refcount.assign((size_t)num_blocks, 0);
    p->prefix.block_entry.assign((size_t)num_blocks, -1);
  } catch (...) {
    delete p;
    return PA_ERR_NOMEM;
  }
  p->used = 0;
  p->shared = 0;
  *out = p;
  return PA_OK;
}

int pa_create_pool_fp8(pa_pool **out, int32_t num_blocks, int32_t block_size,
                       int32_t num_kv_heads, int32_t head_dim, pa_dtype act_dtype,
                       const float *k_scale, const float *v_scale, void *k_cache, void *v_cache) {
  return pa_create_pool_kv8(out, num_blocks, block_size, num_kv_heads, head_dim, PA_FP8_E4M3, act_dtype,
                            k_scale, v_scale, k_cache, v_cache);
}

int pa_create_pool_kv8(pa_pool **out, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                       int32_t head_dim, pa_dtype kv_dtype, pa_dtype act_dtype, const float *k_scale,
                       const float *v_scale, void *k_cache, void *v_cache) {
  if (out == nullptr) return PA_ERR_INVAL;
  *out = nullptr;
  if (kv_dtype != PA_FP8_E4M3 && kv_dtype != PA_FP8_E5M2) return PA_ERR_INVAL;
  if (act_dtype != PA_F16 && act_dtype != PA_BF16) return PA_ERR_INVAL;
  if (num_kv_heads <= 0 || num_kv_heads > pa::kMaxFp8Heads) return PA_ERR_INVAL;
  if (k_scale == nullptr || v_scale == nullptr) return PA_ERR_INVAL;
  for (int h = 0; h < num_kv_heads; ++h) {
    if (!(std::isfinite(k_scale[h]) && k_scale[h] > 0.f)) return PA_ERR_INVAL;
    if (!(std::isfinite(v_scale[h]) && v_scale[h] > 0.f)) return PA_ERR_INVAL;
  }
  pa_pool *p = nullptr;
  const int rc = pa_create_pool(&p, num_blocks, block_size, num_kv_heads, head_dim, act_dtype,
                                k_cache, v_cache);
  if (rc != PA_OK) return rc;
  try {
    p->k_scale.assign(k_scale, k_scale + num_kv_heads);
    p->v_scale.assign(v_scale, v_scale + num_kv_heads);
    p->k_inv.resize(num_kv_heads);
    p->v_inv.resize(num_kv_heads);
  } catch (...) {
    delete p;
    return PA_ERR_NOMEM;
  }
  for (int h = 0; h < num_kv_heads; ++h) {  // float division, rounded once
    volatile float one = 1.0f;
    p->k_inv[h] = one / k_scale[h];
    p->v_inv[h] = one / v_scale[h];
  }
  p->kv_fp8 = true;
  p->kv_dtype = kv_dtype;
  *out = p;
  return PA_OK;
}

void pa_destroy_pool(pa_pool *pool) { delete pool; }

int32_t pa_alloc_block(pa_pool *pool) {
  if (pool == nullptr) return -1;
  std::lock_guard<std::mutex> lock(pool->mu);
  return pa::alloc_block_locked(pool);
}

int pa_incref_block(pa_pool *pool, int32_t block_id) {
  if (pool == nullptr) return PA_ERR_INVAL;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (block_id < 0 || block_id >= pool->num_blocks) return PA_ERR_INVAL;
  const int32_t rc = pool->refcount[(size_t)block_id];
  if (rc == 0 || rc == INT32_MAX) return PA_ERR_STATE;
  pa::add_ref_locked(pool, block_id);
  return PA_OK;
}

int pa_decref_block(pa_pool *pool, int32_t block_id) {
  if (pool == nullptr) return PA_ERR_INVAL;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (block_id < 0 || block_id >= pool->num_blocks) return PA_ERR_INVAL;
  const int32_t rc = pool->refcount[(size_t)block_id];
  if (rc == 0) return PA_ERR_STATE;
  // the prefix index's own reference is dropped by eviction, not here
  if (rc == 1 && pool->prefix.block_entry[(size_t)block_id] >= 0) return PA_ERR_STATE;
  pa::drop_ref_locked(pool, block_id);
  return PA_OK;
}

int32_t pa_get_refcount(const pa_pool *pool, int32_t block_id) {
  if (pool == nullptr) return -1;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (block_id < 0 || block_id >= pool->num_blocks) return -1;
  return pool->refcount[(size_t)block_id];
}

int pa_get_stats(const pa_pool *pool, pa_pool_stats *out) {
  if (pool == nullptr || out == nullptr) return PA_ERR_INVAL;
  std::lock_guard<std::mutex> lock(pool->mu);
  out->total = pool->num_blocks;
  out->used = pool->used;
  out->shared = pool->shared;
  out->free = pool->num_blocks - pool->used;
  return PA_OK;
}

// Slot equation of wzjinhao.cn/news/69573, section "环形上下文与注意力沉淀机制".
int32_t pa_ring_slot(int64_t pos, int32_t sink, int32_t window) {
  if (pos < 0 || sink < 0 || window < 1) return -1;
  if (pos < sink) return (int32_t)pos;
  return (int32_t)(sink + (pos - sink) % window);
}

int pa_compute_slot_mapping(const pa_pool *pool, const int32_t *block_tables, int32_t num_seqs,
                            int32_t max_blocks_per_seq, const int32_t *seq_ids,
                            const int64_t *positions, int32_t n, const pa_ring *ring,
                            int32_t *out) {
  if (pool == nullptr || n < 0 || num_seqs < 0 || max_blocks_per_seq < 0) return PA_ERR_INVAL;
  if (n == 0) return PA_OK;
  if (block_tables == nullptr || seq_ids == nullptr || positions == nullptr || out == nullptr)
    return PA_ERR_INVAL;
  if (!pa::ring_valid(ring)) return PA_ERR_INVAL;
  const int64_t bs = pool->block_size;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = seq_ids[i];
    const int64_t pos = positions[i];
    if (s < 0 || s >= num_seqs || pos < 0) return PA_ERR_INVAL;
    const int64_t r = ring ? (int64_t)pa_ring_slot(pos, ring->sink, ring->window) : pos;
    const int64_t lb = r / bs;
    if (lb >= max_blocks_per_seq) return PA_ERR_INVAL;
    const int32_t phys = block_tables[(int64_t)s * max_blocks_per_seq + lb];
    if (phys < 0 || phys >= pool->num_blocks) return PA_ERR_INVAL;
    const int64_t slot = (int64_t)phys * bs + r % bs;
    if (slot > INT32_MAX) return PA_ERR_INVAL;
    out[i] = (int32_t)slot;
  }
  return PA_OK;
}

const char *pa_status_str(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVAL: return "PA_ERR_INVAL";
    case PA_ERR_NOMEM: return "PA_ERR_NOMEM";
    case PA_ERR_STATE: return "PA_ERR_STATE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    default: return "PA_ERR_UNKNOWN";
  }
}

}  // extern "C"
