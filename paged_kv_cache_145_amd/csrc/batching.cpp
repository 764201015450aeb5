// Continuous-batching host driver over the paged pool: decides every
// iteration which requests run and manages their blocks, after the
// scheduler of "大模型推理内存优化：从 KV Cache 分页到连续批处理的工程实践"
// (pwwt.cn/news/3010209).  One scheduling call takes the page's three steps
// in its order:
//   1. decoding requests stay; one that needs another block for the tokens
//      it holds gets one, or sits this iteration out when none is free;
//   2. waiting requests are admitted first come, first served while the
//      batch has room and the free blocks cover the prompt; the first that
//      does not fit returns to the head of the queue and admission stops;
//   3. requests that reached their token budget leave and free their blocks.
// Decoding requests are visited in admission order (the page's map has no
// order); blocks come from the pool's allocator.  Plain C++17, host only.
#include <algorithm>
#include <deque>
#include <mutex>
#include <new>
#include <unordered_set>
#include <vector>

#include "pool_internal.h"

namespace {

enum class ReqState { kWaiting, kDecoding, kFinished };

struct BatchRequest {
  uint64_t id;
  int32_t prompt_len;
  int32_t max_tokens;
  int32_t generated;
  ReqState state;
  std::vector<int32_t> table;
};

}  // namespace

struct pa_batcher {
  pa_pool *pool;
  int32_t max_batch;
  int32_t max_blocks_per_seq;
  std::mutex mu;
  std::deque<BatchRequest> waiting;
  std::vector<BatchRequest> active;  // admission order
  std::unordered_set<uint64_t> known;
};

extern "C" {

int pa_batcher_create(pa_pool *pool, int32_t max_batch, int32_t max_blocks_per_seq, pa_batcher **out) {
  if (out == nullptr) return PA_ERR_INVAL;
  *out = nullptr;
  if (pool == nullptr || max_batch < 1 || max_blocks_per_seq < 1) return PA_ERR_INVAL;
  pa_batcher *b = new (std::nothrow) pa_batcher();
  if (b == nullptr) return PA_ERR_NOMEM;
  b->pool = pool;
  b->max_batch = max_batch;
  b->max_blocks_per_seq = max_blocks_per_seq;
  *out = b;
  return PA_OK;
}

void pa_batcher_destroy(pa_batcher *b) {
  if (b == nullptr) return;
  for (const BatchRequest &r : b->active)
    for (int32_t blk : r.table) pa_decref_block(b->pool, blk);
  delete b;
}

int pa_batcher_add(pa_batcher *b, uint64_t request_id, int32_t prompt_len, int32_t max_tokens) {
  if (b == nullptr || prompt_len < 1 || max_tokens < 1) return PA_ERR_INVAL;
  const int64_t bs = b->pool->block_size;
  if (pa::ceil_div((int64_t)prompt_len + max_tokens, bs) > b->max_blocks_per_seq) return PA_ERR_INVAL;
  std::lock_guard<std::mutex> lock(b->mu);
  if (b->known.count(request_id) != 0) return PA_ERR_STATE;
  try {
    b->waiting.push_back(BatchRequest{request_id, prompt_len, max_tokens, 0, ReqState::kWaiting, {}});
    b->known.insert(request_id);
  } catch (...) {
    return PA_ERR_NOMEM;
  }
  return PA_OK;
}

int pa_batcher_schedule(pa_batcher *b, uint64_t *ids, int32_t *block_tables, int32_t *context_lens,
                        int32_t *write_start, int32_t *write_count, int32_t *prefill,
                        pa_batch_info *info) {
  if (b == nullptr || ids == nullptr || block_tables == nullptr || context_lens == nullptr ||
      write_start == nullptr || write_count == nullptr || prefill == nullptr || info == nullptr)
    return PA_ERR_INVAL;
  std::lock_guard<std::mutex> lock(b->mu);
  const int64_t bs = b->pool->block_size;
  const int32_t mb = b->max_blocks_per_seq;
  *info = pa_batch_info{};
  int32_t n = 0;
  auto emit = [&](const BatchRequest &r, bool pre, int32_t ctx, int32_t start, int32_t count) {
    ids[n] = r.id;
    int32_t *row = block_tables + (int64_t)n * mb;
    std::fill(row, row + mb, -1);
    std::copy(r.table.begin(), r.table.end(), row);
    context_lens[n] = ctx;
    write_start[n] = start;
    write_count[n] = count;
    prefill[n] = pre ? 1 : 0;
    ++n;
  };
  try {
    // step 1: decoding requests, one more block when the tokens they hold need it
    for (BatchRequest &r : b->active) {
      if (r.state != ReqState::kDecoding) continue;
      const int32_t tokens = r.prompt_len + r.generated;
      if (pa::ceil_div(tokens, bs) > (int64_t)r.table.size()) {
        const int32_t blk = pa_alloc_block(b->pool);
        if (blk < 0) {
          info->preempted += 1;
          continue;
        }
        r.table.push_back(blk);
      }
      emit(r, false, tokens, tokens - 1, 1);
    }
    // step 2: first come, first served admission
    while (n < b->max_batch && !b->waiting.empty()) {
      BatchRequest &r = b->waiting.front();
      const int32_t need = (int32_t)pa::ceil_div(r.prompt_len, bs);
      pa_pool_stats st{};
      pa_get_stats(b->pool, &st);
      if (st.free < need) break;  // it stays at the head of the queue
      std::vector<int32_t> table;
      table.reserve((size_t)pa::ceil_div((int64_t)r.prompt_len + r.max_tokens, bs));
      for (int32_t i = 0; i < need; ++i) {
        const int32_t blk = pa_alloc_block(b->pool);
        if (blk < 0) break;  // another user of the pool took blocks meanwhile
        table.push_back(blk);
      }
      if ((int32_t)table.size() < need) {
        for (int32_t blk : table) pa_decref_block(b->pool, blk);
        break;
      }
      b->active.push_back(std::move(r));
      b->waiting.pop_front();
      BatchRequest &a = b->active.back();
      a.table = std::move(table);
      a.state = ReqState::kDecoding;
      emit(a, true, a.prompt_len, 0, a.prompt_len);
      info->prefill += 1;
    }
    // step 3: finished requests leave
    size_t keep = 0;
    for (size_t i = 0; i < b->active.size(); ++i) {
      BatchRequest &r = b->active[i];
      if (r.generated >= r.max_tokens) {
        for (int32_t blk : r.table) pa_decref_block(b->pool, blk);
        info->freed_requests += 1;
        info->freed_blocks += (int32_t)r.table.size();
        b->known.erase(r.id);
      } else {
        if (keep != i) b->active[keep] = std::move(r);
        ++keep;
      }
    }
    b->active.resize(keep);
  } catch (...) {
    return PA_ERR_NOMEM;
  }
  info->scheduled = n;
  info->waiting = (int32_t)b->waiting.size();
  info->active = (int32_t)b->active.size();
  return PA_OK;
}

int pa_batcher_step(pa_batcher *b, uint64_t request_id) {
  if (b == nullptr) return PA_ERR_INVAL;
  std::lock_guard<std::mutex> lock(b->mu);
  for (BatchRequest &r : b->active) {
    if (r.id != request_id) continue;
    if (r.state != ReqState::kDecoding) return PA_ERR_STATE;
    r.generated += 1;
    if (r.generated >= r.max_tokens) r.state = ReqState::kFinished;
    return PA_OK;
  }
  return PA_ERR_INVAL;
}

}  // extern "C"
