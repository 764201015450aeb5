// C ABI entry points that enqueue device work: argument validation, kernel
// choice, split-K sizing and launch.  The allocator entry points live in
// pool.cpp.
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>

#include "launch.h"
#include "pool_internal.h"

namespace pa {
namespace {

// Kernel-side format of a pool's K/V storage: 0 for 16-bit (or fp32) rows,
// kKvE4M3 / kKvE5M2 for 8-bit codes.
int kv8_format(const pa_pool *pool) {
  if (!pool->kv_fp8) return 0;
  return pool->kv_dtype == PA_FP8_E5M2 ? kKvE5M2 : kKvE4M3;
}

thread_local std::string g_last_hip_error;

int hip_status(hipError_t err) {
  if (err == hipSuccess) return PA_OK;
  g_last_hip_error = hipGetErrorString(err);
  return PA_ERR_HIP;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int env_int(const char *name, int fallback) {
  const char *v = std::getenv(name);
  if (v == nullptr || *v == '\0') return fallback;
  return std::atoi(v);
}

// Overrides of the kernel configuration for tests and measurements
// (pa_set_option).  Each starts from its environment variable, read once
// when the library is loaded; 0 means "the library's own choice".
std::atomic<int32_t> g_options[PA_OPT_COUNT];

int32_t option(pa_option o) { return g_options[o].load(std::memory_order_relaxed); }

struct OptionInit {
  OptionInit() {
    static const char *const names[PA_OPT_COUNT] = {"PA_FORCE_VALU",      "PA_PARTITION_TOKENS",
                                                    "PA_MULTI_WAVES",     "PA_MULTI_ROW_TILES",
                                                    "PA_MULTI_PASS_GROUP", "PA_MULTI_MIN_RANGE",
                                                    "PA_DECODE_SEQ_COST", "PA_MULTI_SEQ_COST",
                                                    "PA_YOUNG_SHARE"};
    for (int i = 0; i < PA_OPT_COUNT; ++i) g_options[i].store(env_int(names[i], 0));
  }
} g_option_init;

int log2_exact(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

struct WorkspaceLayout {
  int partition_tokens;
  int max_parts;
  size_t sched_bytes;  // stream-K tile prefix (MFMA kernel)
  size_t ml_bytes;     // (max, sum) pairs
  size_t o_bytes;      // partial outputs
  size_t total;
};

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

WorkspaceLayout workspace_layout(const pa_pool *pool, int32_t num_seqs, int32_t num_q_heads,
                                 int64_t eff_ctx, bool ring) {
  WorkspaceLayout w{};
  // a partition spans at most 64 blocks (its ids are staged one per lane)
  w.partition_tokens = std::min(choose_partition_tokens(eff_ctx), 64 * pool->block_size);
  w.max_parts = eff_ctx > 0 ? (int)ceil_div(eff_ctx, w.partition_tokens) : 1;
  const int group = num_q_heads / pool->num_kv_heads;
  const int64_t slice = std::min<int64_t>(num_seqs, kMaxSchedSeqsHost);
  if (choose_decode_kernel(pool->dtype, group).kernel == DecodeKernel::kMfma) {
    // stream-K: one slot per wave plus one per (sequence, KV head)
    const size_t waves = (size_t)decode_mfma_waves(pool->dtype, pool->head_dim, ring, kv8_format(pool),
                                                   pool->num_kv_heads);
    const size_t slots = waves + (size_t)slice * pool->num_kv_heads;
    w.sched_bytes = round_up((size_t)(slice + 1) * sizeof(int32_t), 256);
    w.ml_bytes = round_up(slots * group * 2 * sizeof(float), 256);
    w.o_bytes = round_up(slots * group * pool->head_dim * sizeof(float), 256);
    w.total = w.sched_bytes + w.ml_bytes + w.o_bytes;
#ifdef PA_WAVE_TIMELINE
    w.total += kTimelineBytes;  // measurement build: per-wave records after the partials
#endif
    return w;
  }
  if (w.max_parts <= 1) {
    w.max_parts = 1;
    return w;  // single partition: results go straight to the output
  }
  const size_t heads = (size_t)slice * num_q_heads * w.max_parts;
  w.ml_bytes = round_up(heads * 2 * sizeof(float), 256);
  w.o_bytes = round_up(heads * pool->head_dim * sizeof(float), 256);
  w.total = w.ml_bytes + w.o_bytes;
  return w;
}

struct MultiLayout {
  int waves, mt, pass_rows, passes, pass_group, pgroups, seqs_per_launch, grid, groups;
  size_t sched_bytes, ml_bytes, o_bytes, total;
};

// Sizes of one launch slice (at most kMaxMultiSeqsHost (sequence, pass
// group) pairs); slices run one after another and reuse the workspace.
MultiLayout multi_layout(const pa_pool *pool, int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                         bool ring = false) {
  MultiLayout m{};
  const int hkv = pool->num_kv_heads;
  const int group = num_q_heads / hkv;
  const int64_t rows = (int64_t)q_len * group;
  const int max_mt = kMultiMaxRowTiles(pool->head_dim);
  // Many passes (chunked prefill) and 8-bit pools (twice the per-byte
  // arithmetic: verification of the 70B-shaped batch 87.9 us against 99.2 us
  // with one wave) are bound by the per-tile arithmetic: two waves per SIMD
  // with up to three row tiles each (chunked prefill 242 us against 287 us
  // with two); otherwise one wave per SIMD (verification with 16-bit pools:
  // 107 us against 124 us with two waves of three row tiles).
  const int forced_w = option(PA_OPT_MULTI_WAVES);
  m.waves = (forced_w == 1 || forced_w == 2) ? forced_w
            : (pool->kv_fp8 || rows > 3 * 16 * max_mt) ? 2 : 1;
  const int wave_mt = ring ? kMultiMaxRowTilesRing(m.waves) : m.waves == 2 ? std::min(3, max_mt) : max_mt;
  const int forced_mt = option(PA_OPT_MULTI_ROW_TILES);
  m.mt = (int)std::min<int64_t>(forced_mt >= 1 && forced_mt <= wave_mt ? forced_mt : wave_mt, ceil_div(rows, 16));
  m.pass_rows = 16 * m.mt;
  m.passes = (int)ceil_div(rows, m.pass_rows);
  // passes of one head share K/V tiles through L2 when a work-group takes several
  const int forced = option(PA_OPT_MULTI_PASS_GROUP);
  m.pass_group = (forced == 1 || forced == 2 || forced == 4) ? forced
                 : m.passes >= 4 ? 4 : m.passes >= 2 ? 2 : 1;
  m.pgroups = (int)ceil_div(m.passes, m.pass_group);
  m.seqs_per_launch = std::max(1, std::min(num_seqs, kMaxMultiSeqsHost / std::max(1, m.pgroups)));
  const int waves_per_group = hkv * m.pass_group;
  m.grid = std::max(m.waves * multi_grid(), (int)ceil_div(waves_per_group, 4));  // at least one group
  m.groups = (m.grid * 4) / waves_per_group;
  const size_t nv = (size_t)m.seqs_per_launch * m.pgroups;
  const size_t rows_total = (m.groups + nv) * (size_t)waves_per_group * m.pass_rows;
  m.sched_bytes = round_up((nv + 1) * sizeof(int32_t), 256);
  m.ml_bytes = round_up(rows_total * 2 * sizeof(float), 256);
  m.o_bytes = round_up(rows_total * pool->head_dim * sizeof(float), 256);
  m.total = m.sched_bytes + m.ml_bytes + m.o_bytes;
#ifdef PA_WAVE_TIMELINE
  m.total += kTimelineBytes;  // measurement build: per-wave records after the partials
#endif
  return m;
}

constexpr int kMaxMultiQLen = 4096;

// Multi-token decode (ring == nullptr: new tokens already cached) and
// speculative verification over the sink + ring cache (ring != nullptr:
// drafts read from draft_k / draft_v).
int multi_impl(pa_pool *pool, void *out, const void *query, const void *draft_k, const void *draft_v,
               const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
               int32_t num_seqs, int32_t q_len, int32_t num_q_heads, int32_t max_context_len, float scale,
               const pa_ring *ring, void *workspace, size_t workspace_bytes, void *stream) {
  if (pool == nullptr || num_seqs < 0 || q_len < 1 || q_len > pa::kMaxMultiQLen || num_q_heads <= 0 ||
      max_context_len < 0 || max_blocks_per_seq <= 0)
    return PA_ERR_INVAL;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_INVAL;
  const int group = num_q_heads / pool->num_kv_heads;
  // one launch slice must hold every pass of a sequence
  if (pa::ceil_div((int64_t)q_len * group, 16 * pa::kMultiMaxRowTiles(pool->head_dim)) >
      pa::kMaxMultiSeqsHost)
    return PA_ERR_UNSUPPORTED;
  if (pool->dtype != PA_F16 && pool->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (ring != nullptr && pool->kv_fp8) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (out == nullptr || query == nullptr || block_tables == nullptr || context_lens == nullptr)
    return PA_ERR_INVAL;
  if (!pa::aligned16(out) || !pa::aligned16(query)) return PA_ERR_INVAL;
  if ((reinterpret_cast<uintptr_t>(block_tables) | reinterpret_cast<uintptr_t>(context_lens)) & 3u)
    return PA_ERR_INVAL;
  if (ring == nullptr) {
    if (max_context_len > (int64_t)max_blocks_per_seq * pool->block_size) return PA_ERR_INVAL;
  } else {
    // the table covers the ring's slots; the RoPE table covers the drafts'
    // rotations (up to S + W + q_len - 2) at the pool's head size
    if ((int64_t)ring->sink + ring->window > (int64_t)max_blocks_per_seq * pool->block_size) return PA_ERR_INVAL;
    if (ring->rope_table == nullptr || !pa::aligned16(ring->rope_table)) return PA_ERR_INVAL;
    if ((int64_t)ring->rope_capacity < (int64_t)ring->sink + ring->window + q_len - 1 ||
        ring->rope_head_dim != pool->head_dim)
      return PA_ERR_INVAL;
    if (!pa::aligned16(draft_k) || !pa::aligned16(draft_v)) return PA_ERR_INVAL;
  }
  if (!(scale == scale)) return PA_ERR_INVAL;
  const pa::MultiLayout m = pa::multi_layout(pool, num_seqs, q_len, num_q_heads, ring != nullptr);
  if (workspace == nullptr || workspace_bytes < m.total) return PA_ERR_NOMEM;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_INVAL;

  pa::MultiArgs a{};
  a.k_cache = pool->k_cache;
  a.v_cache = pool->v_cache;
  char *ws = static_cast<char *>(workspace);
  a.ws_sched = reinterpret_cast<int32_t *>(ws);
  a.ws_ml = reinterpret_cast<float *>(ws + m.sched_bytes);
  a.ws_o = reinterpret_cast<float *>(ws + m.sched_bytes + m.ml_bytes);
#ifdef PA_WAVE_TIMELINE
  a.timeline = reinterpret_cast<uint64_t *>(ws + m.sched_bytes + m.ml_bytes + m.o_bytes);
#endif
  a.kv_block_stride = (int64_t)pool->block_size * pool->num_kv_heads * pool->head_dim;
  a.num_blocks = pool->num_blocks;
  a.max_context = max_context_len;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.group = group;
  a.q_len = q_len;
  a.rows = q_len * group;
  a.pass_rows = m.pass_rows;
  a.passes = m.passes;
  a.pass_group = m.pass_group;
  a.pgroups = m.pgroups;
  a.groups = m.groups;
  // With two work-groups per CU, the groups past the first work-group of
  // every CU run second on their CU (their waves issue behind the first
  // work-group's) and get 0.8 of the others' ranges: chunked prefill
  // 176.1 -> 168.8 us, E4M3 verification 67.0 -> 65.2 us (0.9: 172.9 /
  // 66.0, 0.7: 173.5 / 65.4, 0.6: 181.2 / 67.8).
  {
    const int wpg = pool->num_kv_heads * m.pass_group;  // waves per group
    const int cus = pa::multi_grid();
    a.young_from = m.grid > cus ? (int)pa::ceil_div((int64_t)cus * 4, wpg) : m.groups;
    const int forced_share = pa::option(PA_OPT_YOUNG_SHARE);
    a.young_share = forced_share >= 1 ? std::min(1024, forced_share * 1024 / 1000) : 819;
  }
  const int forced_range = pa::option(PA_OPT_MULTI_MIN_RANGE);
  a.min_range_tiles = forced_range >= 1 ? forced_range : 4;
  // Stream-K ranges weigh each (sequence, pass group) as this many extra
  // tiles (staging its query rows, writing its output or partial rows).
  // Measured: verification of the 70B-shaped batch 101.7 -> 93.5 us at 6
  // (4: 94.6, 12: 96.9), chunked prefill 211.6 -> 181.0 us, ring
  // verification 36.1 -> 33.6 us.  On the current kernels one wave per
  // SIMD takes 5 (verification 88.4 us at 6, 87.2 at 5, 88.7 at 4; ring
  // verification 0.2 us faster) and two waves per SIMD 6 (chunked prefill
  // 165.8 us against 173.1 at 5; E4M3 verification 63.6 us against 65.9
  // at 8).
  const int forced_cost = pa::option(PA_OPT_MULTI_SEQ_COST);
  a.seq_cost = forced_cost >= 1 ? forced_cost - 1 : m.waves == 1 ? 5 : 6;
  a.block_shift = pa::log2_exact(pool->block_size);
  a.scale_log2 = scale * pa::kLog2eHost;
  if (ring != nullptr) {
    a.rope = ring->rope_table;
    a.ring_sink = ring->sink;
    a.ring_window = ring->window;
  }
  if (pool->kv_fp8)
    for (int h = 0; h < pool->num_kv_heads; ++h) {
      a.kv_scale.k[h] = pool->k_scale[h];
      a.kv_scale.v[h] = pool->v_scale[h];
    }
  const int64_t row_elems = (int64_t)q_len * num_q_heads * pool->head_dim;
  const int esize = pa::dtype_bytes(pool->dtype);
  const int grid = m.grid;
  for (int32_t s0 = 0; s0 < num_seqs; s0 += m.seqs_per_launch) {
    a.num_seqs = std::min(m.seqs_per_launch, num_seqs - s0);
    a.out = static_cast<char *>(out) + s0 * row_elems * esize;
    a.query = static_cast<const char *>(query) + s0 * row_elems * esize;
    a.block_tables = block_tables + (int64_t)s0 * max_blocks_per_seq;
    a.context_lens = context_lens + s0;
    if (ring != nullptr) {
      const int64_t drow = (int64_t)q_len * pool->num_kv_heads * pool->head_dim * esize;
      a.draft_k = static_cast<const char *>(draft_k) + s0 * drow;
      a.draft_v = static_cast<const char *>(draft_v) + s0 * drow;
    }
    const int rc = pa::hip_status(pa::launch_decode_multi(a, pool->dtype, pool->head_dim, pa::kv8_format(pool), m.waves,
                                                          grid, static_cast<hipStream_t>(stream), ring != nullptr));
    if (rc != PA_OK) return rc;
  }
  return PA_OK;
}

}  // namespace

DecodeChoice choose_decode_kernel(pa_dtype dtype, int group) {
  DecodeChoice c;
  const bool force_valu = (option(PA_OPT_FORCE_VALU) != 0);
  // 16-bit and 8-bit pools stream through the MFMA kernel for any group up
  // to 16: it is bound by HBM, so the unused score columns of a small group
  // cost no time (the shared-prefix MHA batch: 61.8 us against 67.1 us for
  // the VALU kernel).
  if (dtype != PA_F32 && group >= 1 && group <= 16 && !force_valu) {
    c.kernel = DecodeKernel::kMfma;
    c.heads_per_pass = group;
    return c;
  }
  c.kernel = DecodeKernel::kValu;
  c.heads_per_pass = group == 1 ? 1 : group == 2 ? 2 : 4;
  return c;
}

int choose_partition_tokens(int64_t eff_ctx) {
  const int forced = option(PA_OPT_PARTITION_TOKENS);
  if (forced >= kTileTokens && forced % kTileTokens == 0) return forced;
  (void)eff_ctx;
  return 512;
}

}  // namespace pa

extern "C" {

const char *pa_last_hip_error(void) { return pa::g_last_hip_error.c_str(); }

int pa_set_option(pa_option opt, int32_t value) {
  if ((int)opt < 0 || (int)opt >= PA_OPT_COUNT || value < 0) return PA_ERR_INVAL;
  pa::g_options[opt].store(value, std::memory_order_relaxed);
  return PA_OK;
}

int32_t pa_get_option(pa_option opt) {
  if ((int)opt < 0 || (int)opt >= PA_OPT_COUNT) return -1;
  return pa::option(opt);
}

int pa_reshape_and_cache(pa_pool *pool, const void *key, const void *value,
                         const int32_t *slot_mapping, int32_t num_tokens, void *stream) {
  if (pool == nullptr || num_tokens < 0) return PA_ERR_INVAL;
  if (num_tokens == 0) return PA_OK;
  if (key == nullptr || value == nullptr || slot_mapping == nullptr) return PA_ERR_INVAL;
  if (!pa::aligned16(key) || !pa::aligned16(value)) return PA_ERR_INVAL;
  if ((reinterpret_cast<uintptr_t>(slot_mapping) & 3u) != 0) return PA_ERR_INVAL;
  if (pool->kv_fp8) {
    pa::KvScales inv{};
    for (int h = 0; h < pool->num_kv_heads; ++h) {
      inv.k[h] = pool->k_inv[h];
      inv.v[h] = pool->v_inv[h];
    }
    return pa::hip_status(pa::launch_reshape_and_cache_fp8(
        pool->dtype, pa::kv8_format(pool), pool->k_cache, pool->v_cache, key, value, slot_mapping, num_tokens,
        pool->num_kv_heads, pool->head_dim, (int64_t)pool->num_blocks * pool->block_size, inv,
        static_cast<hipStream_t>(stream)));
  }
  return pa::hip_status(pa::launch_reshape_and_cache(
      pool->dtype, pool->k_cache, pool->v_cache, key, value, slot_mapping, num_tokens,
      pool->num_kv_heads * pool->head_dim, (int64_t)pool->num_blocks * pool->block_size,
      static_cast<hipStream_t>(stream)));
}

int pa_copy_blocks(pa_pool *pool, const int32_t *src_blocks, const int32_t *dst_blocks,
                   int32_t num_pairs, void *stream) {
  if (pool == nullptr || num_pairs < 0) return PA_ERR_INVAL;
  if (num_pairs == 0) return PA_OK;
  if (src_blocks == nullptr || dst_blocks == nullptr) return PA_ERR_INVAL;
  if ((reinterpret_cast<uintptr_t>(src_blocks) | reinterpret_cast<uintptr_t>(dst_blocks)) & 3u)
    return PA_ERR_INVAL;
  const int64_t elem = pool->kv_fp8 ? 1 : pa::dtype_bytes(pool->dtype);
  const int64_t block_bytes =
      (int64_t)pool->block_size * pool->num_kv_heads * pool->head_dim * elem;
  const int64_t segs = pa::ceil_div(block_bytes / 16, pa::kCopySegChunks);
  if ((int64_t)num_pairs * segs > INT32_MAX) return PA_ERR_UNSUPPORTED;
  return pa::hip_status(pa::launch_copy_blocks(pool->k_cache, pool->v_cache, src_blocks,
                                               dst_blocks, num_pairs, pool->num_blocks, block_bytes,
                                               static_cast<hipStream_t>(stream)));
}

size_t pa_decode_multi_workspace_bytes(const pa_pool *pool, int32_t num_seqs, int32_t q_len,
                                       int32_t num_q_heads, int32_t max_context_len) {
  if (pool == nullptr || num_seqs < 0 || q_len < 1 || q_len > pa::kMaxMultiQLen || num_q_heads <= 0 ||
      max_context_len < 0 || num_q_heads % pool->num_kv_heads != 0)
    return 0;
  if (num_seqs == 0) return 0;
  return pa::multi_layout(pool, num_seqs, q_len, num_q_heads).total;
}

int pa_decode_multi(pa_pool *pool, void *out, const void *query, const int32_t *block_tables,
                    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                    int32_t q_len, int32_t num_q_heads, int32_t max_context_len, float scale,
                    void *workspace, size_t workspace_bytes, void *stream) {
  return pa::multi_impl(pool, out, query, nullptr, nullptr, block_tables, max_blocks_per_seq, context_lens,
                        num_seqs, q_len, num_q_heads, max_context_len, scale, nullptr, workspace, workspace_bytes,
                        stream);
}

size_t pa_decode_verify_ring_workspace_bytes(const pa_pool *pool, int32_t num_seqs, int32_t q_len,
                                             int32_t num_q_heads) {
  if (pool == nullptr || num_seqs <= 0 || q_len < 1 || q_len > pa::kMaxVerifyDrafts || num_q_heads <= 0 ||
      num_q_heads % pool->num_kv_heads != 0)
    return 0;
  return pa::multi_layout(pool, num_seqs, q_len, num_q_heads, true).total;
}

int pa_decode_verify_ring(pa_pool *pool, void *out, const void *query, const void *draft_key,
                          const void *draft_value, const int32_t *block_tables, int32_t max_blocks_per_seq,
                          const int32_t *context_lens, int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                          int32_t max_context_len, float scale, const pa_ring *ring, void *workspace,
                          size_t workspace_bytes, void *stream) {
  if (ring == nullptr || !pa::ring_valid(ring)) return PA_ERR_INVAL;
  if (q_len < 1 || q_len > pa::kMaxVerifyDrafts) return PA_ERR_INVAL;
  if (draft_key == nullptr || draft_value == nullptr) return num_seqs == 0 ? PA_OK : PA_ERR_INVAL;
  return pa::multi_impl(pool, out, query, draft_key, draft_value, block_tables, max_blocks_per_seq, context_lens,
                        num_seqs, q_len, num_q_heads, max_context_len, scale, ring, workspace, workspace_bytes,
                        stream);
}

size_t pa_decode_workspace_bytes(const pa_pool *pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_context_len, const pa_ring *ring) {
  if (pool == nullptr || num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0) return 0;
  if (!pa::ring_valid(ring)) return 0;
  const int64_t eff = pa::effective_context(max_context_len, ring);
  return pa::workspace_layout(pool, num_seqs, num_q_heads, eff, ring != nullptr).total;
}

size_t pa_rope_table_bytes(int32_t capacity, int32_t head_dim) {
  if (capacity <= 0 || head_dim <= 0 || (head_dim & 1)) return 0;
  return (size_t)capacity * (size_t)(head_dim / 2) * 2 * sizeof(float);
}

int pa_check_decode_inputs(const pa_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
                           const pa_ring *ring, const int32_t *slot_mapping, int32_t num_slot_entries,
                           int32_t *counts, void *stream) {
  if (pool == nullptr || counts == nullptr || num_seqs < 0 || num_slot_entries < 0 || max_context_len < 0 ||
      max_blocks_per_seq < 0)
    return PA_ERR_INVAL;
  if (num_seqs > 0 && (block_tables == nullptr || context_lens == nullptr || max_blocks_per_seq == 0))
    return PA_ERR_INVAL;
  if (num_slot_entries > 0 && slot_mapping == nullptr) return PA_ERR_INVAL;
  if ((reinterpret_cast<uintptr_t>(counts) | reinterpret_cast<uintptr_t>(block_tables) |
       reinterpret_cast<uintptr_t>(context_lens) | reinterpret_cast<uintptr_t>(slot_mapping)) & 3u)
    return PA_ERR_INVAL;
  if (ring != nullptr && (ring->sink < 0 || ring->window < 1)) return PA_ERR_INVAL;
  const int32_t capacity = ring != nullptr ? ring->sink + ring->window : 0;
  return pa::hip_status(pa::launch_check_inputs(
      block_tables, max_blocks_per_seq, context_lens, num_seqs, max_context_len, pool->block_size,
      pool->num_blocks, capacity, slot_mapping, num_slot_entries, (int64_t)pool->num_blocks * pool->block_size,
      counts, static_cast<hipStream_t>(stream)));
}

int pa_read_probe(const void *src, size_t bytes, uint32_t *checksums, void *stream) {
  if (src == nullptr || checksums == nullptr || bytes == 0 || (bytes & 15) != 0) return PA_ERR_INVAL;
  if (!pa::aligned16(src) || (reinterpret_cast<uintptr_t>(checksums) & 3u) != 0) return PA_ERR_INVAL;
  // four work-groups per CU
  const int grid = std::min(pa::kReadProbeMaxGrid, 4 * pa::multi_grid());
  return pa::hip_status(pa::launch_read_probe(src, (int64_t)bytes, checksums, grid, static_cast<hipStream_t>(stream)));
}

int pa_rope_table_init(float *table, int32_t capacity, int32_t head_dim, float rope_base,
                       void *stream) {
  if (table == nullptr || capacity <= 0 || (head_dim != 64 && head_dim != 128)) return PA_ERR_INVAL;
  if (!(rope_base > 0.0f) || !pa::aligned16(table)) return PA_ERR_INVAL;
  return pa::hip_status(pa::launch_rope_table_init(table, capacity, head_dim, rope_base,
                                                   static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace pa {
namespace {

// New tokens a decode call appends (one per sequence), or none.
struct AppendInputs {
  const void *key;
  const void *value;
  const int32_t *slots;
};

int decode_impl(pa_pool *pool, void *out, const void *query, const int32_t *block_tables,
                int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                int32_t num_q_heads, int32_t max_context_len, float scale, const pa_ring *ring,
                void *workspace, size_t workspace_bytes, void *stream, const AppendInputs *app) {
  if (pool == nullptr || num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 ||
      max_blocks_per_seq <= 0)
    return PA_ERR_INVAL;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_INVAL;
  const int group = num_q_heads / pool->num_kv_heads;
  if (!pa::ring_valid(ring)) return PA_ERR_INVAL;
  if (pool->kv_fp8 && pa::choose_decode_kernel(pool->dtype, group).kernel != pa::DecodeKernel::kMfma)
    return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (out == nullptr || query == nullptr || block_tables == nullptr || context_lens == nullptr)
    return PA_ERR_INVAL;
  if (!pa::aligned16(out) || !pa::aligned16(query)) return PA_ERR_INVAL;
  if ((reinterpret_cast<uintptr_t>(block_tables) | reinterpret_cast<uintptr_t>(context_lens)) & 3u)
    return PA_ERR_INVAL;
  const int64_t table_tokens = (int64_t)max_blocks_per_seq * pool->block_size;
  if (ring == nullptr) {
    if (max_context_len > table_tokens) return PA_ERR_INVAL;
  } else {
    if ((int64_t)ring->sink + ring->window > table_tokens) return PA_ERR_INVAL;
    if (ring->rope_table == nullptr || !pa::aligned16(ring->rope_table)) return PA_ERR_INVAL;
    // the kernels read table rows 0 .. S+W-1 of head_dim floats each
    if ((int64_t)ring->rope_capacity < (int64_t)ring->sink + ring->window ||
        ring->rope_head_dim != pool->head_dim)
      return PA_ERR_INVAL;
  }
  if (!(scale == scale)) return PA_ERR_INVAL;  // NaN scale

  const int64_t eff = pa::effective_context(max_context_len, ring);
  const pa::WorkspaceLayout w = pa::workspace_layout(pool, num_seqs, num_q_heads, eff, ring != nullptr);
  if (w.total > 0) {
    if (workspace == nullptr || workspace_bytes < w.total) return PA_ERR_NOMEM;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_INVAL;
  }
  if ((int64_t)w.max_parts * num_seqs > INT32_MAX) return PA_ERR_UNSUPPORTED;

  pa::DecodeArgs a{};
  a.out = out;
  a.query = query;
  a.k_cache = pool->k_cache;
  a.v_cache = pool->v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  char *ws = static_cast<char *>(workspace);
  a.ws_sched = w.sched_bytes > 0 ? reinterpret_cast<int32_t *>(ws) : nullptr;
  a.ws_ml = w.ml_bytes > 0 ? reinterpret_cast<float *>(ws + w.sched_bytes) : nullptr;
  a.ws_o = w.o_bytes > 0 ? reinterpret_cast<float *>(ws + w.sched_bytes + w.ml_bytes) : nullptr;
#ifdef PA_WAVE_TIMELINE
  if (w.o_bytes > 0) a.timeline = reinterpret_cast<uint64_t *>(ws + w.sched_bytes + w.ml_bytes + w.o_bytes);
#endif
  a.rope = ring ? ring->rope_table : nullptr;
  a.kv_block_stride = (int64_t)pool->block_size * pool->num_kv_heads * pool->head_dim;
  a.num_seqs = num_seqs;
  a.num_blocks = pool->num_blocks;
  a.max_context = max_context_len;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.group = group;
  a.block_shift = pa::log2_exact(pool->block_size);
  a.partition_tokens = w.partition_tokens;
  a.max_parts = w.max_parts;
  // Plain tiles are cheap, so short ranges lose to start-up and merging;
  // ring tiles also rotate every key and gain from spreading out.
  a.min_range_tiles = ring ? 1 : 4;
  // Stream-K ranges weigh each sequence as this many extra tiles (its start
  // and end: staging, query fragments, output or partial rows).  Measured
  // on the 70B-shaped batch: 8-bit pools 52.0 -> 48.9 us per call at 5
  // (costs 4-6 equal, 9 worse), 16-bit pools 74.1 -> 73.7 us at 1.
  const int forced_cost = pa::option(PA_OPT_DECODE_SEQ_COST);
  a.seq_cost = forced_cost >= 1 ? forced_cost - 1 : pool->kv_fp8 ? 5 : 1;
  // two work-groups per CU (8-bit pools): the second one's share of a range
  // (memory-bound there: 0.9-0.95 measured no faster than equal ranges)
  const int forced_share = pa::option(PA_OPT_YOUNG_SHARE);
  a.young_share = forced_share >= 1 ? std::min(1024, forced_share * 1024 / 1000) : 1024;
  a.young_from = INT32_MAX;  // set by the launcher, which knows the grid
  a.ring_sink = ring ? ring->sink : 0;
  a.ring_window = ring ? ring->window : 1;
  a.scale_log2 = scale * pa::kLog2eHost;
  if (pool->kv_fp8)
    for (int h = 0; h < pool->num_kv_heads; ++h) {
      a.kv_scale.k[h] = pool->k_scale[h];
      a.kv_scale.v[h] = pool->v_scale[h];
      a.kv_inv.k[h] = pool->k_inv[h];
      a.kv_inv.v[h] = pool->v_inv[h];
    }

  const pa::DecodeChoice choice = pa::choose_decode_kernel(pool->dtype, group);
  const int nchunk = choice.kernel == pa::DecodeKernel::kMfma
                         ? 1
                         : (group + choice.heads_per_pass - 1) / choice.heads_per_pass;
  if ((int64_t)pool->num_kv_heads * nchunk > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if (app != nullptr) {
    // the MFMA kernel appends in the same launch; other paths write first
    const bool fused = choice.kernel == pa::DecodeKernel::kMfma && pool->dtype != PA_F32;
    if (fused) {
      a.app_key = app->key;
      a.app_value = app->value;
      a.app_slots = app->slots;
      a.num_slots = (int64_t)pool->num_blocks * pool->block_size;
    } else {
      const int rc = pa_reshape_and_cache(pool, app->key, app->value, app->slots, num_seqs, stream);
      if (rc != PA_OK) return rc;
    }
  }
  return pa::hip_status(pa::launch_decode(a, pool->dtype, pool->head_dim, ring != nullptr,
                                          pa::kv8_format(pool), choice, num_seqs,
                                          static_cast<hipStream_t>(stream)));
}

}  // namespace
}  // namespace pa

// ------------------------------------------------------------------------
// Scratch of the no-allocation entry point.  Device memory the library
// owns: each GPU the library runs on holds one copy of this array until the
// process ends.  Host code never uses the array's name as an address (on
// the host it is only a stand-in for the symbol); it uses the per-device
// address that hipGetSymbolAddress returns.
// ------------------------------------------------------------------------
namespace pa {
namespace {
constexpr size_t kScratchBytes = size_t(32) << 20;
}  // namespace
}  // namespace pa

static __device__ __align__(256) unsigned char scratch[pa::kScratchBytes];

namespace pa {
namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
int scratch_address(void **addr) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxScratchDevices) return PA_ERR_UNSUPPORTED;
  void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (es != hipSuccess) return hip_status(es);
      if (p == nullptr) return PA_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" {

int pa_decode(pa_pool *pool, void *out, const void *query, const int32_t *block_tables,
              int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
              int32_t num_q_heads, int32_t max_context_len, float scale, const pa_ring *ring,
              void *workspace, size_t workspace_bytes, void *stream) {
  return pa::decode_impl(pool, out, query, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                         num_q_heads, max_context_len, scale, ring, workspace, workspace_bytes, stream,
                         nullptr);
}

int pa_decode_append(pa_pool *pool, void *out, const void *query, const void *key, const void *value,
                     const int32_t *slot_mapping, const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                     int32_t max_context_len, float scale, const pa_ring *ring, void *workspace,
                     size_t workspace_bytes, void *stream) {
  if (pool == nullptr || num_seqs < 0) return PA_ERR_INVAL;
  if (num_seqs == 0) return PA_OK;
  if (key == nullptr || value == nullptr || slot_mapping == nullptr) return PA_ERR_INVAL;
  if (!pa::aligned16(key) || !pa::aligned16(value)) return PA_ERR_INVAL;
  if ((reinterpret_cast<uintptr_t>(slot_mapping) & 3u) != 0) return PA_ERR_INVAL;
  const pa::AppendInputs app{key, value, slot_mapping};
  return pa::decode_impl(pool, out, query, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                         num_q_heads, max_context_len, scale, ring, workspace, workspace_bytes, stream,
                         &app);
}

size_t pa_decode_noalloc_scratch_bytes(void) { return pa::kScratchBytes; }

int pa_decode_append_noalloc(pa_pool *pool, void *out, const void *query, const void *key,
                             const void *value, const int32_t *slot_mapping, const int32_t *block_tables,
                             int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t max_context_len, float scale, const pa_ring *ring,
                             void *stream) {
  if (pool == nullptr || num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0) return PA_ERR_INVAL;
  if (num_seqs == 0) return PA_OK;
  if (!pa::ring_valid(ring)) return PA_ERR_INVAL;
  // the same workspace the allocating form needs must fit the scratch array
  const size_t need = pa_decode_workspace_bytes(pool, num_seqs, num_q_heads, max_context_len, ring);
  if (need > pa::kScratchBytes) return PA_ERR_NOMEM;
  void *ws = nullptr;
  const int rc = pa::scratch_address(&ws);
  if (rc != PA_OK) return rc;
  return pa_decode_append(pool, out, query, key, value, slot_mapping, block_tables, max_blocks_per_seq,
                          context_lens, num_seqs, num_q_heads, max_context_len, scale, ring, ws,
                          pa::kScratchBytes, stream);
}

}  // extern "C"
