// Internal (C++ linkage) launch interface between the C ABI entry points and
// the kernels.  Host-side only types.
#ifndef PA_LAUNCH_H_
#define PA_LAUNCH_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Tokens of one split-K partition: one work-group of kDecodeWaves waves per
// (partition, KV head [, head chunk], sequence); tiles of 16 tokens.
constexpr int kTileTokens = 16;
constexpr int kDecodeWaves = 4;
constexpr float kLog2eHost = 1.4426950408889634f;

// Per-KV-head factors of 8-bit pools, passed by value in kernel arguments:
// the decode kernels take the scales, the cache write the inverse scales.
constexpr int kMaxFp8HeadsHost = 64;

// Formats of 8-bit pools, as the launch functions and the kernels' KVF
// template argument name them (0 = 16-bit pools).
constexpr int kKvE4M3 = 1;
constexpr int kKvE5M2 = 2;
struct KvScales {
  float k[kMaxFp8HeadsHost];
  float v[kMaxFp8HeadsHost];
};

struct DecodeArgs {
  void *out;
  const void *query;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  // split-K partials.  MFMA kernel: slots [waves + B * Hkv][G][D] in the
  // activation type and [..][G][2]; VALU kernel: [B][Hq][max_parts][D] fp32
  // and [..][2].
  float *ws_o;   // partition-normalised outputs (see above for the type)
  float *ws_ml;  // (running max in log2 units, sum)
  int32_t *ws_sched;  // MFMA kernel: tile prefix per sequence [B + 1]
  // Append mode (MFMA kernel, plain paging): the new token of each
  // sequence, key/value [B][Hkv][D] in the activation dtype, is stored at
  // app_slots[b] (8-bit pools: quantised with kv_inv) by the wave that
  // streams the sequence's last tile, before it loads that tile.
  const void *app_key;
  const void *app_value;
  const int32_t *app_slots;
  int64_t num_slots;  // num_blocks * block_size (slots past it are not written)
  const float *rope;  // float2 [S+W][D/2] or null
  int64_t kv_block_stride;  // elements per physical block (block_size * Hkv * D)
  int32_t num_seqs;    // sequences of this launch (at most the schedule capacity)
  int32_t num_blocks;
  int32_t max_context;  // host bound of context_lens (lengths are clamped to it)
  int32_t max_blocks_per_seq;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;        // Hq / Hkv
  int32_t block_shift;  // log2(block_size)
  int32_t partition_tokens;
  int32_t max_parts;
  int32_t min_range_tiles;  // MFMA kernel: shortest stream-K range worth a group
  int32_t seq_cost;         // MFMA kernel: extra cost of a sequence in its range, in tiles
  int32_t young_from;       // MFMA kernel: first group run as its CU's second work-group
  int32_t young_share;      // MFMA kernel: their range size relative to the others, / 1024
  int32_t ring_sink;
  int32_t ring_window;
  float scale_log2;  // scale * log2(e)
  KvScales kv_scale;  // 8-bit pools: dequantisation scales per KV head
  KvScales kv_inv;    // 8-bit pools in append mode: fp32(1 / scale), as the cache write uses
  uint64_t *timeline;  // measurement build only (PA_WAVE_TIMELINE), else null and unused
};

// Per-wave timeline of the stream-K decode (single- and multi-token), compiled only into the
// measurement library (PA_WAVE_TIMELINE; the product library has none of
// it).  The records sit after the workspace's other parts:
//   main kernel, wave gw < kTimelineWaves: 8 uint64 at gw * 8:
//     [0] entry stamp, [1] tile schedule ready, [2] first tile consumed,
//     [3] streaming end, [4] (tiles << 32) | segments begun, [5] XCC id,
//     [6] 1 (record valid), [7] work-group id
//   combine kernel, wave cw < kTimelineCombineWaves: 2 uint64 at
//     kTimelineWaves * 8 + cw * 2: [0] entry stamp, [1] exit stamp with
//     bit 63 set when the wave merged a cut sequence.
// Stamps are s_memrealtime counts (100 MHz).  Waves that exit before
// streaming (no range) leave their record untouched.
constexpr int kTimelineWaves = 8192;
constexpr int kTimelineCombineWaves = 65536;
constexpr size_t kTimelineBytes = (size_t)kTimelineWaves * 8 * 8 + (size_t)kTimelineCombineWaves * 2 * 8;

// Multi-token decode (several new tokens per sequence, causal).
constexpr int kMaxMultiSeqsHost = 1024;  // (sequence, pass group) pairs per launch slice
struct MultiArgs {
  void *out;          // [B, q_len, Hq, D]
  const void *query;  // [B, q_len, Hq, D]
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  // stream-K partials: slots [(groups + B * pgroups) * Hkv * pass_group]
  // [pass_rows][D] in the activation type and [..][pass_rows][2] fp32; tile
  // prefix per (sequence, pass group) [B * pgroups + 1]
  float *ws_o;
  float *ws_ml;
  int32_t *ws_sched;
  int64_t kv_block_stride;  // elements per physical block
  int32_t num_seqs;
  int32_t num_blocks;
  int32_t max_context;
  int32_t max_blocks_per_seq;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;      // Hq / Hkv
  int32_t q_len;
  int32_t rows;       // q_len * group query rows per KV head
  int32_t pass_rows;  // 16 * (row tiles per wave)
  int32_t passes;     // ceil(rows / pass_rows)
  int32_t pass_group; // passes one work-group's waves take together (1, 2 or 4)
  int32_t pgroups;    // ceil(passes / pass_group)
  int32_t groups;     // wave groups (Hkv * pass_group waves each) of the grid
  int32_t min_range_tiles;
  int32_t seq_cost;   // extra cost of a (sequence, pass group) in its range, in tiles
  int32_t young_from;  // first group run as its CU's second work-group (W = 2)
  int32_t young_share; // their range size relative to the others, / 1024
  uint64_t *timeline;  // measurement build only (PA_WAVE_TIMELINE), else null and unused
  int32_t block_shift;
  float scale_log2;
  KvScales kv_scale;  // 8-bit pools: dequantisation scales per KV head
  // Speculative verification over the sink + ring cache: context_lens holds
  // the committed positions n; the q_len drafts' K/V rows [B, q_len, Hkv, D]
  // come from draft_k / draft_v (not the cache) as one extra tile per
  // sequence; rope is the float2 (cos, sin) table of at least
  // sink + window + q_len - 1 positions.
  const void *draft_k;
  const void *draft_v;
  const float *rope;
  int32_t ring_sink;
  int32_t ring_window;
};

// CUs of the current device: the multi-token kernel's persistent grid is
// waves-per-SIMD (1 or 2) work-groups per CU.
int multi_grid();
// Row tiles of 16 query rows one wave holds: registers allow four at
// D = 64 and three at D = 128 (with a four-deep load pipeline).
constexpr int kMultiMaxRowTiles(int head_dim) { return head_dim == 128 ? 3 : 4; }
// Ring verification keeps a second (sink-rotated) query copy in registers:
// at most two row tiles with one wave per SIMD, one with two.
constexpr int kMultiMaxRowTilesRing(int waves) { return waves == 2 ? 1 : 2; }
constexpr int kMaxVerifyDrafts = 16;  // drafts of one ring verification (one key tile)

enum class DecodeKernel { kMfma, kValu };

// Upper bounds the host uses to size the workspace.
constexpr int kMaxSchedSeqsHost = 1024;      // sequences per launch slice
constexpr int kMaxPersistentWavesHost = 8192;  // waves of the stream-K grid

struct DecodeChoice {
  DecodeKernel kernel;
  int heads_per_pass;  // VALU: query heads handled per work-group (1, 2 or 4)
};

DecodeChoice choose_decode_kernel(pa_dtype dtype, int group);
// Waves of the MFMA decode kernel's persistent grid on the current device
// (16-bit query/output dtype; kv8 as in launch_decode).
int decode_mfma_waves(pa_dtype dtype, int head_dim, bool ring, int kv8, int num_kv_heads);
int choose_partition_tokens(int64_t effective_max_context);

// dtype: the query/output dtype; kv8: 0 for 16-bit pools, else the format
// of their 8-bit codes (kKvE4M3 = 1, kKvE5M2 = 2).
hipError_t launch_decode(const DecodeArgs &a, pa_dtype dtype, int head_dim, bool ring, int kv8,
                         DecodeChoice choice, int num_seqs, hipStream_t stream);

hipError_t launch_decode_multi(const MultiArgs &a, pa_dtype dtype, int head_dim, int kv8, int waves,
                               int grid, hipStream_t stream, bool ring = false);

hipError_t launch_reshape_and_cache(pa_dtype dtype, void *k_cache, void *v_cache,
                                    const void *key, const void *value,
                                    const int32_t *slot_mapping, int32_t num_tokens,
                                    int32_t row_elems, int64_t num_slots, hipStream_t stream);

// 8-bit pools: quantise rows of act dtype (F16/BF16) with inverse scales to
// codes of format kv8 (1 = E4M3, 2 = E5M2).
hipError_t launch_reshape_and_cache_fp8(pa_dtype act_dtype, int kv8, void *k_cache, void *v_cache,
                                        const void *key, const void *value,
                                        const int32_t *slot_mapping, int32_t num_tokens,
                                        int32_t num_kv_heads, int32_t head_dim, int64_t num_slots,
                                        const KvScales &inv, hipStream_t stream);

// Copy whole blocks (block_bytes each, a multiple of 16) of both pools; one
// work-group per kCopySegChunks 16-byte chunks of a block.
constexpr int kCopySegChunks = 1024;
hipError_t launch_copy_blocks(void *k_cache, void *v_cache, const int32_t *src_blocks,
                              const int32_t *dst_blocks, int32_t num_pairs, int32_t num_blocks,
                              int64_t block_bytes, hipStream_t stream);

// Debug checks of device-resident decode inputs (counts[4], see pa.h).
hipError_t launch_check_inputs(const int32_t *block_tables, int32_t max_blocks_per_seq,
                               const int32_t *context_lens, int32_t num_seqs, int32_t max_context,
                               int32_t block_size, int32_t num_blocks, int32_t ring_capacity,
                               const int32_t *slots, int32_t num_slot_entries, int64_t num_slots,
                               int32_t *counts, hipStream_t stream);

hipError_t launch_rope_table_init(float *table, int32_t capacity, int32_t head_dim,
                                  float rope_base, hipStream_t stream);

// Streaming-read probe: grid work-groups read `bytes` (a multiple of 16) and
// store one XOR checksum each to out[0 .. grid).
constexpr int kReadProbeMaxGrid = 4096;
hipError_t launch_read_probe(const void *src, int64_t bytes, uint32_t *out, int grid, hipStream_t stream);

}  // namespace pa

#endif  // PA_LAUNCH_H_
