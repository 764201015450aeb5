// Paged decode attention kernels for gfx950 (MI355X).
//
// What is computed (cited from the pages, by title and section):
//  * "大模型推理内存优化：从 KV Cache 分页到连续批处理的工程实践"
//    (pwwt.cn/news/3010209), section "KV Cache 的内存开销与分页机制": one new
//    token per sequence attends to every cached K/V vector of its request,
//    which the kernel reaches through the request's block table (logical
//    block -> physical block), one extra indirection per block.
//  * "端侧 SLM 显存保活术…" (sheratonhq.com/news/141880), section
//    "注意力寻址：非连续物理块的间接寻址": logical token T lives in logical block
//    T / block_size at offset T % block_size of the physical block the table
//    names.
//  * wzjinhao.cn/news/69573, sections "环形上下文与注意力沉淀机制" and
//    "C++ 环形 KV 缓存管理内核实现": in ring mode the resident keys are the
//    ring slots 0..L-1 (L = min(n, S+W)); keys are rotated by their cache
//    order so RoPE keeps relative distances as the ring slides.
//
// Work decomposition (MI355X-first, not the pages' CUDA design):
//  * decode_mfma_kernel (16-bit K/V or 8-bit codes, GQA group 1..16, plain
//    or sink + ring): stream-K over 16-token tiles, one work-group of 4
//    waves per CU (two on 8-bit pools), one KV head per wave; both
//    contractions on MFMA; a separate combine kernel merges the partials
//    of sequences cut by a range boundary.
//  * decode_valu_kernel (any dtype, any group): persistent work-groups over
//    (partition, KV head, head chunk, sequence) items with VALU dot
//    products; decode_reduce_kernel merges partitions.
//  * Block ids are never staged in LDS: they are wave-uniform per tile and
//    travel through lanes and v_readlane into scalar registers.
//  * The summation order depends only on logical positions and lengths, so
//    outputs are bit-identical under relabelling of physical blocks.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kNW = kDecodeWaves;

// A new tile maximum must exceed the running reference by this many log2
// units before the accumulators are rescaled; weights stay <= 2^8.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ int ring_cache_index(int r, int n, int sink, int window) {
  if (n <= sink + window || r < sink) return r;
  int x = ((r - sink) - (n - window - sink)) % window;
  if (x < 0) x += window;
  return sink + x;
}

// Keys a sequence attends to.  Lengths are clamped to [0, max_context] so a
// bad device-side length can never walk past the block table or the
// split-K workspace.
__device__ __forceinline__ int effective_len(const DecodeArgs &a, int n, bool ring) {
  int len = n < a.max_context ? n : a.max_context;
  if (ring) {
    const int cap = a.ring_sink + a.ring_window;
    len = len < cap ? len : cap;
  }
  return len > 0 ? len : 0;
}

// ---------------------------------------------------------------------------
// Persistent schedule.  Work items are (sequence b, partition p, KV head g)
// with g fastest, so the heads of one partition run side by side.  Every
// work-group derives the item list itself from the device-resident lengths
// (no host synchronisation): s_first[b] = index of the first (b, p) pair of
// sequence b (an exclusive prefix sum of its partition counts; an empty
// sequence still owns one pair, which writes zeros).  Work-groups then take
// items round-robin.
// ---------------------------------------------------------------------------
constexpr int kMaxSchedSeqs = kMaxSchedSeqsHost;

__device__ int build_schedule(const DecodeArgs &a, bool ring, int *s_first, int *s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = a.partition_tokens;
  int carry = 0;
  for (int base = 0; base < a.num_seqs; base += kNW * kWave) {
    const int b = base + tid;
    int v = 0;
    if (b < a.num_seqs) {
      const int L = effective_len(a, a.context_lens[b], ring);
      v = L > 0 ? (L + P - 1) / P : 1;
    }
    int x = v;  // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1) s_wsum[wave] = x;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      woff += w < wave ? s_wsum[w] : 0;
      tot += s_wsum[w];
    }
    if (b < a.num_seqs) s_first[b] = carry + woff + x - v;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) s_first[a.num_seqs] = carry;
  __syncthreads();
  return carry;
}

// Sequence owning pair index bp (s_first is strictly increasing).
__device__ __forceinline__ int find_seq(const int *s_first, int num_seqs, int bp) {
  int lo = 0, hi = num_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_first[mid] <= bp) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Physical block ids of one partition, staged once per wave in a VGPR:
// lane i holds the id of the partition's i-th logical block (a partition
// spans at most 64 blocks).  Ids outside the pool are clamped into it so
// that the kernel never faults (the result is then unspecified).
struct PartitionBlocks {
  int ids;
  int first;  // first logical block of the partition
  int shift;
  __device__ __forceinline__ PartitionBlocks(const DecodeArgs &a, const int32_t *bt, int begin, int end) {
    shift = a.block_shift;
    first = begin >> shift;
    const int last = (end - 1) >> shift;
    const int lane = threadIdx.x & 63;
    const int phys = first + lane <= last ? bt[first + lane] : 0;
    ids = min(max(phys, 0), a.num_blocks - 1);
  }
  // block id of the logical token r (wave-uniform r)
  __device__ __forceinline__ int of_token(int r) const {
    return __builtin_amdgcn_readlane(ids, (r >> shift) - first);
  }
};

// Buffer descriptor over the rows [r0, r0 + valid) of one head in a block:
// rows past `valid` are out of range, so their loads return zeros without
// touching memory.  `head_base` already includes the head offset.
template <int D, class st>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const DecodeArgs &a, const char *head_base,
                                                           int phys, int row_in_block, int valid,
                                                           int64_t row_stride) {
  const char *p = head_base + ((int64_t)phys * a.kv_block_stride + (int64_t)row_in_block * row_stride) *
                                  (int64_t)sizeof(st);
  const int nrec = valid > 0 ? (int)(((valid - 1) * row_stride + D) * sizeof(st)) : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), (short)0, nrec, kBufferWord3);
}

// Combine the per-wave (m, l, o) of one work-group and store either the
// final output (single partition) or the partition's partial.
template <class T, int D, int HMAX>
__device__ __forceinline__ void finish_partition(const DecodeArgs &a, const float (*s_m)[HMAX],
                                                 const float (*s_l)[HMAX],
                                                 const float (*s_o)[HMAX][D], int nheads,
                                                 int hq0, int b, int p, int parts,
                                                 int wave_stride_bytes = HMAX * D * 4) {
  typedef typename T::storage st;
  for (int idx = threadIdx.x; idx < nheads * D; idx += blockDim.x) {
    const int h = idx / D;
    const int d = idx - h * D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) mx = fmaxf(mx, s_m[w][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float mw = s_m[w][h];
      const float wt = mw == -INFINITY ? 0.f : fast_exp2(mw - mx);
      num += wt * reinterpret_cast<const float(*)[D]>(reinterpret_cast<const char *>(s_o) +
                                                         w * wave_stride_bytes)[h][d];
      den += wt * s_l[w][h];
    }
    const int64_t head = (int64_t)b * a.num_q_heads + hq0 + h;
    if (parts == 1) {
      static_cast<st *>(a.out)[head * D + d] = T::from_float(num / den);
    } else {
      const int64_t slot = head * a.max_parts + p;
      a.ws_o[slot * D + d] = num / den;
      if (d == 0) {
        a.ws_ml[slot * 2] = mx;
        a.ws_ml[slot * 2 + 1] = den;
      }
    }
  }
}

template <class T, int D>
__device__ __forceinline__ void zero_rows(const DecodeArgs &a, int b, int hq0, int nheads) {
  typedef typename T::storage st;
  st *out = static_cast<st *>(a.out) + ((int64_t)b * a.num_q_heads + hq0) * D;
  for (int i = threadIdx.x; i < nheads * D; i += blockDim.x) out[i] = T::from_float(0.f);
}

// 8-bit pools: one lane's V codes for one row (D/16 codes), loaded raw and
// widened to the 16-bit chunk the LDS tile holds.
template <int D>
struct V8Chunk;
template <>
struct V8Chunk<128> {
  typedef uint2 type;
  static __device__ __forceinline__ uint2 load(__amdgpu_buffer_rsrc_t r, int off) {
    return buffer_load8<kCacheStream>(r, off);
  }
  template <class T, int F>
  static __device__ __forceinline__ uint4 widen(const uint2 &v) { return fp8x8_to_16<T, F>(v); }
};
template <>
struct V8Chunk<64> {
  typedef uint32_t type;
  static __device__ __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, int off) {
    return buffer_load4<kCacheStream>(r, off);
  }
  template <class T, int F>
  static __device__ __forceinline__ uint2 widen(const uint32_t &v) { return fp8x4_to_16<T, F>(v); }
};

template <int D>
struct VChunk;
template <>
struct VChunk<128> {
  typedef uint4 type;
  static __device__ __forceinline__ uint4 load(__amdgpu_buffer_rsrc_t r, int off) {
    return buffer_load16<kCacheStream>(r, off);
  }
  static __device__ __forceinline__ uint2 half(const uint4 &v, int h) {
    return h == 0 ? make_uint2(v.x, v.y) : make_uint2(v.z, v.w);
  }
  static __device__ __forceinline__ uint4 select(bool keep, const uint4 &v) {
    return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
  }
};
template <>
struct VChunk<64> {
  typedef uint2 type;
  static __device__ __forceinline__ uint2 load(__amdgpu_buffer_rsrc_t r, int off) {
    return buffer_load8<kCacheStream>(r, off);
  }
  static __device__ __forceinline__ uint2 half(const uint2 &v, int) { return v; }
  static __device__ __forceinline__ uint2 select(bool keep, const uint2 &v) {
    return make_uint2(keep ? v.x : 0u, keep ? v.y : 0u);
  }
};

// ---------------------------------------------------------------------------
// MFMA kernel: 16-bit K/V (or 8-bit codes), GQA group G in [1, 16].
//
// Work split (stream-K over tiles).  The batch is the flattened list of
// (sequence b, 16-token tile t), T tiles in all.  Resident waves form groups
// of Hkv consecutive waves; wave gw streams KV head gw % Hkv over the tile
// range of its group gw / Hkv, ceil(T / groups) tiles.  So all waves carry
// the same number of tiles, and the Hkv heads of one tile (one contiguous
// run of every token row) are read at the same time.  Each wave runs a
// shallow load pipeline straight across sequence boundaries: no per-item
// prologue and no cross-wave barrier.  A sequence that starts and ends
// inside one range writes its final output rows directly; a sequence cut
// by a range boundary leaves a partial (running max, sum and normalised
// output) in slot (group + b) * Hkv + g, and decode_streamk_reduce combines
// the partials.
//
// Scores: S[token][head] = K_tile[16 x D] . Q^T[D x 16] with
//   v_mfma_f32_16x16x32_{bf16,f16}; A = K rows (lane: token row16, 8 dims),
//   B = query (lane: head row16, the same 8 dims), so each lane's 16-byte K
//   load is its A fragment.  Lane l receives S[4*(l/16) + j][l % 16].
// Output: O[head][d] += P[head][token] V[token][d] with
//   v_mfma_f32_16x16x16_{bf16,f16}.  The A operand is the lane's own score
//   output (head l%16, tokens 4*(l/16)..+3); V passes through a per-wave LDS
//   tile and comes back as B operands through transposing LDS reads.
// ---------------------------------------------------------------------------
constexpr int kMaxPersistentWaves = kMaxPersistentWavesHost;
// Depth of the per-wave tile pipeline (tiles in flight + the one consumed).
// HBM saturates with one tile in flight per wave (1024 waves x 8 KiB at
// 16 bits); more only lengthens the queues.  16-bit pools keep one tile
// ahead (the 70B-shaped batch: 85.0 us against 85.6 us at four stages, the
// MHA shared-prefix batch 60.4 against 61.4), 8-bit pools, two waves per
// SIMD with twice the per-byte arithmetic, issue each tile's loads just
// before consuming it (47.0 us against 54.9 us at four stages).
template <bool KV8>
constexpr int kStagesFor = KV8 ? 1 : 2;
// Segment-opening tiles per staged chunk (query fragments kept in LDS);
// 8-bit pools keep two so that two work-groups fit a CU's LDS.
template <bool KV8>
constexpr int kQSlotsFor = KV8 ? 2 : 4;

// Per-wave LDS tile for V: row-major, rows padded so that the transposing
// reads of one instruction spread over all banks.
template <int D>
struct MfmaLds {
  static constexpr int kVRowBytes = D * 2 + 32;
  static constexpr int kVBytes = kTileTokens * kVRowBytes;
};

// Tile schedule shared by a work-group: s_tfirst[b] = tiles of sequences
// before b (exclusive prefix of ceil(L_b / 16)), s_len[b] = L_b.  Work-group
// 0 also publishes s_tfirst to the workspace for the reduce kernel.
__device__ int build_tile_schedule(const DecodeArgs &a, bool ring, int *s_tfirst, int *s_len,
                                   int *s_wsum, int *s_newslot = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < a.num_seqs; base += kNW * kWave) {
    const int b = base + tid;
    int v = 0;
    if (b < a.num_seqs) {
      const int n = a.context_lens[b];
      const int L = effective_len(a, n, ring);
      s_len[b] = L;
      v = (L + kTileTokens - 1) / kTileTokens;
      if (s_newslot != nullptr) {  // ring slot of the newest resident token (-1: none)
        const int pos = (n < a.max_context ? n : a.max_context) - 1;
        s_newslot[b] = L <= 0 ? -1
                       : pos < a.ring_sink ? pos
                                           : a.ring_sink + (pos - a.ring_sink) % a.ring_window;
      }
    }
    int x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1) s_wsum[wave] = x;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      woff += w < wave ? s_wsum[w] : 0;
      tot += s_wsum[w];
    }
    if (b < a.num_seqs) s_tfirst[b] = carry + woff + x - v;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) s_tfirst[a.num_seqs] = carry;
  __syncthreads();
  if (blockIdx.x == 0)
    for (int b = tid; b <= a.num_seqs; b += blockDim.x) a.ws_sched[b] = s_tfirst[b];
  return carry;
}

// Groups that get a tile range.  Ranges shorter than a.min_range_tiles
// cost more in start-up and partial merging than they gain in parallelism,
// so small batches leave some groups idle.
__device__ __forceinline__ int active_groups(const DecodeArgs &a, int total_tiles, int groups) {
  const int m = max(1, a.min_range_tiles);
  return max(1, min(groups, (total_tiles + m - 1) / m));
}

// (b, t) of flattened tile y (y < s_tfirst[num_seqs]).
__device__ __forceinline__ void locate_tile(const int *s_tfirst, int num_seqs, int y, int &b,
                                            int &t, int &tiles) {
  int lo = 0, hi = num_seqs;  // largest b with s_tfirst[b] <= y (it has tiles)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_tfirst[mid] <= y) lo = mid;
    else hi = mid;
  }
  b = lo;
  tiles = s_tfirst[b + 1] - s_tfirst[b];
  t = y - s_tfirst[b];
}

// 16-bit pools: one wave per SIMD (a memory-bound wave paired with an older
// neighbour falls behind it).  8-bit pools halve the bytes per tile and the
// per-tile arithmetic then dominates, so two waves per SIMD overlap it.
// APP: the launch also stores each sequence's new token (8-bit pools: its
// codes); a separate instantiation, so plain decode carries none of it.
// KVF: 0 for 16-bit pools, else the 8-bit format (kKvE4M3 or kKvE5M2).
template <class T, int D, bool RING, int KVF, bool APP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, KVF != 0 ? 2 : 1)))
void decode_mfma_kernel(DecodeArgs a) {
  constexpr bool KV8 = KVF != 0;
  constexpr int KB = D / 32;  // score MFMAs per tile
  constexpr int EV = D / 16;  // V elements per lane per row
  constexpr int NB = D / 16;  // output MFMAs per tile (16 dims each)
  constexpr int kVRow = MfmaLds<D>::kVRowBytes;
  typedef typename T::storage st;
  typedef typename VChunk<D>::type vchunk;
  // 8-bit pools (KV8): one byte per K/V element.  A lane's 16-byte K load
  // then carries 16 dimensions, the A operands of two score MFMAs; the
  // query fragments follow the same dimension order.
  constexpr int kQSlots = kQSlotsFor<KV8>;
  constexpr int KVB = KV8 ? 1 : (int)sizeof(st);  // bytes per K/V element
  constexpr int KLD = KV8 ? D / 64 : KB;          // 16-byte K loads per lane per tile
  typedef typename std::conditional<KV8, typename V8Chunk<D>::type, vchunk>::type vload;

  __shared__ int s_tfirst[kMaxSchedSeqs + 1];
  __shared__ int s_len[kMaxSchedSeqs];
  __shared__ int s_newslot[(RING && APP) ? kMaxSchedSeqs : 1];  // ring append only
  __shared__ int s_wsum[kNW];
  __shared__ __align__(16) char s_vtiles[kNW][MfmaLds<D>::kVBytes];
  __shared__ uint4 s_q[kNW][kQSlots * KB * kWave];  // query fragments, lane-major

#ifdef PA_WAVE_TIMELINE
  const uint64_t tl_entry = tl_now();
#endif
  const int total = build_tile_schedule(a, RING, s_tfirst, s_len, s_wsum, (RING && APP) ? s_newslot : nullptr);
#ifdef PA_WAVE_TIMELINE
  const uint64_t tl_sched = tl_now();
  uint64_t tl_first = 0;
  int tl_segs = 0;
#endif
  const int hkv = a.num_kv_heads;
  const int G = a.group;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row16 = lane & 15, grp = lane >> 4;
  const int groups = active_groups(a, total, (gridDim.x * kNW) / hkv);
  // 8-bit pools: the two work-groups of a group run on one XCD (work-group i
  // runs on XCD i mod 8, so work-groups i and i + 8 pair up): E4M3 70B
  // batch 51.2 -> 50.1 us cold, 49.4 -> 49.1 us hot.  16-bit pools keep
  // consecutive work-groups (on neighbouring XCDs), which measured 1 us
  // faster there.
  const int xw = (KV8 && gridDim.x % 16 == 0)
                     ? ((int)(blockIdx.x >> 4) * 8 + (int)(blockIdx.x & 7)) * 2 + (int)((blockIdx.x >> 3) & 1)
                     : (int)blockIdx.x;
  const int gw = xw * kNW + wave;
  const int grp_id = gw / hkv;  // tile range of this wave
  const int g = gw - grp_id * hkv;  // KV head of this wave
  if (grp_id >= groups) return;
  const RangeSplit rs = range_split(weighted_total(total, a.num_seqs, a.seq_cost), groups, a.young_from, a.young_share);
  const int xbeg = weighted_tile(s_tfirst, a.num_seqs, total, a.seq_cost, range_start(rs, grp_id));
  const int xend = weighted_tile(s_tfirst, a.num_seqs, total, a.seq_cost, range_start(rs, grp_id + 1));
  if (xbeg >= xend) return;  // no barriers follow
  const int hq0 = g * G;
  const int64_t head_off = (int64_t)g * D;

  const int64_t row_stride = (int64_t)hkv * D;  // elements between token rows
  const int bmask = (1 << a.block_shift) - 1;
  char *vt = s_vtiles[wave];
  uint4 *qs = s_q[wave];
  const int k_off = (int)((row16 * row_stride + (KV8 ? 16 : 8) * grp) * KVB);
  // query dimension of element 0 of score MFMA kb's fragment in this lane
  auto q_dim = [&](int kb) { return KV8 ? 64 * (kb >> 1) + 16 * grp + 8 * (kb & 1) : 32 * kb + 8 * grp; };
  int v_off[4];
#pragma unroll
  for (int tau = 0; tau < 4; ++tau)
    v_off[tau] = (int)(((4 * grp + tau) * row_stride + EV * row16) * KVB);
  // dequantisation of 8-bit pools: scores by k_scale, outputs by v_scale
  const float sl2 = KV8 ? a.scale_log2 * a.kv_scale.k[g] : a.scale_log2;
  const float vscale = KV8 ? a.kv_scale.v[g] : 1.f;

  // online-softmax state of the current (b, g) segment
  f32x4 acc[NB];
  float m_run = -INFINITY, l_part = 0.f;
  uint4 qf[KB];
  bool seg_whole = false;  // the segment began at tile 0 of its (b, g)

  // Per-lane staged metadata of a chunk of up to 64 tiles: lane i describes
  // tile c0 + i.  Read back with readlane (wave-uniform SGPR values).
  auto rd = [&](int v, int j) { return __builtin_amdgcn_readlane(v, j); };
  // toff: byte offset of the tile's first row of head g from the pool base
  // (the same for K and V); tnrec: bytes the tile's valid rows span.
  int tb = 0, tt = 0, tvalid = 0, tflag = 0, toff_lo = 0, toff_hi = 0, tnrec = 0, tslot = 0;
  int c0 = 0, cnt = 0;
  int app_hi = 0;  // tiles below this index had their new token stored

  // Append (no ring): the new token of a sequence sits in its last tile, and
  // the wave that streams that tile for head g stores the token's K and V
  // rows of head g (from the inputs; 8-bit pools: quantised exactly as the
  // cache write does) when it stages the tile, before any load of it: the
  // wave's own later loads of those addresses are ordered after its stores,
  // so the result equals a cache write followed by the decode.  A lane
  // group of 2 * D * 2 / 16 lanes carries one sequence's two input rows in
  // 16-byte pieces (K first); a piece stores 16 bytes, or 8 codes.
  // Ring mode: the newest token's ring slot Slot(n - 1) picks its tile,
  // which need not be the sequence's last.
  constexpr int kPiecesPerRow = D * (int)sizeof(st) / 16;
  constexpr int kLanesPerEnd = 2 * kPiecesPerRow;
  constexpr int kEndsPerRound = kWave / kLanesPerEnd;
  constexpr int kAppRounds = 4;  // rounds whose loads are issued together
  const int app_e = lane / kLanesPerEnd;
  const bool app_v = lane % kLanesPerEnd >= kPiecesPerRow;
  const int app_piece = lane % kPiecesPerRow;
  // Loads the rows of the next kAppRounds * kEndsPerRound sequences ending in
  // the staged chunk (bits of `em`, which are consumed); bsel = -1 where none.
  auto app_load = [&](unsigned long long &em, u32x4 (&row)[kAppRounds], int (&slot)[kAppRounds],
                      int (&bsel)[kAppRounds]) {
#pragma unroll
    for (int r = 0; r < kAppRounds; ++r) {
      int bs = -1;
#pragma unroll
      for (int e = 0; e < kEndsPerRound; ++e) {
        const int j = em ? __ffsll((long long)em) - 1 : -1;
        em &= em - 1;
        const int be = j >= 0 ? rd(tb, j) : -1;
        if (e == app_e) bs = be;
      }
      const int b = max(bs, 0);  // in range for every lane
      bsel[r] = bs;
      slot[r] = a.app_slots[b];
      const char *src = static_cast<const char *>(app_v ? a.app_value : a.app_key) +
                        (((int64_t)b * hkv + g) * D) * (int64_t)sizeof(st) + 16 * app_piece;
      row[r] = *reinterpret_cast<const u32x4 *>(src);
    }
  };
  auto app_store = [&](const u32x4 (&row)[kAppRounds], const int (&slot)[kAppRounds],
                       const int (&bsel)[kAppRounds]) {
#pragma unroll
    for (int r = 0; r < kAppRounds; ++r) {
      if (bsel[r] >= 0 && slot[r] >= 0 && slot[r] < a.num_slots) {
        char *dst = static_cast<char *>(const_cast<void *>(app_v ? a.v_cache : a.k_cache)) +
                    (((int64_t)slot[r] * hkv + g) * D) * (int64_t)KVB + (16 / (int)sizeof(st)) * KVB * app_piece;
        if constexpr (KV8) {
          const float inv = app_v ? a.kv_inv.v[g] : a.kv_inv.k[g];
          uint32_t c[2];
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t word = row[r][(4 * w + e) / 2];
              const uint16_t b = (uint16_t)(((4 * w + e) & 1) ? (word >> 16) : (word & 0xFFFFu));
              packed |= fp8_code<KVF>(T::to_float(b) * inv) << (8 * e);
            }
            c[w] = packed;
          }
          *reinterpret_cast<uint2 *>(dst) = make_uint2(c[0], c[1]);
        } else {
          *reinterpret_cast<u32x4 *>(dst) = row[r];
        }
      }
    }
  };

  auto stage = [&](int start) {
    c0 = start;
    cnt = min(kWave, xend - start);
    tb = tt = tvalid = tflag = toff_lo = toff_hi = tnrec = 0;
    int tiles = 0;
    if (lane < cnt) locate_tile(s_tfirst, a.num_seqs, c0 + lane, tb, tt, tiles);
    // new-token rows of the sequences ending in this chunk (not yet stored
    // by an earlier, truncated chunk): requested first, so they have arrived
    // by the time the block ids have
    unsigned long long ends = 0;
    u32x4 arow[kAppRounds];
    int aslot[kAppRounds], absel[kAppRounds];
    if constexpr (APP) {
      const bool holds_new = RING ? (s_newslot[tb] >= 0 && s_newslot[tb] / kTileTokens == tt) : tt == tiles - 1;
      ends = __ballot(lane < cnt && c0 + lane >= app_hi && holds_new);
      app_hi = c0 + cnt;
      app_load(ends, arow, aslot, absel);
    }
    const int r0 = kTileTokens * tt;
    // block id of the tile, loaded before the query fragments are fetched so
    // that both are in flight together (lanes past cnt read entry 0)
    const int phys = a.block_tables[(int64_t)tb * a.max_blocks_per_seq + (r0 >> a.block_shift)];
    if (lane < cnt) {
      tvalid = min(kTileTokens, s_len[tb] - r0);
      tflag = (tt == 0 ? 1 : 0) | (tt == tiles - 1 ? 2 : 0);
    }
    // Tiles that open a segment (first tile of a sequence, or the first
    // tile of this wave's range) get a query slot in LDS; a chunk ends
    // before its (kQSlots + 1)-th opening tile.
    const bool opens = lane < cnt && ((tflag & 1) || c0 + lane == xbeg);
    unsigned long long m = __ballot(opens);
    if (__popcll(m) > kQSlots) {
      unsigned long long r = m;
      for (int i = 0; i < kQSlots; ++i) r &= r - 1;
      cnt = __ffsll((long long)r) - 1;
      m &= (1ull << cnt) - 1;
    }
    tslot = opens && lane < cnt ? __popcll(m & ((1ull << lane) - 1)) : 0;
    // fetch the query fragments of the opening tiles (all loads first)
    uint4 qtmp[kQSlots][KB];
    unsigned long long mm = m;
#pragma unroll
    for (int s2 = 0; s2 < kQSlots; ++s2) {
      const int i = mm ? __ffsll((long long)mm) - 1 : 0;
      const int64_t qoff = ((int64_t)rd(tb, i) * a.num_q_heads + hq0) * D * (int64_t)sizeof(st);
      // lanes of padded heads (row16 >= G) fall outside the record range
      const auto qr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char *>(static_cast<const char *>(a.query) + qoff), (short)0,
          mm ? G * D * (int)sizeof(st) : 0, kBufferWord3);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        qtmp[s2][kb] = buffer_load16(qr, (int)((row16 * D + q_dim(kb)) * sizeof(st)));
      mm &= mm - 1;
    }
    if (lane < cnt) {
      const int64_t off = ((int64_t)min(max(phys, 0), a.num_blocks - 1) * a.kv_block_stride +
                           (int64_t)(r0 & bmask) * row_stride + head_off) *
                          (int64_t)KVB;
      toff_lo = (int)(uint32_t)off;
      toff_hi = (int)(off >> 32);
      tnrec = (int)(((tvalid - 1) * row_stride + D) * KVB);  // tvalid >= 1 here
    }
    if constexpr (APP) {
      app_store(arow, aslot, absel);
      while (ends) {  // more sequence ends than one batch (short contexts)
        app_load(ends, arow, aslot, absel);
        app_store(arow, aslot, absel);
      }
      // The tile loads that follow read rows other lanes of this wave just
      // stored.  Lanes are separate threads, so a wavefront-scope
      // acquire-release fence orders the stores before the loads.  It
      // emits no instruction on gfx9 parts: a wavefront's vector memory
      // operations are performed in program order, so a later load of an
      // address the wave stored to returns the stored value (LLVM AMDGPU
      // memory model, wavefront scope); the fence only keeps the compiler
      // from moving the loads above the stores.
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
#pragma unroll
    for (int s2 = 0; s2 < kQSlots; ++s2)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) qs[(s2 * KB + kb) * kWave + lane] = qtmp[s2][kb];
  };

  // Loads of staged tile j (j >= cnt: an empty tile, no memory access).
  // They are unconditional so that every step has the same wait counts.
  auto load_tile = [&](int j, uint4 (&k)[KLD], vload (&v)[4]) {
    const int jj = min(j, kWave - 1);
    const uint64_t off = ((uint64_t)(uint32_t)rd(toff_hi, jj) << 32) | (uint32_t)rd(toff_lo, jj);
    const int nrec = j < cnt ? rd(tnrec, jj) : 0;
    const auto kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(a.k_cache) + off), (short)0, nrec, kBufferWord3);
    const auto vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(a.v_cache) + off), (short)0, nrec, kBufferWord3);
#pragma unroll
    for (int kb = 0; kb < KLD; ++kb) k[kb] = buffer_load16<kCacheStream>(kr, k_off + 64 * kb);
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      if constexpr (KV8) v[tau] = V8Chunk<D>::load(vr, v_off[tau]);
      else v[tau] = VChunk<D>::load(vr, v_off[tau]);
    }
  };

  // Segment start: the query fragment of the tile's sequence from its slot.
  auto begin_segment = [&](int j, int b, bool whole) {
    const int slot = rd(tslot, j);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qf[kb] = qs[(slot * KB + kb) * kWave + lane];
    if constexpr (RING) {
      if constexpr (KV8) rope_frag16_kv8<T, D>(qf, a.rope + (int64_t)(s_len[b] - 1) * D, grp);
      else rope_frag16<T, KB>(qf, a.rope + (int64_t)(s_len[b] - 1) * D, grp);
    }
    m_run = -INFINITY;
    l_part = 0.f;
#pragma unroll
    for (int e = 0; e < NB; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    seg_whole = whole;
  };

  auto process_tile = [&](int j, uint4 (&kraw)[KLD], vload (&vraw)[4]) {
    uint4 kf[KB];
    vchunk vf[4];
    if constexpr (KV8) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint4 w = kraw[kb >> 1];
        kf[kb] = fp8x8_to_16<T, KVF>((kb & 1) ? make_uint2(w.z, w.w) : make_uint2(w.x, w.y));
      }
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) vf[tau] = V8Chunk<D>::template widen<T, KVF>(vraw[tau]);
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kf[kb] = kraw[kb];
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) vf[tau] = vraw[tau];
    }
    const int jj = min(j, kWave - 1);
    const int valid = j < cnt ? rd(tvalid, jj) : 0;
    if constexpr (RING) {
      // keys are stored un-rotated: rotate each by its cache-order index
      const int b = rd(tb, jj), t = rd(tt, jj);
      const int L = s_len[b];
      const int n = a.context_lens[b];
      const int r = kTileTokens * t + row16;
      const int jc = (j < cnt && r < L) ? ring_cache_index(r, n, a.ring_sink, a.ring_window) : 0;
      if constexpr (KV8) rope_frag16_kv8<T, D>(kf, a.rope + (int64_t)jc * D, grp);
      else rope_frag16<T, KB>(kf, a.rope + (int64_t)jc * D, grp);
    }
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s = T::mfma_16x16x32(kf[kb], qf[kb], s);

    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (4 * grp + r < valid) ? s[r] * sl2 : -INFINITY;
    const float lmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if (__any(lmax > m_run + kRescaleSlack)) {
      float tmax = fmaxf(lmax, __shfl_xor(lmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = fast_exp2(m_run - m_new);
      l_part *= alpha;
      float ah[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ah[r] = __shfl(alpha, 4 * grp + r);
#pragma unroll
      for (int e = 0; e < NB; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[e][r] *= ah[r];
      m_run = m_new;
    }
    // (an empty tile right after a reset sees m_run = -inf; keep exp2 finite)
    const float m_ref = m_run == -INFINITY ? 0.f : m_run;
    float pj[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pj[r] = fast_exp2(sc[r] - m_ref);
    l_part += (pj[0] + pj[1]) + (pj[2] + pj[3]);

    // V rows past the context were loaded as zeros (outside the descriptor
    // range), so a zero weight never meets a NaN sentinel.
#pragma unroll
    for (int tau = 0; tau < 4; ++tau)
      *reinterpret_cast<vchunk *>(vt + (4 * grp + tau) * kVRow + sizeof(vchunk) * row16) = vf[tau];
    const uint2 pa = make_uint2(T::pack_pair(pj[0], pj[1]), T::pack_pair(pj[2], pj[3]));
    const char *vr = vt + (4 * grp + (row16 >> 2)) * kVRow + 8 * (row16 & 3);
    uint2 vtr[NB];
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) vtr[jb] = lds_read_tr16_b64(vr + 32 * jb);
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) acc[jb] = T::mfma_16x16x16(pa, vtr[jb], acc[jb]);
    __builtin_amdgcn_sched_group_barrier(0x100, NB, 0);  // all transposing reads first
    __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);  // then the MFMAs
  };

  // Segment end: final rows if the whole sequence was streamed here, else a
  // partial in workspace slot (group + b) * Hkv + g.
  auto end_segment = [&](int b, bool last_of_pair) {
    float l_tot = l_part + __shfl_xor(l_part, 16);
    l_tot += __shfl_xor(l_tot, 32);  // sum over the tile for head row16
    float lh[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lh[r] = __shfl(l_tot, 4 * grp + r);
    if (seg_whole && last_of_pair) {
      st *out = static_cast<st *>(a.out) + ((int64_t)b * a.num_q_heads + hq0) * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * grp + r;
        if (h < G) {
          const float inv = vscale / lh[r];
#pragma unroll
          for (int e = 0; e < NB; ++e) out[h * D + 16 * e + row16] = T::from_float(acc[e][r] * inv);
        }
      }
    } else {
      // the partial's normalised rows are stored in the activation type, like
      // the output (their (m, l) stay fp32)
      const int64_t slot = ((int64_t)grp_id + b) * hkv + g;
      st *po = reinterpret_cast<st *>(a.ws_o) + slot * G * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * grp + r;
        if (h < G) {
          const float inv = vscale / lh[r];
#pragma unroll
          for (int e = 0; e < NB; ++e) po[h * D + 16 * e + row16] = T::from_float(acc[e][r] * inv);
        }
      }
      if (grp == 0 && row16 < G) {
        a.ws_ml[(slot * G + row16) * 2] = m_run;
        a.ws_ml[(slot * G + row16) * 2 + 1] = l_tot;
      }
    }
  };

  // Pipeline of S register buffers: tile j is consumed from buffer j % S
  // while tiles j+1 .. j+S-1 are in flight.
  constexpr int S = kStagesFor<KV8>;
  uint4 kbuf[S][KLD];
  vload vbuf[S][4];
  auto step = [&](int j, uint4 (&kc)[KLD], vload (&vc)[4], uint4 (&kn)[KLD], vload (&vn)[4]) {
    load_tile(j + S - 1, kn, vn);
    if (j < cnt) {
      const int b = rd(tb, j), flag = rd(tflag, j);
      if ((flag & 1) || c0 + j == xbeg) begin_segment(j, b, (flag & 1) != 0);
      process_tile(j, kc, vc);
#ifdef PA_WAVE_TIMELINE
      if (tl_first == 0) tl_first = tl_now();
      tl_segs += ((flag & 1) || c0 + j == xbeg) ? 1 : 0;
#endif
      const bool last = c0 + j == xend - 1;
      if ((flag & 2) || last) end_segment(b, (flag & 2) != 0);
    }
  };

  for (int start = xbeg; start < xend; start += cnt) {
    stage(start);  // sets cnt
#pragma unroll
    for (int u = 0; u < S - 1; ++u) load_tile(u, kbuf[u], vbuf[u]);
    for (int j = 0; j < cnt; j += S) {
#pragma unroll
      for (int u = 0; u < S; ++u)
        step(j + u, kbuf[u], vbuf[u], kbuf[(u + S - 1) % S], vbuf[(u + S - 1) % S]);
    }
  }
#ifdef PA_WAVE_TIMELINE
  const uint64_t tl_end = tl_now();
  if (lane == 0 && a.timeline != nullptr && gw < kTimelineWaves) {
    uint64_t *r = a.timeline + (int64_t)gw * 8;
    r[0] = tl_entry;
    r[1] = tl_sched;
    r[2] = tl_first;
    r[3] = tl_end;
    r[4] = ((uint64_t)(xend - xbeg) << 32) | (uint32_t)tl_segs;
    r[5] = tl_xcc();
    r[6] = 1;
    r[7] = blockIdx.x;
  }
#endif
}

// ---------------------------------------------------------------------------
// Stream-K combine, one work-group per (KV head g, sequence b): the cut
// segments of sequence b sit in slots (q + b) * Hkv + g for the groups q
// whose tile ranges intersect its tiles.
// out = sum_q l_q 2^(m_q - M) o_q / sum_q l_q 2^(m_q - M).  An empty
// sequence gets zero rows; a sequence streamed by one group was written
// directly and is skipped.
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(256) void decode_streamk_reduce_kernel(DecodeArgs a, int groups) {
  typedef typename T::storage st;
  constexpr int DPL = D / kWave;  // output elements per lane
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * kNW + (threadIdx.x >> 6);  // query head within the group
  const int g = blockIdx.y, b = blockIdx.z;
  const int hkv = a.num_kv_heads, G = a.group;
  if (h >= G) return;
#ifdef PA_WAVE_TIMELINE
  const int64_t tl_cw =
      (((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * kNW + (threadIdx.x >> 6);
  uint64_t *tl_rec = (a.timeline != nullptr && tl_cw < kTimelineCombineWaves)
                         ? a.timeline + (int64_t)kTimelineWaves * 8 + tl_cw * 2
                         : nullptr;
  if (tl_rec != nullptr && lane == 0) tl_rec[0] = tl_now();
#endif
  const int t0 = a.ws_sched[b], t1 = a.ws_sched[b + 1];
  const int total = a.ws_sched[a.num_seqs];
  // lane holds DPL adjacent elements (one 4-byte access at D = 128)
  st *out = static_cast<st *>(a.out) + ((int64_t)b * a.num_q_heads + g * G + h) * D + DPL * lane;
  if (t1 == t0) {
#pragma unroll
    for (int k = 0; k < DPL; ++k) out[k] = T::from_float(0.f);
    return;
  }
  const int active = active_groups(a, total, groups);
  const RangeSplit rs = range_split(weighted_total(total, a.num_seqs, a.seq_cost), active, a.young_from, a.young_share);
  const int64_t w0 = (int64_t)t0 + (int64_t)a.seq_cost * (b + 1);  // weighted position of tile 0
  const int q_lo = range_of(rs, w0), q_hi = range_of(rs, w0 + (t1 - t0) - 1);
  if (q_lo == q_hi) return;
  const int nseg = q_hi - q_lo + 1;
  const int64_t slot0 = ((int64_t)q_lo + b) * hkv + g;  // slot of segment s: slot0 + s * hkv
  const int64_t rstride = (int64_t)hkv * G * D;  // between consecutive segments' rows
  float num[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) num[k] = 0.f;
  float den = 0.f, mx = -INFINITY;
  for (int s0 = 0; s0 < nseg; s0 += kWave) {  // chunks of 64 segments, online rescale
    const int cnt = min(kWave, nseg - s0);
    const st *rows = reinterpret_cast<const st *>(a.ws_o) + ((slot0 + (int64_t)s0 * hkv) * G + h) * D + DPL * lane;
    // the rows of the first 8 segments are requested together with the
    // (m, l) pairs (indices clamped into the chunk; extra copies unused)
    float v[8][DPL];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int k = 0; k < DPL; ++k) v[u][k] = T::to_float(rows[min(u, cnt - 1) * rstride + k]);
    float ms = -INFINITY, ls = 0.f;
    if (lane < cnt) {
      const int64_t slot = slot0 + (int64_t)(s0 + lane) * hkv;
      ms = a.ws_ml[(slot * G + h) * 2];
      ls = a.ws_ml[(slot * G + h) * 2 + 1];
    }
    float cmx = ms;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cmx = fmaxf(cmx, __shfl_xor(cmx, off));
    const float m_new = fmaxf(mx, cmx);
    const float scale_old = mx == -INFINITY ? 0.f : fast_exp2(mx - m_new);
    den *= scale_old;
#pragma unroll
    for (int k = 0; k < DPL; ++k) num[k] *= scale_old;
    mx = m_new;
    const float wq = lane < cnt ? ls * fast_exp2(ms - mx) : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < cnt) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wq), u));
        den += w;
#pragma unroll
        for (int k = 0; k < DPL; ++k) num[k] = fmaf(w, v[u][k], num[k]);
      }
    }
    for (int j = 8; j < cnt; j += 8) {  // rarely: more than 8 segments, 8 rows in flight
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int k = 0; k < DPL; ++k) v[u][k] = T::to_float(rows[min(j + u, cnt - 1) * rstride + k]);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j + u < cnt) {
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wq), j + u));
          den += w;
#pragma unroll
          for (int k = 0; k < DPL; ++k) num[k] = fmaf(w, v[u][k], num[k]);
        }
      }
    }
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int k = 0; k < DPL; ++k) out[k] = T::from_float(num[k] * inv);
#ifdef PA_WAVE_TIMELINE
  if (tl_rec != nullptr && lane == 0) tl_rec[1] = tl_now() | (1ull << 63);
#endif
}

// ---------------------------------------------------------------------------
// VALU kernel: any dtype, NH query heads per work-group (heads chunked when
// G > NH).  Each K/V row is spread over LPR lanes with 16-byte loads; a wave
// covers RPW rows per step, each row group keeping its own online-softmax
// state; dot products reduce within the row group with DPP.
// ---------------------------------------------------------------------------
template <class T, int D, bool RING, int NH>
__device__ __forceinline__ void valu_partition(const DecodeArgs &a, int b, int p, int gc,
                                               float (*s_m)[NH], float (*s_l)[NH],
                                               float (*s_o)[NH][D]) {
  typedef typename T::storage st;
  constexpr int EPL = 16 / T::kBytes;  // elements per lane
  constexpr int LPR = D / EPL;         // lanes per row
  constexpr int RPW = kWave / LPR;     // rows per wave step
  constexpr int STEPS = kTileTokens / RPW;
  static_assert(LPR >= 4 && LPR <= 32, "row split");

  const int G = a.group;
  const int nchunk = (G + NH - 1) / NH;
  const int g = gc / nchunk;
  const int c = gc - g * nchunk;
  const int hq0 = g * G + c * NH;
  const int nh = min(NH, G - c * NH);
  const int n = a.context_lens[b];
  const int L = effective_len(a, n, RING);
  const int P = a.partition_tokens;
  const int parts = L > 0 ? (L + P - 1) / P : 1;
  if (p >= parts) return;
  if (L == 0) {
    zero_rows<T, D>(a, b, hq0, nh);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane % LPR, rg = lane / LPR;
  const int begin = p * P;
  const int end = min(L, begin + P);
  const int ntiles = (end - begin + kTileTokens - 1) / kTileTokens;
  // rotate-half partner lives LPR/2 lanes away; lanes li < LPR/2 hold the low half
  const float rsign = li < LPR / 2 ? -1.f : 1.f;
  const int ridx = (li % (LPR / 2)) * EPL;  // frequency index of element 0

  float q[NH][EPL];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    const bool ok = hh < nh;
    const st *qrow = static_cast<const st *>(a.query) + ((int64_t)b * a.num_q_heads + hq0 + (ok ? hh : 0)) * D;
    const uint4 raw = *reinterpret_cast<const uint4 *>(qrow + li * EPL);
    const st *el = reinterpret_cast<const st *>(&raw);
#pragma unroll
    for (int e = 0; e < EPL; ++e) q[hh][e] = ok ? T::to_float(el[e]) : 0.f;
    if constexpr (RING) {
      const float *cs = a.rope + (int64_t)(L - 1) * D + 2 * ridx;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float partner = __shfl_xor(q[hh][e], LPR / 2);
        q[hh][e] = q[hh][e] * cs[2 * e] + rsign * partner * cs[2 * e + 1];
      }
    }
  }

  const int64_t row_stride = (int64_t)a.num_kv_heads * D;
  const int32_t *bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
  const char *kc = static_cast<const char *>(a.k_cache) + (int64_t)g * D * sizeof(st);
  const char *vc = static_cast<const char *>(a.v_cache) + (int64_t)g * D * sizeof(st);
  const int bmask = (1 << a.block_shift) - 1;
  const PartitionBlocks blocks(a, bt, begin, end);
  int off[STEPS];  // byte offset of this lane's 16 bytes in step s of a tile
#pragma unroll
  for (int s = 0; s < STEPS; ++s) off[s] = (int)(((s * RPW + rg) * row_stride + li * EPL) * sizeof(st));

  float m[NH], l[NH], o[NH][EPL];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[hh][e] = 0.f;
  }

  auto load_tile = [&](int t, uint4 (&k)[STEPS], uint4 (&v)[STEPS]) {
    const int r0 = begin + kTileTokens * min(t, ntiles - 1);
    const int valid = t < ntiles ? min(kTileTokens, end - r0) : 0;
    const int phys = blocks.of_token(r0);
    const auto kr = tile_rsrc<D, st>(a, kc, phys, r0 & bmask, valid, row_stride);
    const auto vr = tile_rsrc<D, st>(a, vc, phys, r0 & bmask, valid, row_stride);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      k[s] = buffer_load16<kCacheStream>(kr, off[s]);
      v[s] = buffer_load16<kCacheStream>(vr, off[s]);
    }
  };

  auto process_tile = [&](int t, const uint4 (&kt)[STEPS], const uint4 (&vt)[STEPS]) {
    const int r0 = begin + kTileTokens * t;
    const int valid = end - r0;  // <= 0 past the partition
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const int tok = s * RPW + rg;
      const bool ok = tok < valid;
      const st *ke = reinterpret_cast<const st *>(&kt[s]);
      const st *ve = reinterpret_cast<const st *>(&vt[s]);
      float kf[EPL], vf[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        kf[e] = T::to_float(ke[e]);
        vf[e] = T::to_float(ve[e]);
      }
      if constexpr (RING) {
        const int r = r0 + tok;
        const int j = (ok && r < L) ? ring_cache_index(r, n, a.ring_sink, a.ring_window) : 0;
        const float *cs = a.rope + (int64_t)j * D + 2 * ridx;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float partner = __shfl_xor(kf[e], LPR / 2);
          kf[e] = kf[e] * cs[2 * e] + rsign * partner * cs[2 * e + 1];
        }
      }
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = fmaf(q[hh][e], kf[e], dot);
        dot = group_sum<LPR>(dot);
        if (ok) {
          const float sc = dot * a.scale_log2;
          const float mn = fmaxf(m[hh], sc);
          const float al = fast_exp2(m[hh] - mn);
          const float pp = fast_exp2(sc - mn);
          l[hh] = l[hh] * al + pp;
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[hh][e] = fmaf(o[hh][e], al, pp * vf[e]);
          m[hh] = mn;
        }
      }
    }
  };

  uint4 ka[STEPS], va[STEPS], kb2[STEPS], vb[STEPS];
  if (wave < ntiles) {
    load_tile(wave, ka, va);
    for (int t = wave; t < ntiles; t += 2 * kNW) {
      load_tile(t + kNW, kb2, vb);
      process_tile(t, ka, va);
      load_tile(t + 2 * kNW, ka, va);
      process_tile(t + kNW, kb2, vb);
    }
  }

  // merge the RPW row groups of the wave
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      const float mo = __shfl_xor(m[hh], off);
      const float lo = __shfl_xor(l[hh], off);
      const float mx = fmaxf(m[hh], mo);
      const float wa = m[hh] == -INFINITY ? 0.f : fast_exp2(m[hh] - mx);
      const float wb = mo == -INFINITY ? 0.f : fast_exp2(mo - mx);
      l[hh] = l[hh] * wa + lo * wb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float oo = __shfl_xor(o[hh][e], off);
        o[hh][e] = o[hh][e] * wa + oo * wb;
      }
      m[hh] = mx;
    }
  }

  if (rg == 0) {
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[wave][hh][li * EPL + e] = o[hh][e];
      if (li == 0) {
        s_m[wave][hh] = m[hh];
        s_l[wave][hh] = l[hh];
      }
    }
  }
  __syncthreads();
  finish_partition<T, D, NH>(a, s_m, s_l, s_o, nh, hq0, b, p, parts);
}

template <class T, int D, bool RING, int NH>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  __shared__ int s_first[kMaxSchedSeqs + 1];
  __shared__ int s_wsum[kNW];
  __shared__ float s_m[kNW][NH];
  __shared__ float s_l[kNW][NH];
  __shared__ float s_o[kNW][NH][D];
  const int nchunk = (a.group + NH - 1) / NH;
  const int per_pair = a.num_kv_heads * nchunk;
  const int pairs = build_schedule(a, RING, s_first, s_wsum);
  const int items = pairs * per_pair;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int bp = it / per_pair;
    const int gc = it - bp * per_pair;
    const int b = find_seq(s_first, a.num_seqs, bp);
    valu_partition<T, D, RING, NH>(a, b, bp - s_first[b], gc, s_m, s_l, s_o);
    __syncthreads();  // the next item reuses the merge buffers
  }
}

// ---------------------------------------------------------------------------
// Split-K combine: out = sum_p w_p o_p / sum_p w_p, w_p = l_p 2^(m_p - M).
// One wave per (query head, sequence), four heads per work-group; only
// multi-partition sequences.  Lanes load the partition weights in parallel;
// the partial outputs are then streamed with independent loads.
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a, int ring) {
  typedef typename T::storage st;
  constexpr int DPL = D / kWave;  // output elements per lane
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * kNW + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (h >= a.num_q_heads) return;
  const int L = effective_len(a, a.context_lens[b], ring != 0);
  const int P = a.partition_tokens;
  const int parts = min((L + P - 1) / P, a.max_parts);
  if (parts <= 1) return;
  const int64_t head = (int64_t)b * a.num_q_heads + h;
  const float *ml = a.ws_ml + head * a.max_parts * 2;
  const float *po = a.ws_o + head * a.max_parts * D;
  float mx = -INFINITY;
  for (int q = lane; q < parts; q += kWave) mx = fmaxf(mx, ml[2 * q]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float num[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) num[k] = 0.f;
  float den = 0.f;
  for (int q0 = 0; q0 < parts; q0 += kWave) {
    const int q = q0 + lane;
    const float wq = q < parts ? ml[2 * q + 1] * fast_exp2(ml[2 * q] - mx) : 0.f;
    const int cnt = min(kWave, parts - q0);
#pragma unroll 8
    for (int j = 0; j < cnt; ++j) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wq), j));
      den += w;
      const float *row = po + (int64_t)(q0 + j) * D + lane;
#pragma unroll
      for (int k = 0; k < DPL; ++k) num[k] = fmaf(w, row[k * kWave], num[k]);
    }
  }
  st *out = static_cast<st *>(a.out) + head * D + lane;
#pragma unroll
  for (int k = 0; k < DPL; ++k) out[k * kWave] = T::from_float(num[k] / den);
}

// Work-groups per CU the device can keep resident for a kernel (at most
// per_cu_cap), times the CU count: the persistent grid.
int persistent_grid(const void *kernel, int per_cu_cap) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kNW * kWave, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  return cus * std::max(1, std::min(per_cu, per_cu_cap));
}

// Persistent grid of the MFMA decode kernel: one work-group per CU for
// 16-bit pools (a lone wave per SIMD is never starved by an older
// neighbour, so equal tile counts finish at nearly equal times), two for
// 8-bit pools; at least one group of Hkv waves.
template <class T, int D, bool RING, int KVF>
int mfma_grid(int num_kv_heads) {
  static const int grid_max = std::min(
      persistent_grid(reinterpret_cast<const void *>(&decode_mfma_kernel<T, D, RING, KVF>), KVF != 0 ? 2 : 1),
      kMaxPersistentWaves / kNW);
  return std::max(grid_max, (num_kv_heads + kNW - 1) / kNW);
}

template <class T, int D, bool RING, int KVF = 0>
hipError_t launch_typed(const DecodeArgs &a, DecodeChoice choice, hipStream_t stream) {
  constexpr bool KV8 = KVF != 0;
  const dim3 block(kNW * kWave);
  if constexpr (KV8) {  // 8-bit pools: the MFMA kernel only
    if (choice.kernel != DecodeKernel::kMfma) return hipErrorInvalidValue;
  }
  if constexpr (T::kBytes == 2) {
    if (choice.kernel == DecodeKernel::kMfma) {
      const int grid = mfma_grid<T, D, RING, KVF>(a.num_kv_heads);
      // groups whose first wave lies past the first work-group of every CU
      // run second on their CU
      DecodeArgs b = a;
      const int cus = multi_grid();
      b.young_from = grid > cus ? (cus * kNW + b.num_kv_heads - 1) / b.num_kv_heads : INT32_MAX;
      if (b.app_key != nullptr) {
        hipLaunchKernelGGL((decode_mfma_kernel<T, D, RING, KVF, true>), dim3(grid), block, 0, stream, b);
      } else {
        hipLaunchKernelGGL((decode_mfma_kernel<T, D, RING, KVF>), dim3(grid), block, 0, stream, b);
      }
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL((decode_streamk_reduce_kernel<T, D>),
                         dim3((b.group + kNW - 1) / kNW, b.num_kv_heads, b.num_seqs), block, 0, stream,
                         b, (grid * kNW) / b.num_kv_heads);
      return hipGetLastError();
    }
  }
  if constexpr (KV8) return hipErrorInvalidValue;
  const int64_t pairs_bound = (int64_t)a.num_seqs * a.max_parts;
  const int nchunk = (a.group + choice.heads_per_pass - 1) / choice.heads_per_pass;
  const int64_t items = pairs_bound * a.num_kv_heads * nchunk;
  switch (choice.heads_per_pass) {
    case 1: {
      static const int gmax = persistent_grid(reinterpret_cast<const void *>(&decode_valu_kernel<T, D, RING, 1>), INT32_MAX);
      hipLaunchKernelGGL((decode_valu_kernel<T, D, RING, 1>), dim3((int)std::min<int64_t>(gmax, items)), block, 0, stream, a);
      break;
    }
    case 2: {
      static const int gmax = persistent_grid(reinterpret_cast<const void *>(&decode_valu_kernel<T, D, RING, 2>), INT32_MAX);
      hipLaunchKernelGGL((decode_valu_kernel<T, D, RING, 2>), dim3((int)std::min<int64_t>(gmax, items)), block, 0, stream, a);
      break;
    }
    default: {
      static const int gmax = persistent_grid(reinterpret_cast<const void *>(&decode_valu_kernel<T, D, RING, 4>), INT32_MAX);
      hipLaunchKernelGGL((decode_valu_kernel<T, D, RING, 4>), dim3((int)std::min<int64_t>(gmax, items)), block, 0, stream, a);
      break;
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.max_parts > 1) {
    const dim3 rgrid((a.num_q_heads + kNW - 1) / kNW, a.num_seqs);
    hipLaunchKernelGGL((decode_reduce_kernel<T, D>), rgrid, block, 0, stream, a, RING ? 1 : 0);
    err = hipGetLastError();
  }
  return err;
}

template <class T>
hipError_t launch_dtype(const DecodeArgs &a, int head_dim, bool ring, int kv8,
                        DecodeChoice choice, hipStream_t stream) {
  if constexpr (T::kBytes == 2) {
    if (kv8 == kKvE4M3 || kv8 == kKvE5M2) {
      if (ring) {
        if (kv8 == kKvE5M2)
          return head_dim == 128 ? launch_typed<T, 128, true, kKvE5M2>(a, choice, stream)
                                 : launch_typed<T, 64, true, kKvE5M2>(a, choice, stream);
        return head_dim == 128 ? launch_typed<T, 128, true, kKvE4M3>(a, choice, stream)
                               : launch_typed<T, 64, true, kKvE4M3>(a, choice, stream);
      }
      if (kv8 == kKvE5M2)
        return head_dim == 128 ? launch_typed<T, 128, false, kKvE5M2>(a, choice, stream)
                               : launch_typed<T, 64, false, kKvE5M2>(a, choice, stream);
      return head_dim == 128 ? launch_typed<T, 128, false, kKvE4M3>(a, choice, stream)
                             : launch_typed<T, 64, false, kKvE4M3>(a, choice, stream);
    }
  }
  if (kv8 != 0) return hipErrorInvalidValue;
  if (head_dim == 128)
    return ring ? launch_typed<T, 128, true>(a, choice, stream)
                : launch_typed<T, 128, false>(a, choice, stream);
  return ring ? launch_typed<T, 64, true>(a, choice, stream)
              : launch_typed<T, 64, false>(a, choice, stream);
}

template <class T, bool RING, int KVF>
int mfma_waves_t(int head_dim, int num_kv_heads) {
  return kNW * (head_dim == 128 ? mfma_grid<T, 128, RING, KVF>(num_kv_heads)
                                : mfma_grid<T, 64, RING, KVF>(num_kv_heads));
}

template <class T, bool RING>
int mfma_waves_r(int head_dim, int kv8, int num_kv_heads) {
  if (kv8 == kKvE4M3) return mfma_waves_t<T, RING, kKvE4M3>(head_dim, num_kv_heads);
  if (kv8 == kKvE5M2) return mfma_waves_t<T, RING, kKvE5M2>(head_dim, num_kv_heads);
  return mfma_waves_t<T, RING, 0>(head_dim, num_kv_heads);
}

}  // namespace

int decode_mfma_waves(pa_dtype dtype, int head_dim, bool ring, int kv8, int num_kv_heads) {
  if (dtype == PA_BF16)
    return ring ? mfma_waves_r<BF16, true>(head_dim, kv8, num_kv_heads)
                : mfma_waves_r<BF16, false>(head_dim, kv8, num_kv_heads);
  if (dtype == PA_F16)
    return ring ? mfma_waves_r<F16, true>(head_dim, kv8, num_kv_heads)
                : mfma_waves_r<F16, false>(head_dim, kv8, num_kv_heads);
  return 0;
}

hipError_t launch_decode(const DecodeArgs &args, pa_dtype dtype, int head_dim, bool ring,
                         int kv8, DecodeChoice choice, int num_seqs, hipStream_t stream) {
  if (dtype == PA_F32) choice.kernel = DecodeKernel::kValu;  // no fp32 MFMA kernel
  // The device-side schedule holds up to kMaxSchedSeqs sequences; larger
  // batches run as consecutive slices on the same stream (each slice reuses
  // the workspace).
  const size_t esz = dtype == PA_F32 ? 4 : 2;
  for (int s0 = 0; s0 < num_seqs; s0 += kMaxSchedSeqs) {
    DecodeArgs a = args;
    a.num_seqs = std::min(kMaxSchedSeqs, num_seqs - s0);
    const int64_t qo = (int64_t)s0 * a.num_q_heads * head_dim;
    a.out = static_cast<char *>(args.out) + qo * esz;
    a.query = static_cast<const char *>(args.query) + qo * esz;
    a.block_tables = args.block_tables + (int64_t)s0 * a.max_blocks_per_seq;
    a.context_lens = args.context_lens + s0;
    if (args.app_key != nullptr) {
      const int64_t ko = (int64_t)s0 * a.num_kv_heads * head_dim;
      a.app_key = static_cast<const char *>(args.app_key) + ko * esz;
      a.app_value = static_cast<const char *>(args.app_value) + ko * esz;
      a.app_slots = args.app_slots + s0;
    }
    hipError_t err;
    switch (dtype) {
      case PA_F16: err = launch_dtype<F16>(a, head_dim, ring, kv8, choice, stream); break;
      case PA_BF16: err = launch_dtype<BF16>(a, head_dim, ring, kv8, choice, stream); break;
      default: err = launch_dtype<F32>(a, head_dim, ring, kv8, choice, stream); break;
    }
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace pa
