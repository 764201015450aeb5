// Multi-token paged attention for gfx950: several new tokens per sequence
// attend causally over the paged cache.  It serves the batched check of
// draft tokens in speculative decoding (wzjinhao.cn/news/69573, section
// "嵌入式流式推理的访存墙与投机瓶颈": the target model scores a step of draft
// tokens in one pass) and chunked prefill ("大模型推理内存优化…"
// (pwwt.cn/news/3010209), section "工程边界与架构取舍": a long prompt is
// processed in pieces between decode steps).
//
// New token i of sequence b sits at position p = L_b - q_len + i (its K/V
// are already cached) and sees positions 0..p.  The q_len * G query rows of
// one KV head (row r = i * G + h) are the M dimension of the MFMA tiles; a
// wave holds MT row tiles (16 * MT rows, a "pass") and longer row sets take
// several passes.
//
// Work split (stream-K, as in the single-token kernel).  Passes are taken
// PG at a time (PG = 1, 2 or 4): a virtual sequence is a (sequence, pass
// group) pair; its tiles are the 16-token tiles up to the last key its rows
// see.  The flattened list of (virtual sequence, tile) is cut into equal
// ranges, one per group of Hkv * PG waves; wave (g, w) of a group streams
// KV head g over the range for pass w of each pass group.  With PG = 1 the
// four waves of a work-group are four heads, so a token row's heads are
// read side by side; with PG = 4 they are four passes of one head over the
// same tiles, so the K/V a pass re-reads comes from the CU's L2 instead of
// HBM.  A virtual sequence that starts and ends inside one range writes its
// output rows directly; one cut by range boundaries leaves normalised
// partials in slots ((group + v) * Hkv + g) * PG + w, merged by
// decode_multi_reduce_kernel.
//
// Ring mode (RING, speculative verification over the sink + ring cache):
// context_lens holds the committed positions n, the resident keys are the
// ring slots 0..L-1 (L = min(n, S + W)) read through the block table, and
// the q_len drafts (positions n..n+q_len-1) are one more tile read from the
// draft K/V buffers, never from the cache.  Row i (draft i, at p = n + i)
// gives what decoding the drafts one at a time would: it sees the sinks,
// the committed window keys its own write would not evict (positions
// >= p + 1 - W) and drafts i + 1 - W .. i.  RoPE keeps the cache's
// relative distances without re-rotating per row: keys are rotated by
// J = pos for sinks and pos - off otherwise (off = max(0, n + 1 - S - W)),
// the row's query by p - off for window keys and by min(p, S + W - 1) for
// sinks (a second score MFMA, only on tiles that hold sinks).
//
// Per 16-token tile:
//   S[token][row] = K_tile . Q^T with v_mfma_f32_16x16x32 (A = the lane's
//   own K row fragment, B = query rows); lane l gets S[4(l/16)+j][l%16];
//   O[row][d] += P[row][token] V[token][d] with v_mfma_f32_16x16x16; V goes
//   through a per-wave LDS tile and returns as B operands through
//   transposing LDS reads, shared by the MT row tiles.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kMqWaves = 4;
constexpr int kMaxMqSeqs = kMaxMultiSeqsHost;  // virtual sequences per launch
constexpr float kMqRescaleSlack = 8.0f;        // log2 units the running max may lag
// Two configurations.  W = 1 (one wave per SIMD, up to three row tiles, a
// two-deep load pipeline: verification of the 70B-shaped batch 102.3 us
// against 103.4 at three stages, 104.4 at four, 106-109 at six): memory-bound
// calls such as draft verification.
// W = 2 (two waves per SIMD, up to three row tiles, one query slot, so two
// work-groups fit a CU): calls with many row passes, where a second wave
// hides the per-tile MFMA -> softmax -> MFMA chain.  Three row tiles fill
// the 256 registers a wave then has with a single load stage (two spill);
// one or two row tiles keep two stages.
template <int W, int MT>
constexpr int kMqStagesFor = (W == 2 && MT >= 3) ? 1 : 2;  // depth of the per-wave tile pipeline
template <int W>
constexpr int kMqQSlotsFor = W == 2 ? 1 : 2;  // segment-opening tiles per staged chunk

// One lane's share of a V row: D / 16 elements, 16 or 8 bytes.
template <int D>
struct MqV;
template <>
struct MqV<128> {
  typedef uint4 type;
  template <int P>
  static __device__ __forceinline__ uint4 load(__amdgpu_buffer_rsrc_t r, int off) {
    return buffer_load16<P>(r, off);
  }
};
template <>
struct MqV<64> {
  typedef uint2 type;
  template <int P>
  static __device__ __forceinline__ uint2 load(__amdgpu_buffer_rsrc_t r, int off) {
    return buffer_load8<P>(r, off);
  }
};

// 8-bit pools: one lane's V codes for a row (D / 16 codes), widened to the
// 16-bit piece the LDS tile holds.
template <int D>
struct MqV8;
template <>
struct MqV8<128> {
  typedef uint2 type;
  template <int P>
  static __device__ __forceinline__ uint2 load(__amdgpu_buffer_rsrc_t r, int off) {
    return buffer_load8<P>(r, off);
  }
  template <class T, int F>
  static __device__ __forceinline__ uint4 widen(const uint2 &v) { return fp8x8_to_16<T, F>(v); }
};
template <>
struct MqV8<64> {
  typedef uint32_t type;
  template <int P>
  static __device__ __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, int off) {
    return buffer_load4<P>(r, off);
  }
  template <class T, int F>
  static __device__ __forceinline__ uint2 widen(const uint32_t &v) { return fp8x4_to_16<T, F>(v); }
};

// Per-wave V tile: row-major, rows padded so the transposing reads of one
// instruction spread over the banks.
template <int D>
struct MqLds {
  static constexpr int kVRowBytes = D * 2 + 32;
  static constexpr int kVBytes = kTileTokens * kVRowBytes;
};

// Rows of pass p and the last key position + 1 that its rows see.
__device__ __forceinline__ void mq_pass(const MultiArgs &a, int L, int p, int &row0, int &row_end,
                                        int &kv_end) {
  row0 = p * a.pass_rows;
  row_end = min(a.rows, row0 + a.pass_rows);
  kv_end = min(max(L - a.q_len + (row_end - 1) / a.group + 1, 0), L);
}

__device__ __forceinline__ int mq_len(const MultiArgs &a, int b) {
  return min(max(a.context_lens[b], 0), a.max_context);
}

// Groups that get a tile range (short ranges cost more than they gain).
__device__ __forceinline__ int mq_active_groups(const MultiArgs &a, int total) {
  const int m = max(1, a.min_range_tiles);
  return max(1, min(a.groups, (total + m - 1) / m));
}

// Tile schedule of the launch: s_tfirst[v] = tiles of virtual sequences
// before v, s_kvend[v] = key positions the rows of v's pass group see.  Work-group 0 also
// publishes s_tfirst to the workspace for the merge kernel.
__device__ int mq_schedule(const MultiArgs &a, int *s_tfirst, int *s_kvend, int *s_wsum, bool ring) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nv = a.num_seqs * a.pgroups;
  int carry = 0;
  for (int base = 0; base < nv; base += kMqWaves * kWave) {
    const int v = base + tid;
    int n = 0;
    if (v < nv) {
      const int b = v / a.pgroups;
      if (ring) {  // committed ring slots, then the draft tile
        const int L = min(mq_len(a, b), a.ring_sink + a.ring_window);
        s_kvend[v] = L;
        n = (L + kTileTokens - 1) / kTileTokens + 1;
      } else {
        const int last = min(a.passes - 1, (v - b * a.pgroups) * a.pass_group + a.pass_group - 1);
        int row0, row_end, kv_end;  // the group's last pass sees the most keys
        mq_pass(a, mq_len(a, b), last, row0, row_end, kv_end);
        s_kvend[v] = kv_end;
        n = (kv_end + kTileTokens - 1) / kTileTokens;
      }
    }
    int x = n;  // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1) s_wsum[wave] = x;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kMqWaves; ++w) {
      woff += w < wave ? s_wsum[w] : 0;
      tot += s_wsum[w];
    }
    if (v < nv) s_tfirst[v] = carry + woff + x - n;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) s_tfirst[nv] = carry;
  __syncthreads();
  if (blockIdx.x == 0)
    for (int v = tid; v <= nv; v += blockDim.x) a.ws_sched[v] = s_tfirst[v];
  return carry;
}

// KVF != 0: the pools hold 8-bit codes of that format (kKvE4M3, kKvE5M2)
// scaled per KV head.  A lane's 16-byte K load then carries 16 dimensions,
// the A operands of two score MFMAs, and the query fragments follow that
// dimension order; codes widen exactly to 16-bit values before the MFMAs and
// the LDS tile.
// NT: the call makes one pass per (sequence, KV head), so each K/V row is
// read once and its loads carry the non-temporal hint.  Calls with several
// passes re-read a head's tiles from L2 (the passes of a work-group share
// them), which the hint would defeat.
// SH: the four waves of a work-group are four passes of one KV head (pass
// group 4), so they walk the same key tiles.  Each tile's K and V then come
// into LDS once for the work-group, a quarter per wave with buffer loads
// that write LDS directly (no registers), kShDepth tiles ahead, one barrier
// per tile; the waves read K fragments and transposed V from there, and a
// segment's query fragments straight from memory.  16-bit pools, D = 128,
// two waves per SIMD (chunked prefill).
template <class T, int D, int MT, int KVF, int W, bool RING, bool NT, bool SH = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(W, W)))
void decode_multi_kernel(MultiArgs a) {
  constexpr bool KV8 = KVF != 0;
  constexpr int kPolicy = NT ? kCacheStream : kCacheNormal;
  static_assert(!(KV8 && RING), "ring verification reads 16-bit pools");
  static_assert(!SH || (!KV8 && !RING && D == 128 && W == 2), "shared tiles: 16-bit pools, D 128, two waves");
  // ring mode keeps a second, sink-rotated copy of each query fragment
  constexpr int kMqQSlots = RING ? 1 : kMqQSlotsFor<W>;
  constexpr int kQCopies = RING ? 2 : 1;
  constexpr int KB = D / 32;  // score MFMAs per row tile and key tile
  constexpr int EV = D / 16;  // V elements per lane per row
  constexpr int NB = D / 16;  // output MFMAs per row tile (16 dims each)
  constexpr int kVRow = MqLds<D>::kVRowBytes;
  constexpr int QF = MT * KB;  // query fragments per lane per segment
  typedef typename T::storage st;
  typedef typename MqV<D>::type vchunk;
  constexpr int KVB = KV8 ? 1 : (int)sizeof(st);  // bytes per K/V element
  constexpr int KLD = KV8 ? D / 64 : KB;          // 16-byte K loads per lane per tile
  typedef typename std::conditional<KV8, typename MqV8<D>::type, vchunk>::type vload;
  __shared__ int s_tfirst[kMaxMqSeqs + 1];
  __shared__ int s_kvend[kMaxMqSeqs];
  __shared__ int s_wsum[kMqWaves];
  __shared__ __align__(16) char s_vt[SH ? 1 : kMqWaves][SH ? 16 : MqLds<D>::kVBytes];
  // SH: [buffer][K rows | V rows], rows of D * 2 bytes without padding; the
  // 16-byte pieces of row r are stored permuted (K: piece p at p ^ r, V: at
  // p ^ 2 (r mod 4)) so that the fragment and transposing reads of one
  // instruction fall in distinct banks
  // SH layout of one buffer: K then V, each four groups (one per loading
  // wave q) of rows q, q + 4, q + 8, q + 12 at 256-byte strides; group q
  // starts at q * kShGroup, 32 bytes past a multiple of 128, so the rows
  // that one fragment or transposing read touches fall in distinct banks.
  // K rows also swap 16-byte pieces within each 64-byte quarter (piece
  // 4 c + e at 4 c + (e ^ (row / 4 mod 2))).  A lane's K fragments and V
  // reads are then one address plus constant offsets.
  constexpr int kShGroup = 4 * D * 2 + 32;       // 1056 bytes
  constexpr int kShHalf = 4 * kShGroup;          // K or V of one tile
  constexpr int kShBuf = 2 * kShHalf;
  constexpr int kShDepth = 3;                    // tiles in flight ahead of the one consumed
  static_assert(kShDepth == 3, "the consuming loop below is unrolled for four buffers");
  __shared__ __align__(16) char s_kv[SH ? (kShDepth + 1) * kShBuf : 16];
  __shared__ uint4 s_q[SH ? 1 : kMqWaves][SH ? 1 : kQCopies * kMqQSlots * QF * kWave];  // query fragments, lane-major

  const int nv = a.num_seqs * a.pgroups;
#ifdef PA_WAVE_TIMELINE
  const uint64_t tl_entry = tl_now();
#endif
  const int total = mq_schedule(a, s_tfirst, s_kvend, s_wsum, RING);
#ifdef PA_WAVE_TIMELINE
  const uint64_t tl_sched = tl_now();
  uint64_t tl_first = 0;
  int tl_segs = 0;
#endif
  const int hkv = a.num_kv_heads, G = a.group, ql = a.q_len, PG = a.pass_group;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row16 = lane & 15, grp = lane >> 4;
  const int groups = mq_active_groups(a, total);
  const int gw = blockIdx.x * kMqWaves + wave;
  const int grp_id = gw / (hkv * PG);  // tile range of this wave
  const int within = gw - grp_id * hkv * PG;
  const int g = within / PG;           // KV head of this wave
  const int w = within - g * PG;       // pass of each pass group
  if (grp_id >= groups) return;        // no barriers follow
  const RangeSplit rs = range_split(weighted_total(total, nv, a.seq_cost), groups, a.young_from, a.young_share);
  const int xbeg = weighted_tile(s_tfirst, nv, total, a.seq_cost, range_start(rs, grp_id));
  const int xend = weighted_tile(s_tfirst, nv, total, a.seq_cost, range_start(rs, grp_id + 1));
  if (xbeg >= xend) return;

  const int64_t row_stride = (int64_t)hkv * D;  // elements between token rows
  const int bmask = (1 << a.block_shift) - 1;
  char *vt = s_vt[SH ? 0 : wave];
  // SH: LDS byte addresses of this lane's first K fragment and first
  // transposing V read in buffer 0 (row row16 = 4 g + q: group q, row g)
  const uint32_t sh_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)s_kv;
  const uint32_t sh_k = sh_lds + (row16 & 3) * kShGroup + (row16 >> 2) * (D * 2) +
                        16 * (grp ^ ((row16 >> 2) & 1));
  const uint32_t sh_v = sh_lds + kShHalf + (row16 >> 2) * kShGroup + grp * (D * 2) + 8 * (row16 & 3);
  uint32_t sh_off = 0;  // SH: byte offset of the consumed tile's buffer
  uint4 *qs = s_q[SH ? 0 : wave];
  const int k_off = (int)((row16 * row_stride + (KV8 ? 16 : 8) * grp) * (int64_t)KVB);
  // query dimension of element 0 of score MFMA kb's fragment in this lane
  auto q_dim = [&](int kb) { return KV8 ? 64 * (kb >> 1) + 16 * grp + 8 * (kb & 1) : 32 * kb + 8 * grp; };
  int v_off[4];
#pragma unroll
  for (int tau = 0; tau < 4; ++tau)
    v_off[tau] = (int)(((4 * grp + tau) * row_stride + EV * row16) * (int64_t)KVB);
  // dequantisation of 8-bit pools: scores by k_scale, outputs by v_scale
  const float kscale = KV8 ? a.kv_scale.k[g] : 1.f;
  const float vscale = KV8 ? a.kv_scale.v[g] : 1.f;

  // segment state
  f32x4 acc[MT][NB];
  float m_run[MT], l_part[MT];
  int limit[MT];  // last key position this lane's row sees in each row tile (-1: none)
  // smallest limit over the valid rows of each row tile (wave-uniform; INT_MAX
  // when the tile holds none): key tiles wholly at or below it need no mask
  int lim_lo[MT];
                  // (ring: the row's draft index i, -1: none)
  int lo_pos[MT];  // ring: oldest window position the row sees (p + 1 - W)
  uint4 qf[MT][KB];
  uint4 qfs[RING ? MT : 1][RING ? KB : 1];  // ring: the sink-rotated copy
  int seg_row0 = 0, seg_row_end = 0;
  bool seg_whole = false;
  // ring: committed length n, resident slots L, rotation offset, the slot
  // of the newest committed position, whether sink rotations differ
  int seg_n = 0, seg_L = 0, seg_off = 0, seg_rn = 0;
  bool seg_dual = false;
  const int S_ = RING ? a.ring_sink : 0, W_ = RING ? a.ring_window : 1;

  // Staged metadata of a chunk of up to 64 tiles (lane i: tile c0 + i),
  // read back with readlane.
  auto rd = [&](int x, int j) { return __builtin_amdgcn_readlane(x, j); };
  int tv = 0, tt = 0, tvalid = 0, tflag = 0, toff_lo = 0, toff_hi = 0, tnrec = 0, tslot = 0;
  int c0 = 0, cnt = 0;
  // query fragments of the staged chunk's opening tiles, between their loads
  // (stage) and their LDS stores (stage_lds)
  uint4 qtmp[kMqQSlots][QF];
  uint4 qsink[RING ? kMqQSlots : 1][RING ? QF : 1];
  auto stage = [&](int start) {
    c0 = start;
    cnt = min(kWave, xend - start);
    tv = tt = tvalid = tflag = toff_lo = toff_hi = tnrec = 0;
    int blk = 0;
    if (lane < cnt) {
      const int y = c0 + lane;
      int lo = 0, hi = nv;  // largest v with s_tfirst[v] <= y (it has tiles)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_tfirst[mid] <= y) lo = mid;
        else hi = mid;
      }
      tv = lo;
      tt = y - s_tfirst[lo];
      const int tiles = s_tfirst[lo + 1] - s_tfirst[lo];
      const int b = lo / a.pgroups;
      const bool draft = RING && tt == tiles - 1;
      if (!draft) {
        blk = a.block_tables[(int64_t)b * a.max_blocks_per_seq + ((kTileTokens * tt) >> a.block_shift)];
        blk = min(max(blk, 0), a.num_blocks - 1);
      }
      tvalid = draft ? ql : min(kTileTokens, s_kvend[lo] - kTileTokens * tt);
      tflag = (tt == 0 ? 1 : 0) | (tt == tiles - 1 ? 2 : 0) | (draft ? 4 : 0);
    }
    // tiles that open a segment get a query slot in LDS; the chunk ends
    // before its (kMqQSlots + 1)-th opening tile
    const bool opens = lane < cnt && ((tflag & 1) || c0 + lane == xbeg);
    unsigned long long m = __ballot(opens);
    if (SH) m = 0;  // segments load their query fragments themselves
    if (__popcll(m) > kMqQSlots) {
      unsigned long long r = m;
      for (int i = 0; i < kMqQSlots; ++i) r &= r - 1;
      cnt = __ffsll((long long)r) - 1;
      m &= (1ull << cnt) - 1;
    }
    tslot = opens && lane < cnt ? __popcll(m & ((1ull << lane) - 1)) : 0;
    unsigned long long mm = m;
#pragma unroll
    for (int s2 = 0; s2 < kMqQSlots; ++s2) {
      const int i = mm ? __ffsll((long long)mm) - 1 : 0;
      const int v = rd(tv, i);
      const int b = v / a.pgroups;
      const int p = (v - b * a.pgroups) * PG + w;  // this wave's pass (none if >= passes)
      const int row_end = min(a.rows, (p + 1) * a.pass_rows);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = p * a.pass_rows + 16 * mt + row16;
        const bool ok = mm != 0 && r < row_end;
        const int qi = ok ? r / G : 0;
        const int h = ok ? r - qi * G : 0;
        const st *q = static_cast<const st *>(a.query) +
                      (((int64_t)b * ql + qi) * a.num_q_heads + (int64_t)g * G + h) * D;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          qtmp[s2][mt * KB + kb] =
              ok ? *reinterpret_cast<const uint4 *>(q + q_dim(kb)) : make_uint4(0u, 0u, 0u, 0u);
        if constexpr (RING) {
          // window copy rotated by p - off, sink copy by min(p, S + W - 1)
          const int n = mq_len(a, b);
          const int p = n + qi;
          const int off = max(0, n + 1 - S_ - W_);
          uint4 fw[KB], fs[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) fw[kb] = fs[kb] = qtmp[s2][mt * KB + kb];
          rope_frag16<T, KB>(fw, a.rope + (int64_t)(p - off) * D, grp);
          rope_frag16<T, KB>(fs, a.rope + (int64_t)min(p, S_ + W_ - 1) * D, grp);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            qtmp[s2][mt * KB + kb] = fw[kb];
            qsink[s2][mt * KB + kb] = fs[kb];
          }
        }
      }
      mm &= mm - 1;
    }
    if (lane < cnt) {
      // the draft tile's rows are those of the draft buffers
      const int64_t off =
          (tflag & 4) ? (((int64_t)(tv / a.pgroups) * ql * hkv + g) * D) * (int64_t)KVB
                      : ((int64_t)blk * a.kv_block_stride + (int64_t)((kTileTokens * tt) & bmask) * row_stride +
                         (int64_t)g * D) * (int64_t)KVB;
      toff_lo = (int)(uint32_t)off;
      toff_hi = (int)(off >> 32);
      tnrec = (int)(((tvalid - 1) * row_stride + D) * (int64_t)KVB);  // tvalid >= 1 here
    }
  };
  // The staged query fragments go to LDS after the chunk's first tile loads
  // have been issued, so those loads overlap the query's arrival.
  auto stage_lds = [&]() {
    if constexpr (!SH) {
#pragma unroll
      for (int s2 = 0; s2 < kMqQSlots; ++s2)
#pragma unroll
        for (int f = 0; f < QF; ++f) qs[(s2 * QF + f) * kWave + lane] = qtmp[s2][f];
    }
    if constexpr (RING) {
#pragma unroll
      for (int s2 = 0; s2 < kMqQSlots; ++s2)
#pragma unroll
        for (int f = 0; f < QF; ++f) qs[((kMqQSlots + s2) * QF + f) * kWave + lane] = qsink[s2][f];
    }
  };

  // Loads of staged tile j (j >= cnt: empty record range, no memory access).
  auto load_tile = [&](int j, uint4 (&k)[KLD], vload (&v)[4]) {
    const int jj = min(j, kWave - 1);
    const uint64_t off = ((uint64_t)(uint32_t)rd(toff_hi, jj) << 32) | (uint32_t)rd(toff_lo, jj);
    const int nrec = j < cnt ? rd(tnrec, jj) : 0;
    const bool draft = RING && (rd(tflag, jj) & 4);
    const char *kbase = static_cast<const char *>(draft ? a.draft_k : a.k_cache);
    const char *vbase = static_cast<const char *>(draft ? a.draft_v : a.v_cache);
    const auto kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(kbase + off), (short)0, nrec, kBufferWord3);
    const auto vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(vbase + off), (short)0, nrec, kBufferWord3);
#pragma unroll
    for (int kb = 0; kb < KLD; ++kb) k[kb] = buffer_load16<kPolicy>(kr, k_off + 64 * kb);
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      if constexpr (KV8) v[tau] = MqV8<D>::template load<kPolicy>(vr, v_off[tau]);
      else v[tau] = MqV<D>::template load<kPolicy>(vr, v_off[tau]);
    }
  };

  // SH: this wave's quarter of staged tile j (rows 4 wave .. 4 wave + 3 of
  // K and of V) into LDS buffer buf; rows past the tile's valid ones fall
  // outside the record range and are written as zeros.
  auto dma_tile = [&](int j, char *buf) {
    if constexpr (SH) {
      // j >= cnt: an empty record (writes zeros into a free buffer), so that
      // every step has the same loads in flight
      const int jj = min(j, kWave - 1);
      const uint64_t off = ((uint64_t)(uint32_t)rd(toff_hi, jj) << 32) | (uint32_t)rd(toff_lo, jj);
      const int nrec = j < cnt ? rd(tnrec, jj) : 0;
      const auto kr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char *>(static_cast<const char *>(a.k_cache) + off), (short)0, nrec, kBufferWord3);
      const auto vr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char *>(static_cast<const char *>(a.v_cache) + off), (short)0, nrec, kBufferWord3);
      // this wave's group: rows 4 g + wave (g = lane / 16), lane's slot s
      const int gq = lane >> 4, slot = lane & 15;
      const int rbytes = (int)((4 * gq + wave) * row_stride * 2);
      const int kpiece = (slot & 12) | ((slot & 3) ^ (gq & 1));
      char *kd = buf + wave * kShGroup;
      char *vd = buf + kShHalf + wave * kShGroup;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (__attribute__((address_space(3))) void *)kd, 16,
                                               rbytes + (kpiece << 4), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void *)vd, 16,
                                               rbytes + (slot << 4), 0, 0, 0);
    }
  };

  auto begin_segment = [&](int j, int v, bool whole) {
    if constexpr (SH) {
      // this wave's pass of virtual sequence v (rows past its last load zeros)
      const int bq = v / a.pgroups;
      const int p = (v - bq * a.pgroups) * PG + w;
      const int row_end = min(a.rows, (p + 1) * a.pass_rows);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = p * a.pass_rows + 16 * mt + row16;
        const bool ok = r < row_end;
        const int qi = ok ? r / G : 0;
        const int h = ok ? r - qi * G : 0;
        const st *q = static_cast<const st *>(a.query) +
                      (((int64_t)bq * ql + qi) * a.num_q_heads + (int64_t)g * G + h) * D;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          qf[mt][kb] = ok ? *reinterpret_cast<const uint4 *>(q + q_dim(kb)) : make_uint4(0u, 0u, 0u, 0u);
      }
    } else {
      const int slot = rd(tslot, j);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qf[mt][kb] = qs[(slot * QF + mt * KB + kb) * kWave + lane];
    }
    const int b = v / a.pgroups;
    const int L = mq_len(a, b);
    int kv_end;
    mq_pass(a, L, (v - b * a.pgroups) * PG + w, seg_row0, seg_row_end, kv_end);  // no rows past the last pass
    if constexpr (RING) {
      seg_n = L;
      seg_L = min(L, S_ + W_);
      seg_off = max(0, L + 1 - S_ - W_);
      seg_rn = L > S_ ? S_ + (L - 1 - S_) % W_ : L - 1;
      seg_dual = L + ql > S_ + W_;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qfs[mt][kb] = qs[((kMqQSlots + rd(tslot, j)) * QF + mt * KB + kb) * kWave + lane];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = seg_row0 + 16 * mt + row16;
      if constexpr (RING) {
        limit[mt] = r < seg_row_end ? r / G : -1;
        lo_pos[mt] = L + r / G + 1 - W_;
      } else {
        limit[mt] = r < seg_row_end ? L - ql + r / G : -1;
        const int r0 = seg_row0 + 16 * mt;
        lim_lo[mt] = __builtin_amdgcn_readfirstlane(r0 < seg_row_end ? L - ql + r0 / G : INT_MAX);
      }
      m_run[mt] = -INFINITY;
      l_part[mt] = 0.f;
#pragma unroll
      for (int e = 0; e < NB; ++e) acc[mt][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    seg_whole = whole;
  };

  const float sl2 = a.scale_log2 * kscale;
  auto process_tile = [&](int j, const uint4 (&kraw)[KLD], const vload (&vraw)[4]) {
    uint4 kf[KB];
    vchunk vf[4];
    // SH: V, already transposed, comes with the K fragments (below)
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 shv[SH ? NB : 1];
    if constexpr (SH) {
      // One asm block reads the tile's K fragments and transposed V and waits
      // for its own reads.  The compiler sees no LDS read of the buffers that
      // the tile loads write, so it adds no waits for those loads of its own
      // (the explicit wait and barrier before this tile order them).
      static_assert(KB == 4 && NB == 8, "SH reads are written for D = 128");
      const uint32_t ka = sh_k + sh_off, va = sh_v + sh_off;
      u32x4 k0, k1, k2, k3;
      asm volatile(
          "ds_read_b128 %0, %12\n\t"
          "ds_read_b128 %1, %12 offset:64\n\t"
          "ds_read_b128 %2, %12 offset:128\n\t"
          "ds_read_b128 %3, %12 offset:192\n\t"
          "ds_read_b64_tr_b16 %4, %13\n\t"
          "ds_read_b64_tr_b16 %5, %13 offset:32\n\t"
          "ds_read_b64_tr_b16 %6, %13 offset:64\n\t"
          "ds_read_b64_tr_b16 %7, %13 offset:96\n\t"
          "ds_read_b64_tr_b16 %8, %13 offset:128\n\t"
          "ds_read_b64_tr_b16 %9, %13 offset:160\n\t"
          "ds_read_b64_tr_b16 %10, %13 offset:192\n\t"
          "ds_read_b64_tr_b16 %11, %13 offset:224\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k0), "=&v"(k1), "=&v"(k2), "=&v"(k3), "=&v"(shv[0]), "=&v"(shv[1]), "=&v"(shv[2]),
            "=&v"(shv[3]), "=&v"(shv[4]), "=&v"(shv[5]), "=&v"(shv[6]), "=&v"(shv[7])
          : "v"(ka), "v"(va)
          : "memory");
      kf[0] = __builtin_bit_cast(uint4, k0);
      kf[1] = __builtin_bit_cast(uint4, k1);
      kf[2] = __builtin_bit_cast(uint4, k2);
      kf[3] = __builtin_bit_cast(uint4, k3);
    } else if constexpr (KV8) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint4 w8 = kraw[kb >> 1];
        kf[kb] = fp8x8_to_16<T, KVF>((kb & 1) ? make_uint2(w8.z, w8.w) : make_uint2(w8.x, w8.y));
      }
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) vf[tau] = MqV8<D>::template widen<T, KVF>(vraw[tau]);
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kf[kb] = kraw[kb];
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) vf[tau] = vraw[tau];
    }
    const int kp0 = kTileTokens * rd(tt, j) + 4 * grp;  // key position of S element 0
    // ring: position of a committed key held by slot r (r < L)
    auto slot_pos = [&](int r) {
      if (r < S_ || seg_n <= S_ + W_) return r;
      int d = seg_rn - r;
      d += d < 0 ? W_ : 0;
      return seg_n - 1 - d;
    };
    const bool dtile = RING && (rd(tflag, j) & 4);
    if constexpr (RING) {
      // rotate this lane's key (row16 of the tile) by J
      const int r = kTileTokens * rd(tt, j) + row16;
      const int pos = dtile ? (row16 < ql ? seg_n + row16 : 0) : (r < seg_L ? slot_pos(r) : 0);
      const int jrot = pos < S_ ? pos : pos - seg_off;
      rope_frag16<T, KB>(kf, a.rope + (int64_t)max(jrot, 0) * D, grp);
    }
    f32x4 sv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sacc = T::mfma_16x16x32(kf[kb], qf[mt][kb], sacc);
      sv[mt] = sacc;
    }
    if constexpr (RING) {
      // sink keys take the sink-rotated query (only tiles holding sinks, and
      // only when the two rotations differ)
      const bool has_sink = dtile ? seg_n < S_ : kTileTokens * rd(tt, j) < S_;
      if (seg_dual && has_sink) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) sacc = T::mfma_16x16x32(kf[kb], qfs[mt][kb], sacc);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int pos = dtile ? seg_n + 4 * grp + r : kp0 + r;  // sink keys: position = slot
            if (pos < S_) sv[mt][r] = sacc[r];
          }
        }
      }
    }
    // V rows past the keys the pass sees were loaded as zeros, so a zero
    // weight never meets a NaN sentinel; rows before hold written values.
    uint2 vtr[NB];
    if constexpr (SH) {
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) vtr[jb] = __builtin_bit_cast(uint2, shv[jb]);
    } else {
#pragma unroll
      for (int tau = 0; tau < 4; ++tau)
        *reinterpret_cast<vchunk *>(vt + (4 * grp + tau) * kVRow + sizeof(vchunk) * row16) = vf[tau];
      const char *vr = vt + (4 * grp + (row16 >> 2)) * kVRow + 8 * (row16 & 3);
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) vtr[jb] = lds_read_tr16_b64(vr + 32 * jb);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float sc[4];
      if constexpr (!RING) {
        // Rows that see the whole tile need no mask; padding rows (past the
        // pass's last) are never stored, so they may see any finite score.
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = sv[mt][r] * sl2;
        if (kTileTokens * rd(tt, j) + kTileTokens - 1 > lim_lo[mt]) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[r] = kp0 + r <= limit[mt] ? sc[r] : -INFINITY;
        }
      } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bool vis;
        if constexpr (RING) {
          if (dtile) {  // draft d: causal, and not evicted by the row's own write
            const int d = 4 * grp + r;
            vis = d < ql && d <= limit[mt] && (seg_n + d < S_ || seg_n + d >= lo_pos[mt]);
          } else {
            const int rs = kp0 + r;
            vis = limit[mt] >= 0 && rs < seg_L && (rs < S_ || slot_pos(rs) >= lo_pos[mt]);
          }
        }
        sc[r] = vis ? sv[mt][r] * sl2 : -INFINITY;
      }
      }
      const float lmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      if (__any(lmax > m_run[mt] + kMqRescaleSlack)) {
        float tmax = fmaxf(lmax, __shfl_xor(lmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run[mt], tmax);
        // a row with no visible key yet keeps m = -inf and alpha = 1
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run[mt] - m_new);
        l_part[mt] *= alpha;
        float ah[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ah[r] = __shfl(alpha, 4 * grp + r);
#pragma unroll
        for (int e = 0; e < NB; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mt][e][r] *= ah[r];
        m_run[mt] = m_new;
      }
      const float m_ref = m_run[mt] == -INFINITY ? 0.f : m_run[mt];
      float pj[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pj[r] = fast_exp2(sc[r] - m_ref);
      l_part[mt] += (pj[0] + pj[1]) + (pj[2] + pj[3]);
      const uint2 pa = make_uint2(T::pack_pair(pj[0], pj[1]), T::pack_pair(pj[2], pj[3]));
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) acc[mt][jb] = T::mfma_16x16x16(pa, vtr[jb], acc[mt][jb]);
    }
  };

  // Segment end: final rows if the whole virtual sequence was streamed here,
  // else partials in slot ((group + v) * Hkv + g) * PG + w.
  auto end_segment = [&](int v, bool last_tile) {
    const bool whole = seg_whole && last_tile;
    const int b = v / a.pgroups;
    const int64_t slot = (((int64_t)grp_id + v) * hkv + g) * PG + w;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float l_tot = l_part[mt] + __shfl_xor(l_part[mt], 16);
      l_tot += __shfl_xor(l_tot, 32);  // the row16 row's sum over this segment
      float lh[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) lh[r] = __shfl(l_tot, 4 * grp + r);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = seg_row0 + 16 * mt + 4 * grp + r;
        if (rr >= seg_row_end) continue;
        const float inv = lh[r] > 0.f ? vscale / lh[r] : 0.f;
        if (whole) {
          const int i = rr / G, h = rr - (rr / G) * G;
          st *out = static_cast<st *>(a.out) +
                    (((int64_t)b * ql + i) * a.num_q_heads + (int64_t)g * G + h) * D;
#pragma unroll
          for (int e = 0; e < NB; ++e) out[16 * e + row16] = T::from_float(acc[mt][e][r] * inv);
        } else {
          // normalised partial rows in the activation type ((m, l) fp32)
          st *po = reinterpret_cast<st *>(a.ws_o) + (slot * a.pass_rows + (rr - seg_row0)) * D;
#pragma unroll
          for (int e = 0; e < NB; ++e) po[16 * e + row16] = T::from_float(acc[mt][e][r] * inv);
        }
      }
      if (!whole && grp == 0) {
        const int rr = seg_row0 + 16 * mt + row16;
        if (rr < seg_row_end) {
          a.ws_ml[(slot * a.pass_rows + (rr - seg_row0)) * 2] = m_run[mt];
          a.ws_ml[(slot * a.pass_rows + (rr - seg_row0)) * 2 + 1] = l_tot;
        }
      }
    }
  };

  auto step = [&](int j, const uint4 (&kc)[KLD], const vload (&vc)[4]) {
    const int v = rd(tv, j), flag = rd(tflag, j);
    if ((flag & 1) || c0 + j == xbeg) begin_segment(j, v, (flag & 1) != 0);
    process_tile(j, kc, vc);
#ifdef PA_WAVE_TIMELINE
    if (tl_first == 0) tl_first = tl_now();
    tl_segs += ((flag & 1) || c0 + j == xbeg) ? 1 : 0;
#endif
    if ((flag & 2) || c0 + j == xend - 1) end_segment(v, (flag & 2) != 0);
  };

  // measurement build: this wave's timeline record
  auto tl_finish = [&]() {
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
  };

  // S register buffers: tile j is consumed from buffer j % S while the next
  // S - 1 tiles are in flight.  Loads are unconditional (empty past cnt) so
  // every step sees the same loads in flight and the same wait counts.
  if constexpr (SH) {
    // Tile j of a chunk sits in buffer j mod 4.  Per tile: this wave's loads
    // of tile j done (two loads per tile, issued in order, those of the
    // kShDepth - 1 later tiles may still be in flight), a barrier (every
    // quarter of tile j in LDS, every wave done with tile j - 1), the loads
    // of tile j + kShDepth into the buffer tile j - 1 used, then tile j.
    // The four waves share the range and the chunking, so they meet the
    // same barriers.  Stores (segment ends) are drained before the next
    // wait, so the count below covers only the tile loads.
    constexpr int kVmWait = 2 * (kShDepth - 1);  // vmcnt field of s_waitcnt (< 16)
    constexpr int kWaitImm = kVmWait | (0x7 << 4) | (0xF << 8);  // expcnt, lgkmcnt unchanged
    uint4 kd[KLD];
    vload vd[4];
    auto sh_step = [&](int j, int cur, int next) {
      if (j >= cnt) return;  // wave-uniform
      __builtin_amdgcn_s_waitcnt(kWaitImm);
      // a bare barrier: __syncthreads() adds a release fence, which waits
      // for every load in flight (the next tiles' too); LDS needs none
      __builtin_amdgcn_s_barrier();
      dma_tile(j + kShDepth, s_kv + next * kShBuf);
      sh_off = cur * kShBuf;
      const bool ends = (rd(tflag, j) & 2) || c0 + j == xend - 1;
      step(j, kd, vd);
      if (ends) __builtin_amdgcn_s_waitcnt(0);  // this segment's stores
    };
    for (int start = xbeg; start < xend; start += cnt) {
      stage(start);  // sets cnt
      stage_lds();
      __syncthreads();  // the previous chunk's tiles are consumed
      dma_tile(0, s_kv);
      dma_tile(1, s_kv + kShBuf);
      dma_tile(2, s_kv + 2 * kShBuf);
      for (int j = 0; j < cnt; j += 4) {
        sh_step(j, 0, 3);
        sh_step(j + 1, 1, 0);
        sh_step(j + 2, 2, 1);
        sh_step(j + 3, 3, 2);
      }
    }
    tl_finish();
    return;
  }
  constexpr int S = kMqStagesFor<W, MT>;
  uint4 kbuf[S][KLD];
  vload vbuf[S][4];
  for (int start = xbeg; start < xend; start += cnt) {
    stage(start);  // sets cnt
#pragma unroll
    for (int u = 0; u < S - 1; ++u) load_tile(u, kbuf[u], vbuf[u]);
    stage_lds();
    for (int j = 0; j < cnt; j += S) {
#pragma unroll
      for (int u = 0; u < S; ++u) {
        load_tile(j + u + S - 1, kbuf[(u + S - 1) % S], vbuf[(u + S - 1) % S]);
        if (j + u < cnt) step(j + u, kbuf[u], vbuf[u]);  // wave-uniform
      }
    }
  }
  tl_finish();
}

// Merge of the passes whose virtual sequence was cut by range boundaries:
// out = sum_k w_k o_k / sum_k w_k, w_k = l_k 2^(m_k - max m), over the
// groups k that covered it, in group order; virtual sequences with no tile
// get zero rows.  A thread owns one row and eight output dimensions (one
// 16-byte load per segment), so a work-group covers a block of 16 rows at
// D = 128.  The grid holds as many work-groups as the CUs keep resident at
// the kernel's register count, each looping over row blocks, rather than one
// work-group per block: dispatching a work-group per block cost verification
// of the 70B-shaped batch about 1 us per call.
template <int D>
struct MqMerge {
  static constexpr int kPerThread = 8;             // output elements per thread
  static constexpr int kThreadsPerRow = D / kPerThread;
  static constexpr int kRowsPerBlock = 256 / kThreadsPerRow;
  static constexpr int kGroupsPerCu = 4;           // resident at up to 128 VGPRs
};

template <class T, int D>
__global__ __launch_bounds__(256) void decode_multi_reduce_kernel(MultiArgs a) {
  typedef typename T::storage st;
  constexpr int QPR = MqMerge<D>::kThreadsPerRow;
  constexpr int RPB = MqMerge<D>::kRowsPerBlock;
  const int bpv = (a.pass_rows + RPB - 1) / RPB;  // row blocks per (sequence, pass, head)
#ifdef PA_WAVE_TIMELINE
  const int64_t tl_cw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  uint64_t *tl_rec = (a.timeline != nullptr && tl_cw < kTimelineCombineWaves)
                         ? a.timeline + (int64_t)kTimelineWaves * 8 + tl_cw * 2
                         : nullptr;
  if (tl_rec != nullptr && (threadIdx.x & 63) == 0) tl_rec[0] = tl_now();
#endif
  const int PG = a.pass_group;
  const int nv = a.num_seqs * a.pgroups;
  const int total = a.ws_sched[nv];
  const int groups = mq_active_groups(a, total);
  const RangeSplit rs = range_split(weighted_total(total, nv, a.seq_cost), groups, a.young_from, a.young_share);
  // item blk: (sequence, pass, KV head, block of RPB rows); returns early when
  // the main kernel wrote the rows (no barriers follow)
  auto item = [&](int blk) {
    const int rb = blk % bpv;
    const int g = (blk / bpv) % a.num_kv_heads;
    const int bp = blk / (bpv * a.num_kv_heads);  // b * passes + pass
    const int b = bp / a.passes;
    const int pass = bp - b * a.passes;
    const int v = b * a.pgroups + pass / PG;
    const int w = pass - (pass / PG) * PG;
    const int t0 = a.ws_sched[v], t1 = a.ws_sched[v + 1];
    const int64_t w0 = (int64_t)t0 + (int64_t)a.seq_cost * (v + 1);  // weighted position of tile 0
    const int ga = t1 > t0 ? range_of(rs, w0) : 0, gb = t1 > t0 ? range_of(rs, w0 + (t1 - t0) - 1) : 0;
    if (t1 > t0 && ga == gb) return;  // written by the main kernel
    const int row0 = pass * a.pass_rows;
    const int row_end = min(a.rows, row0 + a.pass_rows);
    const int row = rb * RPB + (int)threadIdx.x / QPR;
    const int q8 = (int)threadIdx.x % QPR;
    if (row0 + row >= row_end) return;
    float wsum = 0.f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (t1 > t0) {
      // Segments k = ga..gb in windows of kWin: every (m, l) pair and row of a
      // window is requested before the first is used (one round trip per
      // window, not one per segment); windows after the first rescale the
      // running sums to the new maximum.
      constexpr int kWin = 16;
      const int64_t rstep = (int64_t)a.num_kv_heads * PG * a.pass_rows;  // rows between segments
      const int64_t r0 = ((((int64_t)ga + v) * a.num_kv_heads + g) * PG + w) * a.pass_rows + row;
      float m_max = -INFINITY;
      for (int k0 = ga; k0 <= gb; k0 += kWin) {
        const int cnt = min(kWin, gb - k0 + 1);
        float mk[kWin], lk[kWin];
        // rows stay raw (eight 16-bit values) until they are used, so that no
        // conversion waits on a load before the window's other loads issue
        uint4 okr[kWin];
#pragma unroll
        for (int u = 0; u < kWin; ++u) {
          if (u < cnt) {
            const int64_t r = r0 + (int64_t)(k0 - ga + u) * rstep;
            mk[u] = a.ws_ml[r * 2];
            lk[u] = a.ws_ml[r * 2 + 1];
            okr[u] = reinterpret_cast<const uint4 *>(reinterpret_cast<const st *>(a.ws_o) + r * D)[q8];
          } else {
            mk[u] = -INFINITY;
            lk[u] = 0.f;
            okr[u] = make_uint4(0u, 0u, 0u, 0u);
          }
        }
        float m_new = m_max;
#pragma unroll
        for (int u = 0; u < kWin; ++u) m_new = fmaxf(m_new, mk[u]);
        if (k0 > ga && m_new > m_max) {
          const float f = fast_exp2(m_max - m_new);
          wsum *= f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] *= f;
        }
        m_max = m_new;
#pragma unroll
        for (int u = 0; u < kWin; ++u) {
          if (u < cnt) {
            const float wk = lk[u] > 0.f ? lk[u] * fast_exp2(mk[u] - m_max) : 0.f;
            wsum += wk;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += wk * T::to_float(half_of(okr[u], e));
          }
        }
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const int rr = row0 + row;
    const int i = rr / a.group, h = rr - (rr / a.group) * a.group;
    st *out = static_cast<st *>(a.out) +
              (((int64_t)b * a.q_len + i) * a.num_q_heads + (int64_t)g * a.group + h) * D + 8 * q8;
    *reinterpret_cast<uint4 *>(out) =
        make_uint4(T::pack_pair(acc[0] * inv, acc[1] * inv), T::pack_pair(acc[2] * inv, acc[3] * inv),
                   T::pack_pair(acc[4] * inv, acc[5] * inv), T::pack_pair(acc[6] * inv, acc[7] * inv));
#ifdef PA_WAVE_TIMELINE
    if (tl_rec != nullptr && (threadIdx.x & 63) == 0) tl_rec[1] = tl_now() | (1ull << 63);
#endif
  };
  const int items = a.num_seqs * a.passes * a.num_kv_heads * bpv;
  for (int blk = blockIdx.x; blk < items; blk += gridDim.x) item(blk);
}

template <class T, int D, int MT, int KVF, int W, bool RING>
hipError_t launch_mt(const MultiArgs &a, int grid, hipStream_t stream) {
  // one pass per (sequence, KV head): each K/V row is read once (W = 1 only:
  // the two-wave configuration serves calls with several passes)
  constexpr bool kCanShare = W == 2 && KVF == 0 && !RING && D == 128;
  if (W == 1 && a.passes == 1)
    hipLaunchKernelGGL((decode_multi_kernel<T, D, MT, KVF, W, RING, W == 1>), dim3(grid), dim3(kMqWaves * kWave), 0,
                       stream, a);
  else if (kCanShare && a.pass_group == kMqWaves)
    hipLaunchKernelGGL((decode_multi_kernel<T, D, MT, KVF, W, RING, false, kCanShare>), dim3(grid),
                       dim3(kMqWaves * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_multi_kernel<T, D, MT, KVF, W, RING, false>), dim3(grid), dim3(kMqWaves * kWave), 0,
                       stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  constexpr int rpb = MqMerge<D>::kRowsPerBlock;
  const int bpv = (a.pass_rows + rpb - 1) / rpb;
  const int items = a.num_seqs * a.passes * a.num_kv_heads * bpv;
  hipLaunchKernelGGL((decode_multi_reduce_kernel<T, D>),
                     dim3((unsigned)std::min(items, MqMerge<D>::kGroupsPerCu * multi_grid())), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

template <class T, int D, int KVF, bool RING>
hipError_t launch_d(const MultiArgs &a, int mt, int waves, int grid, hipStream_t stream) {
  if constexpr (RING) {  // row tiles per wave: see kMultiMaxRowTilesRing
    if (waves == 2) return mt == 1 ? launch_mt<T, D, 1, KVF, 2, true>(a, grid, stream) : hipErrorInvalidValue;
    if (mt > 2) return hipErrorInvalidValue;
    return mt == 1 ? launch_mt<T, D, 1, KVF, 1, true>(a, grid, stream) : launch_mt<T, D, 2, KVF, 1, true>(a, grid, stream);
  } else {
    if (waves == 2) return mt == 1 ? launch_mt<T, D, 1, KVF, 2, false>(a, grid, stream)
                           : mt == 2 ? launch_mt<T, D, 2, KVF, 2, false>(a, grid, stream)
                                     : launch_mt<T, D, 3, KVF, 2, false>(a, grid, stream);
    switch (mt) {
      case 1: return launch_mt<T, D, 1, KVF, 1, false>(a, grid, stream);
      case 2: return launch_mt<T, D, 2, KVF, 1, false>(a, grid, stream);
      case 3: return launch_mt<T, D, 3, KVF, 1, false>(a, grid, stream);
      default: return launch_mt<T, D, kMultiMaxRowTiles(D), KVF, 1, false>(a, grid, stream);
    }
  }
}

template <class T, int KVF, bool RING>
hipError_t launch_h(const MultiArgs &a, int head_dim, int mt, int waves, int grid, hipStream_t stream) {
  return head_dim == 128 ? launch_d<T, 128, KVF, RING>(a, mt, waves, grid, stream)
                         : launch_d<T, 64, KVF, RING>(a, mt, waves, grid, stream);
}

template <class T>
hipError_t launch_t(const MultiArgs &a, int head_dim, int kv8, int mt, int waves, int grid,
                    hipStream_t stream, bool ring) {
  if (ring) return kv8 == 0 ? launch_h<T, 0, true>(a, head_dim, mt, waves, grid, stream) : hipErrorInvalidValue;
  switch (kv8) {
    case 0: return launch_h<T, 0, false>(a, head_dim, mt, waves, grid, stream);
    case kKvE4M3: return launch_h<T, kKvE4M3, false>(a, head_dim, mt, waves, grid, stream);
    case kKvE5M2: return launch_h<T, kKvE5M2, false>(a, head_dim, mt, waves, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// CUs of the current device (one work-group of four waves per CU and per
// wave-per-SIMD of the configuration).
int multi_grid() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  static std::atomic<int> cached[64];  // CU count per device, looked up once
  const bool slot = dev >= 0 && dev < 64;
  if (slot) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (slot) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

hipError_t launch_decode_multi(const MultiArgs &a, pa_dtype dtype, int head_dim, int kv8, int waves,
                               int grid, hipStream_t stream, bool ring) {
  const int mt = a.pass_rows / 16;
  if (dtype == PA_BF16) return launch_t<BF16>(a, head_dim, kv8, mt, waves, grid, stream, ring);
  return launch_t<F16>(a, head_dim, kv8, mt, waves, grid, stream, ring);
}

}  // namespace pa
