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
//  * One work-group of 4 wave64s per (split-K partition, KV head, sequence).
//    A partition is a contiguous run of `partition_tokens` logical tokens;
//    its 16-token tiles are dealt round-robin to the 4 waves, each keeping
//    its own online-softmax state; the waves merge through LDS at the end.
//  * The block id of a tile is wave-uniform, so it is fetched through the
//    scalar path (one SGPR load per tile) rather than staged in LDS.
//  * A tile's 16 K rows (head g) are read with 16-byte loads; for the MFMA
//    kernel each lane's 16 bytes are exactly its A-operand fragment.
//  * Sequences whose context fits one partition write the final output
//    directly; longer ones write (max, sum, normalised partial) and
//    decode_reduce combines them.
//  * The summation order depends only on logical positions and lengths, so
//    outputs are bit-identical under relabelling of physical blocks.
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
                                                 int hq0, int b, int p, int parts) {
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
      num += wt * s_o[w][h][d];
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

// Rotate-half RoPE on a 16-bit fragment held as KB 16-byte chunks where
// chunk kb covers d = 32 kb + 8 grp + [0, 8); chunk kb + KB/2 holds the
// partner elements d + D/2.  `cs` points at the (cos, sin) row of the angle.
template <class T, int KB>
__device__ __forceinline__ void rope_frag16(uint4 (&f)[KB], const float *cs, int grp) {
#pragma unroll
  for (int kb = 0; kb < KB / 2; ++kb) {
    const float4 *c4 = reinterpret_cast<const float4 *>(cs + 2 * (32 * kb + 8 * grp));
    float c[8], s[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = c4[i];
      c[2 * i] = v.x;
      s[2 * i] = v.y;
      c[2 * i + 1] = v.z;
      s[2 * i + 1] = v.w;
    }
    uint16_t lo[8], hi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = T::to_float(half_of(f[kb], e));
      const float y = T::to_float(half_of(f[kb + KB / 2], e));
      lo[e] = T::from_float(x * c[e] - y * s[e]);
      hi[e] = T::from_float(x * s[e] + y * c[e]);
    }
    f[kb] = make_uint4(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(lo[4], lo[5]),
                       pack2(lo[6], lo[7]));
    f[kb + KB / 2] = make_uint4(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]), pack2(hi[4], hi[5]),
                                pack2(hi[6], hi[7]));
  }
}

template <int D>
struct VChunk;
template <>
struct VChunk<128> {
  typedef uint4 type;
  static __device__ __forceinline__ uint4 load(__amdgpu_buffer_rsrc_t r, int off) {
    return buffer_load16(r, off);
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
    return buffer_load8(r, off);
  }
  static __device__ __forceinline__ uint2 half(const uint2 &v, int) { return v; }
  static __device__ __forceinline__ uint2 select(bool keep, const uint2 &v) {
    return make_uint2(keep ? v.x : 0u, keep ? v.y : 0u);
  }
};

// ---------------------------------------------------------------------------
// MFMA kernel: 16-bit K/V, GQA group G in [1, 16] (used for G >= 4).
//
// Scores: S[token][head] = K_tile[16 x D] . Q^T[D x 16] with
//   v_mfma_f32_16x16x32_{bf16,f16}; A = K rows (lane: token row16, 8 dims),
//   B = query (lane: head row16, the same 8 dims), so each lane's 16-byte K
//   load is its A fragment.  Lane l receives S[4*(l/16) + j][l % 16].
// Output: O[head][d] += P[head][token] V[token][d] with
//   v_mfma_f32_16x16x16_{bf16,f16}.  V rows are d-contiguous, so instead of
//   transposing V the contraction index k = (token group, slot) carries
//   one token per lane group and P is placed in one of the four slots
//   (zeros elsewhere): MFMA e accumulates O[head][EV*(l%16) + e] from the
//   lane's own 16-byte V load, and its A operand is the lane's own score
//   output.  No LDS traffic and no shuffles in the inner loop.
// ---------------------------------------------------------------------------
template <class T, int D, bool RING>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int KB = D / 32;  // score MFMAs per tile
  constexpr int EV = D / 16;  // V elements per lane per row
  typedef typename T::storage st;
  typedef typename VChunk<D>::type vchunk;

  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int n = a.context_lens[b];
  const int L = effective_len(a, n, RING);
  const int P = a.partition_tokens;
  const int parts = L > 0 ? (L + P - 1) / P : 1;
  if (p >= parts) return;
  const int G = a.group;
  const int hq0 = g * G;
  if (L == 0) {
    zero_rows<T, D>(a, b, hq0, G);
    return;
  }
  const int lane = threadIdx.x & 63;
  // wave-uniform (SGPR) so tile indices and block ids stay on the scalar path
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row16 = lane & 15, grp = lane >> 4;
  const int begin = p * P;
  const int end = min(L, begin + P);
  const int ntiles = (end - begin + kTileTokens - 1) / kTileTokens;

  // Query fragment: head row16 of the group, dims 32kb + 8grp + [0, 8).
  uint4 qf[KB];
  const bool head_ok = row16 < G;
  {
    const st *qrow =
        static_cast<const st *>(a.query) + ((int64_t)b * a.num_q_heads + hq0 + (head_ok ? row16 : 0)) * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      qf[kb] = head_ok ? *reinterpret_cast<const uint4 *>(qrow + 32 * kb + 8 * grp) : make_uint4(0, 0, 0, 0);
    if constexpr (RING) rope_frag16<T, KB>(qf, a.rope + (int64_t)(L - 1) * D, grp);
  }

  const int64_t row_stride = (int64_t)a.num_kv_heads * D;  // elements between token rows
  const int32_t *bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
  const char *kc = static_cast<const char *>(a.k_cache) + (int64_t)g * D * sizeof(st);
  const char *vc = static_cast<const char *>(a.v_cache) + (int64_t)g * D * sizeof(st);
  const int bmask = (1 << a.block_shift) - 1;

  f32x4 acc[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_part = 0.f;

  // Per-lane byte offsets inside a tile (K: token row16, dims 8grp..+8 of
  // each 32-dim chunk; V: token 4grp+tau, dims EV*row16..+EV).
  const int k_off = (int)((row16 * row_stride + 8 * grp) * sizeof(st));
  int v_off[4];
#pragma unroll
  for (int tau = 0; tau < 4; ++tau)
    v_off[tau] = (int)(((4 * grp + tau) * row_stride + EV * row16) * sizeof(st));

  const PartitionBlocks blocks(a, bt, begin, end);
  auto load_tile = [&](int t, uint4 (&k)[KB], vchunk (&v)[4]) {
    const int r0 = begin + kTileTokens * min(t, ntiles - 1);
    const int valid = t < ntiles ? min(kTileTokens, end - r0) : 0;
    const int phys = blocks.of_token(r0);
    const auto kr = tile_rsrc<D, st>(a, kc, phys, r0 & bmask, valid, row_stride);
    const auto vr = tile_rsrc<D, st>(a, vc, phys, r0 & bmask, valid, row_stride);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) k[kb] = buffer_load16(kr, k_off + 64 * kb);
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) v[tau] = VChunk<D>::load(vr, v_off[tau]);
  };

  auto process_tile = [&](int t, uint4 (&kf)[KB], vchunk (&vf)[4]) {
    const int r0 = begin + kTileTokens * t;
    const int valid = end - r0;  // <= 0 for a tile past the partition
    if constexpr (RING) {
      const int r = r0 + row16;
      const int j = r < L ? ring_cache_index(r, n, a.ring_sink, a.ring_window) : 0;
      rope_frag16<T, KB>(kf, a.rope + (int64_t)j * D, grp);
    }
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s = T::mfma_16x16x32(kf[kb], qf[kb], s);

    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[j] = (4 * grp + j < valid) ? s[j] * a.scale_log2 : -INFINITY;
    const float lmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if (__any(lmax > m_run + kRescaleSlack)) {
      float tmax = fmaxf(lmax, __shfl_xor(lmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = fast_exp2(m_run - m_new);
      l_part *= alpha;
      float ah[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) ah[jj] = __shfl(alpha, 4 * grp + jj);
#pragma unroll
      for (int e = 0; e < EV; ++e)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[e][jj] *= ah[jj];
      m_run = m_new;
    }
    float pj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pj[j] = fast_exp2(sc[j] - m_run);
    l_part += (pj[0] + pj[1]) + (pj[2] + pj[3]);

    // V rows past the context were loaded as zeros (out of the descriptor's
    // range), so a zero weight never meets a NaN sentinel.
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      const uint32_t x = T::from_float(pj[tau]);
      const uint32_t y = x << 16;
      const uint2 op[4] = {make_uint2(x, 0u), make_uint2(y, 0u), make_uint2(0u, x), make_uint2(0u, y)};
#pragma unroll
      for (int e = 0; e < EV; ++e)
        acc[e] = T::mfma_16x16x16(op[e & 3], VChunk<D>::half(vf[tau], e >> 2), acc[e]);
    }
  };

  // Two register sets in ping-pong: while one tile is consumed the next
  // one's loads are in flight, with no register copies and no branches
  // around loads (so the hardware wait counts stay exact).  A tile past the
  // partition loads nothing and contributes nothing.
  uint4 ka[KB], kb2[KB];
  vchunk va[4], vb[4];
  if (wave < ntiles) {
    load_tile(wave, ka, va);
    for (int t = wave; t < ntiles; t += 2 * kNW) {
      load_tile(t + kNW, kb2, vb);
      process_tile(t, ka, va);
      load_tile(t + 2 * kNW, ka, va);
      process_tile(t + kNW, kb2, vb);
    }
  }

  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot += __shfl_xor(l_tot, 32);

  __shared__ float s_m[kNW][16];
  __shared__ float s_l[kNW][16];
  __shared__ float s_o[kNW][16][D];
  if (grp == 0) {
    s_m[wave][row16] = m_run;
    s_l[wave][row16] = l_tot;
  }
#pragma unroll
  for (int e = 0; e < EV; ++e)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int h = 4 * grp + jj;
      if (h < G) s_o[wave][h][EV * row16 + e] = acc[e][jj];
    }
  __syncthreads();
  finish_partition<T, D, 16>(a, s_m, s_l, s_o, G, hq0, b, p, parts);
}

// ---------------------------------------------------------------------------
// VALU kernel: any dtype, NH query heads per work-group (heads chunked when
// G > NH).  Each K/V row is spread over LPR lanes with 16-byte loads; a wave
// covers RPW rows per step, each row group keeping its own online-softmax
// state; dot products reduce within the row group with DPP.
// ---------------------------------------------------------------------------
template <class T, int D, bool RING, int NH>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  typedef typename T::storage st;
  constexpr int EPL = 16 / T::kBytes;  // elements per lane
  constexpr int LPR = D / EPL;         // lanes per row
  constexpr int RPW = kWave / LPR;     // rows per wave step
  constexpr int STEPS = kTileTokens / RPW;
  static_assert(LPR >= 4 && LPR <= 32, "row split");

  const int p = blockIdx.x, b = blockIdx.z;
  const int G = a.group;
  const int nchunk = (G + NH - 1) / NH;
  const int g = blockIdx.y / nchunk;
  const int c = blockIdx.y - g * nchunk;
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
      k[s] = buffer_load16(kr, off[s]);
      v[s] = buffer_load16(vr, off[s]);
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

  __shared__ float s_m[kNW][NH];
  __shared__ float s_l[kNW][NH];
  __shared__ float s_o[kNW][NH][D];
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

// ---------------------------------------------------------------------------
// Split-K combine: out = sum_p w_p o_p / sum_p w_p, w_p = l_p 2^(m_p - M).
// One work-group per (query head, sequence); only multi-partition sequences.
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(DecodeArgs a, int ring) {
  typedef typename T::storage st;
  const int h = blockIdx.x, b = blockIdx.y;
  const int n = a.context_lens[b];
  const int L = effective_len(a, n, ring != 0);
  const int P = a.partition_tokens;
  const int parts = min((L + P - 1) / P, a.max_parts);
  if (parts <= 1) return;
  const int64_t head = (int64_t)b * a.num_q_heads + h;
  const float *ml = a.ws_ml + head * a.max_parts * 2;
  const float *po = a.ws_o + head * a.max_parts * D;
  float mx = -INFINITY;
  for (int q = 0; q < parts; ++q) mx = fmaxf(mx, ml[2 * q]);
  const int d = threadIdx.x;
  float num = 0.f, den = 0.f;
  for (int q = 0; q < parts; ++q) {
    const float w = ml[2 * q + 1] * fast_exp2(ml[2 * q] - mx);
    num += w * po[(int64_t)q * D + d];
    den += w;
  }
  static_cast<st *>(a.out)[head * D + d] = T::from_float(num / den);
}

template <class T, int D, bool RING>
hipError_t launch_typed(const DecodeArgs &a, DecodeChoice choice, int num_seqs, hipStream_t stream) {
  const dim3 block(kNW * kWave);
  bool launched = false;
  if constexpr (T::kBytes == 2) {
    if (choice.kernel == DecodeKernel::kMfma) {
      const dim3 grid(a.max_parts, a.num_kv_heads, num_seqs);
      hipLaunchKernelGGL((decode_mfma_kernel<T, D, RING>), grid, block, 0, stream, a);
      launched = true;
    }
  }
  if (!launched) {
    const int nchunk = (a.group + choice.heads_per_pass - 1) / choice.heads_per_pass;
    const dim3 grid(a.max_parts, a.num_kv_heads * nchunk, num_seqs);
    switch (choice.heads_per_pass) {
      case 1: hipLaunchKernelGGL((decode_valu_kernel<T, D, RING, 1>), grid, block, 0, stream, a); break;
      case 2: hipLaunchKernelGGL((decode_valu_kernel<T, D, RING, 2>), grid, block, 0, stream, a); break;
      default: hipLaunchKernelGGL((decode_valu_kernel<T, D, RING, 4>), grid, block, 0, stream, a); break;
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.max_parts > 1) {
    const dim3 rgrid(a.num_q_heads, num_seqs);
    hipLaunchKernelGGL((decode_reduce_kernel<T, D>), rgrid, dim3(D), 0, stream, a, RING ? 1 : 0);
    err = hipGetLastError();
  }
  return err;
}

template <class T>
hipError_t launch_dtype(const DecodeArgs &a, int head_dim, bool ring, DecodeChoice choice,
                        int num_seqs, hipStream_t stream) {
  if (head_dim == 128)
    return ring ? launch_typed<T, 128, true>(a, choice, num_seqs, stream)
                : launch_typed<T, 128, false>(a, choice, num_seqs, stream);
  return ring ? launch_typed<T, 64, true>(a, choice, num_seqs, stream)
              : launch_typed<T, 64, false>(a, choice, num_seqs, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, pa_dtype dtype, int head_dim, bool ring,
                         DecodeChoice choice, int num_seqs, hipStream_t stream) {
  switch (dtype) {
    case PA_F16: return launch_dtype<F16>(a, head_dim, ring, choice, num_seqs, stream);
    case PA_BF16: return launch_dtype<BF16>(a, head_dim, ring, choice, num_seqs, stream);
    default: break;
  }
  choice.kernel = DecodeKernel::kValu;  // fp32 always takes the VALU kernel
  return launch_dtype<F32>(a, head_dim, ring, choice, num_seqs, stream);
}

}  // namespace pa
