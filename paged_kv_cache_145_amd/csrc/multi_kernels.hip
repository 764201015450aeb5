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
// one KV head (row r = i * G + h) are the M dimension of the MFMA tiles.
//
// Work split.  Grid (sequence x KV split, 1, head group x row pass): a
// work-group of 4 waves takes 4 consecutive KV heads (so the waves read the
// same token rows side by side), one split of at most split_tiles 16-token
// tiles, and one pass of 16 * MT query rows; each wave keeps its MT row
// tiles in registers and streams its head's K/V tiles once for all of them.
// A (sequence, pass) with one split writes its output rows directly;
// otherwise each split leaves normalised partials and
// decode_multi_reduce_kernel merges them in split order.
//
// Per 16-token tile, as in the single-token kernel but with MT query tiles:
//   S[token][row] = K_tile . Q^T with v_mfma_f32_16x16x32 (A = the lane's
//   own K row fragment, B = query rows); lane l gets S[4(l/16)+j][l%16];
//   O[row][d] += P[row][token] V[token][d] with v_mfma_f32_16x16x16; V goes
//   through a per-wave LDS tile and returns as B operands through
//   transposing LDS reads (shared by the MT row tiles).
#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kMqWaves = 4;
constexpr float kMqRescaleSlack = 8.0f;  // log2 units the running max may lag

// One lane's share of a V row: D / 16 elements, 16 or 8 bytes.
template <int D>
struct MqV;
template <>
struct MqV<128> {
  typedef uint4 type;
  static __device__ __forceinline__ uint4 load(__amdgpu_buffer_rsrc_t r, int off) {
    return buffer_load16(r, off);
  }
};
template <>
struct MqV<64> {
  typedef uint2 type;
  static __device__ __forceinline__ uint2 load(__amdgpu_buffer_rsrc_t r, int off) {
    return buffer_load8(r, off);
  }
};

// Per-wave V tile: row-major, rows padded so the transposing reads of one
// instruction spread over the banks.
template <int D>
struct MqLds {
  static constexpr int kVRowBytes = D * 2 + 32;
  static constexpr int kVBytes = kTileTokens * kVRowBytes;
};

// Key range and split count of (sequence, pass); identical in both kernels.
struct MqRange {
  int L, row0, row_end, kv_end, tiles_end, splits;
};
__device__ __forceinline__ MqRange mq_range(const MultiArgs &a, int b, int pass) {
  MqRange r;
  r.L = min(max(a.context_lens[b], 0), a.max_context);
  r.row0 = pass * a.pass_rows;
  r.row_end = min(a.rows, r.row0 + a.pass_rows);
  // the last row of the pass sees the most keys
  r.kv_end = min(max(r.L - a.q_len + (r.row_end - 1) / a.group + 1, 0), r.L);
  r.tiles_end = (r.kv_end + kTileTokens - 1) / kTileTokens;
  r.splits = max(1, (r.tiles_end + a.split_tiles - 1) / a.split_tiles);
  return r;
}

// Partial slot of (sequence, pass, split, KV head, row within the pass).
__device__ __forceinline__ int64_t mq_slot(const MultiArgs &a, int b, int pass, int s, int g, int row) {
  return ((((int64_t)b * a.passes + pass) * a.max_splits + s) * a.num_kv_heads + g) * a.pass_rows + row;
}

template <class T, int D, int MT>
__global__ __launch_bounds__(256) void decode_multi_kernel(MultiArgs a) {
  constexpr int KB = D / 32;  // score MFMAs per row tile and key tile
  constexpr int EV = D / 16;  // V elements per lane per row
  constexpr int NB = D / 16;  // output MFMAs per row tile (16 dims each)
  constexpr int kVRow = MqLds<D>::kVRowBytes;
  typedef typename T::storage st;
  typedef typename MqV<D>::type vchunk;
  __shared__ __align__(16) char s_vt[kMqWaves][MqLds<D>::kVBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row16 = lane & 15, grp = lane >> 4;
  const int b = blockIdx.x / a.max_splits;
  const int s = blockIdx.x - b * a.max_splits;
  const int hg = blockIdx.z % a.head_groups;
  const int pass = blockIdx.z / a.head_groups;
  const int g = hg * kMqWaves + wave;
  if (g >= a.num_kv_heads) return;  // no barriers in this kernel
  const MqRange rg = mq_range(a, b, pass);
  if (s >= rg.splits) return;
  const int G = a.group, ql = a.q_len;
  const int t_beg = s * a.split_tiles;
  const int ntiles = max(0, min(t_beg + a.split_tiles, rg.tiles_end) - t_beg);  // <= 64

  const int64_t row_stride = (int64_t)a.num_kv_heads * D;  // elements between token rows
  const int bmask = (1 << a.block_shift) - 1;
  char *vt = s_vt[wave];

  // This lane's query row in each row tile: row16 (the S column it holds).
  int limit[MT];  // last key position the row sees (-1: none)
  uint4 qf[MT][KB];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = rg.row0 + 16 * mt + row16;
    const bool ok = r < rg.row_end;
    const int i = ok ? r / G : 0;
    const int h = ok ? r - i * G : 0;
    limit[mt] = ok ? rg.L - ql + i : -1;
    const st *q = static_cast<const st *>(a.query) +
                  (((int64_t)b * ql + i) * a.num_q_heads + (int64_t)g * G + h) * D + 8 * grp;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      qf[mt][kb] = ok ? *reinterpret_cast<const uint4 *>(q + 32 * kb) : make_uint4(0u, 0u, 0u, 0u);
  }

  // block id of tile t_beg + lane, read back per tile with readlane
  int tblk = 0;
  if (lane < ntiles) {
    const int t = t_beg + lane;
    tblk = a.block_tables[(int64_t)b * a.max_blocks_per_seq + ((kTileTokens * t) >> a.block_shift)];
    tblk = min(max(tblk, 0), a.num_blocks - 1);
  }
  const int k_off = (int)((row16 * row_stride + 8 * grp) * (int64_t)sizeof(st));
  int v_off[4];
#pragma unroll
  for (int tau = 0; tau < 4; ++tau)
    v_off[tau] = (int)(((4 * grp + tau) * row_stride + EV * row16) * (int64_t)sizeof(st));

  // Loads of tile j; past ntiles the record range is empty and nothing is read.
  auto load_tile = [&](int j, uint4 (&k)[KB], vchunk (&v)[4]) {
    const int jj = min(j, kWave - 1);
    const int t = t_beg + j;
    const int blk = __builtin_amdgcn_readlane(tblk, jj);
    const int valid = j < ntiles ? min(kTileTokens, rg.kv_end - kTileTokens * t) : 0;
    const int64_t off = ((int64_t)blk * a.kv_block_stride +
                         (int64_t)((kTileTokens * t) & bmask) * row_stride + (int64_t)g * D) *
                        (int64_t)sizeof(st);
    const int nrec = valid > 0 ? (int)(((valid - 1) * row_stride + D) * (int64_t)sizeof(st)) : 0;
    const auto kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(a.k_cache) + off), (short)0, nrec, kBufferWord3);
    const auto vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(a.v_cache) + off), (short)0, nrec, kBufferWord3);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) k[kb] = buffer_load16(kr, k_off + 64 * kb);
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) v[tau] = MqV<D>::load(vr, v_off[tau]);
  };

  f32x4 acc[MT][NB];
  float m_run[MT], l_part[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    m_run[mt] = -INFINITY;
    l_part[mt] = 0.f;
#pragma unroll
    for (int e = 0; e < NB; ++e) acc[mt][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = a.scale_log2;

  auto process_tile = [&](int j, const uint4 (&kf)[KB], const vchunk (&vf)[4]) {
    const int kp0 = kTileTokens * (t_beg + j) + 4 * grp;  // key position of S element 0
    f32x4 sv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sacc = T::mfma_16x16x32(kf[kb], qf[mt][kb], sacc);
      sv[mt] = sacc;
    }
    // V rows past kv_end were loaded as zeros, so a zero weight never meets
    // a NaN sentinel; rows before it hold written values.
#pragma unroll
    for (int tau = 0; tau < 4; ++tau)
      *reinterpret_cast<vchunk *>(vt + (4 * grp + tau) * kVRow + sizeof(vchunk) * row16) = vf[tau];
    const char *vr = vt + (4 * grp + (row16 >> 2)) * kVRow + 8 * (row16 & 3);
    uint2 vtr[NB];
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) vtr[jb] = lds_read_tr16_b64(vr + 32 * jb);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = (kp0 + r <= limit[mt]) ? sv[mt][r] * sl2 : -INFINITY;
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
      const uint2 pa = make_uint2(pack2(T::from_float(pj[0]), T::from_float(pj[1])),
                                  pack2(T::from_float(pj[2]), T::from_float(pj[3])));
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) acc[mt][jb] = T::mfma_16x16x16(pa, vtr[jb], acc[mt][jb]);
    }
  };

  // two register buffers: tile j + 1 is in flight while tile j is consumed
  uint4 ka[KB], kb2[KB];
  vchunk va[4], vb[4];
  load_tile(0, ka, va);
  for (int j = 0; j < ntiles; j += 2) {
    load_tile(j + 1, kb2, vb);
    process_tile(j, ka, va);
    if (j + 1 < ntiles) {
      load_tile(j + 2, ka, va);
      process_tile(j + 1, kb2, vb);
    }
  }

  // Rows of this lane's output fragments: 4 grp + r of each row tile.
  const bool whole = rg.splits == 1;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float l_tot = l_part[mt] + __shfl_xor(l_part[mt], 16);
    l_tot += __shfl_xor(l_tot, 32);  // the row16 row's sum over this split
    float lh[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lh[r] = __shfl(l_tot, 4 * grp + r);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = rg.row0 + 16 * mt + 4 * grp + r;
      if (rr >= rg.row_end) continue;
      const float inv = lh[r] > 0.f ? 1.f / lh[r] : 0.f;
      if (whole) {
        const int i = rr / G, h = rr - (rr / G) * G;
        st *out = static_cast<st *>(a.out) + (((int64_t)b * ql + i) * a.num_q_heads + (int64_t)g * G + h) * D;
#pragma unroll
        for (int e = 0; e < NB; ++e) out[16 * e + row16] = T::from_float(acc[mt][e][r] * inv);
      } else {
        float *po = a.ws_o + mq_slot(a, b, pass, s, g, rr - rg.row0) * D;
#pragma unroll
        for (int e = 0; e < NB; ++e) po[16 * e + row16] = acc[mt][e][r] * inv;
      }
    }
    if (!whole && grp == 0) {
      const int rr = rg.row0 + 16 * mt + row16;
      if (rr < rg.row_end) {
        const int64_t slot = mq_slot(a, b, pass, s, g, rr - rg.row0);
        a.ws_ml[slot * 2] = m_run[mt];
        a.ws_ml[slot * 2 + 1] = l_tot;
      }
    }
  }
}

// Merge the splits of every (sequence, pass, KV head) that had more than
// one: out = sum_s w_s o_s / sum_s w_s with w_s = l_s 2^(m_s - max m), in
// split order.  One work-group per (sequence, pass, KV head).
template <class T, int D>
__global__ __launch_bounds__(256) void decode_multi_reduce_kernel(MultiArgs a) {
  typedef typename T::storage st;
  const int per_seq = a.passes * a.num_kv_heads;
  const int b = blockIdx.x / per_seq;
  const int z = blockIdx.x - b * per_seq;
  const int pass = z / a.num_kv_heads;
  const int g = z - pass * a.num_kv_heads;
  const MqRange rg = mq_range(a, b, pass);
  if (rg.splits <= 1) return;  // written by the main kernel
  const int nrows = rg.row_end - rg.row0;
  const int G = a.group;
  for (int e = threadIdx.x; e < nrows * D; e += blockDim.x) {
    const int row = e / D, d = e - (e / D) * D;
    float m_max = -INFINITY;
    for (int s = 0; s < rg.splits; ++s) m_max = fmaxf(m_max, a.ws_ml[mq_slot(a, b, pass, s, g, row) * 2]);
    float wsum = 0.f, acc = 0.f;
    for (int s = 0; s < rg.splits; ++s) {
      const int64_t slot = mq_slot(a, b, pass, s, g, row);
      const float l = a.ws_ml[slot * 2 + 1];
      if (l > 0.f) {
        const float w = l * fast_exp2(a.ws_ml[slot * 2] - m_max);
        wsum += w;
        acc += w * a.ws_o[slot * D + d];
      }
    }
    const int rr = rg.row0 + row;
    const int i = rr / G, h = rr - (rr / G) * G;
    st *out = static_cast<st *>(a.out) + (((int64_t)b * a.q_len + i) * a.num_q_heads + (int64_t)g * G + h) * D;
    out[d] = T::from_float(wsum > 0.f ? acc / wsum : 0.f);
  }
}

template <class T, int D, int MT>
hipError_t launch_mt(const MultiArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.num_seqs * a.max_splits), 1, (unsigned)(a.head_groups * a.passes));
  hipLaunchKernelGGL((decode_multi_kernel<T, D, MT>), grid, dim3(256), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.max_splits == 1) return err;
  hipLaunchKernelGGL((decode_multi_reduce_kernel<T, D>),
                     dim3((unsigned)(a.num_seqs * a.passes * a.num_kv_heads)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <class T, int D>
hipError_t launch_d(const MultiArgs &a, int mt, hipStream_t stream) {
  switch (mt) {
    case 1: return launch_mt<T, D, 1>(a, stream);
    case 2: return launch_mt<T, D, 2>(a, stream);
    case 3: return launch_mt<T, D, 3>(a, stream);
    default: return launch_mt<T, D, 4>(a, stream);
  }
}

template <class T>
hipError_t launch_t(const MultiArgs &a, int head_dim, int mt, hipStream_t stream) {
  return head_dim == 128 ? launch_d<T, 128>(a, mt, stream) : launch_d<T, 64>(a, mt, stream);
}

}  // namespace

hipError_t launch_decode_multi(const MultiArgs &a, pa_dtype dtype, int head_dim, hipStream_t stream) {
  const int mt = a.pass_rows / 16;
  if (dtype == PA_BF16) return launch_t<BF16>(a, head_dim, mt, stream);
  return launch_t<F16>(a, head_dim, mt, stream);
}

}  // namespace pa
