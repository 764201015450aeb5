// Write side of the paged KV cache and the RoPE table, for gfx950.
//
// reshape_and_cache: a new token's K and V rows ([Hkv, D] each) are copied
// into the flat pool slot the caller computed from the block table, as the
// decode step of "大模型推理内存优化：从 KV Cache 分页到连续批处理的工程实践"
// (pwwt.cn/news/3010209), section "KV Cache 的内存开销与分页机制" writes the new
// token into the request's last block (allocating a block when it is full),
// and as the ring cache of wzjinhao.cn/news/69573, section
// "C++ 环形 KV 缓存管理内核实现", appends one vector per head at the slot of
// the current position.  Pool layout [num_blocks, block_size, Hkv, D] makes
// a slot's rows one contiguous run of Hkv * D elements at slot * Hkv * D.
#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {

// One work-group per token; each thread moves 16-byte chunks of K and V.
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    uint4 *__restrict__ k_cache, uint4 *__restrict__ v_cache, const uint4 *__restrict__ key,
    const uint4 *__restrict__ value, const int32_t *__restrict__ slot_mapping, int32_t chunks,
    int64_t num_slots) {
  const int64_t i = blockIdx.x;
  const int32_t slot = slot_mapping[i];
  // padding (negative) and out-of-pool slots are dropped; the rows are read
  // regardless, so their loads overlap the slot load
  const bool keep = slot >= 0 && slot < num_slots;
  const int64_t src = i * chunks;
  const int64_t dst = (int64_t)(keep ? slot : 0) * chunks;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
    const uint4 kx = key[src + c], vx = value[src + c];
    if (keep) {
      k_cache[dst + c] = kx;
      v_cache[dst + c] = vx;
    }
  }
}

// 8-bit pools: one work-group per token; each thread turns 16 activations
// (one 16-element run inside one head) into 16 codes: x * inv_scale[head]
// in float, then the code of format F (kKvE4M3 or kKvE5M2).
template <class T, int F>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    uint4 *__restrict__ k_cache, uint4 *__restrict__ v_cache, const uint4 *__restrict__ key,
    const uint4 *__restrict__ value, const int32_t *__restrict__ slot_mapping, int32_t chunks,
    int32_t head_dim, int64_t num_slots, KvScales inv) {
  const int64_t i = blockIdx.x;
  const int32_t slot = slot_mapping[i];
  const bool keep = slot >= 0 && slot < num_slots;
  const int64_t dst = (int64_t)(keep ? slot : 0) * chunks;  // 16 codes per chunk
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
    const int h = (c * 16) / head_dim;
    const uint4 k0 = key[(i * chunks + c) * 2], k1 = key[(i * chunks + c) * 2 + 1];
    const uint4 v0 = value[(i * chunks + c) * 2], v1 = value[(i * chunks + c) * 2 + 1];
    auto quant = [&](const uint4 &lo, const uint4 &hi, float s) {
      const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t word = w[(4 * q + e) / 2];
          const uint16_t b = (uint16_t)(((4 * q + e) & 1) ? (word >> 16) : (word & 0xFFFFu));
          packed |= fp8_code<F>(T::to_float(b) * s) << (8 * e);
        }
        o[q] = packed;
      }
      return make_uint4(o[0], o[1], o[2], o[3]);
    };
    const uint4 kq = quant(k0, k1, inv.k[h]);
    const uint4 vq = quant(v0, v1, inv.v[h]);
    if (keep) {
      k_cache[dst + c] = kq;
      v_cache[dst + c] = vq;
    }
  }
}

// Block copy that completes a copy-on-write: a shared block is copied to a
// private one before the private one is written ("Ollama的内存管理策略…"
// (xdnf.cn/news/5086), section "三、KV Cache内存管理的工程实现").  Grid: x =
// (pair, segment), y = pool (0 = K, 1 = V).  A work-group moves one
// kCopySegChunks * 16-byte segment of one block: four independent 16-byte
// loads per thread in flight, then four stores.  The stores are
// non-temporal: the copy's destination is not read again soon, and keeping
// its lines out of the caches took a 512 MiB copy from ~4.6 to ~6.5 TB/s on
// MI355X (non-temporal loads, by contrast, made it slower).
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
static_assert(kCopySegChunks == kCopyThreads * kCopyUnroll, "copy segment size");

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    u32x4 *k_cache, u32x4 *v_cache, const int32_t *__restrict__ src_blocks,
    const int32_t *__restrict__ dst_blocks, int32_t num_blocks, int64_t block_chunks,
    int32_t segs) {
  const int64_t pair = blockIdx.x / segs;
  const int64_t seg = blockIdx.x - pair * segs;
  const int32_t s = src_blocks[pair];
  const int32_t d = dst_blocks[pair];
  if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) return;
  u32x4 *pool = blockIdx.y == 0 ? k_cache : v_cache;
  const u32x4 *from = pool + (int64_t)s * block_chunks;
  u32x4 *to = pool + (int64_t)d * block_chunks;
  const int64_t base = seg * kCopySegChunks + threadIdx.x;
  u32x4 r[kCopyUnroll];
#pragma unroll
  for (int j = 0; j < kCopyUnroll; ++j) {
    const int64_t c = base + j * kCopyThreads;
    if (c < block_chunks) r[j] = from[c];
  }
#pragma unroll
  for (int j = 0; j < kCopyUnroll; ++j) {
    const int64_t c = base + j * kCopyThreads;
    if (c < block_chunks) __builtin_nontemporal_store(r[j], to + c);
  }
}

// table[j][i] = (cos, sin)(j * base^(-2i/D)), double precision, rounded to float.
__global__ __launch_bounds__(256) void rope_table_kernel(float2 *table, int32_t capacity,
                                                         int32_t half_dim, double base) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)capacity * half_dim) return;
  const int j = (int)(idx / half_dim);
  const int i = (int)(idx - (int64_t)j * half_dim);
  const double theta = pow(base, -2.0 * i / (2.0 * half_dim));
  double s, c;
  sincos((double)j * theta, &s, &c);
  table[idx] = make_float2((float)c, (float)s);
}

}  // namespace

hipError_t launch_reshape_and_cache(pa_dtype dtype, void *k_cache, void *v_cache,
                                    const void *key, const void *value,
                                    const int32_t *slot_mapping, int32_t num_tokens,
                                    int32_t row_elems, int64_t num_slots, hipStream_t stream) {
  const int64_t bytes = (int64_t)row_elems * (dtype == PA_F32 ? 4 : 2);
  const int32_t chunks = (int32_t)(bytes / 16);
  const int threads = chunks >= 256 ? 256 : ((chunks + 63) / 64) * 64;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(num_tokens), dim3(threads), 0, stream,
                     static_cast<uint4 *>(k_cache), static_cast<uint4 *>(v_cache),
                     static_cast<const uint4 *>(key), static_cast<const uint4 *>(value),
                     slot_mapping, chunks, num_slots);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(pa_dtype act_dtype, int kv8, void *k_cache, void *v_cache,
                                        const void *key, const void *value,
                                        const int32_t *slot_mapping, int32_t num_tokens,
                                        int32_t num_kv_heads, int32_t head_dim, int64_t num_slots,
                                        const KvScales &inv, hipStream_t stream) {
  if (kv8 != kKvE4M3 && kv8 != kKvE5M2) return hipErrorInvalidValue;
  const int32_t chunks = num_kv_heads * head_dim / 16;
  const int threads = chunks >= 256 ? 256 : ((chunks + 63) / 64) * 64;
  auto *kc = static_cast<uint4 *>(k_cache);
  auto *vc = static_cast<uint4 *>(v_cache);
  auto *kk = static_cast<const uint4 *>(key);
  auto *vv = static_cast<const uint4 *>(value);
  const bool e5 = kv8 == kKvE5M2;
  auto kernel = act_dtype == PA_BF16
                    ? (e5 ? reshape_and_cache_fp8_kernel<BF16, kKvE5M2> : reshape_and_cache_fp8_kernel<BF16, kKvE4M3>)
                    : (e5 ? reshape_and_cache_fp8_kernel<F16, kKvE5M2> : reshape_and_cache_fp8_kernel<F16, kKvE4M3>);
  hipLaunchKernelGGL(kernel, dim3(num_tokens), dim3(threads), 0, stream, kc, vc, kk, vv, slot_mapping, chunks,
                     head_dim, num_slots, inv);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void *k_cache, void *v_cache, const int32_t *src_blocks,
                              const int32_t *dst_blocks, int32_t num_pairs, int32_t num_blocks,
                              int64_t block_bytes, hipStream_t stream) {
  const int64_t chunks = block_bytes / 16;
  const int32_t segs = (int32_t)((chunks + kCopySegChunks - 1) / kCopySegChunks);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)((int64_t)num_pairs * segs), 2),
                     dim3(kCopyThreads), 0, stream, static_cast<u32x4 *>(k_cache),
                     static_cast<u32x4 *>(v_cache), src_blocks, dst_blocks, num_blocks, chunks, segs);
  return hipGetLastError();
}

// Checks of the device-resident inputs the fast path trusts, one work-group:
// counts of lengths outside [0, max_context], of block-table entries a
// decode reads (the first ceil(L / block_size) of each row, L the resident
// key count) outside [0, num_blocks), and of slots at or beyond num_slots.
// Thread 0 stores the three counts and a zero; no atomics, no memset.
__global__ __launch_bounds__(256) void check_inputs_kernel(
    const int32_t *__restrict__ block_tables, int32_t max_blocks_per_seq,
    const int32_t *__restrict__ context_lens, int32_t num_seqs, int32_t max_context,
    int32_t block_size, int32_t num_blocks, int32_t ring_capacity,
    const int32_t *__restrict__ slots, int32_t num_slot_entries, int64_t num_slots,
    int32_t *__restrict__ counts) {
  __shared__ int32_t s_red[3][256];
  int32_t bad_len = 0, bad_block = 0, bad_slot = 0;
  for (int b = threadIdx.x; b < num_seqs; b += blockDim.x) {
    const int32_t n = context_lens[b];
    if (n < 0 || n > max_context) ++bad_len;
  }
  // rows of the tables: one sequence at a time, its entries across threads
  for (int b = 0; b < num_seqs; ++b) {
    int32_t n = context_lens[b];
    n = n < 0 ? 0 : (n > max_context ? max_context : n);
    const int32_t keys = ring_capacity > 0 && n > ring_capacity ? ring_capacity : n;
    const int32_t need = (keys + block_size - 1) / block_size;
    const int32_t lim = need < max_blocks_per_seq ? need : max_blocks_per_seq;
    for (int j = threadIdx.x; j < lim; j += blockDim.x) {
      const int32_t id = block_tables[(int64_t)b * max_blocks_per_seq + j];
      if (id < 0 || id >= num_blocks) ++bad_block;
    }
  }
  for (int i = threadIdx.x; i < num_slot_entries; i += blockDim.x)
    if ((int64_t)slots[i] >= num_slots) ++bad_slot;
  s_red[0][threadIdx.x] = bad_len;
  s_red[1][threadIdx.x] = bad_block;
  s_red[2][threadIdx.x] = bad_slot;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w)
      for (int k = 0; k < 3; ++k) s_red[k][threadIdx.x] += s_red[k][threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    counts[0] = s_red[0][0];
    counts[1] = s_red[1][0];
    counts[2] = s_red[2][0];
    counts[3] = 0;
  }
}

hipError_t launch_check_inputs(const int32_t *block_tables, int32_t max_blocks_per_seq,
                               const int32_t *context_lens, int32_t num_seqs, int32_t max_context,
                               int32_t block_size, int32_t num_blocks, int32_t ring_capacity,
                               const int32_t *slots, int32_t num_slot_entries, int64_t num_slots,
                               int32_t *counts, hipStream_t stream) {
  hipLaunchKernelGGL(check_inputs_kernel, dim3(1), dim3(256), 0, stream, block_tables, max_blocks_per_seq,
                     context_lens, num_seqs, max_context, block_size, num_blocks, ring_capacity, slots,
                     num_slot_entries, num_slots, counts);
  return hipGetLastError();
}

// Streaming-read probe (a measurement aid, not part of the attention path):
// work-group w reads the 16-byte pieces w * U * 256 + u * 256 + t, stepping
// by the grid, with the same non-temporal loads the decode uses for K/V,
// and stores the XOR of every 32-bit word it read to out[w].
constexpr int kProbeUnroll = 8;
__global__ __launch_bounds__(256) void read_probe_kernel(const char *src, int64_t pieces, uint32_t *out) {
  const int64_t step = (int64_t)gridDim.x * kProbeUnroll * 256;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t p0 = (int64_t)blockIdx.x * kProbeUnroll * 256; p0 < pieces; p0 += step) {
    // one descriptor per round keeps every offset below 2^31 bytes
    const int64_t left = pieces - p0;
    const int nrec = (int)(16 * (left < kProbeUnroll * 256 ? left : (int64_t)kProbeUnroll * 256));
    const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(src + 16 * p0), (short)0, nrec,
                                                     kBufferWord3);
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      v[u] = __builtin_bit_cast(u32x4, buffer_load16<kCacheStream>(r, 16 * (u * 256 + (int)threadIdx.x)));
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
  __shared__ uint32_t s_x[4];
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = s_x[0] ^ s_x[1] ^ s_x[2] ^ s_x[3];
}

hipError_t launch_read_probe(const void *src, int64_t bytes, uint32_t *out, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const char *>(src),
                     bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_rope_table_init(float *table, int32_t capacity, int32_t head_dim,
                                  float rope_base, hipStream_t stream) {
  const int64_t total = (int64_t)capacity * (head_dim / 2);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<float2 *>(table), capacity, head_dim / 2, (double)rope_base);
  return hipGetLastError();
}

}  // namespace pa
