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

hipError_t launch_rope_table_init(float *table, int32_t capacity, int32_t head_dim,
                                  float rope_base, hipStream_t stream) {
  const int64_t total = (int64_t)capacity * (head_dim / 2);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<float2 *>(table), capacity, head_dim / 2, (double)rope_base);
  return hipGetLastError();
}

}  // namespace pa
