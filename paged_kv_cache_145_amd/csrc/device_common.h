// Device helpers for the gfx950 kernels: storage-type tags, conversions,
// 16-byte vector loads and wavefront (wave64) cross-lane reductions.
#ifndef PA_DEVICE_COMMON_H_
#define PA_DEVICE_COMMON_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"  // kKvE4M3, kKvE5M2

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 bytes as a vector type: arrays of it stay in registers where arrays of
// the uint4 struct can be placed in memory
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

// ------------------------------------------------------------ type tags ---
// Storage is raw bits: uint16_t for f16/bf16, float for f32.
struct F32 {
  typedef float storage;
  static constexpr int kBytes = 4;
  static __device__ __forceinline__ float to_float(float x) { return x; }
  static __device__ __forceinline__ float from_float(float x) { return x; }
};

struct F16 {
  typedef uint16_t storage;
  typedef f16x8 vec8;
  typedef f16x4 vec4;
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ float to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
  }
  static __device__ __forceinline__ uint16_t from_float(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);  // round to nearest even
  }
  // from_float of two values, lo in bits 0..15 (one v_cvt_pk_f16_f32)
  static __device__ __forceinline__ uint32_t pack_pair(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
  }
  static __device__ __forceinline__ f32x4 mfma_16x16x32(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma_16x16x16(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  // Two E4M3 codes (bytes 2 HI, 2 HI + 1 of w) to two f16 values, exactly.
  template <bool HI>
  static __device__ __forceinline__ uint32_t from_fp8_pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
  // Two E5M2 codes to two f16 values, exactly (E5M2 is f16's top byte).
  template <bool HI>
  static __device__ __forceinline__ uint32_t from_bf8_pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, HI));
  }
};

struct BF16 {
  typedef uint16_t storage;
  typedef bf16x8 vec8;
  typedef bf16x4 vec4;
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ float to_float(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
  }
  static __device__ __forceinline__ uint16_t from_float(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
  }
  // from_float of two values, lo in bits 0..15 (one v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ uint32_t pack_pair(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
  }
  static __device__ __forceinline__ f32x4 mfma_16x16x32(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma_16x16x16(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                     __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
  }
  // Two E4M3 codes (bytes 2 HI, 2 HI + 1 of w) to two bf16 values, exactly
  // (every E4M3 value, subnormals included, is a bf16 value).
  template <bool HI>
  static __device__ __forceinline__ uint32_t from_fp8_pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
  // Two E5M2 codes to two bf16 values, exactly (2^-16 .. 57344 lie well
  // inside bf16's range and 3 significant bits fit its 8).
  template <bool HI>
  static __device__ __forceinline__ uint32_t from_bf8_pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
  }
};

// Unpack the element e (0..7) of a 16-byte vector of 16-bit values.
__device__ __forceinline__ uint16_t half_of(const uint4 &v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// ------------------------------------------------------------ cross-lane ---
// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowRor8 = 0x128;   // rotate right by 8 within a 16-lane row
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N consecutive lanes (N in {4, 8, 16, 32, 64});
// every lane of a group receives the group total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f32<kDppQuadXor1>(x);
  x += dpp_f32<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp_f32<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f32<kDppRowRor8>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------- LDS ------
// gfx950 transposing LDS read of 16-bit data.  Within each group of 16
// lanes, lane i receives element (i % 4) of the 8 bytes that lanes
// 4k + i / 4 (k = 0..3) address, i.e. result[i][k] = supplied[4k + i/4][i%4].
// Reading a row-major [token][d] tile with lane s addressing row
// (4 g + s / 4), column (n0 + 4 (s % 4)) therefore yields, in lane i, the
// four consecutive tokens 4 g .. 4 g + 3 of column n0 + i.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16_b64(const void *lds_addr) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  // an address-space cast, not an integer round trip, so that the compiler
  // still sees which LDS object is read (its waits for loads that write
  // LDS directly then name only that object)
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(__attribute__((address_space(3))) const char *)lds_addr);
  return __builtin_bit_cast(uint2, r);
}

// ------------------------------------------------------- buffer loads ---
// Raw (untyped) buffer descriptor word 3 for gfx9-family parts: 32-bit
// data format, no swizzle.  Loads whose byte offset falls outside the
// descriptor's num_records return zeros and access no memory.
constexpr int kBufferWord3 = 0x00020000;

// Cache policy of a load (the instruction's cache-control bits): kCacheNormal,
// or kCacheStream for data read once (the non-temporal bit: the K/V rows of
// a decode are used once and should not displace reused lines; measured on
// MI355X, a 1 GiB read streams at ~7.0 TB/s with it against ~6.2 TB/s).
constexpr int kCacheNormal = 0;
constexpr int kCacheStream = 2;

template <int POLICY = kCacheNormal>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
}
template <int POLICY = kCacheNormal>
__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POLICY));
}
template <int POLICY = kCacheNormal>
__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POLICY);
}

// Nearest E4M3 code of a float, ties to the even code, magnitudes of 448
// and above saturating to 448, NaN to the NaN code (OCP 8-bit float: bias
// 7, 3 mantissa bits, exponent field 0 = subnormals of step 2^-9).
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: a * 2^9 is exact; round it to an integer
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);  // 8 -> code 8 = 2^-6
  }
  // normal: drop 20 of the 23 fraction bits with round-to-nearest-even
  const uint32_t ab = __float_as_uint(a);
  const uint32_t r = (ab + 0x7FFFFu + ((ab >> 20) & 1u)) & 0xFFF00000u;
  const uint32_t code = ((((r >> 23) - 127u + 7u) & 0xFu) << 3) | ((r >> 20) & 7u);
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// Nearest E5M2 code of a float, ties to the even code, magnitudes of 57344
// and above (infinities too) saturating to 57344, NaN to 0x7F (OCP 8-bit
// float: bias 15, 2 mantissa bits, exponent field 0 = subnormals of step
// 2^-16, exponent field 31 = infinity / NaN, never produced here).
__device__ __forceinline__ uint32_t e5m2_code(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return 0x7Fu;
  if (a >= 57344.0f) return sign | 0x7Bu;
  if (a < 6.103515625e-05f) {  // below 2^-14: a * 2^16 is exact; round it to an integer
    return sign | (uint32_t)__builtin_rintf(a * 65536.0f);  // 4 -> code 4 = 2^-14
  }
  // normal: drop 21 of the 23 fraction bits with round-to-nearest-even
  const uint32_t ab = __float_as_uint(a);
  const uint32_t r = (ab + 0xFFFFFu + ((ab >> 21) & 1u)) & 0xFFE00000u;
  const uint32_t code = ((((r >> 23) - 127u + 15u) & 0x1Fu) << 2) | ((r >> 21) & 3u);
  return sign | (code > 0x7Bu ? 0x7Bu : code);
}

// Code of format F (kKvE4M3 or kKvE5M2) of a float.
template <int F>
__device__ __forceinline__ uint32_t fp8_code(float x) {
  static_assert(F == kKvE4M3 || F == kKvE5M2, "8-bit format");
  if constexpr (F == kKvE5M2) return e5m2_code(x);
  else return e4m3_code(x);
}

template <class T, int F, bool HI>
__device__ __forceinline__ uint32_t code_pair_to_16(uint32_t w) {
  static_assert(F == kKvE4M3 || F == kKvE5M2, "8-bit format");
  if constexpr (F == kKvE5M2) return T::template from_bf8_pair<HI>(w);
  else return T::template from_fp8_pair<HI>(w);
}

// Eight / four 8-bit codes of format F to 16-bit values of the tag T
// (little-endian order kept: code e lands in 16-bit element e).
template <class T, int F>
__device__ __forceinline__ uint4 fp8x8_to_16(uint2 v) {
  return make_uint4(code_pair_to_16<T, F, false>(v.x), code_pair_to_16<T, F, true>(v.x),
                    code_pair_to_16<T, F, false>(v.y), code_pair_to_16<T, F, true>(v.y));
}
template <class T, int F>
__device__ __forceinline__ uint2 fp8x4_to_16(uint32_t v) {
  return make_uint2(code_pair_to_16<T, F, false>(v), code_pair_to_16<T, F, true>(v));
}

#ifdef PA_WAVE_TIMELINE
// Measurement build only: the real-time counter (100 MHz, the same on every
// XCD) and the XCC id of the executing wave (hardware register XCC_ID, bits
// 3:0).
__device__ __forceinline__ uint64_t tl_now() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint64_t tl_xcc() { return (uint64_t)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15); }
#endif

// Cost-weighted stream-K ranges (single- and multi-token decode).  Sequence
// (or virtual sequence) b weighs its tiles plus `cost` tiles' worth of work
// for its start and end, so the weighted position of its tile t is W(b) + cost + t with W(b) = s_tfirst[b] + cost * b (strictly
// increasing in b when cost > 0).  Group q takes the tiles whose weighted
// position lies in [q * per, (q + 1) * per): a range that opens many short
// sequences gets fewer tiles.  Every boundary depends only on the lengths,
// the cost and the grid, so the combine order stays fixed.  cost = 0 gives
// ranges of equal tile counts.
__device__ __forceinline__ int64_t weighted_total(int total, int num_seqs, int cost) {
  return (int64_t)total + (int64_t)cost * num_seqs;
}

// Range sizes when a kernel runs two work-groups per CU.  Work-groups are
// dispatched in index order, one per CU first, so the groups q >= young_from
// (the second work-group of their CU) issue behind the first one and stream
// more slowly; their ranges are young_share / 1024 of the others'.  Group q
// covers weighted positions [range_start(q), range_start(q + 1)); every
// boundary still depends only on the lengths, the costs and the grid.
struct RangeSplit {
  int64_t per, per_young;
  int young_from;
};

__device__ __forceinline__ RangeSplit range_split(int64_t wtotal, int groups, int young_from, int young_share) {
  RangeSplit r;
  r.young_from = min(max(young_from, 0), groups);
  const int ny = groups - r.young_from;
  if (ny == 0 || young_share >= 1024 || young_share <= 0) {
    r.per = (wtotal + groups - 1) / groups;
    r.per_young = r.per;
    r.young_from = groups;
  } else {
    const int64_t den = (int64_t)r.young_from * 1024 + (int64_t)ny * young_share;
    r.per = max((int64_t)1, (wtotal * 1024 + den - 1) / den);
    r.per_young = max((int64_t)1, (r.per * young_share + 1023) / 1024);
  }
  return r;
}

__device__ __forceinline__ int64_t range_start(const RangeSplit &r, int q) {
  return q <= r.young_from ? (int64_t)q * r.per
                           : (int64_t)r.young_from * r.per + (int64_t)(q - r.young_from) * r.per_young;
}

// The group whose range holds weighted position x.
__device__ __forceinline__ int range_of(const RangeSplit &r, int64_t x) {
  const int64_t yo = (int64_t)r.young_from * r.per;
  return x < yo ? (int)(x / r.per) : r.young_from + (int)((x - yo) / r.per_young);
}

// First tile whose weighted position is >= target (total if none).
__device__ __forceinline__ int weighted_tile(const int *s_tfirst, int num_seqs, int total, int cost,
                                             int64_t target) {
  if (target >= weighted_total(total, num_seqs, cost)) return total;
  int lo = 0, hi = num_seqs;  // largest b < num_seqs with W(b) <= target
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)s_tfirst[mid] + (int64_t)cost * mid <= target) lo = mid;
    else hi = mid;
  }
  const int64_t off = target - ((int64_t)s_tfirst[lo] + (int64_t)cost * lo) - cost;
  return s_tfirst[lo] + (off > 0 ? (int)off : 0);
}

// ------------------------------------------------------------- RoPE ---
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

// The same rotation on fragments in the dimension order of 8-bit pools,
// where chunk kb covers d = 64 (kb / 2) + 16 grp + 8 (kb % 2) + [0, 8) (a
// lane's 16-byte load of codes is 16 consecutive dimensions).  D = 128: the
// partner d + 64 is chunk kb + 2 of the same lane.  D = 64: the partner
// d +- 32 is the same chunk of lane ^ 32 (grp ^ 2).
template <class T, int D>
__device__ __forceinline__ void rope_frag16_kv8(uint4 (&f)[D / 32], const float *cs, int grp) {
  constexpr int KB = D / 32;
  auto rotate = [&](uint4 &own, const uint4 &partner, int d0, float sign) {
    const float4 *c4 = reinterpret_cast<const float4 *>(cs + 2 * d0);
    float c[8], s[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = c4[i];
      c[2 * i] = v.x;
      s[2 * i] = v.y;
      c[2 * i + 1] = v.z;
      s[2 * i + 1] = v.w;
    }
    uint16_t r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      r[e] = T::from_float(T::to_float(half_of(own, e)) * c[e] + sign * T::to_float(half_of(partner, e)) * s[e]);
    own = make_uint4(pack2(r[0], r[1]), pack2(r[2], r[3]), pack2(r[4], r[5]), pack2(r[6], r[7]));
  };
  if constexpr (D == 128) {
#pragma unroll
    for (int kb = 0; kb < KB / 2; ++kb) {
      const uint4 lo = f[kb], hi = f[kb + KB / 2];
      const int d0 = 16 * grp + 8 * kb;  // angle index of element 0 (d < D / 2)
      rotate(f[kb], hi, d0, -1.f);
      rotate(f[kb + KB / 2], lo, d0, 1.f);
    }
  } else {
    static_assert(D == 64, "head size");
    const bool low = grp < 2;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      uint4 partner;
      partner.x = __shfl_xor(f[kb].x, 32);
      partner.y = __shfl_xor(f[kb].y, 32);
      partner.z = __shfl_xor(f[kb].z, 32);
      partner.w = __shfl_xor(f[kb].w, 32);
      rotate(f[kb], partner, 16 * (grp & 1) + 8 * kb, low ? -1.f : 1.f);
    }
  }
}

}  // namespace pa

#endif  // PA_DEVICE_COMMON_H_
