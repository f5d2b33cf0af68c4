// Device-side helpers shared by the gfx950 kernels of the DSA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace dsa {

constexpr int WAVE = 64;
constexpr float NEG_INF = -__builtin_inff();

// ---------------------------------------------------------------- scalars --

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}
// Round-to-nearest-even f32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Order-preserving map float -> uint32: a < b as floats iff key(a) < key(b).
// -0 and +0 compare equal, so both take the key of +0: equal scores tie, and
// a tie goes to the lower index whatever the signs of the zeros (a score is
// -0 when every head's ReLU is zero and the head weights are negative).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = u == 0x80000000u ? 0u : u;
  return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}

// Visible prefix length of a query row: keys 0 .. n-1 with n = min(q_pos + 1, kv_len),
// clamped to [0, n_store].
__device__ __forceinline__ int64_t visible_tokens(int32_t q_pos, int64_t kv_len, int64_t n_store) {
  int64_t n = static_cast<int64_t>(q_pos) + 1;
  if (kv_len < n) n = kv_len;
  if (n > n_store) n = n_store;
  return n < 0 ? 0 : n;
}

// ------------------------------------------------------------- MFMA wraps --

__device__ __forceinline__ f32x16_t mfma32x32x16_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32x32x16_f16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16x16x32_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16x16x32_f16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Packs two floats as bf16 (low half = a) / f16.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));   // one v_cvt_pk_bf16_f32
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_f16(a)) | (static_cast<uint32_t>(f32_to_f16(b)) << 16);
}

// Four OCP e4m3fn bytes (one dword) -> four f16 values equal to the fp8 values times 2^-8,
// exactly: the 7 magnitude bits of e4m3 shifted up by 7 form an f16 whose exponent bias
// differs by 8 (15 vs 7), and e4m3 subnormals map to f16 subnormals the same way.
// (The NaN code 0x7f maps to a finite value; stored keys never hold it.)
__device__ __forceinline__ u32x2_t fp8x4_to_f16x4_scaled(uint32_t x) {
  // spread bytes b0..b3 into the low bytes of four 16-bit lanes (byte
  // permutes; selector 0x0c gives a zero byte)
  const uint32_t lo = __builtin_amdgcn_perm(0u, x, 0x0c010c00u);   // [0, b1, 0, b0]
  const uint32_t hi = __builtin_amdgcn_perm(0u, x, 0x0c030c02u);   // [0, b3, 0, b2]
  // per lane: (b + (b & 0x80)) << 7 = ((b & 0x7f) << 7) | ((b & 0x80) << 8),
  // exponent and mantissa up by 7 bits and the sign to bit 15, with no carry
  // out of the 16-bit lane
  u32x2_t r;
  r.x = (lo + (lo & 0x00800080u)) << 7;
  r.y = (hi + (hi & 0x00800080u)) << 7;
  return r;
}

// One element of a tensor of dtype (0 f32, 1 bf16, 2 f16, 3 fp8 e4m3fn) as f32.
__device__ __forceinline__ float load_elem(const void* p, int64_t i, int dtype) {
  switch (dtype) {
    case 0: return static_cast<const float*>(p)[i];
    case 1: return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    case 2: return f16_to_f32(static_cast<const uint16_t*>(p)[i]);
    default: {
      const uint8_t b = static_cast<const uint8_t*>(p)[i];
      const int e = (b >> 3) & 15, m = b & 7;
      float v = e ? ldexpf(1.0f + m * 0.125f, e - 7) : ldexpf(m * 0.125f, -6);
      if (e == 15 && m == 7) v = __builtin_nanf("");
      return (b & 0x80) ? -v : v;
    }
  }
}

// ---------------------------------------------------------- block helpers --

// Exclusive prefix sum over a block of NW waves; also returns the total.
// `scratch` must hold NW uint32 of LDS.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) scratch[wid] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    uint32_t s = scratch[w];
    if (w < wid) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__device__ __forceinline__ uint32_t block_excl_scan_256(uint32_t v, uint32_t* scratch, uint32_t* total) {
  return block_excl_scan<4>(v, scratch, total);
}

}  // namespace dsa
