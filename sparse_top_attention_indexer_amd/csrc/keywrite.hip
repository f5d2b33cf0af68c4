// Indexer-key cache write: rotate new keys and store them in the cache type.
//
// ik_llama.cpp PR #2058, "decode-correct indexer-K cache" commit: the batch's
// Walsh-Hadamard-rotated indexer keys are written into the key cache at the
// batch's cache rows (kv_head), then read back whole for scoring.  The
// ik_llama_opt log ("GLM-DSA: allow for quantized indexer cache") and unsloth
// llama.cpp PR #293 (deepseek41 quantized K cache) store rows in a quantized
// cache type after rotating them in F32.  Here the cache is f16, bf16, or fp8
// e4m3fn with one f32 scale per row.
//
// Arithmetic (fixed bit for bit, so that every stored byte is reproducible):
//   x  = the row in f32 (exact for f32 / bf16 / f16 inputs)
//   y  = fast Walsh-Hadamard butterflies of x (spans 1, 2, ..., 64 in that
//        order, (a, b) -> (a + b, a - b)), unnormalised; or x unrotated
//   f16 / bf16 cache: y times f32(1/sqrt(128)) (rotated rows), rounded to
//        nearest, ties to even
//   fp8 cache: m = max_d |y(d)|, code(d) = e4m3fn(y(d) * (448 / m)) rounded
//        to nearest, ties to the even code, saturating at 448, and scale =
//        m * f32(1 / (448 sqrt(128))) (f32(1 / 448) unrotated), so code *
//        scale is the normalised value; a zero row stores scale 0, zero codes
// Every step is one correctly rounded f32 operation, with one division per
// row (448 / m) and none per element.
//
// Layout: a 16-lane group works on one key row at a time, lane g of the group
// holding elements 8 g .. 8 g + 7 (one 16-byte load of a 16-bit row, two of
// an f32 row).  Spans 1, 2 and 4 of the transform are inside a lane, spans
// 8 .. 64 between lanes g and g ^ 1, 2, 4, 8 (DPP row moves).  A workgroup of 256 threads
// covers 64 consecutive rows of one sequence (4 per group), so loads and
// stores move whole contiguous rows.  Bound: HBM (each row is read once and
// written once).
#include "dsa_device.h"
#include "dsa_internal.h"
#include "../../include/dsa.h"

namespace dsa {

namespace {

constexpr float INV_SQRT128 = 0x1.6a09e6p-4f;    // 1/sqrt(128) rounded to f32
constexpr float FP8_UNIT_ROT = 0x1.9dc22cp-13f;  // 1/(448 sqrt(128)) rounded to f32
constexpr float FP8_UNIT = 0x1.24924ap-9f;       // 1/448 rounded to f32

// Value of lane g ^ M of the same 16-lane row, by DPP moves: quad_perm for
// M = 1, 2; M = 4 as the half-row mirror (g ^ 7) followed by the quad reversal
// (g ^ 3); M = 8 as a rotation of the row by 8 lanes.  Every source lane is
// in the same row and enabled; bound_ctrl lets the compiler fold the move into
// the add that consumes it.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (M == 1) return dpp_mov<0xb1>(v);    // quad_perm [1, 0, 3, 2]
  if constexpr (M == 2) return dpp_mov<0x4e>(v);    // quad_perm [2, 3, 0, 1]
  if constexpr (M == 4) return dpp_mov<0x1b>(dpp_mov<0x141>(v));   // row_half_mirror, quad_perm [3, 2, 1, 0]
  if constexpr (M == 8) return dpp_mov<0x128>(v);   // row_ror:8
}

// One butterfly stage between lanes g and g ^ M: the lower lane keeps a + b,
// the upper lane b - a, computed as (-a) + b (the same IEEE operation); the
// negation is a sign-bit xor.
template <int M>
__device__ __forceinline__ void lane_stage(float (&x)[8], int g) {
  const uint32_t neg = (g & M) ? 0x80000000u : 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float other = lane_xor<M>(x[j]);
    x[j] = __uint_as_float(__float_as_uint(x[j]) ^ neg) + other;
  }
}

template <int M>
__device__ __forceinline__ float row_max_step(float v) {
  return fmaxf(v, lane_xor<M>(v));
}

// Four f32 values -> four e4m3fn codes (one dword, first value in the low
// byte) by the gfx950 conversion: round to nearest, ties to even.  Inputs are
// at most 448 (1 + 2^-22) in magnitude here, which rounds to 448.
__device__ __forceinline__ uint32_t e4m3fn_x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// Rows handled by one 16-lane group; their loads are all issued before any
// of them is transformed, so each lane keeps RPG loads in flight.
constexpr int RPG = 4;
constexpr int ROWS_PER_WG = 16 * RPG;

// Loads elements 8 g .. 8 g + 7 of one key row as f32.
__device__ __forceinline__ void load_row(const void* k_new, int k_dtype, int64_t row, int g, float (&x)[8]) {
  if (k_dtype == DSA_F32) {
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(k_new) + row * 128 + 8 * g);
    const f32x4_t lo = src[0], hi = src[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = lo[j];
      x[4 + j] = hi[j];
    }
  } else {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(k_new) + row * 128 + 8 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t e0 = static_cast<uint16_t>(w[j] & 0xffffu), e1 = static_cast<uint16_t>(w[j] >> 16);
      x[2 * j] = k_dtype == DSA_BF16 ? bf16_to_f32(e0) : f16_to_f32(e0);
      x[2 * j + 1] = k_dtype == DSA_BF16 ? bf16_to_f32(e1) : f16_to_f32(e1);
    }
  }
}

// Grid: x = blocks of ROWS_PER_WG new keys of one sequence, y = the sequence.
// Group q of a workgroup takes rows q, q + 16, q + 32, q + 48 of the block, so
// each load instruction of a wave reads 4 consecutive rows (1 KB of 16-bit keys).
__global__ __launch_bounds__(256) void key_write_kernel(const void* k_new, int k_dtype, int64_t n_new,
                                                        const int32_t* dst_row, int hadamard, void* cache,
                                                        int cache_dtype, float* cache_scale, int64_t n_cache) {
  const int64_t s = blockIdx.y;
  const int g = threadIdx.x & 15;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * ROWS_PER_WG + (threadIdx.x >> 4);

  float x[RPG][8];
  int64_t dst[RPG];
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    const int64_t t = t0 + 16 * i;
    dst[i] = -1;
    if (t < n_new) {   // the same for the 16 lanes of a group
      load_row(k_new, k_dtype, s * n_new + t, g, x[i]);
      const int64_t r = dst_row ? static_cast<int64_t>(dst_row[s * n_new + t]) : t;
      if (r >= 0 && r < n_cache) dst[i] = s * n_cache + r;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[i][j] = 0.f;
    }
  }

  if (hadamard) {
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
#pragma unroll
      for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (!(j & h)) {
            const float a = x[i][j], b = x[i][j + h];
            x[i][j] = a + b;
            x[i][j + h] = a - b;
          }
      lane_stage<1>(x[i], g);
      lane_stage<2>(x[i], g);
      lane_stage<4>(x[i], g);
      lane_stage<8>(x[i], g);
    }
  }

#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    if (cache_dtype == DSA_FP8_E4M3) {
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[i][j]));
      amax = row_max_step<8>(row_max_step<4>(row_max_step<2>(row_max_step<1>(amax))));
      if (dst[i] < 0) continue;
      const float inv = amax > 0.f ? 448.f / amax : 0.f;
      const float scale = amax * (hadamard ? FP8_UNIT_ROT : FP8_UNIT);
      float q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = x[i][j] * inv;
      const u32x2_t packed = {e4m3fn_x4(q[0], q[1], q[2], q[3]), e4m3fn_x4(q[4], q[5], q[6], q[7])};
      *reinterpret_cast<u32x2_t*>(static_cast<uint8_t*>(cache) + dst[i] * 128 + 8 * g) = packed;
      if (g == 0) cache_scale[dst[i]] = scale;
    } else {
      if (dst[i] < 0) continue;
      if (hadamard) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[i][j] *= INV_SQRT128;
      }
      u32x4_t packed;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        packed[j] = cache_dtype == DSA_BF16 ? pack_bf16x2(x[i][2 * j], x[i][2 * j + 1])
                                            : pack_f16x2(x[i][2 * j], x[i][2 * j + 1]);
      *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(cache) + dst[i] * 128 + 8 * g) = packed;
    }
  }
}

}  // namespace

hipError_t launch_key_write(const void* k_new, int k_dtype, int S, int64_t n_new, const int32_t* dst_row,
                            int hadamard, void* cache, int cache_dtype, float* cache_scale, int64_t n_cache,
                            hipStream_t st) {
  if (n_new == 0) return hipSuccess;
  hipLaunchKernelGGL(key_write_kernel,
                     dim3(static_cast<unsigned>((n_new + ROWS_PER_WG - 1) / ROWS_PER_WG), static_cast<unsigned>(S)),
                     dim3(256), 0, st, k_new, k_dtype, n_new, dst_row, hadamard, cache, cache_dtype, cache_scale,
                     n_cache);
  return hipGetLastError();
}

}  // namespace dsa
