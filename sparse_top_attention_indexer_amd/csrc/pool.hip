// Block pooling of raw indexer keys (llama.cpp mirror commit c88c916636: one
// mean-pooled key per complete block of compress_ratio positions, pooled from
// the raw keys, before any norm or rotation), one-shot or incremental
// (offgrid-sys llama-memory-hybrid-idx.h: pooled keys persist across batches,
// each micro-batch re-pools only new pools, an edit stales the pools from its
// position on).
#include "dsa_device.h"
#include "dsa_internal.h"
#include "../../include/dsa.h"

namespace dsa {

// Blocks [from_block[s], floor(min(kv_len[s], n_kv) / c)) of sequence s when
// from_block is given (the incremental form), else every complete block.
__device__ __forceinline__ bool pool_block_live(int64_t s, int64_t b, int64_t n_kv, int c,
                                                const int32_t* from_block, const int32_t* kv_len) {
  if (!from_block) return true;
  int64_t kl = kv_len ? static_cast<int64_t>(kv_len[s]) : n_kv;
  if (kl > n_kv) kl = n_kv;
  return b >= from_block[s] && b < (kl > 0 ? kl / c : 0);
}

// D = 128: one workgroup of 256 threads per (sequence, block).  Lane group g
// (16 lanes, 8 dims each, one 16-byte load of a 16-bit row) sums rows g,
// g + 16, g + 32, ... of the block in that order; the 16 partial sums then
// add in the order g = 0 .. 15 through LDS, and the total is divided by c.
// The order is fixed, so a block's value never depends on which call pools
// it: an incremental pool equals a one-shot pool bit for bit.
__global__ __launch_bounds__(256) void block_pool_kernel(const void* k, int dtype, int64_t n_kv, int c, int64_t nb,
                                                         const int32_t* from_block, const int32_t* kv_len,
                                                         float* out) {
  __shared__ f32x4_t s_part[16][16][2];   // [row group][lane in group][half]
  const int64_t sb = blockIdx.x;
  const int64_t s = sb / nb, b = sb % nb;
  if (!pool_block_live(s, b, n_kv, c, from_block, kv_len)) return;   // whole workgroup
  const int g = threadIdx.x >> 4, l = threadIdx.x & 15;
  const int64_t base = (s * n_kv + b * c) * 128 + 8 * l;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int t = g; t < c; t += 16) {
    const int64_t off = base + static_cast<int64_t>(t) * 128;
    if (dtype == DSA_F32) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(k) + off);
      const f32x4_t e = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(k) + off + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] += a[j];
        acc[4 + j] += e[j];
      }
    } else {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(k) + off);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint16_t lo = static_cast<uint16_t>(w[j] & 0xffffu), hi = static_cast<uint16_t>(w[j] >> 16);
        acc[2 * j] += dtype == DSA_BF16 ? bf16_to_f32(lo) : f16_to_f32(lo);
        acc[2 * j + 1] += dtype == DSA_BF16 ? bf16_to_f32(hi) : f16_to_f32(hi);
      }
    }
  }
  s_part[g][l][0] = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
  s_part[g][l][1] = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
  __syncthreads();
  if (threadIdx.x < 32) {   // lane l of half h: dims 8 l + 4 h .. + 3
    const int ll = threadIdx.x >> 1, h = threadIdx.x & 1;
    f32x4_t tot = s_part[0][ll][h];
    for (int gg = 1; gg < 16; ++gg) tot += s_part[gg][ll][h];
    const float inv_c = static_cast<float>(c);
    *reinterpret_cast<f32x4_t*>(out + sb * 128 + 8 * ll + 4 * h) =
        f32x4_t{tot[0] / inv_c, tot[1] / inv_c, tot[2] / inv_c, tot[3] / inv_c};
  }
}

// Any D: one workgroup per (sequence, block); threads stride over the D dims,
// each summing the c rows in row order.
__global__ __launch_bounds__(256) void block_pool_any_d_kernel(const void* k, int dtype, int64_t n_kv, int D,
                                                               int c, int64_t nb, const int32_t* from_block,
                                                               const int32_t* kv_len, float* out) {
  const int64_t sb = blockIdx.x;
  const int64_t s = sb / nb, b = sb % nb;
  if (!pool_block_live(s, b, n_kv, c, from_block, kv_len)) return;
  const int64_t base = (s * n_kv + b * c) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f;
    for (int t = 0; t < c; ++t) acc += load_elem(k, base + static_cast<int64_t>(t) * D + d, dtype);
    out[sb * D + d] = acc / static_cast<float>(c);
  }
}

hipError_t launch_block_pool(const void* k_raw, int dtype, int S, int64_t n_kv, int D, int c,
                             const int32_t* from_block, const int32_t* kv_len, float* pooled, hipStream_t st) {
  const int64_t nb = n_kv / c;
  if (nb == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(S * nb));
  if (D == 128) {
    hipLaunchKernelGGL(block_pool_kernel, grid, dim3(256), 0, st, k_raw, dtype, n_kv, c, nb, from_block, kv_len,
                       pooled);
  } else {
    const int threads = D >= 256 ? 256 : ((D + 63) / 64) * 64;
    hipLaunchKernelGGL(block_pool_any_d_kernel, grid, dim3(threads), 0, st, k_raw, dtype, n_kv, D, c, nb,
                       from_block, kv_len, pooled);
  }
  return hipGetLastError();
}

}  // namespace dsa
