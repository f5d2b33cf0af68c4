// Block pooling of raw indexer keys (llama.cpp mirror commit c88c916636: one
// mean-pooled key per complete block of compress_ratio positions, pooled from
// the raw keys, before any norm or rotation).
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

// One workgroup per (sequence, block); threads stride over the D dims, so each
// of the c rows is read as one coalesced row.  Sum in f32 in row order, then
// divide by c.
__global__ __launch_bounds__(256) void block_pool_kernel(const void* k, int dtype, int64_t n_kv, int D,
                                                         int c, int64_t nb, float* out) {
  const int64_t sb = blockIdx.x;
  const int64_t s = sb / nb, b = sb % nb;
  const int64_t base = (s * n_kv + b * c) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f;
    for (int t = 0; t < c; ++t) acc += load_elem(k, base + static_cast<int64_t>(t) * D + d, dtype);
    out[sb * D + d] = acc / static_cast<float>(c);
  }
}

hipError_t launch_block_pool(const void* k_raw, int dtype, int S, int64_t n_kv, int D, int c,
                             float* pooled, hipStream_t st) {
  const int64_t nb = n_kv / c;
  if (nb == 0) return hipSuccess;
  const int threads = D >= 256 ? 256 : ((D + 63) / 64) * 64;
  hipLaunchKernelGGL(block_pool_kernel, dim3(static_cast<unsigned>(S * nb)), dim3(threads), 0, st,
                     k_raw, dtype, n_kv, D, c, nb, pooled);
  return hipGetLastError();
}

}  // namespace dsa
