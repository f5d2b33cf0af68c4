// C ABI of the DSA library: argument checks (all on the host, before any
// launch), workspace sizing, dispatch to the kernel launchers, and the fused
// whole-path entry point.  See include/dsa.h for the contract.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/dsa.h"
#include "dsa_internal.h"

using namespace dsa;

// The device scratch of dsa_topk_noalloc: one copy per GPU, held until the
// process ends.  Host code never passes this name to a kernel (on the host it
// is a stand-in, not a device address); it passes the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[DSA_TOPK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxBlocks = 4096;   // idx entries per row in block mode (LDS list)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t esize(int dt) { return dt == DSA_F32 ? 4 : (dt == DSA_FP8_E4M3 ? 1 : 2); }
inline size_t a256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
inline int hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}
hipError_t fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st) {
  int64_t b = (n + 255) / 256;
  if (b > 4096) b = 4096;
  if (b < 1) b = 1;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(static_cast<unsigned>(b)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

// ------------------------------------------------------------------ checks --

int check_index(const dsa_index_desc* d, const float* scores) {
  if (!d || !scores || !d->q || !d->k || !d->w || !d->q_pos) return DSA_ERR_NULL;
  if (d->S < 1 || d->n_q < 1 || d->n_units < 1 || d->n_units > 0x7fffffffLL) return DSA_ERR_SHAPE;
  if (d->H < 1 || d->H > 128 || d->D < 16 || d->D > 256 || d->D % 16) return DSA_ERR_SHAPE;
  if (d->c < 1 || (d->hadamard_q != 0 && d->hadamard_q != 1)) return DSA_ERR_PARAM;
  if (d->hadamard_q && d->D != 128) return DSA_ERR_SHAPE;
  if (d->q_dtype != DSA_F32 && d->q_dtype != DSA_BF16 && d->q_dtype != DSA_F16) return DSA_ERR_DTYPE;
  if (d->k_dtype < DSA_F32 || d->k_dtype > DSA_FP8_E4M3) return DSA_ERR_DTYPE;
  if ((d->k_dtype == DSA_FP8_E4M3) != (d->k_scale != nullptr)) return d->k_scale ? DSA_ERR_PARAM : DSA_ERR_NULL;
  if (!scores_use_mfma(d->q_dtype, d->k_dtype, d->H, d->D) && d->H * d->D > 32768) return DSA_ERR_UNSUPPORTED;
  if (!aligned16(d->q) || !aligned16(d->k) || !aligned16(scores)) return DSA_ERR_ALIGN;
  return DSA_OK;
}

int check_topk(const float* scores, const dsa_topk_desc* d, const int32_t* idx) {
  if (!d || !scores || !idx || !d->q_pos) return DSA_ERR_NULL;
  if (d->S < 1 || d->n_q < 1 || d->n_units < 1 || d->n_units > 0x7fffffffLL) return DSA_ERR_SHAPE;
  if (d->top_k < 1 || d->c < 1 || d->top_k % d->c) return DSA_ERR_PARAM;
  if (d->n_sink < 0 || d->n_sink > d->top_k || (d->n_sink > 0 && d->c > 1)) return DSA_ERR_PARAM;
  return DSA_OK;
}

// Attention family of a descriptor, or a negative status.
int attn_family(const dsa_attn_desc* d) {
  if (d->kv_format != 0 && d->kv_format != d->dtype && d->kv_format != DSA_Q8_0) return DSA_ERR_DTYPE;
  if (d->kv_format == DSA_Q8_0) {   // q8_0 latent rows: the MLA shapes only, byte strides
    if (d->dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (d->Hkv == 1 && d->Dk == 576 && d->Dv == 512 && d->Hq % 16 == 0 && d->v == d->k &&
        d->v_seq_stride == d->k_seq_stride && d->v_tok_stride == d->k_tok_stride &&
        d->n_kv * d->k_tok_stride < (int64_t(1) << 32))
      return ATTN_MLA;
    return DSA_ERR_UNSUPPORTED;
  }
  if (d->dtype == DSA_F32) {
    if (d->Dk > 256 || d->Dv > 256) return DSA_ERR_UNSUPPORTED;
    return ATTN_F32;
  }
  if (d->dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (d->Hkv == 1 && d->Dk == 576 && d->Dv == 512 && d->Hq % 16 == 0 && d->v == d->k &&
      d->v_seq_stride == d->k_seq_stride && d->v_tok_stride == d->k_tok_stride &&
      d->n_kv * d->k_tok_stride * 2 < (int64_t(1) << 32))   // 32-bit row offsets within a sequence
    return ATTN_MLA;
  if (d->Dk == 128 && d->Dv == 128 && d->Hq / d->Hkv <= 16) return ATTN_GQA;
  return DSA_ERR_UNSUPPORTED;
}

int check_attn(const dsa_attn_desc* d, const int32_t* idx, const void* out) {
  if (!d || !d->q || !d->k || !d->v || !d->q_pos || !out) return DSA_ERR_NULL;
  if (d->S < 1 || d->n_q < 1 || d->Hq < 1 || d->Hkv < 1 || d->Hq % d->Hkv || d->Dk < 1 || d->Dv < 1 ||
      d->n_kv < 1 || d->n_kv > 0x7fffffffLL)
    return DSA_ERR_SHAPE;
  if (d->o_dtype != DSA_F32 && d->o_dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (d->c < 1) return DSA_ERR_PARAM;
  if (idx && (d->k_sel < 1 || (d->c > 1 && d->k_sel > kMaxBlocks))) return DSA_ERR_SHAPE;
  if (d->k_tok_stride < 0 || d->k_seq_stride < 0 || d->k_head_stride < 0 || d->v_tok_stride < 0 ||
      d->v_seq_stride < 0 || d->v_head_stride < 0)
    return DSA_ERR_SHAPE;
  const int fam = attn_family(d);
  if (fam < 0) return fam;
  if (fam == ATTN_MLA && idx && d->c > 1 && d->k_sel > MLA_MAX_BLOCKS) return DSA_ERR_SHAPE;
  if (d->kv_format == DSA_Q8_0 && !d->kv_scale) return DSA_ERR_NULL;
  if (!aligned16(d->q) || !aligned16(d->k) || !aligned16(d->v) || !aligned16(out) || !aligned16(d->kv_scale))
    return DSA_ERR_ALIGN;
  const size_t es = d->kv_format == DSA_Q8_0 ? 1 : esize(d->dtype);
  if (fam != ATTN_F32) {
    const int64_t strides[6] = {d->k_seq_stride, d->k_tok_stride, d->k_head_stride,
                                d->v_seq_stride, d->v_tok_stride, d->v_head_stride};
    for (int64_t s : strides)
      if ((s * static_cast<int64_t>(es)) % 16) return DSA_ERR_ALIGN;
  }
  return DSA_OK;
}

AttnParams attn_params(const dsa_attn_desc* d, const int32_t* idx, void* out) {
  AttnParams p{};
  p.q = d->q;
  p.k = d->k;
  p.v = d->v;
  p.k_seq = d->k_seq_stride;
  p.k_tok = d->k_tok_stride;
  p.k_head = d->k_head_stride;
  p.v_seq = d->v_seq_stride;
  p.v_tok = d->v_tok_stride;
  p.v_head = d->v_head_stride;
  p.q_pos = d->q_pos;
  p.kv_len = d->kv_len;
  p.idx = idx;
  p.out = out;
  p.dtype = d->dtype;
  p.o_dtype = d->o_dtype;
  p.S = d->S;
  p.n_q = d->n_q;
  p.Hq = d->Hq;
  p.Hkv = d->Hkv;
  p.Dk = d->Dk;
  p.Dv = d->Dv;
  p.n_kv = d->n_kv;
  p.k_sel = idx ? d->k_sel : 0;
  p.c = d->c;
  const float scale = d->scale > 0.f ? d->scale : 1.0f / sqrtf(static_cast<float>(d->Dk));
  p.scale_log2 = scale * 1.4426950408889634f;
  p.family = attn_family(d);
  p.kq8 = d->kv_format == DSA_Q8_0 ? 1 : 0;
  p.k_scale = p.kq8 ? d->kv_scale : nullptr;
  int64_t list_len = d->n_kv;
  if (idx) list_len = d->c > 1 ? static_cast<int64_t>(d->k_sel) * d->c + d->c - 1 : d->k_sel;
  attn_plan(p, list_len);
  return p;
}

TopkParams topk_params(const float* scores, const dsa_topk_desc* d, int32_t* idx) {
  TopkParams p{};
  p.scores = scores;
  p.idx = idx;
  p.q_pos = d->q_pos;
  p.kv_len = d->kv_len;
  p.S = d->S;
  p.n_q = d->n_q;
  p.n_units = d->n_units;
  p.k_out = d->top_k / d->c;
  p.c = d->c;
  p.n_sink = d->n_sink;
  return p;
}

// ------------------------------------------------ the no-allocation top-k --

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Address of the current device's scratch, looked up once per device.
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DSA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_strerror(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case DSA_ERR_DTYPE: return "unsupported element type combination";
    case DSA_ERR_PARAM: return "invalid top_k, compress_ratio or n_sink";
    case DSA_ERR_ALIGN: return "pointer or row stride not 16-byte aligned";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_HIP: return "HIP runtime error";
    case DSA_ERR_UNSUPPORTED: return "no kernel for this shape";
    default: return "unknown status";
  }
}

int dsa_version(void) { return 100; }

size_t dsa_desc_size(int which) {
  switch (which) {
    case 0: return sizeof(dsa_index_desc);
    case 1: return sizeof(dsa_topk_desc);
    case 2: return sizeof(dsa_attn_desc);
    case 3: return sizeof(dsa_forward_desc);
    default: return 0;
  }
}

int dsa_index_scores(const dsa_index_desc* d, float* scores, void* stream) {
  const int st = check_index(d, scores);
  if (st) return st;
  ScoreParams p{};
  p.q = d->q;
  p.k = d->k;
  p.k_scale = d->k_scale;
  p.w = d->w;
  p.q_pos = d->q_pos;
  p.kv_len = d->kv_len;
  p.scores = scores;
  p.hist = nullptr;
  p.S = d->S;
  p.n_q = d->n_q;
  p.H = d->H;
  p.D = d->D;
  p.n_units = d->n_units;
  p.c = d->c;
  p.hadamard = d->hadamard_q;
  p.q_dtype = d->q_dtype;
  p.k_dtype = d->k_dtype;
  p.fill_invisible = 1;
  p.n_sink = 0;
  p.k_out = 0;
  return hip_status(launch_scores(p, as_stream(stream)));
}

size_t dsa_topk_workspace_bytes(const dsa_topk_desc* d) {
  if (!d || d->S < 1 || d->n_q < 1 || d->n_units < 1) return 0;
  return topk_workspace_bytes(static_cast<int64_t>(d->S) * d->n_q, d->n_units);
}

int dsa_topk(const float* scores, const dsa_topk_desc* d, int32_t* idx, void* workspace,
             size_t workspace_bytes, void* stream) {
  const int st = check_topk(scores, d, idx);
  if (st) return st;
  const size_t need = dsa_topk_workspace_bytes(d);
  if (need && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return DSA_ERR_ALIGN;
  TopkParams p = topk_params(scores, d, idx);
  if (need) topk_bind_workspace(p, workspace);
  return hip_status(launch_topk(p, false, as_stream(stream)));
}

int dsa_topk_noalloc(const float* scores, const dsa_topk_desc* d, int32_t* idx, void* stream) {
  const int st = check_topk(scores, d, idx);
  if (st) return st;
  const size_t need = dsa_topk_workspace_bytes(d);
  if (need > DSA_TOPK_NOALLOC_SCRATCH_BYTES) return DSA_ERR_WORKSPACE;
  TopkParams p = topk_params(scores, d, idx);
  if (need) {
    void* ws = nullptr;
    const int sst = scratch_of_current_device(&ws);
    if (sst) return sst;
    topk_bind_workspace(p, ws);   // the kernels clear what must start at zero
  }
  return hip_status(launch_topk(p, false, as_stream(stream)));
}

int dsa_block_pool(const void* k_raw, int32_t dtype, int32_t S, int64_t n_kv, int32_t D, int32_t c,
                   float* pooled, void* stream) {
  if (!k_raw || !pooled) return DSA_ERR_NULL;
  if (dtype != DSA_F32 && dtype != DSA_BF16 && dtype != DSA_F16) return DSA_ERR_DTYPE;
  if (S < 1 || n_kv < 1 || D < 1 || D > 4096) return DSA_ERR_SHAPE;
  if (c < 1) return DSA_ERR_PARAM;
  if (!aligned16(k_raw) || !aligned16(pooled)) return DSA_ERR_ALIGN;
  return hip_status(launch_block_pool(k_raw, dtype, S, n_kv, D, c, nullptr, nullptr, pooled, as_stream(stream)));
}

int dsa_block_pool_update(const void* k_raw, int32_t dtype, int32_t S, int64_t n_kv, int32_t D, int32_t c,
                          const int32_t* from_block, const int32_t* kv_len, float* pooled, void* stream) {
  if (!k_raw || !pooled || !from_block) return DSA_ERR_NULL;
  if (dtype != DSA_F32 && dtype != DSA_BF16 && dtype != DSA_F16) return DSA_ERR_DTYPE;
  if (S < 1 || n_kv < 1 || D < 1 || D > 4096) return DSA_ERR_SHAPE;
  if (c < 1) return DSA_ERR_PARAM;
  if (S * (n_kv / c) > 0x7fffffffLL) return DSA_ERR_SHAPE;
  if (!aligned16(k_raw) || !aligned16(pooled)) return DSA_ERR_ALIGN;
  return hip_status(launch_block_pool(k_raw, dtype, S, n_kv, D, c, from_block, kv_len, pooled, as_stream(stream)));
}

int32_t dsa_index_share_source(int32_t layer) {
  if (layer < 0) return DSA_ERR_PARAM;
  auto full = [](int32_t il) { return il <= 1 || il % 4 == 2; };
  while (!full(layer)) --layer;
  return layer;
}

int dsa_index_key_write(const void* k_new, int32_t k_dtype, int32_t S, int64_t n_new, int32_t D,
                        const int32_t* dst_row, int32_t hadamard, void* cache, int32_t cache_dtype,
                        float* cache_scale, int64_t n_cache, void* stream) {
  if (!cache || (!k_new && n_new != 0)) return DSA_ERR_NULL;   // an empty batch may pass no key buffer
  if (k_dtype != DSA_F32 && k_dtype != DSA_BF16 && k_dtype != DSA_F16) return DSA_ERR_DTYPE;
  if (cache_dtype != DSA_BF16 && cache_dtype != DSA_F16 && cache_dtype != DSA_FP8_E4M3) return DSA_ERR_DTYPE;
  if ((cache_dtype == DSA_FP8_E4M3) != (cache_scale != nullptr)) return cache_scale ? DSA_ERR_PARAM : DSA_ERR_NULL;
  if (S < 1 || S > 65535 || n_new < 0 || n_cache < 1 || D != 128) return DSA_ERR_SHAPE;
  if ((n_new + 15) / 16 > 0x7fffffffLL) return DSA_ERR_SHAPE;
  if (hadamard != 0 && hadamard != 1) return DSA_ERR_PARAM;
  if (!aligned16(k_new) || !aligned16(cache) || !aligned16(cache_scale) || !aligned16(dst_row)) return DSA_ERR_ALIGN;
  return hip_status(launch_key_write(k_new, k_dtype, S, n_new, dst_row, hadamard, cache, cache_dtype, cache_scale,
                                     n_cache, as_stream(stream)));
}

size_t dsa_sparse_attn_workspace_bytes(const dsa_attn_desc* d, int dense) {
  if (!d || attn_family(d) < 0 || d->S < 1 || d->n_q < 1 || d->n_kv < 1 || d->c < 1) return 0;
  if (!dense && d->k_sel < 1) return 0;
  static const int32_t dummy = 0;
  const AttnParams p = attn_params(d, dense ? nullptr : &dummy, nullptr);
  return attn_workspace_bytes(p);
}

int dsa_sparse_attn(const dsa_attn_desc* d, const int32_t* idx, void* out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  const int st = check_attn(d, idx, out);
  if (st) return st;
  AttnParams p = attn_params(d, idx, out);
  const size_t need = attn_workspace_bytes(p);
  if (need && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return DSA_ERR_ALIGN;
  p.part = static_cast<float*>(workspace);
  return hip_status(launch_attention(p, as_stream(stream)));
}

// ------------------------------------------------------------ forward --

namespace {

struct ForwardPlan {
  dsa_index_desc idx_desc;
  dsa_topk_desc topk_desc;
  dsa_attn_desc attn_desc;
  int64_t n_units;
  int32_t k_out;
  size_t off_pooled, off_scores, off_idx, off_topk, off_prep, off_attn, total;
  bool multiblock;
  bool fuse_hist;    // few long rows: the score epilogue builds the top-k histogram
  bool prep;         // ... in the decode stream kernel, from prepared query operands
  bool attn_dense;   // top_k >= n_kv: every query selects all its visible keys
  AttnParams ap;
};

int plan_forward(const dsa_forward_desc* d, ForwardPlan* f) {
  if (!d || !d->q_idx || !d->k_idx || !d->w || !d->q || !d->k || !d->v || !d->q_pos || !d->out)
    return DSA_ERR_NULL;
  if (d->S < 1 || d->n_q < 1 || d->n_kv < 1 || d->n_kv > 0x7fffffffLL) return DSA_ERR_SHAPE;
  if (d->top_k < 1 || d->c < 1 || d->top_k % d->c) return DSA_ERR_PARAM;
  if (d->n_sink < 0 || d->n_sink > d->top_k || (d->n_sink > 0 && d->c > 1)) return DSA_ERR_PARAM;
  if (d->c > 1 && d->k_idx_dtype == DSA_FP8_E4M3) return DSA_ERR_DTYPE;   // pooling needs raw keys
  if (d->c > 1 && d->top_k / d->c > kMaxBlocks) return DSA_ERR_SHAPE;
  const int64_t n_units = d->c > 1 ? d->n_kv / d->c : d->n_kv;
  f->n_units = n_units;
  f->k_out = d->top_k / d->c;

  dsa_index_desc& id = f->idx_desc;
  memset(&id, 0, sizeof id);
  id.q = d->q_idx;
  id.k = d->k_idx;   // replaced by the pooled keys in block mode
  id.k_scale = d->k_scale;
  id.w = d->w;
  id.q_pos = d->q_pos;
  id.kv_len = d->kv_len;
  id.q_dtype = d->q_idx_dtype;
  id.k_dtype = d->c > 1 ? DSA_F32 : d->k_idx_dtype;
  id.S = d->S;
  id.n_q = d->n_q;
  id.H = d->H;
  id.D = d->D;
  id.n_units = n_units > 0 ? n_units : 1;
  id.c = d->c;
  id.hadamard_q = d->hadamard_q;
  if (d->c > 1 && d->k_idx_dtype != DSA_F32 && d->k_idx_dtype != DSA_BF16 && d->k_idx_dtype != DSA_F16)
    return DSA_ERR_DTYPE;
  if (d->c > 1 && d->k_scale) return DSA_ERR_PARAM;
  {
    static float dummy_scores[4] __attribute__((aligned(16)));
    const int st = check_index(&id, d->scores_out ? d->scores_out : dummy_scores);
    if (st) return st;
  }
  dsa_topk_desc& td = f->topk_desc;
  memset(&td, 0, sizeof td);
  td.q_pos = d->q_pos;
  td.kv_len = d->kv_len;
  td.S = d->S;
  td.n_q = d->n_q;
  td.n_units = id.n_units;
  td.top_k = d->top_k;
  td.c = d->c;
  td.n_sink = d->n_sink;

  dsa_attn_desc& ad = f->attn_desc;
  memset(&ad, 0, sizeof ad);
  ad.q = d->q;
  ad.k = d->k;
  ad.v = d->v;
  ad.k_seq_stride = d->k_seq_stride;
  ad.k_tok_stride = d->k_tok_stride;
  ad.k_head_stride = d->k_head_stride;
  ad.v_seq_stride = d->v_seq_stride;
  ad.v_tok_stride = d->v_tok_stride;
  ad.v_head_stride = d->v_head_stride;
  ad.q_pos = d->q_pos;
  ad.kv_len = d->kv_len;
  ad.dtype = d->a_dtype;
  ad.o_dtype = d->o_dtype;
  ad.S = d->S;
  ad.n_q = d->n_q;
  ad.Hq = d->Hq;
  ad.Hkv = d->Hkv;
  ad.Dk = d->Dk;
  ad.Dv = d->Dv;
  ad.n_kv = d->n_kv;
  ad.k_sel = f->k_out;
  ad.c = d->c;
  ad.scale = d->scale;
  ad.kv_format = d->kv_format;
  ad.kv_scale = d->kv_scale;
  {
    static const int32_t dummy_idx[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
    const int st = check_attn(&ad, dummy_idx, d->out);
    if (st) return st;
  }
  if ((d->idx_out && (reinterpret_cast<uintptr_t>(d->idx_out) & 3u)) ||
      (d->scores_out && !aligned16(d->scores_out)))
    return DSA_ERR_ALIGN;

  const int64_t rows = static_cast<int64_t>(d->S) * d->n_q;
  f->multiblock = n_units > 0 && topk_use_multiblock(rows, n_units);
  size_t off = 0;
  f->off_pooled = off;
  if (d->c > 1 && n_units > 0) off += a256(static_cast<size_t>(d->S) * n_units * d->D * 4);
  f->off_scores = off;
  if (!d->scores_out && n_units > 0) off += a256(static_cast<size_t>(rows) * n_units * 4);
  f->off_idx = off;
  if (!d->idx_out) off += a256(static_cast<size_t>(rows) * f->k_out * 4);
  f->off_topk = off;
  if (n_units > 0) off += a256(topk_workspace_bytes(rows, n_units));
  // few long rows: the score epilogue builds the top-k histogram ([FIDX])
  f->fuse_hist = f->multiblock && !topk_use_long(rows, n_units) &&
                 scores_use_mfma(d->q_idx_dtype, id.k_dtype, d->H, d->D);
  f->prep = f->fuse_hist && scores_use_prep(d->q_idx_dtype, id.k_dtype, d->H, d->D, n_units);
  f->off_prep = off;
  if (f->prep) off += score_prep_bytes(rows, d->q_idx_dtype, id.k_dtype, d->H, d->hadamard_q);
  f->off_attn = off;
  // With top_k >= n_kv the selection is every visible key (in block mode
  // every complete block and the tail), so attention runs as dense causal
  // attention: the same token set, and the result of the dense call bit for
  // bit (ik_llama.cpp PR #2058, first commit: the indexer is an exact no-op).
  f->attn_dense = d->top_k >= d->n_kv;
  f->ap = attn_params(&ad, f->attn_dense ? nullptr : reinterpret_cast<const int32_t*>(16), d->out);   // idx bound later
  off += a256(attn_workspace_bytes(f->ap));
  f->total = off;
  return DSA_OK;
}

}  // namespace

size_t dsa_forward_workspace_bytes(const dsa_forward_desc* d) {
  ForwardPlan f;
  if (plan_forward(d, &f) != DSA_OK) return 0;
  return f.total;
}

int dsa_forward(const dsa_forward_desc* d, void* workspace, size_t workspace_bytes, void* stream) {
  ForwardPlan f;
  const int st = plan_forward(d, &f);
  if (st) return st;
  if (f.total && (!workspace || workspace_bytes < f.total)) return DSA_ERR_WORKSPACE;
  if (f.total && !aligned16(workspace)) return DSA_ERR_ALIGN;
  hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  void* const* ev = d->phase_events;
  const int64_t rows = static_cast<int64_t>(d->S) * d->n_q;
  hipError_t e = hipSuccess;
#define DSA_TRY(x)                         \
  do {                                     \
    if ((e = (x)) != hipSuccess) return DSA_ERR_HIP; \
  } while (0)
  auto mark = [&](int i) -> hipError_t {   // a null entry is skipped
    return ev && ev[i] ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) : hipSuccess;
  };
  int32_t* idx = d->idx_out ? d->idx_out : reinterpret_cast<int32_t*>(ws + f.off_idx);
  DSA_TRY(mark(0));
  if (f.n_units > 0) {
    float* scores = d->scores_out ? d->scores_out : reinterpret_cast<float*>(ws + f.off_scores);
    ScoreParams sp{};
    sp.q = d->q_idx;
    sp.k = d->k_idx;
    sp.k_scale = d->k_scale;
    sp.w = d->w;
    sp.q_pos = d->q_pos;
    sp.kv_len = d->kv_len;
    sp.scores = scores;
    sp.S = d->S;
    sp.n_q = d->n_q;
    sp.H = d->H;
    sp.D = d->D;
    sp.n_units = f.n_units;
    sp.c = d->c;
    sp.hadamard = d->hadamard_q;
    sp.q_dtype = d->q_idx_dtype;
    sp.k_dtype = f.idx_desc.k_dtype;
    sp.fill_invisible = d->scores_out ? 1 : 0;
    sp.n_sink = d->n_sink;
    sp.k_out = f.k_out;
    if (d->c > 1) {
      float* pooled = reinterpret_cast<float*>(ws + f.off_pooled);
      DSA_TRY(launch_block_pool(d->k_idx, d->k_idx_dtype, d->S, d->n_kv, d->D, d->c, nullptr, nullptr, pooled, s));
      sp.k = pooled;
    }
    TopkParams tp = topk_params(scores, &f.topk_desc, idx);
    const bool fuse_hist = f.fuse_hist;
    if (f.multiblock) {
      topk_bind_workspace(tp, ws + f.off_topk);
      if (fuse_hist) {
        sp.hist = tp.hist;
        if (f.prep) score_prep_bind(sp, ws + f.off_prep);
        DSA_TRY(launch_score_prep(sp, tp.cand_cnt, s));
      }
    }
    DSA_TRY(launch_scores(sp, s));
    DSA_TRY(mark(1));
    DSA_TRY(launch_topk(tp, fuse_hist, s));
  } else {
    DSA_TRY(mark(1));
    DSA_TRY(fill_i32(idx, rows * f.k_out, -1, s));
  }
  DSA_TRY(mark(2));
  AttnParams ap = f.ap;
  ap.idx = f.attn_dense ? nullptr : idx;
  ap.part = reinterpret_cast<float*>(ws + f.off_attn);
  DSA_TRY(launch_attention(ap, s, ev ? static_cast<hipEvent_t>(ev[3]) : nullptr));
  DSA_TRY(mark(4));
#undef DSA_TRY
  return DSA_OK;
}

int dsa_event_create(void** event) {
  if (!event) return DSA_ERR_NULL;
  hipEvent_t e;
  if (hipEventCreate(&e) != hipSuccess) return DSA_ERR_HIP;
  *event = e;
  return DSA_OK;
}

int dsa_event_destroy(void* event) {
  if (!event) return DSA_ERR_NULL;
  return hip_status(hipEventDestroy(static_cast<hipEvent_t>(event)));
}

int dsa_event_record(void* event, void* stream) {
  if (!event) return DSA_ERR_NULL;
  return hip_status(hipEventRecord(static_cast<hipEvent_t>(event), as_stream(stream)));
}

int dsa_event_elapsed_ms(void* start, void* end, float* ms) {
  if (!start || !end || !ms) return DSA_ERR_NULL;
  if (hipEventSynchronize(static_cast<hipEvent_t>(end)) != hipSuccess) return DSA_ERR_HIP;
  return hip_status(hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(end)));
}

}  // extern "C"
