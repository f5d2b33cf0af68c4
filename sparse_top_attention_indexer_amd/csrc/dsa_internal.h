// Host-side interfaces between the C ABI layer (api.hip) and the kernel
// launchers (score.hip, topk.hip, pool.hip, attn.hip).  Everything here is
// internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Histogram of the top 12 bits of order-preserving score keys, per row.
constexpr int HIST_BITS = 12;
constexpr int HIST_BINS = 1 << HIST_BITS;

// ------------------------------------------------------------------ scores --
struct ScoreParams {
  const void* q;
  const void* k;
  const float* k_scale;
  const float* w;
  const int32_t* q_pos;
  const int32_t* kv_len;
  float* scores;
  uint32_t* hist;        // [rows][HIST_BINS] when the epilogue feeds top-k, else null
  int32_t S, n_q, H, D;
  int64_t n_units;
  int32_t c;
  int32_t hadamard;
  int32_t q_dtype, k_dtype;
  int32_t chunk_tiles;   // 32-unit tiles per wave
  int32_t n_chunks;      // chunks per row
  int32_t chunk_major;   // 1: a workgroup = 4 chunks of one row; 0: 4 rows x 1 chunk
  int32_t fill_invisible;
  int32_t n_sink;        // hist excludes the forced sinks
  int32_t k_out;         // hist only for rows with more visible units than k_out
  const uint32_t* qop;   // query operands prepared by score_prep_kernel (decode stream kernel), else null
  const float* qw;       // their head weights, in the stream kernel's lane layout
};
// Chooses a kernel variant and launches it; returns a hipError_t.
hipError_t launch_scores(ScoreParams p, hipStream_t st);
// True when the MFMA score kernels cover (q_dtype, k_dtype, H, D).
bool scores_use_mfma(int q_dtype, int k_dtype, int H, int D);
// True when rows with the fused top-k histogram take the decode stream
// kernel, which reads query operands prepared by launch_score_prep.
bool scores_use_prep(int q_dtype, int k_dtype, int H, int D, int64_t n_units);
// Bytes of prepared query operands for `rows` rows (256-byte multiple).
size_t score_prep_bytes(int64_t rows, int q_dtype, int k_dtype, int H, int hadamard);
// Points p.qop and p.qw into a workspace of score_prep_bytes for p's rows.
void score_prep_bind(ScoreParams& p, void* ws);
// Clears the top-k histogram (p.hist) and candidate counts, and when p.qop is
// set writes the query operands and head weights of every row there.
hipError_t launch_score_prep(const ScoreParams& p, uint32_t* cand_cnt, hipStream_t st);

// ------------------------------------------------------------------- top-k --
struct TopkParams {
  const float* scores;
  int32_t* idx;
  const int32_t* q_pos;
  const int32_t* kv_len;
  int32_t S, n_q;
  int64_t n_units;
  int32_t k_out;         // top_k / c
  int32_t c;
  int32_t n_sink;
  // multi-block path workspace
  uint32_t* hist;        // [rows][HIST_BINS]
  uint32_t* cand_cnt;    // [rows]
  uint32_t* cand;        // [rows][cand_cap][2] (key, index): candidates, or the long-row path's staged units
  uint32_t* cnt_hi;      // [rows][n_chunks]
  uint32_t* thr;         // [rows][4]: b1, -, -, units above b1
  int64_t cand_cap;
  int32_t chunk;         // units per multi-block chunk
  int32_t n_chunks;
};
constexpr int TOPK_CHUNK = 4096;
// Long rows take the multi-block path: few of them (decode) spread over many
// workgroups per row (fused or standalone histogram, select, finish); many of
// them (topk_use_long) one workgroup of 1024 threads per row, whose
// workspace holds only the staged units.
bool topk_use_multiblock(int64_t rows, int64_t n_units);
bool topk_use_long(int64_t rows, int64_t n_units);
size_t topk_workspace_bytes(int64_t rows, int64_t n_units);
// Carves the multi-block workspace out of `ws` (256-byte aligned pieces).
void topk_bind_workspace(TopkParams& p, void* ws);
// Zeroes the histogram and candidate counters (must precede scores-with-hist).
hipError_t launch_topk_clear(const TopkParams& p, hipStream_t st);
// Full top-k; `hist_ready` means the score epilogue already filled p.hist.
hipError_t launch_topk(const TopkParams& p, bool hist_ready, hipStream_t st);

// -------------------------------------------------------------- block pool --
// Indexer-key cache write (rotate, then store as f16 / bf16 / fp8 + row scale).
hipError_t launch_key_write(const void* k_new, int k_dtype, int S, int64_t n_new, const int32_t* dst_row,
                            int hadamard, void* cache, int cache_dtype, float* cache_scale, int64_t n_cache,
                            hipStream_t st);
hipError_t launch_block_pool(const void* k_raw, int dtype, int S, int64_t n_kv, int D, int c,
                             const int32_t* from_block, const int32_t* kv_len, float* pooled, hipStream_t st);

// --------------------------------------------------------------- attention --
// floats per split partial record of one (row, split, head): the Dv
// unnormalised output sums, the running max m and the sum l, padded to a
// multiple of 4 floats so that every record starts 16-byte aligned
constexpr int part_width(int dv) { return (dv + 2 + 3) & ~3; }

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t k_seq, k_tok, k_head;
  int64_t v_seq, v_tok, v_head;
  const int32_t* q_pos;
  const int32_t* kv_len;
  const int32_t* idx;    // null = dense
  void* out;
  float* part;           // split partials [rows][n_split][Hq][part_width(Dv)]: o, then m and l
  const void* k_scale;   // q8_0 latent rows: f16 scales [S, n_kv, Dk / 32] (kq8), else null
  int32_t dtype, o_dtype;
  int32_t S, n_q, Hq, Hkv, Dk, Dv;
  int64_t n_kv;
  int32_t k_sel;
  int32_t c;
  float scale_log2;      // softmax scale times log2(e)
  int32_t n_split;       // key-stream splits per row
  int32_t split_len;     // stream entries per split (multiple of 32)
  int32_t family;        // ATTN_F32 / ATTN_MLA / ATTN_GQA
  int32_t kq8;           // MLA: the latent rows are q8_0 codes (int8) with f16 block scales
  int32_t mla_hg;        // MLA (bf16 rows): heads per workgroup, 128 or 64 (0 = 128)
};
enum { ATTN_F32 = 0, ATTN_MLA = 1, ATTN_GQA = 2 };
// Block-mode list length (blocks per row) the MLA kernel keeps in LDS.
constexpr int MLA_MAX_BLOCKS = 1024;
// Split policy and workspace; identical for dense and sparse calls whose
// effective list length min(L, n_kv) agrees (keeps dense == sparse bitwise).
void attn_plan(AttnParams& p, int64_t list_len);
size_t attn_workspace_bytes(const AttnParams& p);
// Main kernel then, for split streams, the combine; `before_combine` (may be
// null) is recorded between the two.
hipError_t launch_attention(const AttnParams& p, hipStream_t st, hipEvent_t before_combine = nullptr);

}  // namespace dsa
