/*
 * dsa.h — C ABI of the MI355X (gfx950) DeepSeek-style sparse attention library.
 *
 * The hot path of DSA: a lightning indexer scores every query against every
 * cached indexer key, each query keeps its top-k keys (or, in block mode, its
 * best mean-pooled blocks plus the incomplete tail block), and softmax
 * attention runs only over the kept keys.
 *
 * Sources of the operations (the pages this library is built from):
 *  - [PR2058]  ik_llama.cpp pull request #2058, first commit ("lightning
 *              indexer", batch-local prefill): score = head sum of per-head
 *              weight times relu(indexer key . indexer query), plus the causal
 *              mask, then a top-k of min(top_k, n_tokens); second commit
 *              (decode-correct indexer-K cache): scores against all cached
 *              keys, Walsh-Hadamard-rotated q/k, attention-sink force-include;
 *              "UPDATE 5" commit: the sink boost belongs to each query's own
 *              sequence.
 *  - [QSA]     llama.cpp mirror, commit c88c916636: one mean-pooled raw key
 *              per complete block of compress_ratio positions, a budget of
 *              whole blocks plus the incomplete tail, exactly dense below
 *              indexer_top_k + compress_ratio - 1 tokens; ReLU per head before
 *              the head sum.
 *  - [FIDX]    ik_llama_opt commit log of src/llama.cpp, the fused indexer
 *              top-k commit (-fidx): head-sum ReLU plus causal mask straight
 *              to top-k rows, never materialising per-head scores.
 *  - [GATHER]  same log, openPangu port, "Gather OpenPangu DSA decode reads"
 *              and the prefill gather commits: attention over the gathered
 *              selected latent rows, values taken from the same rows.
 *  - [HDR]     offgrid-sys llama.cpp llama-memory-hybrid-idx.h: pooled keys
 *              persist in the index cache across batches; each micro-batch
 *              re-pools only its new pools; an edit stales the pools from
 *              its position on.
 *  - [ISHARE]  same log, "GLM-5.2 DSA: IndexShare": full layers (layer <= 1
 *              or layer % 4 == 2) compute their own top-k, shared layers
 *              reuse the most recent full layer's selection.
 *  - [QKC]     same log, "GLM-DSA: allow for quantized indexer cache", and the
 *              unsloth llama.cpp PR #293 (deepseek41 quantized K cache): rows are
 *              rotated in F32 before they are stored in the cache type.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers, row-major, last dimension
 *    innermost.  The caller allocates every buffer, including the workspace
 *    (16-byte aligned, like every tensor pointer, else DSA_ERR_ALIGN);
 *    the library allocates nothing, keeps no pointer after returning and holds
 *    no global state (the one exception is dsa_topk_noalloc's static device
 *    scratch, described there).  Calls are asynchronous on the given stream (a
 *    hipStream_t passed as void*; NULL = the default stream); buffers must stay
 *    alive until the stream reaches them.  Entry points are thread-safe and
 *    re-entrant (dsa_topk_noalloc calls that overlap on one GPU race on its
 *    shared scratch).
 *  - Every argument check runs on the host before anything is launched.  On
 *    failure the call returns a negative DSA_ERR_* code and writes nothing.
 *  - Positions: key j of a sequence is its cache row j, at position j.  A query
 *    at position p sees keys j <= p with j < kv_len (kv_len NULL = all rows).
 *    Device values of q_pos / kv_len are used as given: kv_len is clamped to
 *    the stored rows, q_pos < 0 sees nothing (its output row is zero, its index
 *    row all -1), q_pos >= kv_len sees every stored key.
 *  - Device pointers must be 16-byte aligned, and every strided row (K/V token
 *    rows) must start on a 16-byte boundary (DSA_ERR_ALIGN otherwise).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. DSA_FP8_E4M3 is OCP float8 e4m3fn (max 448, no infinities).
 * DSA_Q8_0 is a storage format of MLA latent rows only: int8 codes with one
 * f16 scale per 32 consecutive values (ggml's q8_0, held as two arrays). */
typedef enum {
  DSA_F32 = 0,
  DSA_BF16 = 1,
  DSA_F16 = 2,
  DSA_FP8_E4M3 = 3,
  DSA_Q8_0 = 4
} dsa_dtype;

/* Status codes. */
#define DSA_OK 0
#define DSA_ERR_NULL (-1)        /* a required pointer is NULL               */
#define DSA_ERR_SHAPE (-2)       /* a size is out of range or inconsistent   */
#define DSA_ERR_DTYPE (-3)       /* unsupported element type combination     */
#define DSA_ERR_PARAM (-4)       /* top_k, compress_ratio or n_sink invalid  */
#define DSA_ERR_ALIGN (-5)       /* pointer or row stride not 16-byte aligned */
#define DSA_ERR_WORKSPACE (-6)   /* workspace NULL or smaller than required  */
#define DSA_ERR_HIP (-7)         /* the HIP runtime reported a launch error  */
#define DSA_ERR_UNSUPPORTED (-8) /* a valid shape the library has no kernel for */

/* Human-readable name of a status code (static string, never NULL). */
const char* dsa_strerror(int status);

/* Library version, as MAJOR*10000 + MINOR*100 + PATCH. */
int dsa_version(void);

/* sizeof() of each descriptor below, so that a binding can check its layout:
 * which = 0 index, 1 topk, 2 attn, 3 forward.  Returns 0 for other values. */
size_t dsa_desc_size(int which);

/* ------------------------------------------------------------------------
 * S2 (+ S0): lightning-indexer scores            [PR2058], [QSA], [FIDX]
 *
 *   s(i,u) = sum_h w(i,h) * max(0, q'(i,h) . k(u)) * k_scale(u)
 *
 * for every unit u visible to query i, -inf for the others.  Units are token
 * keys when c == 1 (visible: u <= q_pos, u < kv_len) or pooled block keys when
 * c > 1 (block u visible iff its last position u*c + c - 1 is a visible
 * token).  q' = H q with H the orthonormal 128-point Sylvester Walsh-Hadamard
 * matrix when hadamard_q != 0 (the keys must then be stored rotated), else q.
 * k_scale is the per-row dequantisation scale of fp8 keys (>= 0) and 1 for
 * other key types.  No other scale is applied (fold any softmax scale into w).
 * Scores are the raw indexer scores: no sink boost.
 * ---------------------------------------------------------------------- */
typedef struct {
  const void* q;          /* [S, n_q, H, D]   q_dtype: F32 | BF16 | F16        */
  const void* k;          /* [S, n_units, D]  k_dtype: F32 | BF16 | F16 | FP8  */
  const float* k_scale;   /* [S, n_units] iff k_dtype == FP8, else NULL        */
  const float* w;         /* [S, n_q, H] head weights                          */
  const int32_t* q_pos;   /* [S, n_q] query positions                          */
  const int32_t* kv_len;  /* [S] stored tokens per sequence, or NULL           */
  int32_t q_dtype;
  int32_t k_dtype;
  int32_t S;              /* >= 1                                              */
  int32_t n_q;            /* >= 1                                              */
  int32_t H;              /* 1..128 indexer heads                              */
  int32_t D;              /* 16..256, multiple of 16 (128 if hadamard_q)       */
  int64_t n_units;        /* >= 1 units per sequence                           */
  int32_t c;              /* compress ratio: 1 token keys, > 1 block keys      */
  int32_t hadamard_q;     /* 0 or 1                                            */
} dsa_index_desc;

/* Writes scores [S, n_q, n_units] f32. */
int dsa_index_scores(const dsa_index_desc* d, float* scores, void* stream);

/* ------------------------------------------------------------------------
 * S3: top-k selection                            [PR2058], [QSA]
 *
 * For each query row: K = min(top_k / c, n_visible_units) units are kept:
 * first the forced sinks (units j < n_sink, token mode only: the sequence's
 * first keys), then the best remaining visible units by (score descending,
 * unit index ascending; scores compare as IEEE values, so -0 and +0 are
 * equal and tie by index).  Writes idx [S, n_q, top_k / c] int32: the kept unit
 * ids in ascending order, then -1 for the dead slots.  A full argsort is never
 * formed.  Scores of invisible units are not read.
 * ---------------------------------------------------------------------- */
typedef struct {
  const int32_t* q_pos;   /* [S, n_q]                                          */
  const int32_t* kv_len;  /* [S] or NULL                                       */
  int32_t S;
  int32_t n_q;
  int64_t n_units;        /* row length of the score matrix                    */
  int32_t top_k;          /* >= 1 tokens; multiple of c                        */
  int32_t c;              /* >= 1                                              */
  int32_t n_sink;         /* 0 .. top_k; must be 0 when c > 1                  */
  int32_t pad_;           /* reserved, set to 0                                */
} dsa_topk_desc;

size_t dsa_topk_workspace_bytes(const dsa_topk_desc* d);
int dsa_topk(const float* scores, const dsa_topk_desc* d, int32_t* idx,
             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * S3 without allocation: dsa_topk with the library's own device scratch
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * selection as dsa_topk, with its long-row workspace (histograms,
 * candidate counters, candidates; or the staged units of many long rows)
 * taken from a static device array of
 * DSA_TOPK_NOALLOC_SCRATCH_BYTES that each GPU holds until the process ends.
 * The call allocates nothing (no hipMalloc, no library allocation).  Calls
 * whose dsa_topk_workspace_bytes(d) exceeds the array return
 * DSA_ERR_WORKSPACE and write nothing (16 MiB covers, e.g., 60 rows of 32768
 * units or 15 rows of 131072).  The stream must belong to the current device.
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents (the call clears what must start at zero): calls that overlap on
 * one GPU (other threads, other streams) race and must be serialised by the
 * caller.
 * ---------------------------------------------------------------------- */
#define DSA_TOPK_NOALLOC_SCRATCH_BYTES (16u << 20)
int dsa_topk_noalloc(const float* scores, const dsa_topk_desc* d, int32_t* idx, void* stream);

/* ------------------------------------------------------------------------
 * S1: block pooling                              [QSA]
 *
 * pooled[s, b, :] = mean of k_raw[s, b*c .. b*c + c - 1, :] for every complete
 * block b < floor(n_kv / c), accumulated in f32.  Pooling uses the raw keys.
 * ---------------------------------------------------------------------- */
int dsa_block_pool(const void* k_raw, int32_t dtype /* F32 | BF16 | F16 */,
                   int32_t S, int64_t n_kv, int32_t D, int32_t c,
                   float* pooled /* [S, n_kv / c, D] */, void* stream);

/* ------------------------------------------------------------------------
 * S1, incremental: re-pool only new or stale blocks      [HDR], [QSA]
 *
 * The pooled keys persist across calls in the caller's buffer; a micro-batch
 * only appends pools, and a sequence edit stales every pool from some
 * position on ([HDR]: pooled keys persist in the index cache across batches,
 * the pools to re-pool per micro-batch, the stale position of an edit).  For
 * each sequence s this recomputes exactly the blocks
 *   from_block[s] <= b < floor(min(kv_len[s], n_kv) / c)
 * of pooled [S, n_kv / c, D] (kv_len NULL: n_kv) and writes nothing else.
 * A block's value does not depend on the call that pools it, so pooling in
 * several calls equals dsa_block_pool bit for bit.  from_block [S] and
 * kv_len [S] are device int32; from_block < 0 counts as 0.
 * ---------------------------------------------------------------------- */
int dsa_block_pool_update(const void* k_raw, int32_t dtype, int32_t S, int64_t n_kv, int32_t D, int32_t c,
                          const int32_t* from_block, const int32_t* kv_len, float* pooled, void* stream);

/* ------------------------------------------------------------------------
 * Indexer-key cache write: rotate new keys, store them in the cache type
 *   [PR2058] decode-correct indexer-K cache commit (rotated keys written at
 *   the batch's cache rows); [QKC] quantized indexer / K caches (rows rotated
 *   in F32, then stored in the cache type)
 *
 * For new key t of sequence s, with destination row r = dst_row[s, t]
 * (dst_row == NULL: r = t), when 0 <= r < n_cache (other rows are skipped):
 *   x = k_new[s, t, :] in f32;  y = sqrt(128) H x when hadamard != 0 (H
 *       the orthonormal 128-point Sylvester Walsh-Hadamard matrix), else x
 *   F16 / BF16 cache: cache[s, r, :] = H x (or x) rounded to nearest, ties
 *       to even
 *   FP8 cache: with m = max_d |y(d)|, cache[s, r, d] = e4m3fn(y(d) * (448 /
 *       m)), nearest, ties to the even code, saturating at 448, and
 *       cache_scale[s, r] = m / (448 sqrt(128)) (m / 448 unrotated), so that
 *       code * scale = H x to fp8 precision; a zero row stores scale 0 and
 *       zero codes
 * Bit-exact definition in f32: y is the fast transform with butterfly spans
 * 1, 2, 4, ..., 64 in that order ((a, b) -> (a + b, a - b)); H x = y *
 * f32(1/sqrt(128)); 448 / m is a correctly rounded division; the scale is m
 * times f32(1/(448 sqrt(128))) (f32(1/448) unrotated).  The stored rows are
 * what dsa_index_scores reads as keys (hadamard_q = 1 when rotated, k_scale =
 * cache_scale for fp8).
 * k_new [S, n_new, D] of k_dtype (F32 | BF16 | F16); cache [S, n_cache, D] of
 * cache_dtype (F16 | BF16 | FP8_E4M3); cache_scale [S, n_cache] f32 iff FP8
 * (else NULL); dst_row [S, n_new] int32 device or NULL.  D must be 128 and
 * S at most 65535;
 * n_new may be 0 (nothing is written; k_new may then be NULL).  Two new keys with the same
 * destination row race: one of them is stored.  Non-finite keys store
 * unspecified codes.
 * ---------------------------------------------------------------------- */
int dsa_index_key_write(const void* k_new, int32_t k_dtype, int32_t S, int64_t n_new, int32_t D,
                        const int32_t* dst_row, int32_t hadamard, void* cache, int32_t cache_dtype,
                        float* cache_scale, int64_t n_cache, void* stream);

/* ------------------------------------------------------------------------
 * IndexShare: which layer's selection a layer attends over     [ISHARE]
 *
 * A layer is full (it runs its own indexer and top-k: dsa_forward with
 * idx_out) when layer <= 1 or layer % 4 == 2; every other layer is shared and
 * attends over the index rows of the most recent full layer
 * (dsa_sparse_attn with those rows).  Returns that layer (the layer itself
 * when it is full), or DSA_ERR_PARAM for layer < 0.  Host-only; no launch.
 * ---------------------------------------------------------------------- */
int32_t dsa_index_share_source(int32_t layer);

/* ------------------------------------------------------------------------
 * S4 + S5 (+ S6): sparse attention over the selected tokens   [GATHER], [PR2058]
 *
 * o(i,h) = sum_{j in T(i)} softmax_j(scale * Q(i,h) . K(j,g)) V(j,g),
 * g = h / (Hq / Hkv).  T(i), in attention order:
 *  - idx == NULL: every visible token 0 .. n_vis-1 (dense causal attention,
 *    the indexer-off reference);
 *  - c == 1: the idx row's entries in list order; -1 entries and ids that are
 *    not visible are skipped; a repeated id is attended once per listing;
 *  - c > 1: the idx row holds block ids; each live complete block expands to
 *    its c positions in list order, followed by the incomplete tail
 *    floor(n_vis / c) * c .. n_vis - 1.
 * Rows with an empty T(i) are written as zeros.
 * Supported families (DSA_ERR_UNSUPPORTED otherwise):
 *  - F32:  Q/K/V f32, Dk, Dv <= 256, any Hq multiple of Hkv;
 *  - MLA:  BF16, Hkv == 1, Dk == 576, Dv == 512, Hq a multiple of 16, V
 *          aliasing the first 512 columns of K (same pointer and strides),
 *          n_kv * k_tok_stride * 2 < 2^32, and in block mode k_sel <= 1024
 *          (DSA_ERR_SHAPE otherwise);
 *  - GQA:  BF16, Dk == Dv == 128, Hq / Hkv <= 16.
 * q8_0 latent rows ([QQ8] below): kv_format = DSA_Q8_0 with the MLA shapes
 * (Q BF16): K = V = int8 codes (the strides count bytes), kv_scale = f16
 * scales [S, n_kv, 18] contiguous, 16-byte aligned; every latent value is
 * code x scale of its 32-value block.  Scores take that value exactly (as the
 * sum of two f16 parts) against the query in f16 (each head scaled by a power
 * of two, undone after); the value product takes it rounded to f16.  Values
 * must lie in the f16 range (|code x scale| <= 65504, i.e. scales <= 515);
 * larger ones give undefined outputs.  Errors: DSA_ERR_NULL without kv_scale,
 * DSA_ERR_DTYPE for other Q types or formats, DSA_ERR_UNSUPPORTED for other
 * shapes, DSA_ERR_ALIGN for a misaligned kv_scale or a row stride not a
 * multiple of 16 bytes.
 *  - [QQ8]  ik_llama_opt log, openPangu port, "Add OpenPangu q8_0 latent
 *           cache type": MLA latent rows cached as q8_0 (0.53x the bytes of
 *           f16), read back by attention.
 * ---------------------------------------------------------------------- */
typedef struct {
  const void* q;          /* [S, n_q, Hq, Dk] contiguous                        */
  const void* k;          /* K(s, j, g, d) at k[s*k_seq_stride + j*k_tok_stride + g*k_head_stride + d] */
  const void* v;          /* V likewise with the v_* strides                    */
  int64_t k_seq_stride, k_tok_stride, k_head_stride;   /* in elements           */
  int64_t v_seq_stride, v_tok_stride, v_head_stride;   /* in elements           */
  const int32_t* q_pos;   /* [S, n_q]                                           */
  const int32_t* kv_len;  /* [S] or NULL                                        */
  int32_t dtype;          /* Q/K/V element type: F32 | BF16                     */
  int32_t o_dtype;        /* output element type: F32 | BF16                    */
  int32_t S, n_q, Hq, Hkv, Dk, Dv;
  int64_t n_kv;           /* stored tokens per sequence                         */
  int32_t k_sel;          /* entries per idx row (ignored when idx == NULL)     */
  int32_t c;              /* >= 1; block mode when > 1                          */
  float scale;            /* softmax scale; <= 0 selects 1/sqrt(Dk)             */
  int32_t kv_format;      /* 0 (K/V of dtype) or DSA_Q8_0 (MLA latent rows)     */
  const void* kv_scale;   /* [S, n_kv, Dk / 32] f16 iff kv_format == DSA_Q8_0   */
} dsa_attn_desc;

/* Workspace for dsa_sparse_attn; dense != 0 sizes the idx == NULL call. */
size_t dsa_sparse_attn_workspace_bytes(const dsa_attn_desc* d, int dense);
/* idx [S, n_q, k_sel] int32 or NULL; out [S, n_q, Hq, Dv] of o_dtype. */
int dsa_sparse_attn(const dsa_attn_desc* d, const int32_t* idx, void* out,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The whole path in one call: [S1 if c > 1] -> S2 -> S3 -> S4/S5 (+S6).
 * Same semantics as the separate calls; the score epilogue feeds the top-k
 * histogram directly on long rows ([FIDX]).  With top_k >= n_kv (token mode)
 * the output is bitwise equal to dsa_sparse_attn(idx = NULL).
 * ---------------------------------------------------------------------- */
#define DSA_N_PHASE_EVENTS 5   /* before S1/S2, before S3, before S5, before S6, end */

typedef struct {
  /* indexer */
  const void* q_idx;      /* [S, n_q, H, D]                                     */
  const void* k_idx;      /* token keys [S, n_kv, D] (c == 1), raw keys (c > 1) */
  const float* k_scale;   /* [S, n_kv] iff k_idx_dtype == FP8 (token mode only) */
  const float* w;         /* [S, n_q, H]                                        */
  int32_t q_idx_dtype, k_idx_dtype;
  int32_t H, D;
  int32_t top_k, c, n_sink, hadamard_q;
  /* attention (same meaning as dsa_attn_desc) */
  const void* q;
  const void* k;
  const void* v;
  int64_t k_seq_stride, k_tok_stride, k_head_stride;
  int64_t v_seq_stride, v_tok_stride, v_head_stride;
  int32_t a_dtype, o_dtype;
  int32_t Hq, Hkv, Dk, Dv;
  float scale;
  int32_t kv_format;      /* as in dsa_attn_desc                                */
  /* shared */
  int32_t S, n_q;
  int64_t n_kv;
  const int32_t* q_pos;
  const int32_t* kv_len;
  /* outputs */
  void* out;              /* [S, n_q, Hq, Dv] of o_dtype                        */
  int32_t* idx_out;       /* optional [S, n_q, top_k / c]                       */
  float* scores_out;      /* optional [S, n_q, n_units] (n_units = n_kv / c in block mode) */
  /* optional timing: NULL, or DSA_N_PHASE_EVENTS hipEvent_t handles recorded
   * on the stream at the phase boundaries (before the first launch, after
   * the scores, after the top-k, before the split merge, after the last
   * launch); a NULL entry is not recorded */
  void* const* phase_events;
  const void* kv_scale;   /* as in dsa_attn_desc                                */
} dsa_forward_desc;

size_t dsa_forward_workspace_bytes(const dsa_forward_desc* d);
int dsa_forward(const dsa_forward_desc* d, void* workspace, size_t workspace_bytes,
                void* stream);

/* ------------------------------------------------------------------------
 * Timing helpers (thin wrappers of the HIP event API, for bindings that have
 * no HIP handle of their own).  Events are created with default flags.
 * ---------------------------------------------------------------------- */
int dsa_event_create(void** event);
int dsa_event_destroy(void* event);
int dsa_event_record(void* event, void* stream);
/* Milliseconds between two recorded events; synchronises on `end`. */
int dsa_event_elapsed_ms(void* start, void* end, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
