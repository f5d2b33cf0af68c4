// Per-row top-k selection on gfx950, without a full sort.
//
// Selection rule (ik_llama.cpp PR #2058, first commit: top-k of
// min(top_k, n_tokens) after the causal mask; "UPDATE 5" commit: the sink keys
// of the query's own sequence are forced in; llama.cpp mirror commit
// c88c916636: in block mode the budget is top_k / compress_ratio blocks):
//   K = min(k_out, n_vis); forced = units 0 .. min(n_sink, n_vis) - 1;
//   the other K - |forced| units are the best of the remaining visible units
//   by (score descending, index ascending); output ascending, -1 padded.
//
// Scores become order-preserving 32-bit keys.  A radix select over the keys
// finds the threshold key T and how many units equal to T are kept (the
// lowest-indexed ones); an ordered compaction then writes the kept indices in
// ascending order.
//   - one workgroup per row when the row has at most 16384 units and there
//     are at least 128 rows or the row has at most 4096 units: the row's keys
//     live in LDS, three radix passes of 11 + 11 + 10 bits over a 2048-bin
//     histogram;
//   - many long rows (at least 128 rows of more than 16384 units): one
//     workgroup of 1024 threads per row, whose two passes over the row's
//     scores (the second from L2) find the threshold bin and stage the units
//     at or above it in index order; the exact threshold comes from the
//     staged units of that bin, and a last compaction of the short staged
//     list writes the kept ids (topk_long_kernel);
//   - few long rows (decode): many workgroups per row.  A global histogram
//     of the top 12 bits (built by the score epilogue in the fused path)
//     locates the threshold bin; units of that bin are gathered as
//     candidates; then every chunk's workgroup resolves the exact threshold
//     among the row's candidates itself and compacts its chunk.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

struct RowInfo {
  int64_t n_vis;   // visible units
  int64_t nf;      // forced sinks
  int64_t K;       // kept units
};

__device__ __forceinline__ RowInfo row_info(const TopkParams& p, int64_t row) {
  const int s = static_cast<int>(row / p.n_q);
  const int64_t kl = p.kv_len ? p.kv_len[s] : p.n_units * p.c;
  RowInfo r;
  r.n_vis = visible_tokens(p.q_pos[row], kl, p.n_units * p.c) / p.c;
  r.nf = p.c == 1 ? (p.n_sink < r.n_vis ? p.n_sink : r.n_vis) : 0;
  r.K = p.k_out < r.n_vis ? p.k_out : r.n_vis;
  return r;
}

// Finds the bin b (scanning from the highest bin down) that holds the need-th
// largest element: above(b) < need <= above(b) + hist[b], with above(b) the
// count of elements in bins > b.  256 threads; nb a multiple of 256.
// Returns b and sets *above.  All threads get the result.
__device__ uint32_t find_bin_desc(const uint32_t* hist, int nb, uint32_t need, uint32_t* scratch,
                                  uint32_t* above) {
  // thread t owns bins [nb - (t+1)*per, nb - t*per): thread 0 owns the top
  // bins; its counts are read once (into registers: the search below then
  // needs no dependent LDS reads)
  const int per = nb / 256;   // 1, 4, 8 or 16
  const int hi = nb - threadIdx.x * per;
  uint32_t c[16];
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    c[i] = i < per ? hist[hi - 1 - i] : 0u;   // c[i]: the i-th bin from the top of the thread's range
    local += c[i];
  }
  uint32_t total;
  const uint32_t excl = block_excl_scan_256(local, scratch, &total);  // elements in higher bins
  if (excl < need && need <= excl + local) {
    uint32_t acc = excl;
    int found = per - 1;
    uint32_t acc_at = 0;
    bool done = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (!done && i < per) {
        if (acc + c[i] >= need) {
          found = i;
          acc_at = acc;
          done = true;
        }
        acc += c[i];
      }
    }
    scratch[4] = static_cast<uint32_t>(hi - 1 - found);
    scratch[5] = acc_at;
  }
  __syncthreads();
  const uint32_t bin = scratch[4];
  *above = scratch[5];
  __syncthreads();
  return bin;
}

// ------------------------------------------------------- one-row-per-block --

// Candidate e of a row lives at s_key[e + e / 16]: the padding word after
// every 16 keys makes the compaction's reads (thread t reads its contiguous
// run 16 t .. 16 t + 15, words 17 t + i) free of bank conflicts.
__device__ __forceinline__ int64_t key_slot(int64_t e) { return e + (e >> 4); }

// Histogram bins of the one-workgroup-per-row select: radix passes of
// 11 + 11 + 10 bits, so that the histogram takes 8 KB of LDS and more rows
// share a compute unit.
constexpr int ROW_BINS = 1 << 11;

// Keys e = tid, tid + 256, ... below m of a row into LDS.  Each thread issues
// the loads of NB keys before converting any (in-range addresses only: past m
// it reloads key m - 1), so a row of 4096 keys costs one memory latency
// instead of sixteen; NB follows the row's length, so that short rows do not
// issue loads they do not use.
template <int NB>
__device__ __forceinline__ void load_row_keys(const float* sc, int64_t m, uint32_t* s_key) {
  for (int64_t e0 = threadIdx.x; e0 < m; e0 += 256 * NB) {
    float v[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t e = e0 + 256 * i;
      v[i] = sc[e < m ? e : m - 1];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t e = e0 + 256 * i;
      if (e < m) s_key[key_slot(e)] = order_key(v[i]);
    }
  }
}

// LONG: rows may exceed 2048 units.  Only then are the batched key loads
// compiled in: their registers (77 VGPRs against 36) would cost launches of
// short rows (pooled blocks, small LDS) two of their eight waves per SIMD.
template <bool LONG>
__global__ __launch_bounds__(256) void topk_row_kernel(TopkParams p) {
  extern __shared__ uint32_t s_mem[];
  uint32_t* s_hist = s_mem;                 // ROW_BINS
  uint32_t* s_scr = s_mem + ROW_BINS;       // 16
  uint32_t* s_key = s_scr + 16;             // row keys, padded (key_slot)
  const int64_t row = blockIdx.x;
  const RowInfo ri = row_info(p, row);
  int32_t* out = p.idx + row * p.k_out;
  const int tid = threadIdx.x;

  if (ri.n_vis <= p.k_out) {   // everything visible is kept
    for (int64_t j = tid; j < p.k_out; j += 256) out[j] = j < ri.n_vis ? static_cast<int32_t>(j) : -1;
    return;
  }
  const int64_t m = ri.n_vis - ri.nf;             // candidates: units nf .. n_vis-1
  const uint32_t need0 = static_cast<uint32_t>(ri.K - ri.nf);
  const float* sc = p.scores + row * p.n_units + ri.nf;
  if constexpr (LONG) {
    if (m > 256 * 8) load_row_keys<16>(sc, m, s_key);
    else if (m > 256 * 2) load_row_keys<4>(sc, m, s_key);
    else load_row_keys<1>(sc, m, s_key);
  } else {
    load_row_keys<1>(sc, m, s_key);
  }
  for (int64_t j = tid; j < p.k_out; j += 256) {
    if (j < ri.nf) out[j] = static_cast<int32_t>(j);
    else if (j >= ri.K) out[j] = -1;
  }
  if (need0 == 0) return;   // every kept slot is a forced sink
  __syncthreads();

  // radix select: 11 + 11 + 10 bits
  uint32_t prefix = 0, pmask = 0, need = need0;
  const int shifts[3] = {21, 10, 0};
  const int nbits[3] = {11, 11, 10};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int nb = 1 << nbits[pass], sh = shifts[pass];
    for (int b = tid; b < nb; b += 256) s_hist[b] = 0;
    __syncthreads();
    for (int64_t e = tid; e < m; e += 256) {
      const uint32_t k = s_key[key_slot(e)];
      if ((k & pmask) == prefix) atomicAdd(&s_hist[(k >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    uint32_t above;
    const uint32_t b = find_bin_desc(s_hist, nb, need, s_scr, &above);
    need -= above;
    prefix |= b << sh;
    pmask |= static_cast<uint32_t>(nb - 1) << sh;
  }
  const uint32_t T = prefix;      // threshold key; keep `need` units equal to T (lowest index)

  // ordered compaction: thread t owns a contiguous range of candidates
  const int64_t per = (m + 255) / 256;
  const int64_t e0 = tid * per < m ? tid * per : m;
  const int64_t e1 = e0 + per < m ? e0 + per : m;
  uint32_t n_gt = 0, n_eq = 0;
  for (int64_t e = e0; e < e1; ++e) {
    const uint32_t k = s_key[key_slot(e)];
    n_gt += k > T;
    n_eq += k == T;
  }
  uint32_t tot;
  const uint32_t eq_before = block_excl_scan_256(n_eq, s_scr, &tot);
  uint32_t take_eq = need > eq_before ? need - eq_before : 0;
  if (take_eq > n_eq) take_eq = n_eq;
  const uint32_t pos0 = block_excl_scan_256(n_gt + take_eq, s_scr, &tot);
  uint32_t pos = static_cast<uint32_t>(ri.nf) + pos0, eq_seen = 0;
  for (int64_t e = e0; e < e1; ++e) {
    const uint32_t k = s_key[key_slot(e)];
    bool keep = k > T;
    if (k == T) {
      keep = eq_seen < take_eq;
      ++eq_seen;
    }
    if (keep) {
      if (pos < ri.K) out[pos] = static_cast<int32_t>(ri.nf + e);   // guard: never past K
      ++pos;
    }
  }
}

// --------------------------------------------------------- multi-block path --

__global__ void topk_clear_kernel(TopkParams p) {
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  const int64_t n = rows * HIST_BINS;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    p.hist[i] = 0;
    if (i < rows) p.cand_cnt[i] = 0;
  }
}

// Top-12-bit histogram of the candidate units of each row (standalone top-k;
// the fused path gets it from the score epilogue instead).
__global__ __launch_bounds__(256) void topk_hist_kernel(TopkParams p) {
  __shared__ uint32_t s_hist[HIST_BINS];
  const int64_t row = blockIdx.x / p.n_chunks;
  const int ch = blockIdx.x % p.n_chunks;
  const RowInfo ri = row_info(p, row);
  if (ri.n_vis <= p.k_out) return;
  for (int b = threadIdx.x; b < HIST_BINS; b += 256) s_hist[b] = 0;
  __syncthreads();
  int64_t j0 = static_cast<int64_t>(ch) * p.chunk, j1 = j0 + p.chunk;
  if (j0 < ri.nf) j0 = ri.nf;
  if (j1 > ri.n_vis) j1 = ri.n_vis;
  const float* sc = p.scores + row * p.n_units;
  for (int64_t jb = j0 + threadIdx.x; jb < j1; jb += 256 * 16) {   // 16 loads in flight per thread
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t j = jb + 256 * i;
      v[i] = sc[j < j1 ? j : j1 - 1];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (jb + 256 * i < j1) atomicAdd(&s_hist[order_key(v[i]) >> 20], 1u);
  }
  __syncthreads();
  uint32_t* g = p.hist + row * HIST_BINS;
  for (int b = threadIdx.x; b < HIST_BINS; b += 256)
    if (s_hist[b]) atomicAdd(g + b, s_hist[b]);
}

// Threshold bin per row; counts units above it per chunk; gathers the units
// of the threshold bin as candidates.  The chunk's keys (16 per thread) are
// loaded first, so that their latency overlaps that of the row's position and
// histogram, and stay in registers for both passes.
static_assert(TOPK_CHUNK == 16 * 256, "16 keys per thread");
__global__ __launch_bounds__(256) void topk_select_kernel(TopkParams p) {
  __shared__ __align__(16) uint32_t s_hist[HIST_BINS];
  __shared__ uint32_t s_scr[16];
  __shared__ uint32_t s_base;
  const int64_t row = blockIdx.x / p.n_chunks;
  const int ch = blockIdx.x % p.n_chunks;
  const int64_t c0 = static_cast<int64_t>(ch) * TOPK_CHUNK;
  const float* sc = p.scores + row * p.n_units;
  // all 16 loads are issued before any key is used (in-range addresses only:
  // past the row's end a lane reloads its last unit)
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t j = c0 + 256 * i + threadIdx.x;
    v[i] = sc[j < p.n_units ? j : p.n_units - 1];
  }
  uint32_t key[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) key[i] = c0 + 256 * i + threadIdx.x < p.n_units ? order_key(v[i]) : 0u;
  const RowInfo ri = row_info(p, row);
  if (ri.n_vis <= p.k_out) return;
  const uint32_t need = static_cast<uint32_t>(ri.K - ri.nf);
  if (need == 0) return;
  // the row's histogram (16 KB, in L2 after the score kernel's atomics):
  // every thread issues its four 16-byte loads before it writes any
  const u32x4_t* g4 = reinterpret_cast<const u32x4_t*>(p.hist + row * HIST_BINS);
  u32x4_t hv[HIST_BINS / 1024];
#pragma unroll
  for (int i = 0; i < HIST_BINS / 1024; ++i) hv[i] = g4[threadIdx.x + 256 * i];
#pragma unroll
  for (int i = 0; i < HIST_BINS / 1024; ++i) reinterpret_cast<u32x4_t*>(s_hist)[threadIdx.x + 256 * i] = hv[i];
  __syncthreads();
  uint32_t above;
  const uint32_t b1 = find_bin_desc(s_hist, HIST_BINS, need, s_scr, &above);
  if (ch == 0 && threadIdx.x == 0) {
    p.thr[row * 4 + 0] = b1;
    p.thr[row * 4 + 3] = above;
  }
  const int64_t j0 = c0 > ri.nf ? c0 : ri.nf;   // candidates: [j0, j1), past the forced sinks
  const int64_t j1 = c0 + TOPK_CHUNK < ri.n_vis ? c0 + TOPK_CHUNK : ri.n_vis;
  // pass 1: count units above the bin and units in it
  uint32_t n_hi = 0, n_in = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t j = c0 + 256 * i + threadIdx.x;
    const bool in = j >= j0 && j < j1;
    const uint32_t bin = key[i] >> 20;
    n_hi += in && bin > b1;
    n_in += in && bin == b1;
  }
  uint32_t tot_hi, tot_in;
  block_excl_scan_256(n_hi, s_scr, &tot_hi);
  const uint32_t my_off = block_excl_scan_256(n_in, s_scr, &tot_in);
  if (threadIdx.x == 0) {
    p.cnt_hi[row * p.n_chunks + ch] = tot_hi;
    s_base = tot_in ? atomicAdd(p.cand_cnt + row, tot_in) : 0;
  }
  __syncthreads();
  // pass 2: write the candidates (key, index)
  uint32_t w = s_base + my_off;
  uint32_t* cand = p.cand + row * p.cand_cap * 2;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t j = c0 + 256 * i + threadIdx.x;
    if (j >= j0 && j < j1 && (key[i] >> 20) == b1) {
      if (w < p.cand_cap) {
        cand[2 * w] = key[i];
        cand[2 * w + 1] = static_cast<uint32_t>(j);
      }
      ++w;
    }
  }
}

// Calls f(key, index) for candidates e = tid, tid + 256, ... below m (this
// thread's share, in that order), with the loads of 8 candidates issued
// before any is used: the candidates come from L2, and a row of a few
// thousand then costs one latency per 2048 instead of one per 256.
template <typename F>
__device__ __forceinline__ void for_candidates(const uint32_t* cand, uint32_t m, F&& f) {
  constexpr int CB = 8;
  for (uint32_t e0 = threadIdx.x; e0 < m; e0 += 256 * CB) {
    u32x2_t kv[CB];
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const uint32_t e = e0 + 256 * i;
      kv[i] = *reinterpret_cast<const u32x2_t*>(cand + 2 * static_cast<size_t>(e < m ? e : m - 1));
    }
#pragma unroll
    for (int i = 0; i < CB; ++i)
      if (e0 + 256 * i < m) f(kv[i].x, kv[i].y);
  }
}

// Exact threshold key T among the candidates of one row, and the largest
// kept index J among the candidates equal to T (0xffffffff when every one of
// them is kept).  The candidates are the units of the threshold bin b1 (the
// units above it are kept whole); radix passes of 12 + 8 bits on the low 20
// bits of the key find T, then, only when the tie at T is cut, 11 + 11 + 10
// bits on the complemented index find J (the need-th smallest index).  The
// candidate order does not matter, so the result is deterministic.  All 256
// threads call it; need > 0.
__device__ void resolve_threshold(const TopkParams& p, int64_t row, uint32_t need, uint32_t* s_hist,
                                  uint32_t* s_scr, uint32_t* T_out, uint32_t* J_out) {
  const int tid = threadIdx.x;
  const uint32_t* cand = p.cand + row * p.cand_cap * 2;
  const uint32_t m = p.cand_cnt[row];
  need -= p.thr[row * 4 + 3];            // minus the units above the threshold bin
  const uint32_t b1 = p.thr[row * 4 + 0];
  uint32_t prefix = b1 << 20, pmask = 0xfff00000u;
  const int shifts[2] = {8, 0};
  const int nbits[2] = {12, 8};
  uint32_t n_eq = 0;   // candidates whose key equals T
  for (int pass = 0; pass < 2; ++pass) {
    const int nb = 1 << nbits[pass], sh = shifts[pass];
    for (int b = tid; b < nb; b += 256) s_hist[b] = 0;
    __syncthreads();
    for_candidates(cand, m, [&](uint32_t k, uint32_t) {
      if ((k & pmask) == prefix) atomicAdd(&s_hist[(k >> sh) & (nb - 1)], 1u);
    });
    __syncthreads();
    uint32_t above;
    const uint32_t b = find_bin_desc(s_hist, nb, need, s_scr, &above);
    need -= above;
    prefix |= b << sh;
    pmask |= static_cast<uint32_t>(nb - 1) << sh;
    if (pass == 1) n_eq = s_hist[b];   // read before the next pass clears the bins
  }
  const uint32_t T = prefix;
  __syncthreads();
  const bool cut = n_eq > need;
  uint32_t jp = 0, jm = 0;
  const int jsh[3] = {21, 10, 0};
  const int jbits[3] = {11, 11, 10};
  for (int pass = 0; pass < (cut ? 3 : 0); ++pass) {
    const int nb = 1 << jbits[pass], sh = jsh[pass];
    for (int b = tid; b < HIST_BINS; b += 256) s_hist[b] = 0;
    __syncthreads();
    for_candidates(cand, m, [&](uint32_t k, uint32_t j) {
      const uint32_t cj = ~j;
      if (k == T && (cj & jm) == jp) atomicAdd(&s_hist[(cj >> sh) & (nb - 1)], 1u);
    });
    __syncthreads();
    uint32_t above;
    const uint32_t b = find_bin_desc(s_hist, nb < 256 ? 256 : nb, need, s_scr, &above);
    need -= above;
    jp |= b << sh;
    jm |= static_cast<uint32_t>(nb - 1) << sh;
  }
  *T_out = T;
  *J_out = cut ? ~jp : 0xffffffffu;
}

// Resolve and ordered compaction of one chunk of a row.  Every workgroup of a
// row resolves (T, J) from the row's candidates on its own (the candidates of
// one 12-bit bin: a few thousand at most, read from L2), so no single
// workgroup per row stands between the select and the compaction.  The
// chunk's output offset is the forced sinks plus the units kept in earlier
// chunks: those above the threshold bin (counted by the select) and the kept
// candidates.  Thread t then owns the 16 units 16 t .. 16 t + 15 of the chunk
// (loaded first, as four 16-byte loads), so an exclusive scan of the
// per-thread counts gives ascending output positions.  Chunk 0 also writes the
// sinks and the -1 padding, or the whole row when every visible unit is kept.
__global__ __launch_bounds__(256) void topk_finish_kernel(TopkParams p) {
  __shared__ uint32_t s_hist[HIST_BINS];
  __shared__ uint32_t s_scr[16];
  const int64_t row = blockIdx.x / p.n_chunks;
  const int ch = blockIdx.x % p.n_chunks;
  const int tid = threadIdx.x;
  const int64_t c0 = static_cast<int64_t>(ch) * TOPK_CHUNK;
  const int64_t a0 = c0 + 16 * tid;
  const float* sc = p.scores + row * p.n_units;
  float v[16];
  if (a0 + 16 <= p.n_units && (p.n_units & 3) == 0) {   // whole, 16-byte aligned run
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4_t q = *reinterpret_cast<const f32x4_t*>(sc + a0 + 4 * i);
      v[4 * i] = q[0];
      v[4 * i + 1] = q[1];
      v[4 * i + 2] = q[2];
      v[4 * i + 3] = q[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = a0 + i < p.n_units ? sc[a0 + i] : 0.f;
  }
  const RowInfo ri = row_info(p, row);
  int32_t* out = p.idx + row * p.k_out;
  if (ri.n_vis <= p.k_out) {
    if (ch == 0)
      for (int64_t j = tid; j < p.k_out; j += 256) out[j] = j < ri.n_vis ? static_cast<int32_t>(j) : -1;
    return;
  }
  if (ch == 0) {
    for (int64_t j = tid; j < p.k_out; j += 256) {
      if (j < ri.nf) out[j] = static_cast<int32_t>(j);
      else if (j >= ri.K) out[j] = -1;
    }
  }
  if (ri.K == ri.nf) return;
  uint32_t T, J;
  resolve_threshold(p, row, static_cast<uint32_t>(ri.K - ri.nf), s_hist, s_scr, &T, &J);
  // units kept before this chunk
  uint32_t before = 0;
  for (int c = tid; c < ch; c += 256) before += p.cnt_hi[row * p.n_chunks + c];
  {
    const uint32_t* cand = p.cand + row * p.cand_cap * 2;
    const uint32_t m = p.cand_cnt[row];
    for_candidates(cand, m, [&](uint32_t k, uint32_t j) { before += j < c0 && (k > T || (k == T && j <= J)); });
  }
  uint32_t tot_before;
  block_excl_scan_256(before, s_scr, &tot_before);
  const uint32_t off = static_cast<uint32_t>(ri.nf) + tot_before;
  const int64_t j0 = c0 > ri.nf ? c0 : ri.nf;
  const int64_t j1 = c0 + TOPK_CHUNK < ri.n_vis ? c0 + TOPK_CHUNK : ri.n_vis;
  uint32_t sel = 0;   // bit i: unit a0 + i is kept
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t j = a0 + i;
    const uint32_t k = order_key(v[i]);
    const bool keep = j >= j0 && j < j1 && (k > T || (k == T && static_cast<uint32_t>(j) <= J));
    sel |= static_cast<uint32_t>(keep) << i;
  }
  uint32_t tot;
  uint32_t pos = off + block_excl_scan_256(__builtin_popcount(sel), s_scr, &tot);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if ((sel >> i) & 1u) {
      if (pos < ri.K) out[pos] = static_cast<int32_t>(a0 + i);   // guard: never past K
      ++pos;
    }
  }
}

// ------------------------------------------------------------- long rows --

constexpr int LONG_NT = 1024;                 // threads of the long-row kernel (16 waves)
constexpr int LONG_NW = LONG_NT / 64;
constexpr int LONG_SUB = 4 * LONG_NT;         // units of one coalesced sub-block (a float4 per thread)
constexpr int LONG_NS = 4;                    // sub-blocks per iteration
constexpr int LONG_IT = LONG_NS * LONG_SUB;   // 16384 units per iteration
constexpr int LONG_BINS = 4096;               // 12-bit histogram
constexpr int LONG_COPIES = 8;                // histogram copies (lane l adds into copy l % 8)
constexpr int LONG_STRIDE = LONG_BINS + 1;    // words between copies: a bin's copies fall in different banks
constexpr size_t LONG_LDS = static_cast<size_t>(LONG_COPIES) * LONG_STRIDE * sizeof(uint32_t);

// Finds the bin b (scanning from the highest bin down) that holds the need-th
// largest element: above(b) < need <= above(b) + hist[b].  NT threads, nb a
// multiple of NT (at most 16 bins per thread).  All threads get the result.
template <int NT>
__device__ uint32_t find_bin_desc_nt(const uint32_t* hist, int nb, uint32_t need, uint32_t* scratch,
                                     uint32_t* above) {
  const int per = nb / NT;
  const int hi = nb - threadIdx.x * per;
  uint32_t c[16];
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    c[i] = i < per ? hist[hi - 1 - i] : 0u;
    local += c[i];
  }
  uint32_t total;
  const uint32_t excl = block_excl_scan<NT / 64>(local, scratch, &total);
  if (excl < need && need <= excl + local) {
    uint32_t acc = excl, acc_at = 0;
    int found = per - 1;
    bool done = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (!done && i < per) {
        if (acc + c[i] >= need) {
          found = i;
          acc_at = acc;
          done = true;
        }
        acc += c[i];
      }
    }
    scratch[NT / 64] = static_cast<uint32_t>(hi - 1 - found);
    scratch[NT / 64 + 1] = acc_at;
  }
  __syncthreads();
  const uint32_t bin = scratch[NT / 64];
  *above = scratch[NT / 64 + 1];
  __syncthreads();
  return bin;
}

// Raw scores of one iteration of the long-row kernel: thread t holds units
// a + 4096 i + 4 t + r (sub-block i < 4, r < 4), so that every load
// instruction of a wave reads 1 KB of contiguous scores.  Every load is
// unconditional at an in-range address, so that the next iteration's loads
// stay in flight while this one is processed: ALIGNED (units a multiple of
// 4, rows 16-byte aligned) loads float4s, clamped to the last whole one
// (whose units, past the row, are never used); otherwise one clamped load
// per unit.
template <bool ALIGNED>
__device__ __forceinline__ void long_load(const float* sc, int64_t n_units, int64_t a, float (&v)[4 * LONG_NS]) {
#pragma unroll
  for (int i = 0; i < LONG_NS; ++i) {
    const int64_t u0 = a + static_cast<int64_t>(i) * LONG_SUB + 4 * threadIdx.x;
    if constexpr (ALIGNED) {
      const f32x4_t q = *reinterpret_cast<const f32x4_t*>(sc + (u0 + 4 <= n_units ? u0 : n_units - 4));
      v[4 * i] = q[0];
      v[4 * i + 1] = q[1];
      v[4 * i + 2] = q[2];
      v[4 * i + 3] = q[3];
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * i + r] = sc[u0 + r < n_units ? u0 + r : n_units - 1];
    }
  }
}

// Keys of the loaded units; bit 4 i + r of the result says the unit lies in [lo, hi).
__device__ __forceinline__ uint32_t long_keys(const float (&v)[4 * LONG_NS], int64_t a, int64_t lo, int64_t hi,
                                              uint32_t (&key)[4 * LONG_NS]) {
  uint32_t valid = 0;
#pragma unroll
  for (int i = 0; i < LONG_NS; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t u = a + static_cast<int64_t>(i) * LONG_SUB + 4 * threadIdx.x + r;
      key[4 * i + r] = order_key(v[4 * i + r]);
      valid |= static_cast<uint32_t>(u >= lo && u < hi) << (4 * i + r);
    }
  return valid;
}

// Ordered compaction of one iteration: writes the selected units (bit 4 i + r
// of sel: unit a + 4096 i + 4 t + r) at base + their rank in index order
// (sub-blocks, then waves, then lanes, then r), through put(position, slot);
// returns the number selected.  A lane's selected units of lower lanes come
// from the four ballots of its sub-block; per-wave totals through LDS.  All
// threads call it; it holds two barriers.
template <typename F>
__device__ __forceinline__ uint32_t long_compact(uint32_t sel, uint32_t base, uint32_t* s_wt, F&& put) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t lane_before[LONG_NS];
#pragma unroll
  for (int i = 0; i < LONG_NS; ++i) {
    uint32_t lb = 0, wt = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint64_t bal = __ballot((sel >> (4 * i + r)) & 1u);
      lb += __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u));
      wt += static_cast<uint32_t>(__popcll(bal));
    }
    lane_before[i] = lb;
    if (lane == 0) s_wt[i * LONG_NW + wid] = wt;
  }
  __syncthreads();
  uint32_t sub_base = 0;
#pragma unroll
  for (int i = 0; i < LONG_NS; ++i) {
    uint32_t before = 0, st = 0;
    for (int w = 0; w < LONG_NW; ++w) {
      const uint32_t t = s_wt[i * LONG_NW + w];
      before += w < wid ? t : 0u;
      st += t;
    }
    uint32_t pos = base + sub_base + before + lane_before[i];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if ((sel >> (4 * i + r)) & 1u) {
        put(pos, 4 * i + r);
        ++pos;
      }
    }
    sub_base += st;
  }
  __syncthreads();   // s_wt is rewritten by the next call
  return sub_base;
}

// One workgroup of 1024 threads per row, for rows longer than the row kernel
// holds in LDS, and for the few long rows of decode.  The row's scores are
// read twice (the second time from the L2), each pass with the next
// iteration's loads in flight while the current one is processed:
//   1. a histogram of the top 12 bits of the keys of the candidate units (the
//      visible units past the forced sinks), in eight bank-shifted copies
//      (lane l adds into copy l % 8, so that lanes of one instruction rarely
//      hit one address), finds the threshold bin b1;
//   2. every unit at or above bin b1 is staged in the workspace as (key,
//      index), in index order (ordered compaction: ballots within a wave,
//      per-wave totals through LDS): the kept units of bins above b1 plus
//      the units of bin b1, a few thousand for a real score row;
// then the staged units of bin b1 give the exact threshold key T and, when
// the tie at T is cut, the largest kept index J among the units equal to T;
// a last ordered compaction over the staged list writes the kept ids in
// ascending order.  The staging count lives in registers (one workgroup per
// row), so nothing needs clearing before the launch.
template <bool ALIGNED>
__device__ void topk_long_row(const TopkParams& p, int64_t row, uint32_t* s_hist, uint32_t* s_scr, uint32_t* s_wt) {
  const int tid = threadIdx.x, lane = tid & 63;
  const RowInfo ri = row_info(p, row);
  int32_t* out = p.idx + row * p.k_out;
  if (ri.n_vis <= p.k_out) {   // everything visible is kept
    for (int64_t j = tid; j < p.k_out; j += LONG_NT) out[j] = j < ri.n_vis ? static_cast<int32_t>(j) : -1;
    return;
  }
  for (int64_t j = tid; j < p.k_out; j += LONG_NT) {
    if (j < ri.nf) out[j] = static_cast<int32_t>(j);
    else if (j >= ri.K) out[j] = -1;
  }
  uint32_t need = static_cast<uint32_t>(ri.K - ri.nf);
  if (need == 0) return;   // every kept slot is a forced sink
  const float* sc = p.scores + row * p.n_units;
  const int64_t lo = ri.nf, hi = ri.n_vis;
  const int64_t a_end = (hi + LONG_IT - 1) / LONG_IT * LONG_IT;   // whole iterations covering [0, hi)

  // pass 1: histogram of the top 12 bits
  for (int b = tid; b < LONG_COPIES * LONG_STRIDE; b += LONG_NT) s_hist[b] = 0;
  __syncthreads();
  uint32_t* my_hist = s_hist + (lane & (LONG_COPIES - 1)) * LONG_STRIDE;
  {
    float cur[4 * LONG_NS];
    long_load<ALIGNED>(sc, p.n_units, 0, cur);
    for (int64_t a = 0; a < a_end; a += LONG_IT) {
      float nxt[4 * LONG_NS];
      long_load<ALIGNED>(sc, p.n_units, a + LONG_IT < a_end ? a + LONG_IT : a, nxt);
      uint32_t k[4 * LONG_NS];
      const uint32_t v = long_keys(cur, a, lo, hi, k);
#pragma unroll
      for (int i = 0; i < 4 * LONG_NS; ++i)
        if ((v >> i) & 1u) atomicAdd(&my_hist[k[i] >> 20], 1u);
#pragma unroll
      for (int i = 0; i < 4 * LONG_NS; ++i) cur[i] = nxt[i];
    }
  }
  __syncthreads();
  for (int b = tid; b < LONG_BINS; b += LONG_NT) {
    uint32_t t = 0;
#pragma unroll
    for (int c = 0; c < LONG_COPIES; ++c) t += s_hist[c * LONG_STRIDE + b];
    s_hist[b] = t;   // copy 0 holds the sum (each bin has one owner thread)
  }
  __syncthreads();
  uint32_t above;
  const uint32_t b1 = find_bin_desc_nt<LONG_NT>(s_hist, LONG_BINS, need, s_scr, &above);
  need -= above;   // to keep from bin b1

  // pass 2: stage the units at or above bin b1, in index order
  uint32_t* stage = p.cand + row * p.cand_cap * 2;
  uint32_t m = 0;   // staged units
  {
    float cur[4 * LONG_NS];
    long_load<ALIGNED>(sc, p.n_units, 0, cur);
    for (int64_t a = 0; a < a_end; a += LONG_IT) {
      float nxt[4 * LONG_NS];
      long_load<ALIGNED>(sc, p.n_units, a + LONG_IT < a_end ? a + LONG_IT : a, nxt);
      uint32_t k[4 * LONG_NS];
      const uint32_t v = long_keys(cur, a, lo, hi, k);
      uint32_t sel = 0;
#pragma unroll
      for (int i = 0; i < 4 * LONG_NS; ++i) sel |= static_cast<uint32_t>(((v >> i) & 1u) && (k[i] >> 20) >= b1) << i;
      m += long_compact(sel, m, s_wt, [&](uint32_t pos, int slot) {
        if (pos < p.cand_cap) {
          stage[2 * pos] = k[slot];
          stage[2 * pos + 1] = static_cast<uint32_t>(a + (slot >> 2) * LONG_SUB + 4 * tid + (slot & 3));
        }
      });
#pragma unroll
      for (int i = 0; i < 4 * LONG_NS; ++i) cur[i] = nxt[i];
    }
  }
  // (long_compact's last barrier: the staged list is complete and visible)

  // exact threshold among the staged units of bin b1: 12 + 8 more bits of the
  // key, then, only when the tie at T is cut, 11 + 11 + 10 bits of the
  // complemented index
  uint32_t prefix = b1 << 20, pmask = 0xfff00000u, n_eq = 0;
  {
    const int shifts[2] = {8, 0};
    const int nbits[2] = {12, 8};
    for (int pass = 0; pass < 2; ++pass) {
      const int nb = 1 << nbits[pass], sh = shifts[pass];
      for (int b = tid; b < LONG_BINS; b += LONG_NT) s_hist[b] = 0;
      __syncthreads();
      for (uint32_t e = tid; e < m; e += LONG_NT) {
        const uint32_t kk = stage[2 * e];
        if ((kk & pmask) == prefix) atomicAdd(&s_hist[(kk >> sh) & (nb - 1)], 1u);
      }
      __syncthreads();
      uint32_t ab;
      const uint32_t b = find_bin_desc_nt<LONG_NT>(s_hist, LONG_BINS, need, s_scr, &ab);
      need -= ab;
      prefix |= b << sh;
      pmask |= static_cast<uint32_t>(nb - 1) << sh;
      if (pass == 1) n_eq = s_hist[b];
      __syncthreads();   // every thread has read s_hist[b] before the next clear
    }
  }
  const uint32_t T = prefix;
  uint32_t J = 0xffffffffu;   // the largest kept index among the units equal to T
  if (n_eq > need) {
    uint32_t jp = 0, jm = 0;
    const int jsh[3] = {21, 10, 0};
    const int jbits[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
      const int nb = 1 << jbits[pass], sh = jsh[pass];
      for (int b = tid; b < LONG_BINS; b += LONG_NT) s_hist[b] = 0;
      __syncthreads();
      for (uint32_t e = tid; e < m; e += LONG_NT) {
        const uint32_t kk = stage[2 * e], cj = ~stage[2 * e + 1];
        if (kk == T && (cj & jm) == jp) atomicAdd(&s_hist[(cj >> sh) & (nb - 1)], 1u);
      }
      __syncthreads();
      uint32_t ab;
      const uint32_t b = find_bin_desc_nt<LONG_NT>(s_hist, LONG_BINS, need, s_scr, &ab);
      need -= ab;
      jp |= b << sh;
      jm |= static_cast<uint32_t>(nb - 1) << sh;
    }
    J = ~jp;
  }

  // the kept units of the staged list, in its (index) order: thread t owns a
  // contiguous run of it
  const uint32_t per = (m + LONG_NT - 1) / LONG_NT;
  const uint32_t e0 = tid * per < m ? tid * per : m;
  const uint32_t e1 = e0 + per < m ? e0 + per : m;
  uint32_t n_keep = 0;
  for (uint32_t e = e0; e < e1; ++e) {
    const uint32_t kk = stage[2 * e], j = stage[2 * e + 1];
    n_keep += kk > T || (kk == T && j <= J);
  }
  uint32_t tot;
  uint32_t pos = static_cast<uint32_t>(ri.nf) + block_excl_scan<LONG_NW>(n_keep, s_scr, &tot);
  for (uint32_t e = e0; e < e1; ++e) {
    const uint32_t kk = stage[2 * e], j = stage[2 * e + 1];
    if (kk > T || (kk == T && j <= J)) {
      if (pos < ri.K) out[pos] = static_cast<int32_t>(j);   // guard: never past K
      ++pos;
    }
  }
}

__global__ __launch_bounds__(LONG_NT) void topk_long_kernel(TopkParams p) {
  extern __shared__ uint32_t s_hist[];   // LONG_COPIES x LONG_STRIDE
  __shared__ uint32_t s_scr[LONG_NW + 4];
  __shared__ uint32_t s_wt[LONG_NS * LONG_NW];   // selected units per (sub-block, wave)
  if ((p.n_units & 3) == 0) topk_long_row<true>(p, blockIdx.x, s_hist, s_scr, s_wt);
  else topk_long_row<false>(p, blockIdx.x, s_hist, s_scr, s_wt);
}

// ------------------------------------------------------------------ host --

bool topk_use_multiblock(int64_t rows, int64_t n_units) {
  return n_units > 16384 || (rows < 128 && n_units > TOPK_CHUNK);
}

bool topk_use_long(int64_t rows, int64_t n_units) { return rows >= 128 && n_units > 16384; }

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t topk_workspace_bytes(int64_t rows, int64_t n_units) {
  if (!topk_use_multiblock(rows, n_units)) return 0;
  if (topk_use_long(rows, n_units)) return align256(static_cast<size_t>(rows) * n_units * 8);   // staged units
  const int64_t nch = (n_units + TOPK_CHUNK - 1) / TOPK_CHUNK;
  size_t b = 0;
  b += align256(rows * HIST_BINS * 4);
  b += align256(rows * 4);
  b += align256(rows * n_units * 8);
  b += align256(rows * nch * 4);
  b += align256(rows * 16);
  return b;
}

void topk_bind_workspace(TopkParams& p, void* ws) {
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  p.cand_cap = p.n_units;
  if (topk_use_long(rows, p.n_units)) {
    p.cand = static_cast<uint32_t*>(ws);
    return;
  }
  p.chunk = TOPK_CHUNK;
  p.n_chunks = static_cast<int32_t>((p.n_units + TOPK_CHUNK - 1) / TOPK_CHUNK);
  char* c = static_cast<char*>(ws);
  p.hist = reinterpret_cast<uint32_t*>(c);     c += align256(rows * HIST_BINS * 4);
  p.cand_cnt = reinterpret_cast<uint32_t*>(c); c += align256(rows * 4);
  p.cand = reinterpret_cast<uint32_t*>(c);     c += align256(rows * p.n_units * 8);
  p.cnt_hi = reinterpret_cast<uint32_t*>(c);   c += align256(rows * p.n_chunks * 4);
  p.thr = reinterpret_cast<uint32_t*>(c);
}

hipError_t launch_topk_clear(const TopkParams& p, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  int64_t blocks = (rows * HIST_BINS + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(topk_clear_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkParams& p, bool hist_ready, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  hipError_t e;
  if (!topk_use_multiblock(rows, p.n_units)) {
    const size_t lds = (ROW_BINS + 16 + static_cast<size_t>(p.n_units + p.n_units / 16 + 1)) * sizeof(uint32_t);
    const bool long_rows = p.n_units > 2048;
    const void* fn = long_rows ? reinterpret_cast<const void*>(topk_row_kernel<true>)
                               : reinterpret_cast<const void*>(topk_row_kernel<false>);
    if (lds > 65536) {
      // the largest size this path uses (rows of 16384 units), the same value
      // on every call: no state kept between calls, and concurrent calls agree
      constexpr size_t lds_max = (ROW_BINS + 16 + 16384 + 16384 / 16 + 1) * sizeof(uint32_t);
      if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_max))) !=
          hipSuccess)
        return e;
    }
    if (long_rows) hipLaunchKernelGGL(topk_row_kernel<true>, dim3(static_cast<unsigned>(rows)), dim3(256), lds, st, p);
    else hipLaunchKernelGGL(topk_row_kernel<false>, dim3(static_cast<unsigned>(rows)), dim3(256), lds, st, p);
    return hipGetLastError();
  }
  if (topk_use_long(rows, p.n_units)) {
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_long_kernel),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(LONG_LDS))) != hipSuccess)
      return e;
    hipLaunchKernelGGL(topk_long_kernel, dim3(static_cast<unsigned>(rows)), dim3(LONG_NT), LONG_LDS, st, p);
    return hipGetLastError();
  }
  const dim3 g(static_cast<unsigned>(rows * p.n_chunks));
  if (!hist_ready) {
    if ((e = launch_topk_clear(p, st)) != hipSuccess) return e;
    hipLaunchKernelGGL(topk_hist_kernel, g, dim3(256), 0, st, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(topk_select_kernel, g, dim3(256), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_finish_kernel, g, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace dsa
