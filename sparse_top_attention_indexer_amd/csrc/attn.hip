// Softmax attention over the selected tokens on gfx950.
//
// o(i, h) = sum_{j in T(i)} softmax_j(scale * Q(i, h) . K(j, g)) V(j, g)
//
// T(i) is the query's token stream: the idx row in list order (token mode),
// the live selected blocks expanded to their positions followed by the
// incomplete tail (block mode; llama.cpp mirror commit c88c916636), or every
// visible token (dense, the indexer-off reference of ik_llama.cpp PR #2058).
// The selected rows are gathered straight from the cache (ik_llama_opt log,
// openPangu "Gather ... DSA decode reads" and the gathered prefill commits:
// attention over the gathered latent rows, values taken from the same rows).
//
// The stream is cut into tiles of 32 entries.  An online softmax runs over the
// tiles in order; invisible or dead entries are masked by position: their
// logits are -inf, so their weights are exactly zero.  The GQA and f32 kernels
// zero-fill their rows; the MLA kernel gathers the sequence's row 0 in their
// place (a written, visible row whenever the stream has a live entry), which
// its zero weight cancels.  A row that sees no key at all is written as
// zeros.  Long streams are split into contiguous chunks whose partial (max,
// sum, unnormalised output) are merged in a fixed order by
// attn_combine_kernel, so results are deterministic and identical for the
// same stream whatever the call that produced it.
//
// Kernels:
//   attn_f32_kernel   f32 Q/K/V, any head grouping, Dk, Dv <= 256 (VALU)
//   attn_mla_kernel   MLA: 576-wide latent K, V = its first 512 columns, bf16,
//                     8 waves x 16 heads on 16x16x32 MFMAs
//   attn_gqa_kernel   GQA: Dk = Dv = 128, up to 16 heads per KV group, bf16,
//                     one wave per KV group on 16x16x32 MFMAs
#include <type_traits>

#include "dsa_device.h"
#include "dsa_internal.h"
#include "../../include/dsa.h"

namespace dsa {

constexpr int TILE = 32;
constexpr int MAX_BLOCKS = 4096;   // idx entries per row in block mode

// ----------------------------------------------------------- token stream --

struct StreamInfo {
  int64_t n_vis;    // visible tokens
  int64_t n_cb;     // complete visible blocks (block mode)
  int64_t nb_live;  // live selected blocks (block mode)
  int64_t len;      // stream length
};

// Prepares the stream of one row; in block mode compacts the live block ids
// (0 <= b < n_cb) of the idx row into s_blk, in list order.  All NW * 64
// threads of the workgroup must call it.
template <int NW>
__device__ StreamInfo stream_setup(const AttnParams& p, int64_t row, int32_t* s_blk, uint32_t* s_scr) {
  const int s = static_cast<int>(row / p.n_q);
  const int64_t kl = p.kv_len ? p.kv_len[s] : p.n_kv;
  StreamInfo si;
  si.n_vis = visible_tokens(p.q_pos[row], kl, p.n_kv);
  si.n_cb = 0;
  si.nb_live = 0;
  if (p.idx == nullptr) {
    si.len = si.n_vis;
  } else if (p.c == 1) {
    si.len = p.k_sel;
  } else {
    si.n_cb = si.n_vis / p.c;
    const int32_t* ir = p.idx + row * p.k_sel;
    constexpr int NT = NW * 64;
    const int per = (p.k_sel + NT - 1) / NT;
    const int e0 = threadIdx.x * per < p.k_sel ? threadIdx.x * per : p.k_sel;
    const int e1 = e0 + per < p.k_sel ? e0 + per : p.k_sel;
    uint32_t cnt = 0;
    for (int e = e0; e < e1; ++e) cnt += (ir[e] >= 0 && ir[e] < si.n_cb);
    uint32_t tot;
    uint32_t w = block_excl_scan<NW>(cnt, s_scr, &tot);
    for (int e = e0; e < e1; ++e)
      if (ir[e] >= 0 && ir[e] < si.n_cb) s_blk[w++] = ir[e];
    __syncthreads();
    si.nb_live = tot;
    si.len = si.nb_live * p.c + (si.n_vis - si.n_cb * p.c);
  }
  return si;
}

// Token of stream position `pos` (0 <= pos), or -1 when dead / invisible.
__device__ __forceinline__ int64_t stream_token(const AttnParams& p, int64_t row, const StreamInfo& si,
                                                const int32_t* s_blk, int64_t pos) {
  if (pos >= si.len) return -1;
  if (p.idx == nullptr) return pos;
  if (p.c == 1) {
    const int64_t t = p.idx[row * p.k_sel + pos];
    return (t >= 0 && t < si.n_vis) ? t : -1;
  }
  const int64_t nbt = si.nb_live * p.c;
  if (pos < nbt) return static_cast<int64_t>(s_blk[pos / p.c]) * p.c + pos % p.c;
  return si.n_cb * p.c + (pos - nbt);
}

__device__ __forceinline__ void split_range(const AttnParams& p, int sp, int64_t len, int64_t* p0, int64_t* p1) {
  *p0 = static_cast<int64_t>(sp) * p.split_len;
  *p1 = sp == p.n_split - 1 ? len : *p0 + p.split_len;
  if (*p1 > len) *p1 = len;
}

// Writes 4 consecutive output values (f32 or bf16).
__device__ __forceinline__ void store4(void* out, int o_dtype, int64_t off, float a, float b, float c, float d) {
  if (o_dtype == DSA_F32) {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + off) = f32x4_t{a, b, c, d};
  } else {
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(out) + off) = u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)};
  }
}

// ============================================================== MLA kernel ==

constexpr int MLA_DK = 576, MLA_DV = 512;
constexpr int MLA_WAVES = 8;                     // 16 query heads each
constexpr int KT_MAIN = TILE * 1024;             // dims 0..511 of the tile rows, 1 KB per row
constexpr int KT_ROPE = TILE * 128;              // dims 512..575, 128 B per row
constexpr int KT_BYTES = KT_MAIN + KT_ROPE;      // one gathered tile (36 KB)
constexpr int KT_NBUF = 3;                       // tiles read by the two wave groups + one in flight
constexpr int TOK_RING = 1024;                   // validated token ids of 32 tiles
constexpr size_t MLA_LDS = KT_NBUF * KT_BYTES + TOK_RING * 4 + 64 + MLA_MAX_BLOCKS * 4;

// Softmax weights reach the PV product rounded to bf16 (relative error up to
// 2^-9).  If the normaliser is summed from the same rounded weights, the
// output is an exact average under perturbed weights w_j (1 + e_j), and
// its error is sum_j w_j e_j (v_j - o): independent small terms when the
// weights are spread, but up to 2^-9 |v_j - o| when one weight dominates
// (x8 outlier rows: several 1e-2).  So a tile whose largest weight in some
// head of the wave exceeds LO_SHARE of that head's normaliser so far also
// runs the bf16 residual of its weights (exact to ~2^-17); every other tile
// uses the high part alone, and every later weight only shrinks its share.
constexpr float LO_SHARE = 1.f / 16.f;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// One wave-wide global -> LDS load: lane L copies 16 bytes from sbase + voff
// (sbase wave-uniform) to LDS byte address lds_base + 16 L.  Issued as inline
// assembly so that the compiler does not treat every later LDS read as a
// possible alias of the in-flight copy; the caller waits (vmcnt) and
// synchronises before the destination is read.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}

// XOR mask of the 16-byte slots of dims 0..511 in tile row r (1 KB rows).  16
// aligned rows read at one chunk land on 16 distinct slots mod 16 (8 aligned
// rows on 8 distinct slots mod 8), and 8 aligned rows read at an aligned pair
// of chunks on 16 distinct slots mod 16 (4 rows on 8 mod 8).  The 16-byte
// reads of the key fragments and the transposing 8-byte reads of the value
// fragments are thus free of bank conflicts for 32 or 64 banks of 4 bytes.
__device__ __forceinline__ uint32_t main_swz(uint32_t r) {
  r &= 15;
  return 2 * (r & 7) + (((r >> 2) ^ (r >> 3)) & 1);
}
// Same for the 8 slots of dims 512..575 (128-byte rows): 16 aligned rows at one
// chunk fall on distinct slots of a 256-byte bank period, 8 on distinct slots
// of a 128-byte one.
__device__ __forceinline__ uint32_t rope_swz(uint32_t r) { return ((r & 15) ^ ((r & 15) >> 3)) & 7; }

// lane l receives the values of lanes l ^ 16 and l ^ 32 folded in: max / sum
// over the four lanes that hold one head's 32 keys; every lane of the four
// adds in the same order, so all hold the same result
__device__ __forceinline__ float quad_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// IEEE maximum (NaN-propagating): no operand canonicalisation, and three
// operands in one instruction on gfx950
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
__device__ __forceinline__ float quad_vmax(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One workgroup = one query row x one stream chunk x 128 heads, 8 waves; wave
// w owns heads 16 w .. 16 w + 15 and all 576 contraction dims.  Per tile of 32
// gathered latent rows:
//   S^T (32 keys x 16 heads) = K_tile . Q^T on 16x16x32 MFMAs (two 16-key
//       blocks), K fragments read from the LDS tile, Q in registers
//   online softmax over the 32 keys of each head (8 per lane + two lane
//       swaps); the running max is only raised when it grows by more than 2^8
//       in weight.  The weights enter the PV product as a bf16 high part,
//       plus a bf16 residual when some weight of the tile is large against
//       the running normaliser (see LO_SHARE)
//   O^T (512 dims x 16 heads) += V^T . P^T: V^T fragments come straight from
//       the key-major tile through the transposing LDS read; P^T is the S^T
//       accumulator layout, so no data moves between lanes
// Work runs in segments separated by barriers: a wave computes the scores of
// tile u, their running max and the residual decision in one segment, and
// the exponentials, the bf16 weights and the PV products in the next; waves
// 4..7 run one segment behind waves 0..3, so on every SIMD (waves w and w + 4)
// one wave's score products overlap the other wave's exponentials and PV
// products.  Tiles are gathered with direct global -> LDS loads two
// segments ahead (three tile buffers).  Token ids of the stream sit in an LDS
// ring of 32 tiles, refilled 16 tiles ahead.  HG64: a workgroup of 64 heads
// (few rows: the decode split), whose heads sit on waves 0, 1, 6 and 7, one
// computing wave per SIMD; the other four gather and synchronise only.
template <bool HG64>
__global__ __launch_bounds__(64 * MLA_WAVES, 1) void attn_mla_kernel(AttnParams p) {
  constexpr int NW = MLA_WAVES;
  constexpr int GW = NW / 2;   // waves per group
  extern __shared__ __align__(16) uint8_t s_raw[];
  uint8_t* s_kb = s_raw;                                                      // KT_NBUF tiles
  int32_t* s_tok = reinterpret_cast<int32_t*>(s_raw + KT_NBUF * KT_BYTES);   // token ring
  uint32_t* s_scr = reinterpret_cast<uint32_t*>(s_tok + TOK_RING);
  int32_t* s_blk = reinterpret_cast<int32_t*>(s_scr + 16);                   // MLA_MAX_BLOCKS

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar registers
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  const int64_t row = rows - 1 - blockIdx.x / p.n_split;     // latest (longest causal) rows first
  const int sp = blockIdx.x % p.n_split;
  const int s = static_cast<int>(row / p.n_q);
  const int grp = wid / GW;
  const int col = lane & 15, q = lane >> 4;
  // Heads per workgroup: 128 (16 a wave), or 64 (HG64) when few rows would
  // leave CUs idle.  Then waves 0, 1 (first group) and 6, 7 (second group)
  // hold the heads, one per SIMD (waves w and w + 4 share one), and the
  // other four only gather and synchronise.  A head's arithmetic does not
  // depend on the workgroup that computes it.
  const bool has_heads = !HG64 || wid < 2 || wid >= 6;
  const int slot = HG64 ? (wid < 2 ? wid : wid - 4) : wid;
  const int head0 = blockIdx.y * (HG64 ? 64 : 16 * NW) + slot * 16;
  const bool wvalid = has_heads && head0 < p.Hq;   // Hq is a multiple of 16
  const int head = head0 + col;

  // In token mode the stream is the idx row itself (its length k_sel needs no
  // load), so the row's first 2 TOK_RING entries are fetched first, then the Q
  // fragments.  Vector loads complete in issue order: the token ring waits for
  // the index entries alone while Q is still in flight, and Q lands while the
  // ring is filled and the first two tiles are gathered.
  const bool token_mode = p.idx != nullptr && p.c == 1;
  constexpr int RPT0 = TOK_RING / (64 * NW);   // ring entries per thread
  static_assert(RPT0 * 64 * NW == TOK_RING, "the ring is filled in whole passes");
  int64_t p0 = 0, p1 = 0;
  int32_t pre[2 * RPT0];
  if (token_mode) {
    split_range(p, sp, p.k_sel, &p0, &p1);
    const int32_t* ir = p.idx + row * p.k_sel;
#pragma unroll
    for (int j = 0; j < 2 * RPT0; ++j) {
      const int64_t e = p0 + tid + 64 * NW * j;
      pre[j] = e < p1 ? ir[e] : -1;
    }
  }

  // Contraction step ks takes four 8-dim chunks, one per lane group q: for
  // ks < 16 chunk 16 (ks >> 2) + 4 q + (ks & 3), for ks = 16, 17 the rope chunk
  // 64 + 2 q + ks - 16 (a fixed permutation of the 576 dims, the same for K and
  // Q; this spread keeps the 16-byte LDS reads free of bank conflicts).
  // Q^T fragments: lane (head col, q) holds the 8 dims of its chunk (147 KB
  // per row), issued behind the index entries.  The loads are unconditional,
  // so that the wait before the ring counts exactly; a wave without heads
  // (Hq < 128) loads head 0's query in every column, and its outputs are
  // never written.
  u32x4_t qf[18];
  {
    const uint16_t* qr = static_cast<const uint16_t*>(p.q) + (row * p.Hq + (wvalid ? head : 0)) * MLA_DK;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const int chunk = ks < 16 ? 16 * (ks >> 2) + 4 * q + (ks & 3) : 64 + 2 * q + (ks - 16);
      qf[ks] = *reinterpret_cast<const u32x4_t*>(qr + 8 * chunk);
    }
  }

  const StreamInfo si = stream_setup<NW>(p, row, s_blk, s_scr);
  if (!token_mode) split_range(p, sp, si.len, &p0, &p1);
  // The token ring takes the first TOK_RING stream entries.  In token mode
  // the trailing dead entries (the -1 padding of short selections) are cut
  // off in the same pass over the index row; they would add nothing.
  uint32_t last = 0;   // 1 + offset of the last live entry
#pragma unroll
  for (int j = 0; j < RPT0; ++j) {
    const int i = tid + 64 * NW * j;
    int32_t t;
    if (token_mode) t = pre[j] >= 0 && pre[j] < si.n_vis ? pre[j] : -1;
    else t = p0 + i < p1 ? static_cast<int32_t>(stream_token(p, row, si, s_blk, p0 + i)) : -1;
    s_tok[i] = t;
    if (t >= 0) last = static_cast<uint32_t>(i + 1);
  }
  const bool trim = token_mode && p1 > p0;
  if (trim) {
#pragma unroll
    for (int j = RPT0; j < 2 * RPT0; ++j)
      if (pre[j] >= 0 && pre[j] < si.n_vis) last = static_cast<uint32_t>(tid + 64 * NW * j + 1);
    const int32_t* ir = p.idx + row * p.k_sel;
    for (int64_t e = p0 + 2 * TOK_RING + tid; e < p1; e += 64 * NW) {
      const int32_t v = ir[e];
      if (v >= 0 && v < si.n_vis) last = static_cast<uint32_t>(e - p0 + 1);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) last = max(last, static_cast<uint32_t>(__shfl_xor(static_cast<int>(last), o, 64)));
    if (lane == 0) s_scr[8 + wid] = last;
  }
  __syncthreads();   // the ring and the per-wave ends
  if (trim) {
    uint32_t e = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) e = max(e, s_scr[8 + w]);
    p1 = p0 + e;
  }
  const int n_tiles = p1 > p0 ? static_cast<int>((p1 - p0 + TILE - 1) / TILE) : 0;

  // o[db]: O^T dims 16 db + 4 q + j of head `head`; o[32]: the head's
  // normaliser in every register, the product of the weights with a block of
  // ones, so that it sums exactly the bf16 weights the value products take
  f32x4_t o[33];
#pragma unroll
  for (int db = 0; db < 33; ++db) o[db] = f32x4_t{};
  const u32x4_t ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};   // bf16 1.0 pairs
  float m_run = NEG_INF;
  const float c2 = p.scale_log2;

  const uint32_t kb_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)s_kb));
  const char* kseq_b = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.k) + s * p.k_seq);
  const uint64_t pitch = static_cast<uint64_t>(p.k_tok) * 2u;   // bytes per token row
  auto tokens_of = [&](int u) __attribute__((always_inline)) -> int32_t {
    return s_tok[(u * TILE + (lane & 31)) & (TOK_RING - 1)];
  };
  // Each group gathers its part of a tile in its score segments, spread
  // between the products (a load stalls the wave that issues it; the other
  // group's products keep the SIMD busy meanwhile).  Wave l of the second
  // group loads the 1 KB main parts of rows l, l + GW, ... below 16 and the
  // rope parts of rows (32 / GW) l .. (32 / GW) (l + 1) - 1 of tile u + 2 in
  // segment 2 u + 1; wave l of the first group loads the main parts of rows
  // 16 + l, 16 + l + GW, ... of tile u + 1 in segment 2 u.  A group waits
  // for its own loads at the end of the next segment (the second group at
  // even segment ends, the first at odd ones).  The token ids come in a
  // register read from the ring beforehand: lane r of tl holds the token of
  // row r.
  const int gl = wid % GW;
  constexpr int N_MAIN = 16 / GW;   // main-part loads per wave and half tile
  constexpr int N_ROPE = 4 / GW;    // rope loads per wave and tile (8 rows each)
  auto gather_main = [&](int r, int32_t tl, uint32_t lb, int ln) __attribute__((always_inline)) {
    const int32_t tk = __builtin_amdgcn_readlane(tl, r);
    const char* src = kseq_b + static_cast<uint64_t>(tk > 0 ? tk : 0) * pitch;
    dma16(src, (16u * ln) ^ (16u * main_swz(r)), lb + 1024u * r);
  };
  auto gather_rope = [&](int j, int32_t tl, uint32_t lb, int ln) __attribute__((always_inline)) {
    const int g8 = N_ROPE * gl + j;   // rows 8 g8 .. 8 g8 + 7
    const uint32_t rr = 8 * g8 + (ln >> 3);
    const int32_t t8 = __shfl(tl, static_cast<int>(rr), 64);
    const uint32_t voff = static_cast<uint32_t>(t8 > 0 ? t8 : 0) * static_cast<uint32_t>(pitch) + 1024u +
                          16u * ((ln & 7) ^ rope_swz(rr));
    dma16(kseq_b, voff, lb + KT_MAIN + 1024u * g8);
  };
  // load c of a wave's share of one tile: the second group (plan 1) takes
  // N_MAIN main rows below 16, then N_ROPE rope loads; the first group
  // (plan 2) N_MAIN main rows from 16
  auto gather_c = [&](auto plan, int c, int32_t tl, uint32_t lb, int ln) __attribute__((always_inline)) {
    if constexpr (decltype(plan)::value == 1) {
      if (c < N_MAIN) gather_main(gl + GW * c, tl, lb, ln);
      else gather_rope(c - N_MAIN, tl, lb, ln);
    } else {
      gather_main(16 + gl + GW * c, tl, lb, ln);
    }
  };
  auto live_of = [&](int u) __attribute__((always_inline)) -> uint32_t {
    return static_cast<uint32_t>(__ballot(tokens_of(u) >= 0));
  };

  // K fragment of key block mb, contraction step ks: lane (col, q) reads its
  // chunk of tile row 16 mb + col, at (cs ^ 16 (ks & 3)) + 256 (ks >> 2)
  // + 16 KB mb (main part, ks < 16) or (cr ^ 16 (ks - 16)) + 2 KB mb (rope);
  // the xor terms only touch bits 4..5
  const uint32_t cs = col * 1024u + ((64u * q) ^ (16u * main_swz(col)));
  const uint32_t cr = KT_MAIN + col * 128u + ((32u * q) ^ (16u * rope_swz(col)));
  constexpr int SD = 4;   // K fragments read ahead (products in the order ks, mb)
  // scores of the tile in buffer bs, for key blocks 0 and 1
  auto scores = [&](auto with_gather, int bs, f32x4_t& s0, f32x4_t& s1, int32_t tl,
                    int bg) __attribute__((always_inline)) {
    uint32_t xs = cs, xr = cr;
    int ln = lane;
    asm volatile("" : "+v"(xs), "+v"(xr), "+v"(ln));   // a few bases per tile, not 36 live offsets
    const uint32_t lb = kb_lds + bg * KT_BYTES;
    const uint8_t* kt = s_kb + bs * KT_BYTES;
    auto frag = [&](int i) __attribute__((always_inline)) -> u32x4_t {
      const int ks = i >> 1, mb = i & 1;
      const uint8_t* ad = ks < 16 ? kt + (xs ^ (16u * (ks & 3))) + 256 * (ks >> 2) + 16384 * mb
                                  : kt + (xr ^ (16u * (ks - 16))) + 2048 * mb;
      return *reinterpret_cast<const u32x4_t*>(ad);
    };
    u32x4_t kf[SD];
#pragma unroll
    for (int i = 0; i < SD; ++i) kf[i] = frag(i);
    __builtin_amdgcn_sched_group_barrier(0x100, SD, 0);   // the first SD LDS reads lead
    s0 = f32x4_t{};
    s1 = f32x4_t{};
#pragma unroll
    for (int i = 0; i < 36; ++i) {
      if (i & 1) s1 = mfma16x16x32_bf16(kf[i % SD], qf[i >> 1], s1);
      else s0 = mfma16x16x32_bf16(kf[i % SD], qf[i >> 1], s0);
      if (i + SD < 36) kf[i % SD] = frag(i + SD);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // then one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // and one LDS read, in turn
      // the group's loads, spread evenly over the 36 products
      constexpr int plan = decltype(with_gather)::value;   // 0: none, 1: second group, 2: first group
      if constexpr (plan != 0) {
        constexpr int NL = plan == 1 ? N_MAIN + N_ROPE : N_MAIN;
        if ((i + 1) * NL / 36 != i * NL / 36) gather_c(with_gather, (i + 1) * NL / 36 - 1, tl, lb, ln);
      }
    }
  };
  // a wave without heads (64-head workgroups): its share of the gather alone
  auto gather_only = [&](auto plan, int32_t tl, int bg) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const uint32_t lb = kb_lds + bg * KT_BYTES;
    constexpr int NL = decltype(plan)::value == 1 ? N_MAIN + N_ROPE : N_MAIN;
#pragma unroll
    for (int c = 0; c < NL; ++c) gather_c(plan, c, tl, lb, ln);
  };
  // softmax: s_mb reg j holds key 16 mb + 4 q + j of head col.  Produces the
  // P^T fragments (k slot j < 4: key 4 q + j; j >= 4: key 16 + 4 q + j - 4)
  // and returns the factor that rescales what was accumulated before.
  // online softmax, first half (in the score segment): masks dead entries,
  // moves the running max, decides the residual pass, and returns the factor
  // that rescales what was accumulated before; the exponent offset goes to mb
  auto softmax_a = [&](f32x4_t& s0, f32x4_t& s1, uint32_t live, float& mb, bool& need_lo)
                       __attribute__((always_inline)) -> float {
    if (live != 0xffffffffu) {
      const uint32_t lm = live >> (4 * q);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!((lm >> j) & 1u)) s0[j] = NEG_INF;
        if (!((lm >> (16 + j)) & 1u)) s1[j] = NEG_INF;
      }
    }
    float tmax = vmax3(vmax3(s0[0], s0[1], s0[2]), vmax3(s0[3], s1[0], s1[1]), vmax3(s1[2], s1[3], NEG_INF));
    tmax = quad_vmax(tmax);
    const bool first = m_run == NEG_INF;
    const bool grow = !first && (tmax - m_run) * c2 > 8.f;
    float alpha = 1.f;   // the rescale factor, computed only when some head's max moves
    if (__ballot(grow) != 0) {
      asm volatile("" ::: "memory");   // not speculated into the common path
      const float a = __builtin_amdgcn_exp2f((m_run - tmax) * c2);
      alpha = grow ? a : 1.f;
    }
    m_run = (first || grow) ? tmax : m_run;
    mb = m_run == NEG_INF ? 0.f : m_run * c2;   // an all-dead prefix gives zero weights
    const float xmax = __builtin_amdgcn_exp2f(fmaf(tmax, c2, -mb));   // the head's largest weight in the tile
    need_lo = __ballot(xmax * (1.f - LO_SHARE) > LO_SHARE * o[32][0] * alpha) != 0;   // wave-uniform
    return alpha;
  };
  // second half (in the PV segment): the weights as bf16 high parts, and
  // their residual when the tile runs the residual pass
  auto softmax_b = [&](f32x4_t s0, f32x4_t s1, float mb, bool need_lo, u32x4_t& ph, u32x4_t& pl)
                       __attribute__((always_inline)) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = __builtin_amdgcn_exp2f(fmaf(s0[j], c2, -mb));
      x[4 + j] = __builtin_amdgcn_exp2f(fmaf(s1[j], c2, -mb));
    }
    uint32_t hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    ph = u32x4_t{hv[0], hv[1], hv[2], hv[3]};
    if (need_lo) {
      uint32_t lv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lv[i] = pack_bf16x2(x[2 * i] - __uint_as_float(hv[i] << 16), x[2 * i + 1] - __uint_as_float(hv[i] & 0xffff0000u));
      pl = u32x4_t{lv[0], lv[1], lv[2], lv[3]};
    }
  };
  auto rescale = [&](float alpha) __attribute__((always_inline)) {
    if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
      for (int db = 0; db < 33; ++db) o[db] *= alpha;
    }
  };
  // V^T fragment of dim block db: lane (q, source slot 4 m + r) addresses key
  // 4 q + m (then 16 + 4 q + m), dims 16 db + 4 r; the transposing read hands
  // lane j of each 16-lane group dim 16 db + j of those four keys.  Tile
  // offset: (cv ^ 32 (db & 7)) + 256 (db >> 3) (+ 16 KB for the second read),
  // the xor touching bits 5..7.
  uint32_t cv;
  {
    const uint32_t m4 = (lane >> 2) & 3, r4 = lane & 3, R = 4 * q + m4, f = main_swz(R);
    cv = R * 1024 + 16 * ((r4 >> 1) ^ (f & 1)) + 16 * (f & 14) + 8 * (r4 & 1);
  }
  constexpr int VD = 3;   // V^T fragments read ahead
  // one pass of O^T += V^T . P^T over the 32 dim blocks, P^T = the weights'
  // high part or (a second pass over the same tile) their residual
  auto pv = [&](int bp, const u32x4_t& pw) __attribute__((always_inline)) {
    uint32_t x1 = cv;
    asm volatile("" : "+v"(x1));
    uint8_t* kt = s_kb + bp * KT_BYTES;
    auto vfrag = [&](int db) __attribute__((always_inline)) -> u32x4_t {
      uint8_t* ad = kt + (x1 ^ (32u * (db & 7))) + 256 * (db >> 3);
      const v4i16_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)ad);
      const v4i16_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(ad + 16384));
      const u32x2_t a2 = __builtin_bit_cast(u32x2_t, a), b2 = __builtin_bit_cast(u32x2_t, b);
      return u32x4_t{a2.x, a2.y, b2.x, b2.y};
    };
    u32x4_t vf[VD];
#pragma unroll
    for (int i = 0; i < VD; ++i) vf[i] = vfrag(i);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * VD, 0);
    o[32] = mfma16x16x32_bf16(ones, pw, o[32]);
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      o[db] = mfma16x16x32_bf16(vf[db % VD], pw, o[db]);
      if (db + VD < 32) vf[db % VD] = vfrag(db + VD);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // the first two tiles
  __syncthreads();   // token ring filled
  // All waves load the main parts (wave w: rows w, w + NW, ...), so that
  // each issues half the loads (a load stalls the wave that issues it); the
  // second group also loads the rope parts.
  int32_t g_tl = 0;   // token ids of the next tile to gather (second group)
  {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    for (int u = 0; u < 2 && u < n_tiles; ++u) {
      const int32_t tl = tokens_of(u);
#pragma unroll
      for (int k = 0; k < 32 / NW; ++k) gather_main(wid + NW * k, tl, kb_lds + u * KT_BYTES, ln);
      if (grp == 1) {
#pragma unroll
        for (int j = 0; j < N_ROPE; ++j) gather_rope(j, tl, kb_lds + u * KT_BYTES, ln);
      }
    }
    if (grp == 1 && n_tiles > 2) g_tl = tokens_of(2);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
  __syncthreads();

  // token ring refill: entries of tiles 16 j + 16 .. 16 j + 31 are fetched in
  // segment 32 j + 1, land by the wait that closes segment 32 j + 2, and are
  // validated and stored in segment 32 j + 3, into the slots of tiles
  // 16 j - 16 .. 16 j - 1, which segment 32 j read last
  constexpr int RPT = 16 * TILE / (64 * NW);   // refill entries per thread
  int32_t ring_v[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) ring_v[i] = -1;
  // the part of segment sg that every wave does: its share of the ring refill
  auto segment_io = [&](int sg) __attribute__((always_inline)) {
    const int m = sg >> 1;
    if ((sg & 31) == 1 && sg > 32 && m + 16 < n_tiles) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int64_t pos = p0 + static_cast<int64_t>(m + 16) * TILE + tid + 64 * NW * i;
        if (token_mode) ring_v[i] = p.idx[row * p.k_sel + (pos < p1 ? pos : p1 - 1)];
        else ring_v[i] = pos < p1 ? static_cast<int32_t>(stream_token(p, row, si, s_blk, pos)) : -1;
      }
    }
    if ((sg & 31) == 3 && sg > 32 && m + 15 < n_tiles) {
      const int base = (m + 15) * TILE;   // m + 15 = 16 j + 16
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int e = tid + 64 * NW * i;
        const int64_t pos = p0 + base + e;
        int32_t v = ring_v[i];
        if (pos >= p1) v = -1;
        else if (token_mode && !(v >= 0 && v < si.n_vis)) v = -1;
        s_tok[(base + e) & (TOK_RING - 1)] = v;
      }
    }
  };
  auto segment_end = [&](int sg) __attribute__((always_inline)) {
    if ((sg & 1) == (grp == 0 ? 1 : 0)) __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this group's loads have landed
    __syncthreads();
  };
  // accumulator (db, j) holds dim 16 db + 4 q + j of head `head`
  auto write_out = [&]() __attribute__((always_inline)) {
    if (!(wvalid && head < p.Hq)) return;
    if (p.n_split == 1) {
      const float inv = o[32][0] > 0.f ? 1.f / o[32][0] : 0.f;
      const int64_t ob = (row * p.Hq + head) * MLA_DV + 4 * q;
#pragma unroll
      for (int db = 0; db < 32; ++db)
        store4(p.out, p.o_dtype, ob + 16 * db, o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
    } else {
      float* pp = p.part + ((row * p.n_split + sp) * p.Hq + head) * part_width(MLA_DV);
#pragma unroll
      for (int db = 0; db < 32; ++db)
        *reinterpret_cast<f32x4_t*>(pp + 16 * db + 4 * q) = o[db];
      if (q == 0) {
        pp[MLA_DV] = m_run;
        pp[MLA_DV + 1] = o[32][0];
      }
    }
  };

  // Segment sg: waves 0..3 compute the scores and softmax of tile sg / 2
  // (even sg) or its PV products (odd sg); waves 4..7 do the same one segment
  // later.  Waves without heads in a 128-head workgroup (Hq < 128) run the
  // same products on head 0's query, so that every wave takes the same
  // straight-line path; in a 64-head workgroup the four waves without heads
  // run a loop of their own that issues their gather share and meets the
  // same barriers.
  using plan_hi = std::integral_constant<int, 1>;   // the gather share of waves 4..7
  using plan_lo = std::integral_constant<int, 2>;   // the gather share of waves 0..3
  if (grp == 0) {
    if (!HG64 || has_heads) {
      for (int u = 0; u < n_tiles; ++u) {
        segment_io(2 * u);
        f32x4_t s0, s1;
        u32x4_t ph, pl;
        bool need_lo;
        float mb;
        // tile u + 1 past tile 1 (the first two come whole from the prologue;
        // at u = 0 this reloads rows of tile 1 with the same bytes, and past
        // the stream it loads rows nothing reads)
        __builtin_amdgcn_s_setprio(2);   // the score chain first; the other group's PV fills the gaps
        scores(plan_lo{}, u % KT_NBUF, s0, s1, tokens_of(u + 1), (u + 1) % KT_NBUF);
        rescale(softmax_a(s0, s1, live_of(u), mb, need_lo));
        __builtin_amdgcn_s_setprio(0);
        segment_end(2 * u);
        segment_io(2 * u + 1);
        softmax_b(s0, s1, mb, need_lo, ph, pl);
        u32x4_t pw = ph;
#pragma clang loop unroll(disable)
        for (int ps = 0; ps < 1 + need_lo; ++ps) {
          pv(u % KT_NBUF, pw);
          pw = pl;
        }
        segment_end(2 * u + 1);
      }
    } else {
      for (int u = 0; u < n_tiles; ++u) {
        segment_io(2 * u);
        gather_only(plan_lo{}, tokens_of(u + 1), (u + 1) % KT_NBUF);
        segment_end(2 * u);
        segment_io(2 * u + 1);
        segment_end(2 * u + 1);
      }
    }
    // the last segment is the other group's last PV: this group's outputs
    // are final and are written meanwhile
    segment_io(2 * n_tiles);
    write_out();
    segment_end(2 * n_tiles);
  } else {
    segment_io(0);
    segment_end(0);
    if (!HG64 || has_heads) {
      for (int u = 0; u < n_tiles; ++u) {
        // the gather of tile u + 2 also runs past the end: it then reloads rows
        // (ring entries past the stream: token 0 or stale valid ids) into the
        // buffer of tile u - 1, which nothing reads again
        segment_io(2 * u + 1);
        f32x4_t s0, s1;
        u32x4_t ph, pl;
        bool need_lo;
        float mb;
        __builtin_amdgcn_s_setprio(2);
        scores(plan_hi{}, u % KT_NBUF, s0, s1, g_tl, (u + 2) % KT_NBUF);
        rescale(softmax_a(s0, s1, live_of(u), mb, need_lo));
        __builtin_amdgcn_s_setprio(0);
        segment_end(2 * u + 1);
        segment_io(2 * u + 2);
        g_tl = tokens_of(u + 3);   // for the next score segment
        softmax_b(s0, s1, mb, need_lo, ph, pl);
        u32x4_t pw = ph;
#pragma clang loop unroll(disable)
        for (int ps = 0; ps < 1 + need_lo; ++ps) {
          pv(u % KT_NBUF, pw);
          pw = pl;
        }
        segment_end(2 * u + 2);
      }
    } else {
      for (int u = 0; u < n_tiles; ++u) {
        segment_io(2 * u + 1);
        gather_only(plan_hi{}, g_tl, (u + 2) % KT_NBUF);
        segment_end(2 * u + 1);
        segment_io(2 * u + 2);
        g_tl = tokens_of(u + 3);
        segment_end(2 * u + 2);
      }
    }
  }
  if (grp == 1) write_out();
}

// ========================================================= MLA, q8_0 rows ==

// The latent rows as q8_0 (ik_llama_opt log, openPangu port, "Add OpenPangu
// q8_0 latent cache type": int8 codes, one f16 scale per 32 values; 612 bytes
// a row against 1152 in bf16).  Layout: codes [S, n_kv, 576] int8 at the K
// strides (bytes), scales [S, n_kv, 18] f16, contiguous.
//
// Precision.  A dequantised value c s (a 7-bit code times an 11-bit scale)
// carries up to 18 significant bits: bf16 (8) or f16 (11) alone would lose
// the score accuracy of bf16 rows (rows with outliers magnify a key error
// through the softmax).  Scores take it exactly, as the sum of hi = f16(c s)
// and lo = c s - hi (the residual is a multiple of the scale's last bit below
// half an ulp of hi: an f16 value, exact).  Queries enter as f16, each head's
// scaled by the power of two that puts its largest component in [2^14, 2^15)
// (exact for components down to 2^-24 of the largest); the factor is folded
// back into that head's softmax scale and running max.  Values take hi alone
// (relative error 2^-12), the weights f16 with attn_mla_kernel's residual
// rule.  The dequantised values must lie in the f16 range (|c s| <= 65504,
// so scales up to 515).
constexpr int Q8_BLOCKS = MLA_DK / 32;                     // scales per row
constexpr int Q8_STAGE = TILE * MLA_DK;                    // one tile's codes (18 KB)
// one tile's scales: 9 dwords a row, 288 in all, loaded by 5 whole waves
// (each lane writes its own dword; the last 32 lanes' land past the 288)
constexpr int Q8_SSTAGE = (TILE * 9 + 63) / 64 * 256;
// tile of hi values, tile of lo values (attn_mla_kernel's layout each), code
// and scale staging, token ids of three tiles
constexpr size_t MLA_Q8_LDS = 2 * KT_BYTES + Q8_STAGE + Q8_SSTAGE + 3 * TILE * 4 + 64 + MLA_MAX_BLOCKS * 4;

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// One lane-wide global -> LDS load of 4 bytes (lane L: lds_base + 4 L), as dma16.
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}

// 16 codes (4 per dword) and their f16 scale s -> hi = f16(c s) and
// lo = f16(c s - hi), 8 dims per u32x4 (h0, l0: dims 0..7; h1, l1: 8..15).
// A code byte c, offset to c + 128 and placed under the f16 exponent of 1024,
// reads as 1024 + c + 128; taking 1152 off gives c exactly.  The product is
// rounded once, and the fused residual is exact.
__device__ __forceinline__ void q8_split16(u32x4_t c, uint16_t sbits, u32x4_t& h0, u32x4_t& h1, u32x4_t& l0,
                                           u32x4_t& l1) {
#pragma clang fp contract(off)
  const _Float16 sh = __builtin_bit_cast(_Float16, sbits);
  const f16x2_t s2 = {sh, sh};
  const f16x2_t bias = {static_cast<_Float16>(1152.f), static_cast<_Float16>(1152.f)};
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = w[i] ^ 0x80808080u;
    const uint32_t e[2] = {__builtin_amdgcn_perm(0x64646464u, x, 0x04010400u),    // codes 0, 1
                           __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u)};   // codes 2, 3
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f16x2_t cv = __builtin_bit_cast(f16x2_t, e[j]) - bias;
      const f16x2_t hv = cv * s2;
      const f16x2_t lv = __builtin_elementwise_fma(cv, s2, -hv);
      h[2 * i + j] = __builtin_bit_cast(uint32_t, hv);
      l[2 * i + j] = __builtin_bit_cast(uint32_t, lv);
    }
  }
  h0 = u32x4_t{h[0], h[1], h[2], h[3]};
  h1 = u32x4_t{h[4], h[5], h[6], h[7]};
  l0 = u32x4_t{l[0], l[1], l[2], l[3]};
  l1 = u32x4_t{l[4], l[5], l[6], l[7]};
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}

// One workgroup = one query row x one stream chunk x 128 heads, 8 waves of 16
// heads, as attn_mla_kernel, for q8_0 latent rows.  Per tile of 32 stream
// entries: the codes and scales of the next tile go straight to LDS staging
// areas (direct global -> LDS loads) while the tile in LDS is computed; after
// the barrier that ends the tile's products they are split into hi and lo
// f16 tiles (see above) over it, and a second barrier completes them.
// Scores run on f16 MFMAs over hi and lo (72 per wave and tile), the PV
// products over hi with f16 weights; the contraction order, the online
// softmax (lazy running max, weights plus their residual on tiles where one
// weight is large against the normaliser) and the output follow
// attn_mla_kernel, in one wave group.  Token ids of tile u + 2 are fetched
// during tile u.
__global__ __launch_bounds__(64 * MLA_WAVES, 1) void attn_mla_q8_kernel(AttnParams p) {
  constexpr int NW = MLA_WAVES;
  extern __shared__ __align__(16) uint8_t s_raw[];
  uint8_t* s_kb = s_raw;                                                     // hi tile, then lo tile
  uint8_t* s_st = s_raw + 2 * KT_BYTES;                                     // code staging (Q8_STAGE)
  const uint16_t* s_ss = reinterpret_cast<const uint16_t*>(s_st + Q8_STAGE); // scale staging: row r at 18 r
  int32_t* s_tk = reinterpret_cast<int32_t*>(s_st + Q8_STAGE + Q8_SSTAGE);  // token ids of 3 tiles
  uint32_t* s_scr = reinterpret_cast<uint32_t*>(s_tk + 3 * TILE);
  int32_t* s_blk = reinterpret_cast<int32_t*>(s_scr + 16);                  // MLA_MAX_BLOCKS

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  const int64_t row = rows - 1 - blockIdx.x / p.n_split;   // latest (longest causal) rows first
  const int sp = blockIdx.x % p.n_split;
  const int s = static_cast<int>(row / p.n_q);
  const int col = lane & 15, q = lane >> 4;
  const int head0 = blockIdx.y * (16 * NW) + wid * 16;
  const bool wvalid = head0 < p.Hq;
  const int head = head0 + col;

  // Q^T fragments in attn_mla_kernel's permutation (a wave without heads
  // loads head 0's query; its outputs are never written), as f16 of the
  // query times 2^qk, qk from the head's largest |component| (the four
  // lanes col + 16 q hold all 576 dims of head col)
  u32x4_t qf[18];
  int qk;
  {
    const uint16_t* qr = static_cast<const uint16_t*>(p.q) + (row * p.Hq + (wvalid ? head : 0)) * MLA_DK;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const int chunk = ks < 16 ? 16 * (ks >> 2) + 4 * q + (ks & 3) : 64 + 2 * q + (ks - 16);
      qf[ks] = *reinterpret_cast<const u32x4_t*>(qr + 8 * chunk);
    }
    uint32_t m = 0;   // largest bf16 magnitude (bits), monotone in the value
#pragma unroll
    for (int ks = 0; ks < 18; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = max(m, max(qf[ks][i] & 0x7fffu, (qf[ks][i] >> 16) & 0x7fffu));
    m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 16, 64)));
    m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 32, 64)));
    // largest component 2^E (1 + f), E = (m >> 7) - 127: scale by 2^(14 - E)
    qk = m == 0 ? 0 : min(141 - static_cast<int>(m >> 7), 64);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      u32x4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = pack_h2(__builtin_amdgcn_ldexpf(__uint_as_float(qf[ks][i] << 16), qk),
                       __builtin_amdgcn_ldexpf(__uint_as_float(qf[ks][i] & 0xffff0000u), qk));
      qf[ks] = v;
    }
  }
  const float c2 = __builtin_amdgcn_ldexpf(p.scale_log2, -qk);   // scores arrive times 2^qk
  const StreamInfo si = stream_setup<NW>(p, row, s_blk, s_scr);
  int64_t p0, p1;
  split_range(p, sp, si.len, &p0, &p1);
  const int n_tiles = p1 > p0 ? static_cast<int>((p1 - p0 + TILE - 1) / TILE) : 0;

  const int8_t* kseq = static_cast<const int8_t*>(p.k) + s * p.k_seq;
  const uint16_t* sseq = static_cast<const uint16_t*>(p.k_scale) + static_cast<int64_t>(s) * p.n_kv * Q8_BLOCKS;
  // token id of stream entry r of tile u (-1: dead or past the chunk); tile
  // v's ids sit in s_tk[v % 3], written by wave 0 one tile ahead of the loads
  auto tok = [&](int u, int r) __attribute__((always_inline)) -> int32_t {
    const int64_t pos = p0 + static_cast<int64_t>(u) * TILE + r;
    return pos < p1 ? static_cast<int32_t>(stream_token(p, row, si, s_blk, pos)) : -1;
  };
  // The codes and scales of a tile go straight to LDS staging areas (direct
  // global -> LDS loads; no registers held across the products): code chunk c
  // (16 bytes) at 16 c, in the order main chunks t (rows t / 32, dims
  // 16 (t % 32) ..) and t + 512 (rows + 16), then rope chunks 1024 + t (t <
  // 128: row t / 4, dims 512 + 16 (t % 4) ..); scale dword d of row r (the
  // row's 18 scales are 9 dwords) at 4 (9 r + d).  Wave w, load i, lane L
  // fetches chunk 512 i + 64 w + L.  Dead entries read row 0 (their weights
  // are zero).
  const uint8_t* sbytes = reinterpret_cast<const uint8_t*>(sseq);
  const uint32_t st_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)s_st));
  const uint32_t pitch = static_cast<uint32_t>(p.k_tok);   // bytes per latent row
  auto load_stage = [&](int u) __attribute__((always_inline)) {
    int t = tid;
    asm volatile("" : "+v"(t));   // addresses from tid at each use, not held across the loop
    const int32_t* tk = s_tk + (u % 3) * TILE;
    const int32_t a = tk[t >> 5], b = tk[(t >> 5) + 16], r = tk[(t >> 2) & 31];
    const uint32_t ta = a > 0 ? a : 0, tb = b > 0 ? b : 0, tr = r > 0 ? r : 0;
    const uint32_t c = t & 31, rcc = t & 3;
    dma16(kseq, ta * pitch + 16u * c, __builtin_amdgcn_readfirstlane(st_lds + 1024u * wid));
    dma16(kseq, tb * pitch + 16u * c, __builtin_amdgcn_readfirstlane(st_lds + 1024u * (8 + wid)));
    if (wid < 2) dma16(kseq, tr * pitch + 512u + 16u * rcc, __builtin_amdgcn_readfirstlane(st_lds + 1024u * (16 + wid)));
    if (wid < (TILE * 9 + 63) / 64) {   // 288 scale dwords
      const int d = (t < TILE * 9 ? t : TILE * 9 - 1), sr = d / 9, sj = d % 9;
      const int32_t ts = tk[sr];
      const uint32_t tsu = ts > 0 ? ts : 0;
      dma4(sbytes, tsu * (Q8_BLOCKS * 2u) + 4u * sj, __builtin_amdgcn_readfirstlane(st_lds + Q8_STAGE + 256u * wid));
    }
  };
  // the staged tile, split, into the hi and lo tiles: main row r keeps its
  // 16-byte chunk c (dims 8 c ..) in slot c ^ main_swz(r), rope row r its
  // chunk c in slot c ^ rope_swz(r)
  auto store_stage = [&]() __attribute__((always_inline)) {
    int t = tid;
    asm volatile("" : "+v"(t));
    const int ra = t >> 5, c = t & 31, rb = ra + 16, rw = (t >> 2) & 31, rcc = t & 3;
    u32x4_t h0, h1, l0, l1;
    auto put = [&](uint32_t o0, uint32_t o1) __attribute__((always_inline)) {
      *reinterpret_cast<u32x4_t*>(s_kb + o0) = h0;
      *reinterpret_cast<u32x4_t*>(s_kb + o1) = h1;
      *reinterpret_cast<u32x4_t*>(s_kb + KT_BYTES + o0) = l0;
      *reinterpret_cast<u32x4_t*>(s_kb + KT_BYTES + o1) = l1;
    };
    q8_split16(*reinterpret_cast<const u32x4_t*>(s_st + 16 * t), s_ss[Q8_BLOCKS * ra + (c >> 1)], h0, h1, l0, l1);
    put(ra * 1024 + 16 * ((2 * c) ^ main_swz(ra)), ra * 1024 + 16 * ((2 * c + 1) ^ main_swz(ra)));
    q8_split16(*reinterpret_cast<const u32x4_t*>(s_st + 16 * (512 + t)), s_ss[Q8_BLOCKS * rb + (c >> 1)], h0, h1, l0,
               l1);
    put(rb * 1024 + 16 * ((2 * c) ^ main_swz(rb)), rb * 1024 + 16 * ((2 * c + 1) ^ main_swz(rb)));
    if (wid < 2) {
      q8_split16(*reinterpret_cast<const u32x4_t*>(s_st + 16 * (1024 + t)), s_ss[Q8_BLOCKS * rw + 16 + (rcc >> 1)],
                 h0, h1, l0, l1);
      put(KT_MAIN + rw * 128 + 16 * ((2 * rcc) ^ rope_swz(rw)), KT_MAIN + rw * 128 + 16 * ((2 * rcc + 1) ^ rope_swz(rw)));
    }
  };

  f32x4_t o[32];
#pragma unroll
  for (int db = 0; db < 32; ++db) o[db] = f32x4_t{};
  float m_run = NEG_INF, l_run = 0.f;

  // K fragment of key block mb, contraction step ks (attn_mla_kernel's
  // addressing; + KT_BYTES for the lo tile)
  const uint32_t cs = col * 1024u + ((64u * q) ^ (16u * main_swz(col)));
  const uint32_t cr = KT_MAIN + col * 128u + ((32u * q) ^ (16u * rope_swz(col)));
  auto scores = [&](f32x4_t& s0, f32x4_t& s1) __attribute__((always_inline)) {
    uint32_t xs = cs, xr = cr;
    asm volatile("" : "+v"(xs), "+v"(xr));
    auto frag = [&](int i) __attribute__((always_inline)) -> u32x4_t {
      const int ks = i >> 2, mb = (i >> 1) & 1, lo = i & 1;
      const uint8_t* ad = ks < 16 ? s_kb + (xs ^ (16u * (ks & 3))) + 256 * (ks >> 2) + 16384 * mb
                                  : s_kb + (xr ^ (16u * (ks - 16))) + 2048 * mb;
      return *reinterpret_cast<const u32x4_t*>(ad + lo * KT_BYTES);
    };
    constexpr int SD = 2;   // K fragments read ahead
    u32x4_t kf[SD];
#pragma unroll
    for (int i = 0; i < SD; ++i) kf[i] = frag(i);
    s0 = f32x4_t{};
    s1 = f32x4_t{};
    // product i: step i / 4, key block (i / 2) & 1, hi (i even) or lo
#pragma unroll
    for (int i = 0; i < 72; ++i) {
      if ((i >> 1) & 1) s1 = mfma16x16x32_f16(kf[i % SD], qf[i >> 2], s1);
      else s0 = mfma16x16x32_f16(kf[i % SD], qf[i >> 2], s0);
      if (i + SD < 72) kf[i % SD] = frag(i + SD);
    }
  };
  // online softmax of the tile (attn_mla_kernel's rule, f16 weights);
  // returns the factor that rescales what was accumulated before
  auto softmax = [&](f32x4_t s0, f32x4_t s1, uint32_t live, u32x4_t& ph, u32x4_t& pl,
                     bool& need_lo) __attribute__((always_inline)) -> float {
    if (live != 0xffffffffu) {
      const uint32_t lm = live >> (4 * q);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!((lm >> j) & 1u)) s0[j] = NEG_INF;
        if (!((lm >> (16 + j)) & 1u)) s1[j] = NEG_INF;
      }
    }
    float tmax = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])), fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    tmax = quad_max(tmax);
    const bool first = m_run == NEG_INF;
    const bool grow = !first && (tmax - m_run) * c2 > 8.f;
    const float a = __builtin_amdgcn_exp2f((m_run - tmax) * c2);
    const float alpha = grow ? a : 1.f;
    m_run = (first || grow) ? tmax : m_run;
    const float mb = m_run == NEG_INF ? 0.f : m_run * c2;
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = __builtin_amdgcn_exp2f(fmaf(s0[j], c2, -mb));
      x[4 + j] = __builtin_amdgcn_exp2f(fmaf(s1[j], c2, -mb));
    }
    uint32_t hv[4], lv[4];
    float psum = 0.f, hsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hv[i] = pack_h2(x[2 * i], x[2 * i + 1]);
      const f16x2_t hh = __builtin_bit_cast(f16x2_t, hv[i]);
      const float h0 = static_cast<float>(hh.x), h1 = static_cast<float>(hh.y);
      lv[i] = pack_h2(x[2 * i] - h0, x[2 * i + 1] - h1);
      psum += x[2 * i] + x[2 * i + 1];
      hsum += h0 + h1;
    }
    ph = u32x4_t{hv[0], hv[1], hv[2], hv[3]};
    pl = u32x4_t{lv[0], lv[1], lv[2], lv[3]};
    const float la = l_run * alpha, l_full = la + quad_sum(psum);
    const float xmax = __builtin_amdgcn_exp2f(fmaf(tmax, c2, -mb));
    need_lo = __ballot(xmax > LO_SHARE * l_full) != 0;
    l_run = need_lo ? l_full : la + quad_sum(hsum);
    return alpha;
  };
  uint32_t cv;
  {
    const uint32_t m4 = (lane >> 2) & 3, r4 = lane & 3, R = 4 * q + m4, f = main_swz(R);
    cv = R * 1024 + 16 * ((r4 >> 1) ^ (f & 1)) + 16 * (f & 14) + 8 * (r4 & 1);
  }
  constexpr int VD = 2;   // V^T fragments read ahead
  auto pv = [&](const u32x4_t& pw) __attribute__((always_inline)) {
    uint32_t x1 = cv;
    asm volatile("" : "+v"(x1));
    auto vfrag = [&](int db) __attribute__((always_inline)) -> u32x4_t {
      uint8_t* ad = s_kb + (x1 ^ (32u * (db & 7))) + 256 * (db >> 3);
      const v4i16_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)ad);
      const v4i16_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(ad + 16384));
      const u32x2_t a2 = __builtin_bit_cast(u32x2_t, a), b2 = __builtin_bit_cast(u32x2_t, b);
      return u32x4_t{a2.x, a2.y, b2.x, b2.y};
    };
    u32x4_t vf[VD];
#pragma unroll
    for (int i = 0; i < VD; ++i) vf[i] = vfrag(i);
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      o[db] = mfma16x16x32_f16(vf[db % VD], pw, o[db]);
      if (db + VD < 32) vf[db % VD] = vfrag(db + VD);
    }
  };

  // prologue: token ids of tiles 0 and 1, tile 0 split into the tiles
  if (wid == 0) s_tk[lane] = tok(lane >> 5, lane & 31);   // tiles 0 and 1 (entries past the chunk: -1)
  __syncthreads();
  if (n_tiles > 0) load_stage(0);
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's staging loads have landed
  __syncthreads();
  if (n_tiles > 0) store_stage();
  __syncthreads();
  for (int u = 0; u < n_tiles; ++u) {
    // the codes and scales of tile u + 1 and the token ids of tile u + 2 are
    // in flight during the products of tile u; then, after a barrier, tile
    // u + 1 is split over tile u
    const bool more = u + 1 < n_tiles;
    if (more) load_stage(u + 1);
    int32_t t2 = -1;
    if (wid == 0 && lane < 32) t2 = tok(u + 2, lane);
    const uint32_t live = static_cast<uint32_t>(__ballot(s_tk[(u % 3) * TILE + (lane & 31)] >= 0));
    f32x4_t s0, s1;
    u32x4_t ph, pl;
    bool need_lo;
    scores(s0, s1);
    const float alpha = softmax(s0, s1, live, ph, pl, need_lo);
    if (alpha != 1.f) {
#pragma unroll
      for (int db = 0; db < 32; ++db) o[db] *= alpha;
    }
    u32x4_t pw = ph;
#pragma clang loop unroll(disable)
    for (int ps = 0; ps < 1 + need_lo; ++ps) {
      pv(pw);
      pw = pl;
    }
    if (wid == 0 && lane < 32) s_tk[((u + 2) % 3) * TILE + lane] = t2;   // over tile u - 1's ids
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's staging loads have landed
    __syncthreads();                      // all of the staging, the ids of tile u + 2; tile u read
    if (more) store_stage();
    __syncthreads();                      // tile u + 1 complete; the staging is free
  }

  // output (accumulator (db, j) holds dim 16 db + 4 q + j of head `head`)
  if (!(wvalid && head < p.Hq)) return;
  if (p.n_split == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const int64_t ob = (row * p.Hq + head) * MLA_DV + 4 * q;
#pragma unroll
    for (int db = 0; db < 32; ++db)
      store4(p.out, p.o_dtype, ob + 16 * db, o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
  } else {
    float* pp = p.part + ((row * p.n_split + sp) * p.Hq + head) * part_width(MLA_DV);
#pragma unroll
    for (int db = 0; db < 32; ++db) *reinterpret_cast<f32x4_t*>(pp + 16 * db + 4 * q) = o[db];
    if (q == 0) {
      pp[MLA_DV] = __builtin_amdgcn_ldexpf(m_run, -qk);   // the running max in score units
      pp[MLA_DV + 1] = l_run;
    }
  }
}

// ============================================================== GQA kernel ==

constexpr int GQA_D = 128;
constexpr int GQA_VT = TILE * GQA_D * 2;   // one V tile of one wave in LDS (8 KB)

// LDS of a GQA workgroup (one wave): two V tiles, the stream scratch, and the
// row's block list in block mode
static size_t gqa_lds_bytes(const AttnParams& p) {
  return 2 * GQA_VT + 64 + (p.idx != nullptr && p.c > 1 ? static_cast<size_t>(p.k_sel) * 4 : 0);
}

// Workgroups of the GQA kernel: one per (query row, stream chunk, KV group).
// Workgroup b runs on XCD b % 8; when the group count divides 8, the group is
// taken from b % 8, so that each XCD's L2 holds the K/V rows of one group
// (of an XCD pair, for 4 groups) instead of all of them.
static int64_t gqa_grid(const AttnParams& p) {
  const int64_t n = static_cast<int64_t>(p.S) * p.n_q * p.n_split * p.Hkv;
  return 8 % p.Hkv == 0 ? (n + 7) / 8 * 8 : n;
}

struct GqaK {   // K fragments of one tile: key block mb, contraction step ks
  u32x4_t a[2][4];
};
struct GqaV {   // one lane's share of a V tile: rows 4 i + lane / 16, 16-byte chunk lane % 16
  u32x4_t v[8];
};

// One workgroup = one wave = one query row x one stream chunk x one KV group
// g and its G <= 16 query heads (the MFMA columns, padded to 16); see
// gqa_grid for the group of a workgroup.  After the stream set-up the wave
// runs its own pipeline over tiles of 32 stream entries: the
// token ids of tile j + 3 are fetched while tile j is computed; the K
// fragments of tile j + 1 (A operand of S^T = K Q^T, straight from the cache
// rows) and its V rows (coalesced, 1 KB per load) are in flight in registers;
// the wave writes the V rows of tile j into one of its two LDS buffers and
// reads them back transposed with ds_read_b64_tr_b16 as the A operand of
// O^T = V^T P^T.  V row t keeps its 32-byte dim block b in slot b ^ (t & 7),
// which keeps both the row writes and the transposing reads free of bank
// conflicts.  With 8 heads per KV group the gathered K/V rows (16 KB per tile
// and group) outweigh the products: the kernel is bound by L2 / last-level
// cache bandwidth, not by the MFMAs.
__global__ __launch_bounds__(64, 2) void attn_gqa_kernel(AttnParams p) {
  extern __shared__ __align__(16) uint8_t s_raw[];
  const int lane = threadIdx.x;
  uint8_t* s_vt = s_raw;
  uint32_t* s_scr = reinterpret_cast<uint32_t*>(s_raw + 2 * GQA_VT);
  int32_t* s_blk = reinterpret_cast<int32_t*>(s_scr + 16);

  const int64_t b = blockIdx.x;
  int64_t unit;   // (row, chunk)
  int g;
  if (8 % p.Hkv == 0) {
    g = static_cast<int>((b & 7) % p.Hkv);
    unit = (b >> 3) * (8 / p.Hkv) + (b & 7) / p.Hkv;
  } else {
    g = static_cast<int>(b % p.Hkv);
    unit = b / p.Hkv;
  }
  if (unit >= static_cast<int64_t>(p.S) * p.n_q * p.n_split) return;   // padding of the last group of 8
  const int64_t row = unit / p.n_split;
  const int sp = static_cast<int>(unit % p.n_split);
  const int s = static_cast<int>(row / p.n_q);
  const StreamInfo si = stream_setup<1>(p, row, s_blk, s_scr);
  int64_t p0, p1;
  split_range(p, sp, si.len, &p0, &p1);
  const int n_tiles = p1 > p0 ? static_cast<int>((p1 - p0 + TILE - 1) / TILE) : 0;

  const int G = p.Hq / p.Hkv;
  const int col = lane & 15, quad = lane >> 4;
  const bool hvalid = col < G;
  const int head = g * G + col;

  u32x4_t qf[4];
  {
    const uint16_t* qr = static_cast<const uint16_t*>(p.q) + (row * p.Hq + (hvalid ? head : 0)) * GQA_D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[ks] = hvalid ? *reinterpret_cast<const u32x4_t*>(qr + 32 * ks + 8 * quad) : u32x4_t{0u, 0u, 0u, 0u};
  }
  f32x4_t o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4_t{};
  float m_run = NEG_INF, l_run = 0.f;
  const float c2 = p.scale_log2;
  const uint16_t* kbase = static_cast<const uint16_t*>(p.k) + s * p.k_seq + g * p.k_head;
  const uint16_t* vbase = static_cast<const uint16_t*>(p.v) + s * p.v_seq + g * p.v_head;

  // token id of entry lane % 32 of tile j (-1: dead or past the chunk)
  auto tile_tokens = [&](int j) __attribute__((always_inline)) -> int32_t {
    const int64_t pos = p0 + static_cast<int64_t>(j) * TILE + (lane & 31);
    return pos < p1 ? static_cast<int32_t>(stream_token(p, row, si, s_blk, pos)) : -1;
  };
  auto load_k = [&](GqaK& kk, int32_t tok) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int32_t t = __shfl(tok, 16 * mb + col, 64);
      const uint16_t* kr = kbase + static_cast<int64_t>(t >= 0 ? t : 0) * p.k_tok + 8 * quad;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kk.a[mb][ks] = t >= 0 ? *reinterpret_cast<const u32x4_t*>(kr + 32 * ks) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto load_v = [&](GqaV& vv, int32_t tok) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int32_t t = __shfl(tok, 4 * i + (lane >> 4), 64);
      const uint16_t* vr = vbase + static_cast<int64_t>(t >= 0 ? t : 0) * p.v_tok + 8 * col;
      vv.v[i] = t >= 0 ? *reinterpret_cast<const u32x4_t*>(vr) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store_v = [&](const GqaV& vv, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = 4 * i + (lane >> 4);
      *reinterpret_cast<u32x4_t*>(s_vt + b * GQA_VT + t * 256 + 32 * ((col >> 1) ^ (t & 7)) + 16 * (col & 1)) =
          vv.v[i];
    }
  };
  // V^T fragment of dim block db from buffer b: source lane (quad, 4 m + r)
  // addresses row R = 4 quad + m (then R + 16), dims 16 db + 4 r; the
  // transposing read hands lane j of each 16-lane group dim 16 db + j of
  // those four rows
  const uint32_t vr_m = (lane >> 2) & 3, vr_r = lane & 3, vr_R = 4 * quad + vr_m;
  auto vfrag = [&](int b, int db) __attribute__((always_inline)) -> u32x4_t {
    uint8_t* ad = s_vt + b * GQA_VT + vr_R * 256 + 32 * (db ^ (vr_R & 7)) + 8 * vr_r;
    const v4i16_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)ad);
    const v4i16_t c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(ad + 16 * 256));
    const u32x2_t a2 = __builtin_bit_cast(u32x2_t, a), c2_ = __builtin_bit_cast(u32x2_t, c);
    return u32x4_t{a2.x, a2.y, c2_.x, c2_.y};
  };
  // scores, online softmax and PV products of the tile in buffer b
  auto compute = [&](const GqaK& kk, int b, uint32_t live) __attribute__((always_inline)) {
    // S^T = K (32 keys x 128) . Q^T (128 x 16 heads): two 16-key blocks;
    // accumulator (mb, j) holds key 16 mb + 4 quad + j of head column col
    f32x4_t sacc[2] = {f32x4_t{}, f32x4_t{}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) sacc[mb] = mfma16x16x32_bf16(kk.a[mb][ks], qf[ks], sacc[mb]);
    float sv[8];
    float tmax = NEG_INF;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = 16 * (j >> 2) + 4 * quad + (j & 3);
      sv[j] = (live >> key) & 1u ? sacc[j >> 2][j & 3] : NEG_INF;
      tmax = fmaxf(tmax, sv[j]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    if (m_run == NEG_INF) {
      m_run = tmax;
    } else if (tmax > m_run) {   // exact running max
      const float alpha = exp2f((m_run - tmax) * c2);
      m_run = tmax;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) o[db] *= alpha;
    }
    // weights as bf16 high part + bf16 residual (see the MLA kernel)
    const float mb_ = m_run * c2;
    uint32_t pk[4], pl[4];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float a = m_run == NEG_INF ? 0.f : exp2f(fmaf(sv[j], c2, -mb_));
      const float bb = m_run == NEG_INF ? 0.f : exp2f(fmaf(sv[j + 1], c2, -mb_));
      pk[j >> 1] = pack_bf16x2(a, bb);
      pl[j >> 1] = pack_bf16x2(a - __uint_as_float(pk[j >> 1] << 16), bb - __uint_as_float(pk[j >> 1] & 0xffff0000u));
      psum += a + bb;
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run += psum;
    // P^T operand: slot (quad, j) <-> key 4 quad + j (j < 4), 16 + 4 quad + j - 4 (j >= 4)
    const u32x4_t pb = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
    const u32x4_t pr = u32x4_t{pl[0], pl[1], pl[2], pl[3]};
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const u32x4_t va = vfrag(b, db);
      o[db] = mfma16x16x32_bf16(va, pb, o[db]);
      o[db] = mfma16x16x32_bf16(va, pr, o[db]);
    }
  };

  GqaK kA, kB;
  GqaV vA, vB;
  int32_t tj = n_tiles > 0 ? tile_tokens(0) : -1;    // tokens of tile j
  int32_t tj1 = n_tiles > 1 ? tile_tokens(1) : -1;   // of tile j + 1
  int32_t tj2 = n_tiles > 2 ? tile_tokens(2) : -1;   // of tile j + 2
  if (n_tiles > 0) {
    load_k(kA, tj);
    load_v(vA, tj);
  }
  // one tile: its V rows into LDS buffer j & 1 (which held tile j - 2, read
  // by this wave before), the loads of tile j + 1, the token ids of tile
  // j + 3, then the products of tile j (fully dead tiles are skipped)
  auto step = [&](const GqaK& kc, const GqaV& vc, GqaK& kn, GqaV& vn, int j) __attribute__((always_inline)) {
    store_v(vc, j & 1);
    if (j + 1 < n_tiles) {
      load_k(kn, tj1);
      load_v(vn, tj1);
    }
    const int32_t tj3 = j + 3 < n_tiles ? tile_tokens(j + 3) : -1;
    const uint32_t live = static_cast<uint32_t>(__ballot(tj >= 0));
    asm volatile("" ::: "memory");   // the V rows are in LDS before they are read back
    if (live != 0u) compute(kc, j & 1, live);
    tj = tj1;
    tj1 = tj2;
    tj2 = tj3;
  };
  for (int j = 0; j < n_tiles; j += 2) {
    step(kA, vA, kB, vB, j);
    if (j + 1 >= n_tiles) break;
    step(kB, vB, kA, vA, j + 1);
  }

  if (!hvalid) return;
  // accumulator (db, j) holds dim 16 db + 4 quad + j of head column `col`
  if (p.n_split == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const int64_t ob = (row * p.Hq + head) * GQA_D;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      store4(p.out, p.o_dtype, ob + 16 * db + 4 * quad, o[db][0] * inv, o[db][1] * inv, o[db][2] * inv,
             o[db][3] * inv);
  } else {
    float* pp = p.part + ((row * p.n_split + sp) * p.Hq + head) * part_width(GQA_D);
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4_t*>(pp + 16 * db + 4 * quad) = o[db];
    if (quad == 0) {
      pp[GQA_D] = m_run;
      pp[GQA_D + 1] = l_run;
    }
  }
}

// ===================================================== GQA query tiles ==

// Workgroup of the query-tile kernel: GT_WAVES waves, each with one group of
// 16 MFMA columns; a column is a (query, head) pair of one KV group, so a
// workgroup takes 256 / G consecutive queries of one sequence (G = heads per
// group, a divisor of 16).  One workgroup fills a CU (1024 threads, up to
// 160 KB of LDS).
constexpr int GT_WAVES = 16;
constexpr int GT_KV = TILE * GQA_D * 2;      // K (or V) rows of one tile of one group (8 KB)
constexpr int GT_BUF = 2 * GT_KV;            // one tile: K rows, then V rows
constexpr int GT_RING = 4;                   // pairs of tiles resident in LDS
constexpr int GT_NBUF = 2 * GT_RING;         // tile buffers
constexpr int GT_JOBS = 2;                   // load jobs of a pair: one tile each (16 KB: K rows, then V rows)
constexpr int GT_QMAX = GT_WAVES * 16;       // queries of a workgroup (G = 1)
constexpr int GT_MAX_TILES = 2048;           // key tiles of one split
constexpr int GT_MAX_CNT = 12288;            // (query, block) multiplicities in LDS (u16)

static int gt_queries(const AttnParams& p) { return GT_WAVES * 16 / (p.Hq / p.Hkv); }
static int64_t gt_blocks(const AttnParams& p) { return p.idx ? p.n_kv / p.c : 0; }

// The query-tile kernel takes GQA calls in dense mode and in block mode with
// blocks of a multiple of 32 tokens, when a sequence has enough queries to
// share the K/V tiles (decode rows stay on attn_gqa_kernel's gather).
bool gqa_tiled(const AttnParams& p) {
  if (p.family != ATTN_GQA) return false;
  const int G = p.Hq / p.Hkv;
  if (16 % G || p.n_q < 8) return false;
  if (p.idx && (p.c == 1 || p.c % TILE)) return false;
  if (gt_queries(p) * gt_blocks(p) > GT_MAX_CNT) return false;
  const int64_t lim = int64_t(1) << 32;   // 32-bit row offsets within a sequence
  return p.n_kv * p.k_tok * 2 < lim && p.n_kv * p.v_tok * 2 < lim;
}

static size_t gt_lds_bytes(const AttnParams& p) {
  const size_t cnt = (static_cast<size_t>(gt_queries(p)) * gt_blocks(p) + 1) / 2 * 4;
  return GT_NBUF * GT_BUF + 128 + 2 * GT_QMAX * 4 + GT_MAX_TILES * 2 + cnt;
}
static constexpr size_t GT_LDS_MAX = GT_NBUF * GT_BUF + 128 + 2 * GT_QMAX * 4 + GT_MAX_TILES * 2 + GT_MAX_CNT * 2;
static_assert(GT_LDS_MAX <= 160 * 1024, "query-tile kernel LDS");

// Workgroups: (sequence, split, query tile) units times the KV groups; as in
// gqa_grid, workgroup b runs on XCD b % 8 and takes its group from b % 8
// when the group count divides 8, so that the workgroups of one XCD stream
// the K/V tiles of one group, in the same order, through its L2.
static int64_t gt_grid(const AttnParams& p) {
  const int64_t n_qt = (p.n_q + gt_queries(p) - 1) / gt_queries(p);
  const int64_t n = static_cast<int64_t>(p.S) * p.n_split * n_qt * p.Hkv;
  return 8 % p.Hkv == 0 ? (n + 7) / 8 * 8 : n;
}

// One workgroup = a tile of consecutive queries of one sequence x one KV group
// g x one split of the key positions.  Attention over a query's selected
// tokens is attention over all positions with the others weighted zero: the
// workgroup walks the key positions of its split in tiles of 32, skipping
// tiles that no query of the tile attends to, and each tile's K and V rows
// go once into LDS (direct global -> LDS loads into a ring of four pairs of
// tiles), where all 256 columns read them.  A query's weight for a token is
// its multiplicity:
// in block mode the number of times its idx row lists the token's block
// (live entries: 0 <= b < n_cb), and 1 for the incomplete tail n_cb c ..
// n_vis - 1; in dense mode 1 for every visible token.  A list that names a
// block twice thus counts its tokens twice, as the list semantics of the
// gathered stream do; the summation runs in position order instead of list
// order.  A tile lies in one block (32 | c), so its multiplicity per query
// is one count, read from an LDS table built from the idx rows.
// Each wave holds 16 columns (query, head) and takes the tiles in pairs, at
// its own pace (no workgroup barrier in the loop), both tiles of a pair in
// one step:
//   scores  S^T (32 keys x 16 columns) = K_tile . Q^T per tile, 16x16x32
//           MFMAs, Q in registers
//   softmax per column over the 64 keys of the pair (attn_mla_kernel's lazy
//           running max and bf16 weights plus residual), masked entries -inf
//   PV      O^T (128 dims x 16 columns) += V^T . P^T per tile, V^T fragments
//           through the transposing LDS read
// A wave whose columns all skip both tiles of a pair skips the step; a tile
// of the step that every column skips gets zero weights.  The step runs at a
// wave priority that grows with the number of waves already past its pair,
// so that the waves the ring waits for issue first.
// K row t keeps 16-byte chunk c of its 256 bytes in slot c ^ (t & 15) and
// V row t its 32-byte dim block b in slot b ^ (t & 7) (attn_gqa_kernel's V
// layout): the fragment reads are free of bank conflicts.
__global__ __launch_bounds__(64 * GT_WAVES, 4) void attn_gqa_tile_kernel(AttnParams p) {
  constexpr int NT = 64 * GT_WAVES;
  extern __shared__ __align__(16) uint8_t s_raw[];
  uint8_t* s_kv = s_raw;                                                          // GT_NBUF tiles
  uint32_t* s_scr = reinterpret_cast<uint32_t*>(s_raw + GT_NBUF * GT_BUF);      // 16 words
  uint32_t* s_sync = s_scr + 16;                                                 // ring counters, 16 words
  int32_t* s_nv = reinterpret_cast<int32_t*>(s_sync + 16);                       // n_vis per query
  int32_t* s_tl = s_nv + GT_QMAX;                                                // first tail token per query
  uint16_t* s_tiles = reinterpret_cast<uint16_t*>(s_tl + GT_QMAX);               // needed tiles of the split
  uint32_t* s_cnt = reinterpret_cast<uint32_t*>(s_tiles + GT_MAX_TILES);         // multiplicities, u16 pairs

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.Hq / p.Hkv, QPC = 16 / G, QT = GT_WAVES * QPC;
  const int64_t n_qt = (p.n_q + QT - 1) / QT;
  const int64_t b = blockIdx.x;
  int64_t unit;
  int g;
  if (8 % p.Hkv == 0) {
    g = static_cast<int>((b & 7) % p.Hkv);
    unit = (b >> 3) * (8 / p.Hkv) + (b & 7) / p.Hkv;
  } else {
    g = static_cast<int>(b % p.Hkv);
    unit = b / p.Hkv;
  }
  if (unit >= static_cast<int64_t>(p.S) * p.n_split * n_qt) return;   // padding of the last group of 8
  const int qt = static_cast<int>(unit % n_qt);
  const int sp = static_cast<int>((unit / n_qt) % p.n_split);
  const int s = static_cast<int>(unit / n_qt / p.n_split);
  const int64_t row0 = static_cast<int64_t>(s) * p.n_q + static_cast<int64_t>(qt) * QT;
  const int nqt = min(QT, static_cast<int>(p.n_q - static_cast<int64_t>(qt) * QT));   // real queries
  const bool blk = p.idx != nullptr;
  const int nb = blk ? static_cast<int>(p.n_kv / p.c) : 0;
  const int64_t kl = p.kv_len ? p.kv_len[s] : p.n_kv;

  // per query: visible tokens and the first tail token (dense: 0)
  if (tid < GT_QMAX) {
    int32_t nv = 0, tl = 0;
    if (tid < nqt) {
      nv = static_cast<int32_t>(visible_tokens(p.q_pos[row0 + tid], kl, p.n_kv));
      tl = blk ? nv / p.c * p.c : 0;
    }
    s_nv[tid] = nv;
    s_tl[tid] = tl;
  }
  const int cnt_words = (QT * nb + 1) / 2;
  for (int i = tid; i < cnt_words; i += NT) s_cnt[i] = 0u;
  if (tid < 16) s_sync[tid] = 0u;
  __syncthreads();
  auto count = [&](int qi, int bl) __attribute__((always_inline)) -> uint32_t {
    const uint32_t at = static_cast<uint32_t>(qi * nb + bl);
    return (s_cnt[at >> 1] >> (16 * (at & 1))) & 0xffffu;
  };
  if (blk) {
    const int ne = nqt * p.k_sel;
    for (int e = tid; e < ne; e += NT) {
      const int qi = e / p.k_sel;
      const int32_t bl = p.idx[(row0 + qi) * p.k_sel + (e - qi * p.k_sel)];
      if (bl >= 0 && bl < s_tl[qi] / p.c) {
        const uint32_t at = static_cast<uint32_t>(qi * nb + bl);
        atomicAdd(&s_cnt[at >> 1], 1u << (16 * (at & 1)));
      }
    }
  }
  int32_t vmax = 0;
  for (int i = 0; i < nqt; ++i) vmax = max(vmax, s_nv[i]);
  __syncthreads();   // the multiplicities

  // the split's key tiles that some query attends to, in position order
  const int64_t k0 = static_cast<int64_t>(sp) * p.split_len;
  const int64_t k1 = min(k0 + p.split_len, static_cast<int64_t>(vmax));
  const int kt0 = static_cast<int>(k0 / TILE);
  const int ntl = k1 > k0 ? static_cast<int>((k1 - k0 + TILE - 1) / TILE) : 0;
  auto needed = [&](int kt) __attribute__((always_inline)) -> bool {
    const int t0 = kt * TILE;
    const int bl = blk ? t0 / p.c : 0;
    for (int qi = 0; qi < nqt; ++qi) {
      if (t0 >= s_nv[qi]) continue;
      if (t0 >= s_tl[qi] || count(qi, bl) != 0u) return true;
    }
    return false;
  };
  {
    const int per = (ntl + NT - 1) / NT;
    const int e0 = min(tid * per, ntl), e1 = min(e0 + per, ntl);
    uint32_t n = 0;
    for (int e = e0; e < e1; ++e) n += needed(kt0 + e);
    uint32_t tot;
    uint32_t w = block_excl_scan<GT_WAVES>(n, s_scr, &tot);
    for (int e = e0; e < e1; ++e)
      if (needed(kt0 + e)) s_tiles[w++] = static_cast<uint16_t>(e);
    if (tid == 0) s_scr[8] = tot;
  }
  __syncthreads();
  const int n_need = static_cast<int>(s_scr[8]);

  // columns: wave wid holds queries wid QPC .. wid QPC + QPC - 1 of the tile,
  // G heads each; lane (col, q) holds column col
  const int col = lane & 15, q = lane >> 4;
  const int head = g * G + col % G;
  const int qi = wid * QPC + col / G;
  const bool c_ok = qi < nqt;
  const int32_t c_nv = s_nv[qi], c_tl = s_tl[qi];
  // the smallest visible count among the wave's queries (wave-uniform): a
  // tile that ends below it crosses no query's last visible token
  int32_t nv_min = c_ok ? c_nv : INT32_MAX;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) nv_min = min(nv_min, __shfl_xor(nv_min, o, 64));
  nv_min = __builtin_amdgcn_readfirstlane(nv_min);
  u32x4_t qf[4];
  {
    const uint16_t* qr = static_cast<const uint16_t*>(p.q) + ((row0 + (c_ok ? qi : 0)) * p.Hq + head) * GQA_D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[ks] = c_ok ? *reinterpret_cast<const u32x4_t*>(qr + 32 * ks + 8 * q) : u32x4_t{0u, 0u, 0u, 0u};
  }

  // K and V rows of the tiles: K row t keeps 16-byte chunk c of its 256 bytes
  // in slot c ^ (t & 15), V row t its 32-byte dim block b in slot b ^ (t & 7).
  // Rows no query of the tile sees read row 0 (zero weight).
  const uint32_t kv_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)s_kv));
  const char* kb = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.k) + s * p.k_seq + g * p.k_head);
  const char* vb = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.v) + s * p.v_seq + g * p.v_head);
  const uint32_t kpitch = static_cast<uint32_t>(p.k_tok) * 2u, vpitch = static_cast<uint32_t>(p.v_tok) * 2u;

  // o[db], db < 8: dims 16 db + 4 q + j of column col (O^T); o[8]: the
  // column's normaliser in every register, as the product of the weights
  // with a block of ones, so that it sums exactly the bf16 weights the value
  // products take
  f32x4_t o[9];
#pragma unroll
  for (int db = 0; db < 9; ++db) o[db] = f32x4_t{};
  float m_run = NEG_INF;
  const u32x4_t ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};   // bf16 1.0 pairs
  const float c2 = p.scale_log2;
  const uint32_t vr_m = (lane >> 2) & 3, vr_r = lane & 3, vr_R = 4 * q + vr_m;
  // V^T fragment db of lane (vr_R, vr_r): row vr_R, slot 2 (db ^ (vr_R & 7)) +
  // vr_r / 2; the xor with 32 db only touches bits 5..7 of this offset (the
  // buffer bases are multiples of 8 KB)
  const uint32_t v_lane = vr_R * 256u + 32u * (vr_R & 7u) + 8u * vr_r;
  // K fragment (mb, ks) of lane (col, q): row 16 mb + col, slot (4 ks + q) ^ col;
  // (4 ks + q) ^ col = 4 ks ^ (q ^ col), so the offset is k_lane ^ 64 ks + 4096 mb
  const uint32_t k_lane = static_cast<uint32_t>(col) * 256u + 16u * static_cast<uint32_t>(q ^ col);

  // O^T += V^T . P^T over the N tiles in buffers bf[0..N-1], weights pw[i],
  // straight-line: the normaliser first, then tile 0's 8 dim blocks, then
  // tile 1's (so each accumulator's two products are 8 apart), V^T fragments
  // read two ahead (attn_gqa_kernel's addressing)
  auto pv = [&](auto n_t, const int (&bf)[2], const u32x4_t (&pw)[2]) __attribute__((always_inline)) {
    constexpr int N = decltype(n_t)::value;
    auto vfrag = [&](int e) __attribute__((always_inline)) -> u32x4_t {
      const uint32_t vt_off = static_cast<uint32_t>(bf[e / 8] * GT_BUF + GT_KV) + v_lane;
      const uint8_t* a2 = s_kv + (vt_off ^ (32u * (e % 8)));
      const v4i16_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)a2);
      const v4i16_t vc = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(a2 + 16 * 256));
      const u32x2_t u2 = __builtin_bit_cast(u32x2_t, va), w2 = __builtin_bit_cast(u32x2_t, vc);
      return u32x4_t{u2.x, u2.y, w2.x, w2.y};
    };
    constexpr int VD = 2;
    u32x4_t vf[VD];
#pragma unroll
    for (int e = 0; e < VD; ++e) vf[e] = vfrag(e);
#pragma unroll
    for (int i = 0; i < N; ++i) o[8] = mfma16x16x32_bf16(ones, pw[i], o[8]);
#pragma unroll
    for (int e = 0; e < 8 * N; ++e) {
      o[e % 8] = mfma16x16x32_bf16(vf[e % VD], pw[e / 8], o[e % 8]);
      if (e + VD < 8 * N) vf[e % VD] = vfrag(e + VD);
    }
  };

  // the column's multiplicity for key tile kt of block bl: 0 when its query
  // skips the tile
  const int32_t c_cb = qi * nb;   // the query's row of the multiplicity table
  // In two halves, so that the table read can be issued a step before its
  // value is used: cnt_word reads the table word, mult_of finishes.
  auto cnt_word = [&](int bl) __attribute__((always_inline)) -> uint32_t {
    if (nb == 0) return 0u;
    const int blc = bl < nb ? bl : nb - 1;   // a tile past the complete blocks is every query's tail
    return s_cnt[static_cast<uint32_t>(c_cb + blc) >> 1];
  };
  auto mult_of = [&](int kt, int bl, uint32_t w) __attribute__((always_inline)) -> uint32_t {
    const int t0 = kt * TILE;
    uint32_t cnt = 1u;
    if (nb > 0) {
      const int blc = bl < nb ? bl : nb - 1;
      cnt = (w >> (16 * (static_cast<uint32_t>(c_cb + blc) & 1))) & 0xffffu;
    }
    const bool vis = c_ok && t0 < c_nv;
    return vis ? (t0 >= c_tl ? 1u : cnt) : 0u;
  };

  // One online-softmax step over N = 1 or 2 tiles (buffers bf, key tiles kt,
  // multiplicities mult) that some column of the wave attends to: the scores
  // of all N tiles, one running-max update and one residual decision, then
  // the value products of the N tiles in position order.
  // wave priority lv (0..3; s_setprio takes an immediate)
  auto set_prio = [](int lv) __attribute__((always_inline)) {
    if (lv >= 3) __builtin_amdgcn_s_setprio(3);
    else if (lv == 2) __builtin_amdgcn_s_setprio(2);
    else if (lv == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  };
  auto step = [&](auto n_t, const int (&bf)[2], const int (&kt)[2], const uint32_t (&mult)[2])
                  __attribute__((always_inline)) {
    constexpr int N = decltype(n_t)::value;
    // reg j of s[i][mb]: key 32 kt[i] + 16 mb + 4 q + j of column col
    f32x4_t s[2][2];
    uint32_t kt_off[2];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      kt_off[i] = static_cast<uint32_t>(bf[i] * GT_BUF) + k_lane;
      s[i][0] = s[i][1] = f32x4_t{};
    }
    // the N x 2 accumulation chains interleaved, step ks of every chain in turn
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < N; ++i)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          s[i][mb] = mfma16x16x32_bf16(*reinterpret_cast<const u32x4_t*>(s_kv + (kt_off[i] ^ (64u * ks)) + 4096 * mb),
                                       qf[ks], s[i][mb]);
    // A column whose query skips a tile (mult 0) keeps that tile's scores out
    // of the max and gets zero weights through an infinite offset; keys past a
    // query's last visible token (only in a tile that crosses it) are -inf.
    float tmax = NEG_INF;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int t0 = kt[i] * TILE;
      if (t0 + TILE > nv_min) {
        if (__ballot(mult[i] != 0u && t0 + TILE > c_nv) != 0) {
          const int lim = c_nv - t0 - 4 * q;   // keys j < lim (+ 16 mb) are visible
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (j >= lim) s[i][0][j] = NEG_INF;
            if (16 + j >= lim) s[i][1][j] = NEG_INF;
          }
        }
      }
      const float t = vmax3(vmax3(s[i][0][0], s[i][0][1], s[i][0][2]), vmax3(s[i][0][3], s[i][1][0], s[i][1][1]),
                            vmax3(s[i][1][2], s[i][1][3], NEG_INF));
      tmax = mult[i] != 0u ? __builtin_elementwise_maximum(tmax, t) : tmax;
    }
    tmax = quad_vmax(tmax);
    const bool first = m_run == NEG_INF;
    const bool grow = !first && (tmax - m_run) * c2 > 8.f;
    const float a = __builtin_amdgcn_exp2f((m_run - tmax) * c2);
    const float alpha = grow ? a : 1.f;
    m_run = (first || grow) ? tmax : m_run;
    const float mc = m_run == NEG_INF ? 0.f : m_run * c2;
    // the multiplicity scales the weights: offset log2(mult), zero -> +inf
    // (a listing count above 1 comes only from a list that names a block
    // twice: a branch of its own, kept out of the common path)
    float mo[2];
    float mo_min = __builtin_inff();
#pragma unroll
    for (int i = 0; i < N; ++i) mo[i] = mc;
    bool rep = false;
#pragma unroll
    for (int i = 0; i < N; ++i) rep = rep || mult[i] > 1u;
    if (__ballot(rep) != 0) {
      asm volatile("" ::: "memory");   // not speculated into the common path
#pragma unroll
      for (int i = 0; i < N; ++i)
        mo[i] -= __builtin_amdgcn_logf(static_cast<float>(mult[i] > 1u ? mult[i] : 1u));
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      mo[i] = mult[i] != 0u ? mo[i] : __builtin_inff();
      mo_min = fminf(mo_min, mo[i]);
    }
    // the step adds at least its largest weight (at most this bound) to the
    // rescaled normaliser
    const float xmax = __builtin_amdgcn_exp2f(fmaf(tmax, c2, -mo_min));
    const bool lo = __ballot(xmax * (1.f - LO_SHARE) > LO_SHARE * o[8][0] * alpha) != 0;
    u32x4_t ph[2], pl[2];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = __builtin_amdgcn_exp2f(fmaf(s[i][0][j], c2, -mo[i]));
        x[4 + j] = __builtin_amdgcn_exp2f(fmaf(s[i][1][j], c2, -mo[i]));
      }
      ph[i] = u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
      if (lo) {
        uint32_t lv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t hv = ph[i][k];
          lv[k] = pack_bf16x2(x[2 * k] - __uint_as_float(hv << 16), x[2 * k + 1] - __uint_as_float(hv & 0xffff0000u));
        }
        pl[i] = u32x4_t{lv[0], lv[1], lv[2], lv[3]};
      }
    }
    if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
      for (int db = 0; db < 9; ++db) o[db] *= alpha;
    }
    pv(n_t, bf, ph);
    if (lo) pv(n_t, bf, pl);
  };
  using two_t = std::integral_constant<int, 2>;

  // The tiles go through a ring of GT_RING pairs in LDS, and the waves do
  // not meet at barriers: each wave walks the pairs at its own pace and
  // computes only those its columns attend to, so a pair costs the waves that
  // compute it, not the slowest wave of the workgroup.  Words of s_sync:
  //   [i]            releases of ring slot i, over all its pairs: a wave
  //                  releases pair u when done with it (or at once if it
  //                  skips it); pair u + GT_RING may load into the slot once
  //                  all GT_WAVES waves released pair u
  //   [GT_RING + i]  load jobs of slot i landed, over all its pairs
  //   [8]            the next load job to claim (job j: pair j / GT_JOBS)
  // A wave that waits (for a slot or for a pair's loads) claims load jobs of
  // pairs whose slot is free, issues them, waits for them and counts them.
  // A wave enters pair u only once the slot holds pair u's generation (all
  // waves released pair u - GT_RING), so the counts of one slot never mix
  // generations; every pair has a wave that computes it (its tiles are
  // needed), and that wave releases it only after its loads landed.  The
  // slowest wave can always claim and load what it waits for itself, so
  // every wait ends; a wait is still bounded by an iteration limit.
  const int n_pairs = (n_need + 1) / 2;
  constexpr uint32_t NWV = GT_WAVES;
  constexpr int SPIN_MAX = 1 << 16;
  auto sync_ld = [&](int i) __attribute__((always_inline)) -> uint32_t {
    return __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(&s_sync[i], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
  };
  // load job j: tile j % 2 of pair j / 2, K rows then V rows in 1 KB loads;
  // load l of a part takes rows 4 l .. 4 l + 3, lane L slot L % 16 of row
  // 4 l + L / 16
  auto issue_job = [&](uint32_t j) __attribute__((always_inline)) {
    const int pj = static_cast<int>(j / GT_JOBS), ti = static_cast<int>(j % GT_JOBS);
    const int e = 2 * pj + ti;
    const int kt = kt0 + static_cast<int>(__builtin_amdgcn_readfirstlane(s_tiles[e < n_need ? e : n_need - 1]));
    const int t0 = kt * TILE;
    const uint32_t lb0 = kv_lds + static_cast<uint32_t>((2 * (pj % GT_RING) + ti) * GT_BUF);
    const uint32_t sl16 = lane & 15;
    const bool whole = t0 + TILE <= vmax;
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      const uint32_t r = 4u * l + (lane >> 4);
      const uint32_t rk = 16u * (sl16 ^ (r & 15)), rv = 16u * ((2u * ((sl16 >> 1) ^ (r & 7))) | (sl16 & 1u));
      uint32_t ko = (static_cast<uint32_t>(t0) + r) * kpitch + rk, vo = (static_cast<uint32_t>(t0) + r) * vpitch + rv;
      if (!whole) {
        const bool in = t0 + static_cast<int>(r) < vmax;
        ko = in ? ko : rk;
        vo = in ? vo : rv;
      }
      dma16(kb, ko, __builtin_amdgcn_readfirstlane(lb0 + 1024u * l));
      dma16(vb, vo, __builtin_amdgcn_readfirstlane(lb0 + GT_KV + 1024u * l));
    }
  };
  // claims one load job whose slot is free, loads it and counts it; false
  // when there is none
  auto try_claim = [&]() __attribute__((always_inline)) -> bool {
    uint32_t job = 0xffffffffu;
    if (lane == 0) {
      uint32_t j = __hip_atomic_load(&s_sync[8], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
      for (;;) {
        const uint32_t pj = j / GT_JOBS;
        if (pj >= static_cast<uint32_t>(n_pairs)) break;
        if (pj >= GT_RING && __hip_atomic_load(&s_sync[pj % GT_RING], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) <
                                 NWV * (pj / GT_RING))
          break;
        uint32_t exp = j;
        if (__hip_atomic_compare_exchange_strong(&s_sync[8], &exp, j + 1, __ATOMIC_ACQ_REL, __ATOMIC_ACQUIRE,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP)) {
          job = j;
          break;
        }
        j = exp;
      }
    }
    job = __builtin_amdgcn_readfirstlane(job);
    if (job == 0xffffffffu) return false;
    issue_job(job);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the job's rows are in LDS
    if (lane == 0)
      __hip_atomic_fetch_add(&s_sync[GT_RING + (job / GT_JOBS) % GT_RING], 1u, __ATOMIC_RELEASE,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
    return true;
  };
  auto wait_for = [&](int i, uint32_t target) __attribute__((always_inline)) {
    for (int it = 0; it < SPIN_MAX && sync_ld(i) < target; ++it)
      if (!try_claim()) __builtin_amdgcn_s_sleep(1);
  };

  const int tpb = blk ? p.c / TILE : 1;   // tiles per block
  // kt / tpb for kt < 2^16 as the high word of kt * (floor(2^32 / tpb) + 1):
  // the product overshoots kt / tpb by less than 2^-16 < 1 / tpb
  const uint32_t tpb_m = tpb > 1 ? 0xffffffffu / static_cast<uint32_t>(tpb) + 1u : 0u;
  auto block_of = [&](int kt) __attribute__((always_inline)) -> int {
    return tpb > 1 ? static_cast<int>(__umulhi(static_cast<uint32_t>(kt), tpb_m)) : kt;
  };
  // the list entry of position e as read from LDS (a position past the list
  // reads its last entry: such a tile gets multiplicity 0), and its tile id
  auto tile_raw = [&](int e) __attribute__((always_inline)) -> uint32_t {
    return s_tiles[e < n_need ? e : n_need - 1];
  };
  auto tile_id = [&](uint32_t raw) __attribute__((always_inline)) -> int {
    return kt0 + static_cast<int>(__builtin_amdgcn_readfirstlane(raw));
  };
  // The bookkeeping runs ahead: while pair u is computed, the table words of
  // pair u + 1 and the tile ids of pair u + 2 are read.  A pair without a
  // second tile loads the first tile's rows again and gives that tile
  // multiplicity 0 for every column (finite scores, zero weights).
  int ka = 0, kb_ = 0, kc = 0, kd = 0;
  uint32_t ma = 0u, mb_ = 0u;
  if (n_need > 0) {
    ka = tile_id(tile_raw(0));
    kb_ = tile_id(tile_raw(1));
    ma = mult_of(ka, block_of(ka), cnt_word(block_of(ka)));
    mb_ = n_need > 1 ? mult_of(kb_, block_of(kb_), cnt_word(block_of(kb_))) : 0u;
    kc = tile_id(tile_raw(2));
    kd = tile_id(tile_raw(3));
  }
  for (int u = 0; u < n_pairs; ++u) {
    const int sl = u % GT_RING;
    const uint32_t gen = static_cast<uint32_t>(u / GT_RING);
    const int blc_ = block_of(kc), bld = block_of(kd);
    const uint32_t wc = cnt_word(blc_), wd = cnt_word(bld);
    const uint32_t re = tile_raw(2 * u + 4), rf = tile_raw(2 * u + 5);
    const bool act = __ballot(ma != 0u || mb_ != 0u) != 0;
    if (u >= GT_RING) wait_for(sl, NWV * gen);   // the slot holds pair u's generation
    if (act) {
      wait_for(GT_RING + sl, GT_JOBS * (gen + 1));   // pair u's rows have landed
      // the more waves are past pair u, the higher this wave's priority
      const int lv = static_cast<int>((sync_ld(sl) - NWV * gen) / (NWV / 4));
      set_prio(lv);
      step(two_t{}, {2 * sl, 2 * sl + 1}, {ka, kb_}, {ma, mb_});
      __builtin_amdgcn_s_setprio(0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's reads of the slot are done
    if (lane == 0) __hip_atomic_fetch_add(&s_sync[sl], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    ma = 2 * u + 2 < n_need ? mult_of(kc, blc_, wc) : 0u;
    mb_ = 2 * u + 3 < n_need ? mult_of(kd, bld, wd) : 0u;
    ka = kc;
    kb_ = kd;
    kc = tile_id(re);
    kd = tile_id(rf);
  }

  // output: accumulator (db, j) holds dim 16 db + 4 q + j of column col.
  // The column's query and head are derived again from the lane id (opaque
  // to the compiler), so that no 64-bit index stays live across the loop.
  int lid = lane;
  asm volatile("" : "+v"(lid));
  const int qi_o = wid * QPC + (lid & 15) / G, head_o = g * G + (lid & 15) % G;
  if (qi_o < nqt) {
    const int64_t row = row0 + qi_o;
    if (p.n_split == 1) {
      const float inv = o[8][0] > 0.f ? 1.f / o[8][0] : 0.f;
      const int64_t ob = (row * p.Hq + head_o) * GQA_D + 4 * q;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        store4(p.out, p.o_dtype, ob + 16 * db, o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
    } else {
      float* pp = p.part + ((row * p.n_split + sp) * p.Hq + head_o) * part_width(GQA_D);
#pragma unroll
      for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4_t*>(pp + 16 * db + 4 * q) = o[db];
      if (q == 0) {
        pp[GQA_D] = m_run;
        pp[GQA_D + 1] = o[8][0];
      }
    }
  }
}

// ============================================================== f32 kernel ==

constexpr size_t F32_LDS = 64 * 4 * 2 + 64 + MAX_BLOCKS * 4;

// One wave per (query row, head, chunk).  64 tokens at a time: lane t scores
// token t of the batch (16-byte key loads when VEC: Dk and the strides are
// multiples of 4), the batch softmax updates the running state, then lane t
// accumulates output dims t, t + 64, ..., with the value loads of 32 tokens
// issued before their products (which still add in token order).
template <bool VEC>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnParams p) {
  constexpr int VB = 32;   // tokens whose value loads are in flight together
  extern __shared__ __align__(16) uint8_t s_raw[];
  float* s_p = reinterpret_cast<float*>(s_raw);
  int32_t* s_t = reinterpret_cast<int32_t*>(s_p + 64);
  uint32_t* s_scr = reinterpret_cast<uint32_t*>(s_t + 64);
  int32_t* s_blk = reinterpret_cast<int32_t*>(s_scr + 16);
  // stream_setup expects 256 threads; emulate with a 64-thread strided scan
  const int lane = threadIdx.x;
  const int64_t rh = blockIdx.x / p.n_split;
  const int sp = blockIdx.x % p.n_split;
  const int64_t row = rh / p.Hq;
  const int h = static_cast<int>(rh % p.Hq);
  const int s = static_cast<int>(row / p.n_q);
  const int g = h / (p.Hq / p.Hkv);
  StreamInfo si;
  {
    const int64_t kl = p.kv_len ? p.kv_len[s] : p.n_kv;
    si.n_vis = visible_tokens(p.q_pos[row], kl, p.n_kv);
    si.n_cb = 0;
    si.nb_live = 0;
    if (p.idx == nullptr) si.len = si.n_vis;
    else if (p.c == 1) si.len = p.k_sel;
    else {
      si.n_cb = si.n_vis / p.c;
      const int32_t* ir = p.idx + row * p.k_sel;
      if (lane == 0) {
        int64_t w = 0;
        for (int e = 0; e < p.k_sel; ++e)
          if (ir[e] >= 0 && ir[e] < si.n_cb) s_blk[w++] = ir[e];
        s_scr[0] = static_cast<uint32_t>(w);
      }
      __syncthreads();
      si.nb_live = s_scr[0];
      si.len = si.nb_live * p.c + (si.n_vis - si.n_cb * p.c);
    }
  }
  int64_t p0, p1;
  split_range(p, sp, si.len, &p0, &p1);
  const float* Q = static_cast<const float*>(p.q) + (row * p.Hq + h) * p.Dk;
  const float* K = static_cast<const float*>(p.k) + s * p.k_seq + g * p.k_head;
  const float* V = static_cast<const float*>(p.v) + s * p.v_seq + g * p.v_head;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float m_run = NEG_INF, l_run = 0.f;
  const float c2 = p.scale_log2;
  for (int64_t t0 = p0; t0 < p1; t0 += 64) {
    const int64_t tok = t0 + lane < p1 ? stream_token(p, row, si, s_blk, t0 + lane) : -1;
    float lg = NEG_INF;
    if (tok >= 0) {
      const float* kr = K + tok * p.k_tok;
      float d = 0.f;
      if constexpr (VEC) {
        for (int i = 0; i < p.Dk; i += 4) {
          const f32x4_t k4 = *reinterpret_cast<const f32x4_t*>(kr + i);
          d = fmaf(Q[i], k4[0], d);
          d = fmaf(Q[i + 1], k4[1], d);
          d = fmaf(Q[i + 2], k4[2], d);
          d = fmaf(Q[i + 3], k4[3], d);
        }
      } else {
        for (int i = 0; i < p.Dk; ++i) d = fmaf(Q[i], kr[i], d);
      }
      lg = d;
    }
    float tmax = lg;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 64));
    if (tmax == NEG_INF) continue;
    if (m_run == NEG_INF) {
      m_run = tmax;
    } else if (tmax > m_run) {
      const float alpha = exp2f((m_run - tmax) * c2);
      m_run = tmax;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;
    }
    const float pr = tok >= 0 ? exp2f((lg - m_run) * c2) : 0.f;
    float ps = pr;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ps += __shfl_xor(ps, o, 64);
    l_run += ps;
    s_p[lane] = pr;
    s_t[lane] = static_cast<int32_t>(tok);
    __syncthreads();
    for (int u0 = 0; u0 < 64; u0 += VB) {
      float vv[VB][4], pu[VB];
      bool ok[VB];
#pragma unroll
      for (int j = 0; j < VB; ++j) {
        const int64_t tk = s_t[u0 + j];
        ok[j] = tk >= 0;
        pu[j] = s_p[u0 + j];
        const float* vr = V + (ok[j] ? tk : 0) * p.v_tok;
#pragma unroll
        for (int i = 0; i < 4; ++i) vv[j][i] = lane + 64 * i < p.Dv ? vr[lane + 64 * i] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < VB; ++j) {
        if (!ok[j]) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (lane + 64 * i < p.Dv) acc[i] = fmaf(pu[j], vv[j][i], acc[i]);
      }
    }
    __syncthreads();
  }
  if (p.n_split == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    for (int i = 0; i < 4; ++i) {
      const int d = lane + 64 * i;
      if (d >= p.Dv) break;
      const int64_t off = (row * p.Hq + h) * p.Dv + d;
      if (p.o_dtype == DSA_F32) static_cast<float*>(p.out)[off] = acc[i] * inv;
      else static_cast<uint16_t*>(p.out)[off] = f32_to_bf16(acc[i] * inv);
    }
  } else {
    float* pp = p.part + ((row * p.n_split + sp) * p.Hq + h) * part_width(p.Dv);
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i < p.Dv) pp[lane + 64 * i] = acc[i];
    if (lane == 0) {
      pp[p.Dv] = m_run;
      pp[p.Dv + 1] = l_run;
    }
  }
}

// ========================================================= split combine ==

// One wave per (row, head, 64 float4 columns of the record), four waves per
// workgroup: merges the partials of the splits in split order.  Lane L owns
// float4 column 64 c + L (Dv rounded up to 4; the padded tail of the last
// column is read, never written).  The running maxima are reduced across the
// lanes first; the split loop then keeps several splits' loads in flight.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p) {
  const int lane = threadIdx.x & 63;
  const int nv = (p.Dv + 3) >> 2;   // float4 columns
  const int ncb = (nv + 63) >> 6;   // column blocks of 64
  const int64_t wv = static_cast<int64_t>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  if (wv >= rows * p.Hq * ncb) return;
  const int64_t rh = wv / ncb;
  const int v = static_cast<int>(wv % ncb) * 64 + lane;
  const int64_t row = rh / p.Hq;
  const int h = static_cast<int>(rh % p.Hq);
  const int W = part_width(p.Dv);
  const float* base = p.part + (row * p.n_split * p.Hq + h) * static_cast<int64_t>(W);
  const int64_t sstride = static_cast<int64_t>(p.Hq) * W;
  float M = NEG_INF;
  for (int c = lane; c < p.n_split; c += 64) M = fmaxf(M, base[c * sstride + p.Dv]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != NEG_INF) {
    const int vc = v < nv ? v : nv - 1;   // lanes past the record read a valid column, write nothing
#pragma unroll 8
    for (int c = 0; c < p.n_split; ++c) {
      const float* rec = base + c * sstride;
      const float mc = rec[p.Dv];
      const float wc = mc != NEG_INF ? exp2f((mc - M) * p.scale_log2) : 0.f;
      L += wc * rec[p.Dv + 1];
      const f32x4_t o = *reinterpret_cast<const f32x4_t*>(rec + 4 * vc);
      acc[0] += wc * o[0];
      acc[1] += wc * o[1];
      acc[2] += wc * o[2];
      acc[3] += wc * o[3];
    }
  }
  if (v >= nv) return;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int64_t off = (row * p.Hq + h) * p.Dv + 4 * v;
  if (p.Dv % 4 == 0) {
    store4(p.out, p.o_dtype, off, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  } else {
    for (int j = 0; j < 4 && 4 * v + j < p.Dv; ++j) {
      if (p.o_dtype == DSA_F32) static_cast<float*>(p.out)[off + j] = acc[j] * inv;
      else static_cast<uint16_t*>(p.out)[off + j] = f32_to_bf16(acc[j] * inv);
    }
  }
}

// ================================================================== host ==

void attn_plan(AttnParams& p, int64_t list_len) {
  if (gqa_tiled(p)) {
    // splits of the key positions: one workgroup per CU, at least 16 tiles
    // and at most GT_MAX_TILES tiles a split
    const int64_t wgs = static_cast<int64_t>(p.S) * ((p.n_q + gt_queries(p) - 1) / gt_queries(p)) * p.Hkv;
    int64_t ns = wgs < 256 ? (256 + wgs - 1) / wgs : 1;
    const int64_t max_ns = (p.n_kv + 16 * TILE - 1) / (16 * TILE);
    if (ns > max_ns) ns = max_ns;
    const int64_t min_ns = (p.n_kv + int64_t(GT_MAX_TILES) * TILE - 1) / (int64_t(GT_MAX_TILES) * TILE);
    if (ns < min_ns) ns = min_ns;
    int64_t sl = (p.n_kv + ns - 1) / ns;
    sl = (sl + TILE - 1) / TILE * TILE;
    p.n_split = static_cast<int32_t>((p.n_kv + sl - 1) / sl);
    p.split_len = static_cast<int32_t>(sl);
    return;
  }
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  int64_t wgs;   // workgroups per split
  int64_t target;
  if (p.family == ATTN_MLA) {
    wgs = rows * ((p.Hq + 127) / 128);
    target = 128;   // the f32 partials of a split weigh as much as its gathered rows: few, long splits
  } else if (p.family == ATTN_GQA) {
    wgs = rows * ((p.Hkv + 3) / 4);
    target = 1024;
  } else {
    wgs = rows * p.Hq;
    target = 2048;
  }
  int64_t lmin = list_len < p.n_kv ? list_len : p.n_kv;
  if (lmin < 1) lmin = 1;
  int64_t ns = 1;
  if (wgs < target) {
    ns = (target + wgs - 1) / wgs;
    const int64_t max_ns = (lmin + 63) / 64;   // at least two tiles per split
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
  }
  int64_t sl = (lmin + ns - 1) / ns;
  sl = (sl + 63) / 64 * 64;   // whole tiles for every kernel (64 covers the f32 batch)
  ns = (lmin + sl - 1) / sl;
  if (ns < 1) ns = 1;
  p.n_split = static_cast<int32_t>(ns);
  p.split_len = static_cast<int32_t>(sl);
  // MLA over bf16 rows: workgroups of 64 heads when those of 128 would leave
  // half the CUs idle (decode)
  p.mla_hg = 128;
  if (p.family == ATTN_MLA && !p.kq8 && p.Hq % 64 == 0 && wgs * ns <= 128) p.mla_hg = 64;
}

size_t attn_workspace_bytes(const AttnParams& p) {
  if (p.n_split <= 1) return 0;
  return static_cast<size_t>(p.S) * p.n_q * p.n_split * p.Hq * part_width(p.Dv) * sizeof(float);
}

hipError_t launch_attention(const AttnParams& p, hipStream_t st, hipEvent_t before_combine) {
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  hipError_t e;
  if (p.family == ATTN_MLA && p.kq8) {
    // set on every call (the same value each time, no state kept between calls)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_mla_q8_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(MLA_Q8_LDS));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_mla_q8_kernel, dim3(static_cast<unsigned>(rows * p.n_split), (p.Hq + 127) / 128),
                       dim3(64 * MLA_WAVES), MLA_Q8_LDS, st, p);
  } else if (p.family == ATTN_MLA) {
    // set on every call (the same value each time, no state kept between calls)
    const bool hg64 = p.mla_hg == 64;
    const void* fn = hg64 ? reinterpret_cast<const void*>(attn_mla_kernel<true>)
                          : reinterpret_cast<const void*>(attn_mla_kernel<false>);
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(MLA_LDS));
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(rows * p.n_split), hg64 ? (p.Hq + 63) / 64 : (p.Hq + 127) / 128);
    if (hg64)
      hipLaunchKernelGGL(attn_mla_kernel<true>, grid, dim3(64 * MLA_WAVES), MLA_LDS, st, p);
    else
      hipLaunchKernelGGL(attn_mla_kernel<false>, grid, dim3(64 * MLA_WAVES), MLA_LDS, st, p);
  } else if (gqa_tiled(p)) {
    // the largest size any call uses, so that concurrent calls set the same value
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_gqa_tile_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(GT_LDS_MAX));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_gqa_tile_kernel, dim3(static_cast<unsigned>(gt_grid(p))), dim3(64 * GT_WAVES),
                       gt_lds_bytes(p), st, p);
  } else if (p.family == ATTN_GQA) {
    // the largest size any call uses, so that concurrent calls set the same value
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_gqa_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(2 * GQA_VT + 64 + MAX_BLOCKS * 4));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_gqa_kernel, dim3(static_cast<unsigned>(gqa_grid(p))), dim3(64), gqa_lds_bytes(p), st,
                       p);
  } else {
    // 16-byte key loads when every key row starts 16-byte aligned
    const bool vec = p.Dk % 4 == 0 && p.k_tok % 4 == 0 && p.k_seq % 4 == 0 && p.k_head % 4 == 0 &&
                     (reinterpret_cast<uintptr_t>(p.k) & 15) == 0;
    if (vec)
      hipLaunchKernelGGL(attn_f32_kernel<true>, dim3(static_cast<unsigned>(rows * p.Hq * p.n_split)), dim3(64),
                         F32_LDS, st, p);
    else
      hipLaunchKernelGGL(attn_f32_kernel<false>, dim3(static_cast<unsigned>(rows * p.Hq * p.n_split)), dim3(64),
                         F32_LDS, st, p);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (before_combine && (e = hipEventRecord(before_combine, st)) != hipSuccess) return e;
  if (p.n_split > 1) {
    const int64_t waves = rows * p.Hq * ((p.Dv + 255) / 256);   // (row, head, 64 float4 columns)
    hipLaunchKernelGGL(attn_combine_kernel, dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0, st, p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace dsa
