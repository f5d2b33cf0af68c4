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
// tiles in order; invisible or dead entries are masked by position (their rows
// are zero-filled and their logits -inf, never multiplied), and a row that sees
// no key at all is written as zeros.  Long streams are split into contiguous
// chunks whose partial (max, sum, unnormalised output) are merged in a fixed
// order by attn_combine_kernel, so results are deterministic and identical for
// the same stream whatever the call that produced it.
//
// Kernels:
//   attn_f32_kernel   f32 Q/K/V, any head grouping, Dk, Dv <= 256 (VALU)
//   attn_mla_kernel   MLA: 576-wide latent K, V = its first 512 columns, bf16,
//                     32 heads per wave on 32x32x16 MFMAs
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
constexpr int MLA_WAVES = 4;                     // 32 query heads per wave
constexpr int KT_MAIN = TILE * 1024;             // dims 0..511 of the tile rows, 1 KB per row
constexpr int KT_ROPE = TILE * 128;              // dims 512..575, 128 B per row
constexpr int KT_BYTES = KT_MAIN + KT_ROPE;      // one gathered tile (36 KB)
constexpr int KT_NBUF = 3;                       // tiles t (PV), t + 1 (S), t + 2 (in flight)
constexpr int TOK_RING = 1024;                   // validated token ids of 32 tiles
constexpr int TOK_REFILL = TOK_RING / 2 / TILE;  // tiles per ring refill (16)
constexpr int MLA_QL = 8;                        // 16-dim steps of Q kept in LDS (the last ones)
constexpr int MLA_QR = 36 - MLA_QL;              // 16-dim steps of Q kept in registers
constexpr int MLA_QBYTES = MLA_WAVES * MLA_QL * 64 * 16;
constexpr size_t MLA_LDS = KT_NBUF * KT_BYTES + MLA_QBYTES + TOK_RING * 4 + 64 + MLA_MAX_BLOCKS * 4;

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
// aligned rows read at one chunk, or 4 aligned rows at 4 aligned neighbouring
// chunks, land on 16 distinct slots mod 16; 8 aligned rows at one chunk, or 4
// rows at 2 neighbouring chunks, on 8 distinct slots mod 8.  The 16-byte reads
// of the key fragments and the transposing 8-byte reads of the value
// fragments are thus free of bank conflicts for 32 or 64 banks of 4 bytes.
__device__ __forceinline__ uint32_t main_swz(uint32_t r) {
  const uint32_t m = r & 3, b = (r >> 2) & 3;
  return (b & 1) | ((m & 1) << 1) | ((m >> 1) << 2) | (((m & 1) ^ (b >> 1)) << 3);
}
// Same for the 8 slots of dims 512..575 (128-byte rows): 16 aligned rows at one
// chunk fall on distinct slots of a 256-byte bank period, 8 on distinct slots
// of a 128-byte one.
__device__ __forceinline__ uint32_t rope_swz(uint32_t r) { return ((r & 15) ^ ((r & 15) >> 3)) & 7; }

// lane l receives the value of lane l ^ 32 (max / sum across the two key halves)
__device__ __forceinline__ float swap_halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  // both halves add (lower, upper) in the same order: identical sums
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One workgroup = one query row x one stream chunk x 128 heads, 4 waves; wave
// w owns heads 32 w .. 32 w + 31 and all 576 contraction dims.  Per tile of 32
// gathered latent rows:
//   S^T (32 keys x 32 heads) = K_tile . Q^T on 32x32x16 MFMAs, K fragments
//       read from the LDS tile, Q in registers
//   online softmax over the 32 keys of each head (16 per lane + one lane
//       swap); the running max is only raised when it grows by more than 2^8
//       in weight, and the weights enter the PV product as a bf16 high part
//       plus a bf16 residual, so they stay exact to ~2^-17 even above 1
//   O^T (512 dims x 32 heads) += V^T . P^T: V^T fragments come straight from
//       the key-major tile through the transposing LDS read; P^T is the S^T
//       accumulator layout, so no data moves between lanes
// Software pipeline: iteration t computes S of tile t + 1, then the PV
// product of tile t, then the softmax of tile t + 1, so the exponentials and
// packing overlap the PV matrix products; tile t + 2 is gathered meanwhile
// with direct global -> LDS loads (three tile buffers).  Token ids of the
// stream sit in an LDS ring of 32 tiles, refilled 16 tiles ahead.
__global__ __launch_bounds__(256, 1) void attn_mla_kernel(AttnParams p) {
  extern __shared__ __align__(16) uint8_t s_raw[];
  uint8_t* s_kb = s_raw;                                                       // KT_NBUF tiles
  uint8_t* s_q = s_raw + KT_NBUF * KT_BYTES;                                   // Q fragments
  int32_t* s_tok = reinterpret_cast<int32_t*>(s_q + MLA_QBYTES);               // token ring
  uint32_t* s_scr = reinterpret_cast<uint32_t*>(s_tok + TOK_RING);
  int32_t* s_blk = reinterpret_cast<int32_t*>(s_scr + 16);                    // MLA_MAX_BLOCKS

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar registers
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  const int64_t row = rows - 1 - blockIdx.x / p.n_split;     // latest (longest causal) rows first
  const int sp = blockIdx.x % p.n_split;
  const int s = static_cast<int>(row / p.n_q);
  const StreamInfo si = stream_setup<MLA_WAVES>(p, row, s_blk, s_scr);
  int64_t p0, p1;
  split_range(p, sp, si.len, &p0, &p1);
  // token mode: trailing dead entries (the -1 padding of short selections)
  // are cut off; they would add nothing
  if (p.idx != nullptr && p.c == 1 && p1 > p0) {
    if (tid == 0) s_scr[8] = 0u;
    __syncthreads();
    const int32_t* ir = p.idx + row * p.k_sel;
    uint32_t last = 0;   // 1 + offset of the last live entry
    for (int64_t e = p0 + tid; e < p1; e += 64 * MLA_WAVES) {
      const int32_t v = ir[e];
      if (v >= 0 && v < si.n_vis) last = static_cast<uint32_t>(e - p0 + 1);
    }
    if (last) atomicMax(&s_scr[8], last);
    __syncthreads();
    p1 = p0 + s_scr[8];
  }
  const int n_tiles = p1 > p0 ? static_cast<int>((p1 - p0 + TILE - 1) / TILE) : 0;
  auto token_at = [&](int64_t pos) __attribute__((always_inline)) -> int32_t {
    return pos < p1 ? static_cast<int32_t>(stream_token(p, row, si, s_blk, pos)) : -1;
  };
  for (int i = tid; i < TOK_RING; i += 64 * MLA_WAVES) s_tok[i] = token_at(p0 + i);

  const int r32 = lane & 31, h = lane >> 5;
  const int head0 = blockIdx.y * 128 + wid * 32;
  const bool wvalid = head0 < p.Hq;   // Hq is a multiple of 16
  const int head = head0 + r32;
  const bool hvalid = head < p.Hq;

  // Q^T fragments: lane (head, h) holds dims 16 ks + 8 h .. + 7 (chunk 2 ks + h);
  // steps ks < MLA_QR in registers, the others in LDS in fragment order (the
  // registers are what the accumulators and the pipelined loads need most)
  u32x4_t qf[MLA_QR];
  u32x4_t* s_qw = reinterpret_cast<u32x4_t*>(s_q) + wid * MLA_QL * 64 + lane;
  {
    const uint16_t* qr = static_cast<const uint16_t*>(p.q) + (row * p.Hq + (hvalid ? head : 0)) * MLA_DK + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      const u32x4_t v = hvalid ? *reinterpret_cast<const u32x4_t*>(qr + 16 * ks) : u32x4_t{0u, 0u, 0u, 0u};
      if (ks < MLA_QR) qf[ks] = v;
      else s_qw[(ks - MLA_QR) * 64] = v;
    }
  }
  f32x16_t o[16];
#pragma unroll
  for (int db = 0; db < 16; ++db) o[db] = f32x16_t{};
  float m_run = NEG_INF, l_run = 0.f;
  const float c2 = p.scale_log2;

  const uint32_t kb_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)s_kb));
  const char* kseq_b = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.k) + s * p.k_seq);
  const uint64_t pitch = static_cast<uint64_t>(p.k_tok) * 2u;   // bytes per token row
  // Gather of tile u into buffer lb: wave w loads the 1 KB main parts of rows
  // w, w + 4, ..., w + 28 (instruction k < 8: row w + 4 k, its token id read
  // from lane r of tl) and the rope parts of rows 8 w .. 8 w + 7 (k = 8).
  // The nine instructions are spread over the matrix products of a tile, so
  // that the address unit takes them as it frees up instead of stalling the
  // wave.  ln is the lane id, opaque to the compiler (recomputed per tile).
  auto dma_k = [&](int k, int32_t tl, uint32_t lb, int ln) __attribute__((always_inline)) {
    if (k < 8) {
      const int r = wid + MLA_WAVES * k;
      const int32_t tok = __builtin_amdgcn_readlane(tl, r);
      const char* src = kseq_b + static_cast<uint64_t>(tok > 0 ? tok : 0) * pitch;
      dma16(src, (16u * ln) ^ (16u * main_swz(r)), lb + 1024u * r);
    } else {
      const uint32_t rr = 8 * wid + (ln >> 3);
      const int32_t tok = __shfl(tl, rr, 64);
      const uint32_t voff = static_cast<uint32_t>(tok > 0 ? tok : 0) * static_cast<uint32_t>(pitch) + 1024u +
                            16u * ((ln & 7) ^ rope_swz(rr));
      dma16(kseq_b, voff, lb + KT_MAIN + 1024u * wid);
    }
  };
  auto tokens_of = [&](int u) __attribute__((always_inline)) -> int32_t {
    return s_tok[(u * TILE + (lane & 31)) & (TOK_RING - 1)];
  };
  auto issue = [&](int u, int buf) __attribute__((always_inline)) {
    const int32_t tl = tokens_of(u);
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = 0; k < 9; ++k) dma_k(k, tl, kb_lds + buf * KT_BYTES, ln);
  };
  auto live_of = [&](int u) __attribute__((always_inline)) -> uint32_t {
    return static_cast<uint32_t>(__ballot(tokens_of(u) >= 0));
  };

  // K fragment of S: lane (row r32, half h) reads chunk 2 ks + h of row r32,
  // at tile offset (cs ^ 32 (ks & 7)) + 256 (ks >> 3) (main) or
  // (cr ^ 32 (ks - 32)) (rope); the xor terms only touch bits 5..7.  The 36
  // products run in a fixed order: product i < 32 takes chunk pair k8 = i >> 2
  // of 256-byte group a = i & 3 (ks = 8 a + k8), i >= 32 the rope chunk pair
  // i - 32.
  const uint32_t cs = r32 * 1024u + 16u * (h ^ main_swz(r32));
  const uint32_t cr = KT_MAIN + r32 * 128u + 16u * (h ^ rope_swz(r32));
  auto kfrag = [&](const uint8_t* kt, uint32_t xs, uint32_t xr, int i) __attribute__((always_inline)) -> u32x4_t {
    const uint8_t* ad = i < 32 ? kt + (xs ^ (32u * (i >> 2))) + 256 * (i & 3) : kt + (xr ^ (32u * (i - 32)));
    return *reinterpret_cast<const u32x4_t*>(ad);
  };
  auto qfrag = [&](int i) __attribute__((always_inline)) -> u32x4_t {
    const int ks = i < 32 ? 8 * (i & 3) + (i >> 2) : i;
    return ks < MLA_QR ? qf[ks < MLA_QR ? ks : 0] : s_qw[(ks - MLA_QR) * 64];
  };
  // V^T fragment of dim block db, key half kk: lane (group g, source slot
  // 4 m + q) addresses key 16 kk + 4 (g >> 1) + m (then + 8), dims
  // 32 db + 16 (g & 1) + 4 q; the transposing read hands lane j of each 16-lane
  // group dim 32 db + 16 (g & 1) + j of those four keys.  Tile offset:
  // (cv ^ 64 (db & 3)) + 256 (db >> 2) + 16 KB kk, the xor touching bits 6..7.
  // PV step i (of 32): dim quarter dq = i >> 3, 256-byte group dh = (i >> 1) & 3
  // (dim block db = 4 dh + dq), key half kk = i & 1.
  uint32_t cv1, cv2;
  {
    const uint32_t g4 = lane >> 4, m4 = (lane >> 2) & 3, q4 = lane & 3;
    const uint32_t R1 = 4 * (g4 >> 1) + m4, R2 = R1 + 8;
    const uint32_t f1 = main_swz(R1), f2 = main_swz(R2), lo_c = 2 * (g4 & 1) + (q4 >> 1);
    cv1 = R1 * 1024 + 64 * (f1 >> 2) + 16 * (lo_c ^ (f1 & 3)) + 8 * (q4 & 1);
    cv2 = R2 * 1024 + 64 * (f2 >> 2) + 16 * (lo_c ^ (f2 & 3)) + 8 * (q4 & 1);
  }
  auto vfrag = [&](uint8_t* kt, uint32_t x1, uint32_t x2, int i) __attribute__((always_inline)) -> u32x4_t {
    const int dq = i >> 3, off = 16384 * (i & 1) + 256 * ((i >> 1) & 3);
    const v4i16_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(kt + (x1 ^ (64u * dq)) + off));
    const v4i16_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(kt + (x2 ^ (64u * dq)) + off));
    const u32x2_t a2 = __builtin_bit_cast(u32x2_t, a), b2 = __builtin_bit_cast(u32x2_t, b);
    return u32x4_t{a2.x, a2.y, b2.x, b2.y};
  };
  // dead keys of a tile (bit clear in `live`) get score -inf
  auto mask_dead = [&](f32x16_t& sacc, uint32_t live) __attribute__((always_inline)) {
    const uint32_t lm = live >> (4 * h);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (!((lm >> (8 * (j >> 2) + (j & 3))) & 1u)) sacc[j] = NEG_INF;
  };
  // softmax of a tile's S^T accumulator: reg j holds key 8 (j >> 2) + 4 h + (j & 3)
  // of head r32.  Returns the factor that rescales what was accumulated before.
  auto softmax = [&](const f32x16_t& sacc, u32x4_t (&ph)[2], u32x4_t (&pl)[2]) __attribute__((always_inline)) -> float {
    float sv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) sv[j] = sacc[j];
    float tmax = sv[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) tmax = fmaxf(tmax, sv[j]);
    tmax = swap_halves_max(tmax);
    // branch-free, so that it can run between the matrix products
    const bool first = m_run == NEG_INF;
    const bool grow = !first && (tmax - m_run) * c2 > 8.f;
    const float a = __builtin_amdgcn_exp2f((m_run - tmax) * c2);
    const float alpha = grow ? a : 1.f;
    m_run = (first || grow) ? tmax : m_run;
    const float mb = m_run == NEG_INF ? 0.f : m_run * c2;   // an all-dead prefix gives zero weights
    float psum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t hv[4], lv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = __builtin_amdgcn_exp2f(fmaf(sv[8 * kk + 2 * i], c2, -mb));
        const float x1 = __builtin_amdgcn_exp2f(fmaf(sv[8 * kk + 2 * i + 1], c2, -mb));
        hv[i] = pack_bf16x2(x0, x1);
        lv[i] = pack_bf16x2(x0 - __uint_as_float(hv[i] << 16), x1 - __uint_as_float(hv[i] & 0xffff0000u));
        psum += x0 + x1;
      }
      ph[kk] = u32x4_t{hv[0], hv[1], hv[2], hv[3]};
      pl[kk] = u32x4_t{lv[0], lv[1], lv[2], lv[3]};
    }
    l_run = l_run * alpha + swap_halves_sum(psum);
    return alpha;
  };
  // o *= alpha (rare): element by element through one VGPR, written so that
  // the accumulators keep living in the accumulation registers
  auto rescale = [&](float alpha) __attribute__((always_inline)) {
    if (alpha != 1.f) {
#pragma unroll
      for (int db = 0; db < 16; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          float x = o[db][j], tmp;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                       : "+a"(x), "=&v"(tmp)
                       : "v"(alpha));
          o[db][j] = x;
        }
    }
  };
  u32x4_t ph[2] = {u32x4_t{}, u32x4_t{}}, pl[2] = {u32x4_t{}, u32x4_t{}};
  auto pv_mfma = [&](int i, const u32x4_t& va) __attribute__((always_inline)) {
    const int db = 4 * ((i >> 1) & 3) + (i >> 3), kk = i & 1;
    o[db] = mfma32x32x16_bf16(va, ph[kk], o[db]);
    o[db] = mfma32x32x16_bf16(va, pl[kk], o[db]);
  };
  constexpr int SD = 4;   // K fragments read ahead
  constexpr int VD = 2;   // V^T fragments read ahead

  // One tile step: PV of tile t (buffer bp) with the pending weights, S of
  // tile t + 1 (buffer bs), its softmax, and the gather of tile t + 2 (buffer
  // bg).  Phase 1 interleaves the 36 S products with the first 16 PV steps
  // and the nine gather loads; phase 2 runs the softmax between the last 16
  // PV steps.  The S products accumulate in one fixed order, so results do
  // not depend on the schedule.
  auto tile_step = [&](int bp, int bs, int bg, uint32_t live_n, int u_gather) __attribute__((always_inline)) {
    uint32_t xs = cs, xr = cr, x1 = cv1, x2 = cv2;
    int ln = lane;
    asm volatile("" : "+v"(xs), "+v"(xr), "+v"(x1), "+v"(x2), "+v"(ln));   // recomputed per tile
    const uint8_t* ks_t = s_kb + bs * KT_BYTES;
    uint8_t* kp_t = s_kb + bp * KT_BYTES;
    const int32_t tl = tokens_of(u_gather);
    const uint32_t lb = kb_lds + bg * KT_BYTES;
    u32x4_t kf[SD], vf[VD];
#pragma unroll
    for (int i = 0; i < SD; ++i) kf[i] = kfrag(ks_t, xs, xr, i);
#pragma unroll
    for (int i = 0; i < VD; ++i) vf[i] = vfrag(kp_t, x1, x2, i);
    __builtin_amdgcn_sched_group_barrier(0x100, SD + 2 * VD, 0);
    f32x16_t sacc = f32x16_t{};
    auto s_item = [&](int si) __attribute__((always_inline)) {
      sacc = mfma32x32x16_bf16(kf[si % SD], qfrag(si), sacc);
      if (si + SD < 36) kf[si % SD] = kfrag(ks_t, xs, xr, si + SD);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    };
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s_item(2 * i);
      s_item(2 * i + 1);
      pv_mfma(i, vf[i % VD]);
      vf[i % VD] = vfrag(kp_t, x1, x2, i + VD);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      if ((i & 1) && i < 16) dma_k(i >> 1, tl, lb, ln);
    }
#pragma unroll
    for (int i = 32; i < 36; ++i) s_item(i);
    dma_k(8, tl, lb, ln);
    if (live_n != 0xffffffffu) mask_dead(sacc, live_n);
    u32x4_t nh[2], nl[2];
    const float alpha = softmax(sacc, nh, nl);
#pragma unroll
    for (int i = 16; i < 32; ++i) {
      pv_mfma(i, vf[i % VD]);
      if (i + VD < 32) vf[i % VD] = vfrag(kp_t, x1, x2, i + VD);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    rescale(alpha);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      ph[kk] = nh[kk];
      pl[kk] = nl[kk];
    }
  };
  // PV of the last tile
  auto pv_last = [&](int bp) __attribute__((always_inline)) {
    uint32_t x1 = cv1, x2 = cv2;
    asm volatile("" : "+v"(x1), "+v"(x2));
    uint8_t* kp_t = s_kb + bp * KT_BYTES;
    u32x4_t vf[VD];
#pragma unroll
    for (int i = 0; i < VD; ++i) vf[i] = vfrag(kp_t, x1, x2, i);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      pv_mfma(i, vf[i % VD]);
      if (i + VD < 32) vf[i % VD] = vfrag(kp_t, x1, x2, i + VD);
    }
  };
  // S and softmax of the first tile
  auto s_first = [&](uint32_t live0) __attribute__((always_inline)) {
    uint32_t xs = cs, xr = cr;
    const uint8_t* ks_t = s_kb;
    f32x16_t sacc = f32x16_t{};
#pragma unroll
    for (int i = 0; i < 36; ++i) sacc = mfma32x32x16_bf16(kfrag(ks_t, xs, xr, i), qfrag(i), sacc);
    if (live0 != 0xffffffffu) mask_dead(sacc, live0);
    softmax(sacc, ph, pl);
  };

  // token ring refill: entries of tiles t + 16 .. t + 31 are fetched at t = 16 j
  // and validated and stored one iteration later (their loads have landed by
  // then) into the slots of tiles t - 16 .. t - 1
  const bool token_mode = p.idx != nullptr && p.c == 1;
  auto ring_fetch = [&](int64_t pos) __attribute__((always_inline)) -> int32_t {
    if (token_mode) return p.idx[row * p.k_sel + (pos < p1 ? pos : p1 - 1)];
    return pos < p1 ? static_cast<int32_t>(stream_token(p, row, si, s_blk, pos)) : -1;
  };
  auto ring_value = [&](int64_t pos, int32_t v) __attribute__((always_inline)) -> int32_t {
    if (pos >= p1) return -1;
    if (token_mode) return (v >= 0 && v < si.n_vis) ? v : -1;
    return v;
  };
  int32_t ring_v[2] = {-1, -1};
  __syncthreads();   // token ring filled
  if (n_tiles > 0) issue(0, 0);
  if (n_tiles > 1) issue(1, 1);
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
  __syncthreads();
  if (n_tiles > 0 && wvalid) s_first(live_of(0));

  for (int t = 0; t + 1 < n_tiles; ++t) {
    if (t > 0) {
      __builtin_amdgcn_s_waitcnt(0x0f70);   // this thread's part of tile t + 1 has landed
      __syncthreads();                      // tile t + 1 complete; tile t - 1 released
    }
    if ((t % TOK_REFILL) == 1 && t > TOK_REFILL && (t - 1 + TOK_REFILL) < n_tiles) {
      const int base = (t - 1 + TOK_REFILL) * TILE;
#pragma unroll
      for (int k = 0; k < 2; ++k)
        s_tok[(base + tid + 256 * k) & (TOK_RING - 1)] = ring_value(p0 + base + tid + 256 * k, ring_v[k]);
    }
    if ((t % TOK_REFILL) == 0 && t >= TOK_REFILL && (t + TOK_REFILL) < n_tiles) {
      const int base = (t + TOK_REFILL) * TILE;
#pragma unroll
      for (int k = 0; k < 2; ++k) ring_v[k] = ring_fetch(p0 + base + tid + 256 * k);
    }
    // the gather of tile t + 2 also runs past the end: it then reloads rows
    // (of token 0) into the buffer of tile t - 1, which nothing reads again
    const int bg = (t + 2) % KT_NBUF;
    if (wvalid) {
      tile_step(t % KT_NBUF, (t + 1) % KT_NBUF, bg, live_of(t + 1), t + 2);
    } else {
      issue(t + 2, bg);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);   // no gather left in flight
  if (n_tiles > 0 && wvalid) pv_last((n_tiles - 1) % KT_NBUF);
  if (!hvalid) return;

  // accumulator (db, j) holds dim 32 db + 8 (j >> 2) + 4 h + (j & 3) of head `head`
  if (p.n_split == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const int64_t ob = (row * p.Hq + head) * MLA_DV + 4 * h;
#pragma unroll
    for (int db = 0; db < 16; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        store4(p.out, p.o_dtype, ob + 32 * db + 8 * a, o[db][4 * a] * inv, o[db][4 * a + 1] * inv,
               o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv);
  } else {
    float* pp = p.part + ((row * p.n_split + sp) * p.Hq + head) * (MLA_DV + 2);
#pragma unroll
    for (int db = 0; db < 16; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<f32x4_t*>(pp + 32 * db + 8 * a + 4 * h) =
            f32x4_t{o[db][4 * a], o[db][4 * a + 1], o[db][4 * a + 2], o[db][4 * a + 3]};
    if (h == 0) {
      pp[MLA_DV] = m_run;
      pp[MLA_DV + 1] = l_run;
    }
  }
}

// ============================================================== GQA kernel ==

constexpr int GQA_D = 128;
constexpr int GVROW = TILE + 4;
constexpr size_t GQA_LDS = 4 * (GQA_D * GVROW) * 2 + TILE * 4 + 64 + MAX_BLOCKS * 4;

// One workgroup = one query row x one stream chunk x 4 KV groups; wave w owns
// KV group g = 4 * blockIdx.y + w and its G <= 16 query heads (MFMA columns,
// padded to 16).  K fragments come straight from the cache rows; each wave
// transposes its V tile through a private LDS region.
__global__ __launch_bounds__(256, 2) void attn_gqa_kernel(AttnParams p) {
  extern __shared__ __align__(16) uint8_t s_raw[];
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  uint16_t* s_vt = reinterpret_cast<uint16_t*>(s_raw) + wid * (GQA_D * GVROW);
  int32_t* s_tok = reinterpret_cast<int32_t*>(reinterpret_cast<uint16_t*>(s_raw) + 4 * GQA_D * GVROW);
  uint32_t* s_scr = reinterpret_cast<uint32_t*>(s_tok + TILE);
  int32_t* s_blk = reinterpret_cast<int32_t*>(s_scr + 16);

  const int64_t row = blockIdx.x / p.n_split;
  const int sp = blockIdx.x % p.n_split;
  const int s = static_cast<int>(row / p.n_q);
  const StreamInfo si = stream_setup<4>(p, row, s_blk, s_scr);
  int64_t p0, p1;
  split_range(p, sp, si.len, &p0, &p1);

  const int G = p.Hq / p.Hkv;
  const int g = blockIdx.y * 4 + wid;
  const bool gvalid = g < p.Hkv;
  const int col = lane & 15, quad = lane >> 4;
  const bool hvalid = gvalid && col < G;
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
  const uint16_t* kbase = static_cast<const uint16_t*>(p.k) + s * p.k_seq + (gvalid ? g : 0) * p.k_head;
  const uint16_t* vbase = static_cast<const uint16_t*>(p.v) + s * p.v_seq + (gvalid ? g : 0) * p.v_head;

  for (int64_t t0 = p0; t0 < p1; t0 += TILE) {
    __syncthreads();   // s_tok of the previous tile is no longer read
    if (tid < TILE) s_tok[tid] = static_cast<int32_t>(t0 + tid < p1 ? stream_token(p, row, si, s_blk, t0 + tid) : -1);
    __syncthreads();
    bool any = false;
#pragma unroll
    for (int r = 0; r < TILE; ++r) any |= s_tok[r] >= 0;
    if (!any || !gvalid) continue;

    // V tile: lane loads token (lane & 31), dims [64 * (lane >> 5), +64), writes V^T
    {
      const int vt = lane & 31, vh = lane >> 5;
      const int64_t tok = s_tok[vt];
      const uint16_t* vr = vbase + (tok >= 0 ? tok : 0) * p.v_tok + 64 * vh;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4_t v = tok >= 0 ? *reinterpret_cast<const u32x4_t*>(vr + 8 * i) : u32x4_t{0u, 0u, 0u, 0u};
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          s_vt[(64 * vh + 8 * i + jj) * GVROW + vt] = static_cast<uint16_t>(wv[jj >> 1] >> (16 * (jj & 1)));
      }
    }
    // S^T = K (32 keys x 128) . Q^T (128 x 16 heads): two 16-key blocks
    f32x4_t sacc[2] = {f32x4_t{}, f32x4_t{}};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int64_t tok = s_tok[16 * mb + col];
      const uint16_t* kr = kbase + (tok >= 0 ? tok : 0) * p.k_tok;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4_t a = tok >= 0 ? *reinterpret_cast<const u32x4_t*>(kr + 32 * ks + 8 * quad) : u32x4_t{0u, 0u, 0u, 0u};
        sacc[mb] = mfma16x16x32_bf16(a, qf[ks], sacc[mb]);
      }
    }
    // accumulator (mb, j) holds key 16 mb + 4 quad + j of head column `col`
    float sv[8];
    float tmax = NEG_INF;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = 16 * (j >> 2) + 4 * quad + (j & 3);
      sv[j] = s_tok[key] >= 0 ? sacc[j >> 2][j & 3] : NEG_INF;
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
      const float b = m_run == NEG_INF ? 0.f : exp2f(fmaf(sv[j + 1], c2, -mb_));
      pk[j >> 1] = pack_bf16x2(a, b);
      pl[j >> 1] = pack_bf16x2(a - bf16_to_f32(static_cast<uint16_t>(pk[j >> 1] & 0xffffu)),
                               b - bf16_to_f32(static_cast<uint16_t>(pk[j >> 1] >> 16)));
      psum += a + b;
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run += psum;
    // P^T operand: slot (quad, j) <-> key 4 quad + j (j < 4), 16 + 4 quad + j - 4 (j >= 4)
    const u32x4_t pb = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
    const u32x4_t pr = u32x4_t{pl[0], pl[1], pl[2], pl[3]};
    __builtin_amdgcn_s_waitcnt(0);   // V^T writes of this wave are visible to its own reads
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint16_t* vr = s_vt + (16 * db + col) * GVROW + 4 * quad;
      const u32x2_t a0 = *reinterpret_cast<const u32x2_t*>(vr);
      const u32x2_t a1 = *reinterpret_cast<const u32x2_t*>(vr + 16);
      const u32x4_t va = u32x4_t{a0.x, a0.y, a1.x, a1.y};
      o[db] = mfma16x16x32_bf16(va, pb, o[db]);
      o[db] = mfma16x16x32_bf16(va, pr, o[db]);
    }
    __builtin_amdgcn_wave_barrier();
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
    float* pp = p.part + ((row * p.n_split + sp) * p.Hq + head) * (GQA_D + 2);
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) pp[16 * db + 4 * quad + j] = o[db][j];
    if (quad == 0) {
      pp[GQA_D] = m_run;
      pp[GQA_D + 1] = l_run;
    }
  }
}

// ============================================================== f32 kernel ==

constexpr size_t F32_LDS = 64 * 4 * 2 + 64 + MAX_BLOCKS * 4;

// One wave per (query row, head, chunk).  64 tokens at a time: lane t scores
// token t of the batch, the batch softmax updates the running state, then lane
// t accumulates output dims t, t + 64, ...
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnParams p) {
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
      for (int i = 0; i < p.Dk; ++i) d = fmaf(Q[i], kr[i], d);
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
    for (int u = 0; u < 64; ++u) {
      const int64_t tk = s_t[u];
      if (tk < 0) continue;
      const float* vr = V + tk * p.v_tok;
      const float pu = s_p[u];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < p.Dv) acc[i] = fmaf(pu, vr[lane + 64 * i], acc[i]);
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
    float* pp = p.part + ((row * p.n_split + sp) * p.Hq + h) * (p.Dv + 2);
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i < p.Dv) pp[lane + 64 * i] = acc[i];
    if (lane == 0) {
      pp[p.Dv] = m_run;
      pp[p.Dv + 1] = l_run;
    }
  }
}

// ========================================================= split combine ==

// One workgroup per (row, head): merges the partials of the splits in order.
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnParams p) {
  const int64_t rh = blockIdx.x;
  const int64_t row = rh / p.Hq;
  const int h = static_cast<int>(rh % p.Hq);
  const int W = p.Dv + 2;
  const float* base = p.part + (row * p.n_split * p.Hq + h) * static_cast<int64_t>(W);
  const int64_t sstride = static_cast<int64_t>(p.Hq) * W;
  float M = NEG_INF;
  for (int c = 0; c < p.n_split; ++c) M = fmaxf(M, base[c * sstride + p.Dv]);
  float L = 0.f;
  if (M != NEG_INF)
    for (int c = 0; c < p.n_split; ++c) {
      const float mc = base[c * sstride + p.Dv];
      if (mc != NEG_INF) L += exp2f((mc - M) * p.scale_log2) * base[c * sstride + p.Dv + 1];
    }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int d = threadIdx.x; d < p.Dv; d += blockDim.x) {
    float acc = 0.f;
    if (M != NEG_INF)
      for (int c = 0; c < p.n_split; ++c) {
        const float mc = base[c * sstride + p.Dv];
        if (mc != NEG_INF) acc += exp2f((mc - M) * p.scale_log2) * base[c * sstride + d];
      }
    const int64_t off = (row * p.Hq + h) * p.Dv + d;
    if (p.o_dtype == DSA_F32) static_cast<float*>(p.out)[off] = acc * inv;
    else static_cast<uint16_t*>(p.out)[off] = f32_to_bf16(acc * inv);
  }
}

// ================================================================== host ==

void attn_plan(AttnParams& p, int64_t list_len) {
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  int64_t wgs;   // workgroups per split
  int64_t target;
  if (p.family == ATTN_MLA) {
    wgs = rows * ((p.Hq + 127) / 128);
    target = 512;
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
}

size_t attn_workspace_bytes(const AttnParams& p) {
  if (p.n_split <= 1) return 0;
  return static_cast<size_t>(p.S) * p.n_q * p.n_split * p.Hq * (p.Dv + 2) * sizeof(float);
}

hipError_t launch_attention(const AttnParams& p, hipStream_t st, hipEvent_t before_combine) {
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  hipError_t e;
  if (p.family == ATTN_MLA) {
    static bool attr = false;
    if (!attr) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_mla_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(MLA_LDS));
      if (e != hipSuccess) return e;
      attr = true;
    }
    hipLaunchKernelGGL(attn_mla_kernel, dim3(static_cast<unsigned>(rows * p.n_split), (p.Hq + 127) / 128),
                       dim3(64 * MLA_WAVES), MLA_LDS, st, p);
  } else if (p.family == ATTN_GQA) {
    static bool attr = false;
    if (!attr) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_gqa_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(GQA_LDS));
      if (e != hipSuccess) return e;
      attr = true;
    }
    hipLaunchKernelGGL(attn_gqa_kernel, dim3(static_cast<unsigned>(rows * p.n_split), (p.Hkv + 3) / 4),
                       dim3(256), GQA_LDS, st, p);
  } else {
    hipLaunchKernelGGL(attn_f32_kernel, dim3(static_cast<unsigned>(rows * p.Hq * p.n_split)), dim3(64),
                       F32_LDS, st, p);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (before_combine && (e = hipEventRecord(before_combine, st)) != hipSuccess) return e;
  if (p.n_split > 1) {
    hipLaunchKernelGGL(attn_combine_kernel, dim3(static_cast<unsigned>(rows * p.Hq)), dim3(128), 0, st, p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace dsa
