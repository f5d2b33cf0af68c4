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
constexpr int KT_CHUNKS = MLA_DK / 8;              // 16-byte chunks of data per gathered row (72)
constexpr int KT_SLOTS = KT_CHUNKS + 2;            // per LDS row, with a 32-byte pad (74)
constexpr int KT_ROW = KT_SLOTS * 16;              // 1184 B: rows start 8 banks apart
constexpr int KT_BYTES = TILE * KT_ROW;            // one gathered tile
constexpr int KT_INSTR = TILE * KT_SLOTS / 64;     // wave-wide 1 KB loads per tile (37)
constexpr int MLA_WAVES = 8;
constexpr size_t MLA_LDS = 2 * KT_BYTES + 3 * TILE * 4 + 64 + MAX_BLOCKS * 4;

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// One wave-wide global -> LDS load: lane L copies 16 bytes from its `src` to
// LDS byte address lds_base + 16 L (lds_base wave-uniform).  Issued as inline
// assembly so that the compiler does not treat every later LDS read as a
// possible alias of the in-flight copy; the caller waits (vmcnt) and
// synchronises before the destination is read.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base) : "memory", "m0");
}

// Workgroup barrier that waits for this thread's LDS accesses only (not for
// outstanding global memory operations, such as global -> LDS loads of a tile
// that nobody reads before the next full barrier).
__device__ __forceinline__ void barrier_lds_only() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// Physical 16-byte slot of data chunk c in row r: the chunks of rows 4..7 of
// every 8 are swapped pairwise (c ^ 1), so that 8 consecutive rows read at one
// column (16-byte reads) and 4 consecutive rows read at 4 neighbouring 8-byte
// columns (transposing reads) both spread over all 32 banks.
__device__ __forceinline__ int kt_slot(int r, int c) { return c ^ ((r >> 2) & 1); }

// One workgroup = one query row x one stream chunk x 128 heads, 8 waves; wave
// w owns heads 16 w .. 16 w + 15 and all 576 contraction dims.  Per tile of 32
// gathered latent rows:
//   S^T (32 keys x 16 heads) = K_tile . Q^T on 16x16x32 MFMAs, K fragments
//       read from the LDS tile, Q in registers
//   online softmax over the 32 keys of each head (in-lane + two swaps); the
//       running max is only raised when it grows by more than 2^8 in weight,
//       and the weights enter the PV product as a bf16 high part plus a bf16
//       residual, so they stay exact to ~2^-17 even when they exceed 1
//   O^T (512 dims x 16 heads) += V^T . P^T: V^T fragments come straight from
//       the key-major tile through the transposing LDS read; P^T is the S^T
//       accumulator layout
// Tiles are gathered with direct global -> LDS loads, double buffered.
__global__ __launch_bounds__(512, 1) void attn_mla_kernel(AttnParams p) {
  extern __shared__ __align__(16) uint8_t s_raw[];
  uint8_t* s_kb = s_raw;                                                    // 2 tiles
  int32_t* s_tok = reinterpret_cast<int32_t*>(s_raw + 2 * KT_BYTES);        // [3][32]
  uint32_t* s_scr = reinterpret_cast<uint32_t*>(s_tok + 3 * TILE);
  int32_t* s_blk = reinterpret_cast<int32_t*>(s_scr + 16);

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, quad = lane >> 4;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar registers
  const int64_t row = blockIdx.x / p.n_split;
  const int sp = blockIdx.x % p.n_split;
  const int s = static_cast<int>(row / p.n_q);
  const StreamInfo si = stream_setup<MLA_WAVES>(p, row, s_blk, s_scr);
  int64_t p0, p1;
  split_range(p, sp, si.len, &p0, &p1);
  const int n_tiles = static_cast<int>((p1 - p0 + TILE - 1) / TILE);

  const int head0 = blockIdx.y * 128 + wid * 16;
  const bool hvalid = head0 < p.Hq;   // Hq is a multiple of 16
  const int head = head0 + col;

  u32x4_t qf[18];
  {
    const uint16_t* qr = static_cast<const uint16_t*>(p.q) + (row * p.Hq + (hvalid ? head : 0)) * MLA_DK;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks)
      qf[ks] = hvalid ? *reinterpret_cast<const u32x4_t*>(qr + 32 * ks + 8 * quad) : u32x4_t{0u, 0u, 0u, 0u};
  }
  f32x4_t o[32];
#pragma unroll
  for (int db = 0; db < 32; ++db) o[db] = f32x4_t{};
  float m_run = NEG_INF, l_run = 0.f;
  const float c2 = p.scale_log2;
  const uint16_t* kseq = static_cast<const uint16_t*>(p.k) + s * p.k_seq;

  // gather of one tile: 37 wave-instructions of 64 x 16 B; lane L of
  // instruction I fills physical slot 64 I + L of the tile (pad slots reload
  // the row's first chunk)
  constexpr int MAXI = (KT_INSTR + MLA_WAVES - 1) / MLA_WAVES;   // 5
  const uint32_t kb_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)s_kb));
  const char* kseq_b = reinterpret_cast<const char*>(kseq);
  const uint32_t pitch = static_cast<uint32_t>(p.k_tok) * 2u;   // bytes per token row (< 4 GiB per sequence)
  auto issue = [&](int t, int buf) {
    const int32_t* tk = s_tok + (t % 3) * TILE;
    // recomputed at every call: keeping these per-lane constants live across
    // the tile loop would cost registers the MFMA operands need
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = 0; k < MAXI; ++k) {
      const int I = wid + MLA_WAVES * k;
      if (I < KT_INSTR) {
        const int q = 64 * I + ln;
        const int r = q / KT_SLOTS, pc = q - KT_SLOTS * r;
        const int c = pc < KT_CHUNKS ? kt_slot(r, pc) : 0;
        const int32_t tok = tk[r];
        const uint32_t off = static_cast<uint32_t>(tok >= 0 ? tok : 0) * pitch + 16u * static_cast<uint32_t>(c);
        dma16(kseq_b + off, __builtin_amdgcn_readfirstlane(kb_lds + buf * KT_BYTES + 1024 * I));
      }
    }
  };
  // token ids run two tiles ahead of their use: lane < 32 of wave 0 loads the
  // raw idx entry of tile t + 2 (from a clamped position, unconditionally, so
  // nothing waits for it) while tile t is computed, and validates it when it
  // stores it one tile later
  const bool token_mode = p.idx != nullptr && p.c == 1;
  auto fetch = [&](int64_t pos) -> int32_t {
    return token_mode ? p.idx[row * p.k_sel + (pos < p1 ? pos : p1 - 1)] : 0;
  };
  auto store_token = [&](int slot, int64_t pos, int32_t raw) {
    int32_t t = -1;
    if (pos < p1) {
      if (token_mode) t = (raw >= 0 && raw < si.n_vis) ? raw : -1;
      else t = static_cast<int32_t>(stream_token(p, row, si, s_blk, pos));
    }
    s_tok[slot * TILE + tid] = t;
  };
  int32_t pending = 0;
  if (tid < TILE && n_tiles > 0) {
    store_token(0, p0 + tid, fetch(p0 + tid));
    pending = fetch(p0 + TILE + tid);
  }
  __syncthreads();
  if (n_tiles > 0) issue(0, 0);

  // per-lane byte offsets inside a tile (the swizzle bit of a row depends on
  // row bits 2, which the 16-row and 4-row groups below never change)
  const int sw = (col >> 2) & 1;
  const uint32_t s_off = col * KT_ROW + 16 * (quad ^ sw);                   // S: row col (+16 mb), chunk 4 ks + quad
  const int tm = col >> 2, tr = col & 3;
  const uint32_t v_off = (4 * quad + tm) * KT_ROW + 16 * ((tr >> 1) ^ (quad & 1)) + 8 * (tr & 1);  // PV

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (tid < TILE) store_token((t + 1) % 3, p0 + static_cast<int64_t>(t + 1) * TILE + tid, pending);
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this thread's part of tile t has landed
    __syncthreads();                      // tile t complete; tile t-1 no longer read
    if (t + 1 < n_tiles) issue(t + 1, buf ^ 1);
    if (tid < TILE) pending = fetch(p0 + static_cast<int64_t>(t + 2) * TILE + tid);
    __builtin_amdgcn_sched_barrier(0);

    // live entries of the tile as a bit mask (uniform)
    const int32_t* tk = s_tok + (t % 3) * TILE;
    const uint64_t live = __ballot(lane < TILE && tk[lane] >= 0) & 0xffffffffull;
    if (live == 0 || !hvalid) continue;

    const uint8_t* kt = s_kb + buf * KT_BYTES;
    f32x4_t sacc[2] = {f32x4_t{}, f32x4_t{}};
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(kt + s_off + mb * 16 * KT_ROW + 64 * ks);
        sacc[mb] = mfma16x16x32_bf16(a, qf[ks], sacc[mb]);
      }
    }
    // accumulator (mb, j) holds key 16 mb + 4 quad + j of head `col`
    float sv[8];
    float tmax = NEG_INF;
    const uint32_t lm = static_cast<uint32_t>(live) >> (4 * quad);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sv[j] = ((lm >> (16 * (j >> 2) + (j & 3))) & 1u) ? sacc[j >> 2][j & 3] : NEG_INF;
      tmax = fmaxf(tmax, sv[j]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    if (m_run == NEG_INF) {
      m_run = tmax;
    } else if ((tmax - m_run) * c2 > 8.f) {
      const float alpha = __builtin_amdgcn_exp2f((m_run - tmax) * c2);
      m_run = tmax;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 32; ++db) o[db] *= alpha;
    }
    const float mb_ = m_run * c2;
    uint32_t pk[4], pl[4];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float x0 = __builtin_amdgcn_exp2f(fmaf(sv[j], c2, -mb_));
      const float x1 = __builtin_amdgcn_exp2f(fmaf(sv[j + 1], c2, -mb_));
      pk[j >> 1] = pack_bf16x2(x0, x1);
      pl[j >> 1] = pack_bf16x2(x0 - bf16_to_f32(static_cast<uint16_t>(pk[j >> 1] & 0xffffu)),
                               x1 - bf16_to_f32(static_cast<uint16_t>(pk[j >> 1] >> 16)));
      psum += x0 + x1;
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run += psum;
    // P^T slot (quad, j) <-> key 4 quad + j (j < 4) / 16 + 4 quad + j - 4 (j >= 4)
    const u32x4_t pb = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
    const u32x4_t pr = u32x4_t{pl[0], pl[1], pl[2], pl[3]};
    // V^T fragment of dim block db: lane (quad, j) needs dim 16 db + j for keys
    // 4 quad + {0..3} and 16 + 4 quad + {0..3}.  The transposing read hands lane
    // j of a 16-lane group element j % 4 of the rows addressed by lanes
    // j / 4 + 4 m, so lane 4 m + r addresses key 4 quad + m, dims 16 db + 4 r.
    const uint8_t* vb = kt + v_off;
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      const uint8_t* a0 = vb + 32 * db;
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(const_cast<uint8_t*>(a0)));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(const_cast<uint8_t*>(a0 + 16 * KT_ROW)));
      const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2v = __builtin_bit_cast(u32x2_t, hi);
      const u32x4_t va = u32x4_t{l2.x, l2.y, h2v.x, h2v.y};
      o[db] = mfma16x16x32_bf16(va, pb, o[db]);
      o[db] = mfma16x16x32_bf16(va, pr, o[db]);
    }
  }
  if (!hvalid) return;

  // accumulator (db, j) holds dim 16 db + 4 quad + j of head `col`
  if (p.n_split == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const int64_t ob = (row * p.Hq + head) * MLA_DV;
#pragma unroll
    for (int db = 0; db < 32; ++db)
      store4(p.out, p.o_dtype, ob + 16 * db + 4 * quad, o[db][0] * inv, o[db][1] * inv, o[db][2] * inv,
             o[db][3] * inv);
  } else {
    float* pp = p.part + ((row * p.n_split + sp) * p.Hq + head) * (MLA_DV + 2);
#pragma unroll
    for (int db = 0; db < 32; ++db)
      *reinterpret_cast<f32x4_t*>(pp + 16 * db + 4 * quad) = f32x4_t{o[db][0], o[db][1], o[db][2], o[db][3]};
    if (quad == 0) {
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
