// Lightning-indexer scores on gfx950.
//
//   s(i, u) = sum_h w(i, h) * max(0, q'(i, h) . k(u)) [* k_scale(u)]
//
// (ik_llama.cpp PR #2058, first commit: per-head ReLU of the key/query
// product, weighted head sum, causal mask; llama.cpp mirror commit c88c916636,
// last paragraph: the ReLU acts on each head before the sum.)  The per-head
// products are never written out: they live in MFMA accumulators and the ReLU,
// the head weights and the head sum run in the epilogue (ik_llama_opt log,
// fused indexer top-k commit).
//
// MFMA kernel layout (D = 128, H <= 64):
//   one wave = one query row x one chunk of 32-unit tiles.  Rows of the MFMA
//   are heads (32 per row block, up to 2 blocks), columns are 32 keys, the
//   contraction runs over the 128 dims in 8 steps of 16.  The contraction
//   order is permuted so that lane half h reads dims [64h, 64h + 64) of its
//   key: each lane streams 64 contiguous dims, and the same permutation is
//   applied to q.  The head sum is an in-lane sum of 16 accumulators per row
//   block plus one exchange between lane halves.
#include <type_traits>

#include "dsa_device.h"
#include "dsa_internal.h"
#include "../../include/dsa.h"

namespace dsa {

enum KeyKind { KK_BF16 = 0, KK_F16 = 1, KK_FP8 = 2, KK_F32 = 3 };

template <int KK>
struct KeyTile;  // raw bytes of one lane's 64 dims of one key

template <> struct KeyTile<KK_BF16> { u32x4_t v[8]; };
template <> struct KeyTile<KK_F16> { u32x4_t v[8]; };
template <> struct KeyTile<KK_FP8> { u32x4_t v[4]; };
template <> struct KeyTile<KK_F32> { u32x4_t v[16]; };

template <int KK>
__device__ __forceinline__ void load_key(KeyTile<KK>& t, const void* base, int64_t elem_off, bool ok) {
  constexpr int N = sizeof(KeyTile<KK>) / 16;
  constexpr int ESZ = KK == KK_FP8 ? 1 : (KK == KK_F32 ? 4 : 2);
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(
      static_cast<const char*>(base) + elem_off * ESZ);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (ok) t.v[i] = p[i];
    else t.v[i] = u32x4_t{0u, 0u, 0u, 0u};
  }
}

// B operand(s) of contraction step ks from a lane's key slice.
template <int KK>
__device__ __forceinline__ void key_operand(const KeyTile<KK>& t, int ks, u32x4_t& hi, u32x4_t& lo) {
  if constexpr (KK == KK_BF16 || KK == KK_F16) {
    hi = t.v[ks];
  } else if constexpr (KK == KK_FP8) {
    const u32x4_t v = t.v[ks >> 1];
    const uint32_t a = (ks & 1) ? v.z : v.x;
    const uint32_t b = (ks & 1) ? v.w : v.y;
    u32x2_t ca = fp8x4_to_f16x4_scaled(a), cb = fp8x4_to_f16x4_scaled(b);
    hi = u32x4_t{ca.x, ca.y, cb.x, cb.y};
  } else {
    const u32x4_t a = t.v[2 * ks], b = t.v[2 * ks + 1];
    float f[8] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w),
                  __uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z), __uint_as_float(b.w)};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float h0 = bf16_to_f32(f32_to_bf16(f[2 * i])), h1 = bf16_to_f32(f32_to_bf16(f[2 * i + 1]));
      h[i] = pack_bf16x2(h0, h1);
      l[i] = pack_bf16x2(f[2 * i] - h0, f[2 * i + 1] - h1);
    }
    hi = u32x4_t{h[0], h[1], h[2], h[3]};
    lo = u32x4_t{l[0], l[1], l[2], l[3]};
  }
}

// Unnormalised Walsh-Hadamard butterflies on the 6 in-lane index bits of x[64].
__device__ __forceinline__ void fwht64(float (&x)[64]) {
#pragma unroll
  for (int b = 1; b < 64; b <<= 1) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (i & b) continue;
      const float u = x[i], v = x[i | b];
      x[i] = u + v;
      x[i | b] = u - v;
    }
  }
}

// Query operands of one row for the MFMA kernels: qa[rb][ks][*] is the A
// operand of contraction step ks for heads 32 rb .. 32 rb + 31 (lane n: head
// 32 rb + n, lane half h2: dims 64 h2 + 8 ks .. + 7), after the optional
// rotation and the f16 prescale or bf16 split; wv[rb][j] is the head weight
// (times the undoing scale) of accumulator row j of block rb held by the lane.
// max(x, 0) as one integer max on the bit pattern: a float with the sign bit
// set is a negative integer, and a non-negative float orders as its integer
// (fmaxf would first quiet a NaN input with a second max instruction)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// the sum of x over the two 32-lane halves of the wave, in the same order in
// every lane
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int KK, int QK, int RB, int NQ>
__device__ __forceinline__ void query_operands(const ScoreParams& p, int64_t row, int n, int h2,
                                               u32x4_t (&qa)[RB][8][NQ], float (&wv)[RB][16]) {
  constexpr bool F16OP = (KK == KK_F16 || KK == KK_FP8);
  float fw[RB];
  const int Hh = p.H;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int head = rb * 32 + n;
    if constexpr (QK == 0 && !F16OP && NQ == 1) {   // bf16 q, used as it is
      const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p.q) +
                                                           (row * Hh + (head < Hh ? head : 0)) * 128 + 64 * h2);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qa[rb][ks][0] = head < Hh ? qp[ks] : u32x4_t{0u, 0u, 0u, 0u};
      fw[rb] = head < Hh ? p.w[row * Hh + head] : 0.f;
      continue;
    }
    float x[64];
    if (head < Hh) {
      const int64_t base = (row * Hh + head) * 128 + 64 * h2;
      if constexpr (QK == 0 || QK == 1) {
        const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p.q) + base);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const u32x4_t v = qp[i];
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint16_t lo16 = w4[j] & 0xffffu, hi16 = w4[j] >> 16;
            x[8 * i + 2 * j] = QK == 0 ? bf16_to_f32(lo16) : f16_to_f32(lo16);
            x[8 * i + 2 * j + 1] = QK == 0 ? bf16_to_f32(hi16) : f16_to_f32(hi16);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 64; ++i) x[i] = 0.f;
    }
    if (p.hadamard) {
      fwht64(x);
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const float o = __shfl_xor(x[i], 32, 64);
        x[i] = (h2 == 0 ? x[i] + o : o - x[i]) * 0.088388347648318440550f;   // 1/sqrt(128)
      }
    }
    float factor = 1.f;
    if constexpr (F16OP) {
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(x[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      int e = 0;
      if (amax > 0.f) {
        int E;
        frexpf(amax, &E);
        e = 14 - E;   // amax * 2^e < 2^14: inside the f16 range with headroom
      }
      factor = ldexpf(1.f, -e);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        uint32_t wv4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          wv4[j] = pack_f16x2(ldexpf(x[8 * ks + 2 * j], e), ldexpf(x[8 * ks + 2 * j + 1], e));
        qa[rb][ks][0] = u32x4_t{wv4[0], wv4[1], wv4[2], wv4[3]};
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        uint32_t hv[4], lv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = x[8 * ks + 2 * j], b = x[8 * ks + 2 * j + 1];
          const float ah = bf16_to_f32(f32_to_bf16(a)), bh = bf16_to_f32(f32_to_bf16(b));
          hv[j] = pack_bf16x2(ah, bh);
          lv[j] = pack_bf16x2(a - ah, b - bh);
        }
        qa[rb][ks][0] = u32x4_t{hv[0], hv[1], hv[2], hv[3]};
        if constexpr (NQ == 2) qa[rb][ks][NQ - 1] = u32x4_t{lv[0], lv[1], lv[2], lv[3]};
      }
    }
    float wh = head < Hh ? p.w[row * Hh + head] : 0.f;
    if constexpr (KK == KK_FP8) factor *= 256.f;   // undo the 2^-8 of the fp8 -> f16 map
    fw[rb] = wh * factor;
  }

  // head weight of each accumulator row held by this lane
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < 16; ++j) wv[rb][j] = __shfl(fw[rb], 8 * (j >> 2) + 4 * h2 + (j & 3), 64);

}

template <int KK, int QK, int RB, int NQ>
__global__ __launch_bounds__(256, 2) void score_mfma_kernel(ScoreParams p) {
  constexpr bool F16OP = (KK == KK_F16 || KK == KK_FP8);
  constexpr int NK = KK == KK_F32 ? 2 : 1;
  extern __shared__ uint32_t s_hist[];

  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, h2 = lane >> 5;
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  int64_t row;
  int chunk;
  if (p.chunk_major) {
    const int ncg = (p.n_chunks + 3) >> 2;
    row = blockIdx.x / ncg;
    chunk = (blockIdx.x % ncg) * 4 + wid;
  } else {
    const int64_t nrg = (rows + 3) >> 2;
    row = (nrg - 1 - static_cast<int64_t>(blockIdx.x) / p.n_chunks) * 4 + wid;
    chunk = blockIdx.x % p.n_chunks;
  }
  const bool use_hist = p.hist != nullptr;
  if (use_hist) {
    for (int b = threadIdx.x; b < HIST_BINS; b += 256) s_hist[b] = 0;
    __syncthreads();
  }

  bool active = row < rows && chunk < p.n_chunks;
  const int s = active ? static_cast<int>(row / p.n_q) : 0;
  int64_t n_vis = 0, u_begin = 0, u_end = 0;
  if (active) {
    const int64_t kl = p.kv_len ? p.kv_len[s] : p.n_units * p.c;
    n_vis = visible_tokens(p.q_pos[row], kl, p.n_units * p.c) / p.c;
    u_begin = static_cast<int64_t>(chunk) * p.chunk_tiles * 32;
    u_end = u_begin + static_cast<int64_t>(p.chunk_tiles) * 32;
    if (u_end > p.n_units) u_end = p.n_units;
  }
  const int64_t c_end = n_vis < u_end ? n_vis : u_end;     // compute [u_begin, c_end)
  const bool do_hist = use_hist && n_vis > p.k_out;
  const int64_t nf = (p.c == 1 && p.n_sink < n_vis) ? p.n_sink : (p.c == 1 ? n_vis : 0);

  if (active && c_end > u_begin) {
    u32x4_t qa[RB][8][NQ];
    float wv[RB][16];
    query_operands<KK, QK, RB, NQ>(p, row, n, h2, qa, wv);

    // -------------------------------------------------------- key stream --
    const int64_t key_row0 = static_cast<int64_t>(s) * p.n_units;
    const int t_begin = static_cast<int>(u_begin >> 5);
    const int t_end = static_cast<int>((c_end + 31) >> 5);
    KeyTile<KK> cur, nxt;
    {
      const int64_t u = static_cast<int64_t>(t_begin) * 32 + n;
      load_key<KK>(cur, p.k, (key_row0 + (u < p.n_units ? u : 0)) * 128 + 64 * h2, u < p.n_units);
    }
    for (int t = t_begin; t < t_end; ++t) {
      if (t + 1 < t_end) {
        const int64_t u = static_cast<int64_t>(t + 1) * 32 + n;
        load_key<KK>(nxt, p.k, (key_row0 + (u < p.n_units ? u : 0)) * 128 + 64 * h2, u < p.n_units);
      }
      f32x16_t acc[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        u32x4_t bh, bl;
        key_operand<KK>(cur, ks, bh, bl);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if constexpr (F16OP) {
            acc[rb] = mfma32x32x16_f16(qa[rb][ks][0], bh, acc[rb]);
          } else {
            acc[rb] = mfma32x32x16_bf16(qa[rb][ks][0], bh, acc[rb]);
            if constexpr (NK == 2) acc[rb] = mfma32x32x16_bf16(qa[rb][ks][0], bl, acc[rb]);
            if constexpr (NQ == 2) acc[rb] = mfma32x32x16_bf16(qa[rb][ks][NQ - 1], bh, acc[rb]);
          }
        }
      }
      // epilogue: ReLU, head weight, head sum
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < 16; ++j) part[j & 3] = fmaf(wv[rb][j], relu(acc[rb][j]), part[j & 3]);
      float tot = half_sum((part[0] + part[1]) + (part[2] + part[3]));
      const int64_t u = static_cast<int64_t>(t) * 32 + n;
      if constexpr (KK == KK_FP8) {
        if (u < p.n_units) tot *= p.k_scale[key_row0 + u];
      }
      const float val = u < n_vis ? tot : NEG_INF;
      if (h2 == 0 && u < u_end) p.scores[row * p.n_units + u] = val;
      if (do_hist && h2 == 0 && u >= nf && u < n_vis) atomicAdd(&s_hist[order_key(val) >> 20], 1u);
      cur = nxt;
    }
  }
  if (active && p.fill_invisible) {
    const int64_t f0 = c_end > u_begin ? ((c_end + 31) & ~int64_t(31)) : u_begin;
    for (int64_t u = f0 + lane; u < u_end; u += 64) p.scores[row * p.n_units + u] = NEG_INF;
    // the partially computed last tile already holds -inf past n_vis
  }
  if (use_hist) {
    __syncthreads();
    if (row < rows) {
      uint32_t* g = p.hist + row * HIST_BINS;
      for (int b = threadIdx.x; b < HIST_BINS; b += 256) {
        const uint32_t v = s_hist[b];
        if (v) atomicAdd(g + b, v);
      }
    }
  }
}

// Prefill variant (n_q a multiple of 4, no histogram): one workgroup = 4
// consecutive query rows of one sequence (one wave each) x one chunk of
// 32-key tiles.  The key tiles are gathered once per workgroup into LDS with
// direct global -> LDS loads in pairs (four tile buffers: one pair is
// computed while the next lands, one barrier per pair), and read by all four
// waves.  Three workgroups share a CU (148 registers, 48 KB of
// LDS), so that three waves per SIMD interleave their products and
// epilogues; with a rotated or non-bf16 q split into two operands, two
// workgroups (more registers).  The scores of the chunk
// collect in LDS and leave in one coalesced pass at the end (so that no store
// sits between the tile loads in the memory queue).  Tile layout: key row r
// (256 bytes, 2-byte keys, D = 128) keeps its 16-byte chunk c in slot
// c ^ (r & 15), so that a wave's B-operand read (lane n: row n, chunk
// 8 h2 + ks) is free of LDS bank conflicts.
constexpr int SC_NBUF = 4;                      // tiles: a pair computed, a pair in flight
constexpr int SC_MAX_TILES = 32;                // chunk_tiles bound for this kernel
// 2-byte keys: 256-byte rows; f32 keys (pooled blocks): 512-byte rows, two
// workgroups per CU
template <int KK> struct TiledGeom {
  static constexpr int ROW = KK == KK_F32 ? 512 : 256;   // bytes per key row
  static constexpr int TB = 32 * ROW;                     // bytes per tile
  static constexpr int NLD = 8 * ROW / 1024;              // 1 KB gather loads per wave and tile
  static constexpr size_t LDS = SC_NBUF * TB + 4 * SC_MAX_TILES * 32 * 4 + 16;
};

typedef __attribute__((address_space(3))) void sc_lds_void_t;

__device__ __forceinline__ void sc_dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}

template <int KK, int QK, int RB, int NQ>
__global__ __launch_bounds__(256, NQ == 2 || KK == KK_F32 ? 2 : 3) void score_tiled_kernel(ScoreParams p) {
  static_assert(KK == KK_BF16 || KK == KK_F16 || KK == KK_F32, "2- or 4-byte keys");
  using G = TiledGeom<KK>;
  constexpr bool F16OP = KK == KK_F16;
  constexpr int NK = KK == KK_F32 ? 2 : 1;   // key operands a step: f32 keys as bf16 high part + residual
  extern __shared__ __align__(16) uint8_t s_raw[];
  uint8_t* s_kt = s_raw;                                                  // SC_NBUF tiles
  float* s_sc = reinterpret_cast<float*>(s_raw + SC_NBUF * G::TB);       // [4][chunk_tiles * 32]
  int32_t* s_tend = reinterpret_cast<int32_t*>(s_sc + 4 * SC_MAX_TILES * 32);

  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 31, h2 = lane >> 5;
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  // Workgroups go to the 8 XCDs in turn (block b to XCD b % 8), and inside an
  // XCD to its 4 shader engines in turn.  XCD x takes row groups x, x + 8,
  // x + 16, ... (the longest rows first), each with all of its chunks back to
  // back, so that the causal work is spread evenly over the XCDs and the
  // chunks of a row group find its q in the same L2; the chunk order turns
  // by one from one row group to the next, so that no shader engine always
  // draws the same chunk (the causal mask makes the late chunks the short
  // ones).
  const int64_t nrg = rows >> 2;
  const int64_t jx = static_cast<int64_t>(blockIdx.x >> 3);
  const int64_t gl = jx / p.n_chunks;
  const int64_t g = gl * 8 + (blockIdx.x & 7);
  if (g >= nrg) return;   // the padding of the last round (whole workgroup)
  const int64_t row = (nrg - 1 - g) * 4 + wid;
  const int chunk = static_cast<int>((jx % p.n_chunks + gl) % p.n_chunks);
  const int s = static_cast<int>(row / p.n_q);   // the same for the 4 rows (n_q % 4 == 0)
  const int64_t kl = p.kv_len ? p.kv_len[s] : p.n_units * p.c;
  const int64_t n_vis = visible_tokens(p.q_pos[row], kl, p.n_units * p.c) / p.c;
  const int64_t u_begin = static_cast<int64_t>(chunk) * p.chunk_tiles * 32;
  int64_t u_end = u_begin + static_cast<int64_t>(p.chunk_tiles) * 32;
  if (u_end > p.n_units) u_end = p.n_units;
  const int64_t c_end = n_vis < u_end ? n_vis : u_end;   // this row computes [u_begin, c_end)
  const int t_own = c_end > u_begin ? static_cast<int>((c_end - u_begin + 31) >> 5) : 0;
  if (lane == 0) s_tend[wid] = t_own;
  __syncthreads();
  const int n_t = max(max(s_tend[0], s_tend[1]), max(s_tend[2], s_tend[3]));   // tiles of the workgroup

  // gather of tile T into slot T % SC_NBUF: wave w loads rows 8 w .. 8 w + 7
  // (NLD 1 KB loads; lane L of load i: row 8 w + (1024 i + 16 L) / ROW, the
  // 16-byte slot (16 L % ROW) / 16 of that row)
  const uint32_t kt_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((sc_lds_void_t*)s_kt));
  const char* kbase = static_cast<const char*>(p.k) + static_cast<int64_t>(s) * p.n_units * G::ROW;
  // lane parts of the gather (row r of the tile, the chunk that belongs in
  // its swizzled slot) and the tile base; rows past the keys read the last row
  const uint32_t n_units32 = static_cast<uint32_t>(p.n_units), u_begin32 = static_cast<uint32_t>(u_begin);
  constexpr int LPR = G::ROW / 16;   // lanes per row of a load
  uint32_t g_r[G::NLD], g_sl[G::NLD];
#pragma unroll
  for (int i = 0; i < G::NLD; ++i) {
    const uint32_t r = 8 * wid + (1024 / G::ROW) * i + lane / LPR;
    g_r[i] = r;
    g_sl[i] = 16u * ((lane & (LPR - 1)) ^ (r & 15));
  }
  auto issue = [&](int T) __attribute__((always_inline)) {
    const uint32_t t0 = u_begin32 + 32u * static_cast<uint32_t>(T);
#pragma unroll
    for (int i = 0; i < G::NLD; ++i) {
      uint32_t u = t0 + g_r[i];
      u = u < n_units32 ? u : n_units32 - 1;   // past the end: any valid row, never used
      sc_dma16(kbase, u * static_cast<uint32_t>(G::ROW) + g_sl[i],
               __builtin_amdgcn_readfirstlane(kt_lds + (T % SC_NBUF) * G::TB + 1024u * (G::NLD * wid + i)));
    }
  };
  if (n_t > 0) issue(0);
  if (n_t > 1) issue(1);

  u32x4_t qa[RB][8][NQ];
  float wv[RB][16];
  if (n_t > 0) query_operands<KK, QK, RB, NQ>(p, row, n, h2, qa, wv);
  // B operand of step ks: row n, dims 64 h2 + 8 ks .. + 7.  2-byte keys:
  // chunk 8 h2 + ks in slot (8 h2 + ks) ^ (n & 15) = ((8 h2) ^ (n & 15)) ^ ks,
  // so the step only flips the low 3 slot bits.  f32 keys: chunks
  // 16 h2 + 2 ks + j (j = 0, 1) in slots 16 h2 + ((n & 15) ^ 2 ks ^ j).
  const uint32_t b_off = KK == KK_F32 ? n * 512u + 16u * (16u * h2 + (n & 15))
                                      : n * 256u + 16u * ((8u * h2) ^ (n & 15));

  auto products = [&](uint32_t kof, f32x16_t (&acc)[RB]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4_t bh, bl;
      if constexpr (KK == KK_F32) {
        KeyTile<KK_F32> kt2;   // the two chunks of step ks, as key_operand reads them
        kt2.v[2 * ks] = *reinterpret_cast<const u32x4_t*>(s_kt + (kof ^ (32u * ks)));
        kt2.v[2 * ks + 1] = *reinterpret_cast<const u32x4_t*>(s_kt + (kof ^ (32u * ks + 16u)));
        key_operand<KK_F32>(kt2, ks, bh, bl);
      } else {
        bh = *reinterpret_cast<const u32x4_t*>(s_kt + (kof ^ (16u * ks)));
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if constexpr (F16OP) {
          acc[rb] = mfma32x32x16_f16(qa[rb][ks][0], bh, acc[rb]);
        } else {
          acc[rb] = mfma32x32x16_bf16(qa[rb][ks][0], bh, acc[rb]);
          if constexpr (NK == 2) acc[rb] = mfma32x32x16_bf16(qa[rb][ks][0], bl, acc[rb]);
          if constexpr (NQ == 2) acc[rb] = mfma32x32x16_bf16(qa[rb][ks][NQ - 1], bh, acc[rb]);
        }
      }
    }
  };
  // ReLU, head weight and head sum (four partial sums, then the lane halves)
  auto epilogue = [&](const f32x16_t (&acc)[RB], int t) __attribute__((always_inline)) {
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < 16; ++j) part[j & 3] = fmaf(wv[rb][j], relu(acc[rb][j]), part[j & 3]);
    const float tot = half_sum((part[0] + part[1]) + (part[2] + part[3]));
    const int32_t u = static_cast<int32_t>(u_begin) + t * 32 + n;
    if (h2 == 0) s_sc[wid * (SC_MAX_TILES * 32) + t * 32 + n] = u < static_cast<int32_t>(n_vis) ? tot : NEG_INF;
  };

  // pairs of tiles: the loads of tiles T + 2, T + 3 run while T, T + 1 are
  // computed; one barrier per pair (before the loads into the slots of
  // T - 2, T - 1)
  for (int T = 0; T < n_t; T += 2) {
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this pair has landed
    __syncthreads();
    if (T + 2 < n_t) issue(T + 2);
    if (T + 3 < n_t) issue(T + 3);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int Tt = T + d;
      if (Tt < t_own) {
        uint32_t kof = (Tt % SC_NBUF) * G::TB + b_off;
        asm volatile("" : "+v"(kof));
        f32x16_t acc0[RB];
        __builtin_amdgcn_s_setprio(1);   // the product chain first; the other waves' epilogues fill the gaps
        products(kof, acc0);
        __builtin_amdgcn_s_setprio(0);
        epilogue(acc0, Tt);
      }
    }
  }
  // write-out: computed tiles, then -inf for the invisible rest when asked
  __syncthreads();
  const int64_t w_end = p.fill_invisible ? u_end : u_begin + static_cast<int64_t>(t_own) * 32 < u_end
                                                       ? u_begin + static_cast<int64_t>(t_own) * 32 : u_end;
  float* orow = p.scores + row * p.n_units;
  for (int64_t u = u_begin + lane; u < w_end; u += 64) {
    const int i = static_cast<int>(u - u_begin);
    orow[u] = i < t_own * 32 ? s_sc[wid * (SC_MAX_TILES * 32) + i] : NEG_INF;
  }
}

// Query operands of the decode stream kernel, prepared once per row instead
// of once per wave (a row's query is shared by every wave that streams its
// keys).  One wave per (row, head), lane l holding dims 2 l and 2 l + 1; the
// rotation runs the butterflies of query_operands in the same order (index
// bit 0 in the lane, bits 1..5 across lanes, bit 6 with the 1/sqrt(128)
// scale), each output the same f32 sum or difference of the same two values,
// so the operands are bit for bit those of query_operands.  Outputs, per row
// r and head block rb (RB = 1 or 2 blocks of 32 heads):
//   qop: u32x4 [r][rb][ks][nq][64]: the operand qa[rb][ks][nq] of stream lane
//        n + 32 h2 (head 32 rb + n, dims 64 h2 + 8 ks .. + 7)
//   qw:  f32 [r][rb][j / 4][64][4]: the head weight wv[rb][j] of each lane
// The same launch clears the top-k histogram and candidate counts.
template <int KK, int QK, int NQ>
__global__ __launch_bounds__(256) void score_prep_kernel(ScoreParams p, uint32_t* cand_cnt) {
  constexpr bool F16OP = (KK == KK_F16 || KK == KK_FP8);
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  const int64_t n_clear = rows * HIST_BINS;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n_clear;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    p.hist[i] = 0;
    if (i < rows) cand_cnt[i] = 0;
  }
  if (p.qop == nullptr) return;
  const int lane = threadIdx.x & 63;
  const int RB = p.H <= 32 ? 1 : 2;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (wave >= rows * RB * 32) return;
  const int64_t row = wave / (RB * 32);
  const int h = static_cast<int>(wave - row * (RB * 32));
  const int rb = h >> 5, hh = h & 31;
  float x0 = 0.f, x1 = 0.f, wh = 0.f;
  uint32_t raw = 0;
  if (h < p.H) {
    raw = reinterpret_cast<const uint32_t*>(p.q)[(row * p.H + h) * 64 + lane];
    const uint16_t lo16 = raw & 0xffffu, hi16 = raw >> 16;
    x0 = QK == 0 ? bf16_to_f32(lo16) : f16_to_f32(lo16);
    x1 = QK == 0 ? bf16_to_f32(hi16) : f16_to_f32(hi16);
    wh = p.w[row * p.H + h];
  }
  if (p.hadamard) {
    {
      const float u = x0, v = x1;
      x0 = u + v;
      x1 = u - v;
    }
#pragma unroll
    for (int b = 1; b <= 32; b <<= 1) {   // the lower index keeps u + v, the upper u - v
      const float o0 = __shfl_xor(x0, b, 64), o1 = __shfl_xor(x1, b, 64);
      const bool up = (lane & b) != 0;
      x0 = up ? o0 - x0 : x0 + o0;
      x1 = up ? o1 - x1 : x1 + o1;
      if (b == 32) {
        x0 *= 0.088388347648318440550f;   // 1/sqrt(128)
        x1 *= 0.088388347648318440550f;
      }
    }
  }
  uint32_t word[NQ];
  float factor = 1.f;
  if constexpr (F16OP) {
    float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    int e = 0;
    if (amax > 0.f) {
      int E;
      frexpf(amax, &E);
      e = 14 - E;   // amax * 2^e < 2^14: inside the f16 range with headroom
    }
    factor = ldexpf(1.f, -e);
    word[0] = pack_f16x2(ldexpf(x0, e), ldexpf(x1, e));
  } else if constexpr (QK == 0 && NQ == 1) {
    word[0] = raw;   // bf16 q, used as it is
  } else {
    const float ah = bf16_to_f32(f32_to_bf16(x0)), bh = bf16_to_f32(f32_to_bf16(x1));
    word[0] = pack_bf16x2(ah, bh);
    word[NQ - 1] = pack_bf16x2(x0 - ah, x1 - bh);
  }
  if constexpr (KK == KK_FP8) factor *= 256.f;   // undo the 2^-8 of the fp8 -> f16 map
  const float fw = wh * factor;
  const int h2 = lane >> 5, ks = (lane & 31) >> 2, j = lane & 3;
  uint32_t* qo = const_cast<uint32_t*>(p.qop) + row * (RB * 8 * NQ * 64 * 4);
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) qo[(((rb * 8 + ks) * NQ + nq) * 64 + hh + 32 * h2) * 4 + j] = word[nq];
  if (lane < 32) {
    float* qw = const_cast<float*>(p.qw) + row * (RB * 4 * 64 * 4);
    const int hw2 = (hh >> 2) & 1;
    qw[((rb * 4 + (hh >> 3)) * 64 + lane + 32 * hw2) * 4 + (hh & 3)] = fw;
  }
}

// Decode variant (rows with the fused top-k histogram, 1- or 2-byte keys):
// one wave per (query row, chunk of 32-key tiles), four chunks of one row per
// workgroup, one wave per SIMD.  Each wave streams its own key tiles with
// coalesced non-temporal loads (every load instruction moves 1 KB of
// contiguous key rows; a lane-per-key load would touch 64 cache lines per
// instruction for 16 bytes each) through a ring of four tiles in registers
// (the loads of three tiles stay in flight while one is stored), and
// writes each tile into one of two LDS buffers from which the B operands are
// read in the MFMA layout.  Row r of a tile keeps its 16-byte chunk c in slot
// c ^ swz(r) (2-byte keys: 256-byte rows, swz(r) = r & 15; fp8: 128-byte
// rows, swz(r) = (r >> 1) & 7), which keeps the B-operand reads free of bank
// conflicts.  Scores collect in LDS and leave in one coalesced pass per wave
// at the end.
template <int KK> struct StreamGeom {
  static constexpr int ROW = KK == KK_FP8 ? 128 : 256;   // bytes per key
  static constexpr int TB = 32 * ROW;                     // bytes per tile
  static constexpr int NLD = TB / 1024;                   // 1 KB loads per tile
};

template <int KK>
constexpr size_t stream_lds_bytes(int chunk_tiles) {
  return HIST_BINS * 4 + 4 * 2 * StreamGeom<KK>::TB + 4 * static_cast<size_t>(chunk_tiles) * 32 * 4;
}

template <int KK>
struct StreamTile {   // one lane's share of a tile in flight: NLD x 16 bytes, plus its fp8 row scale
  u32x4_t v[StreamGeom<KK>::NLD];
  float sc;
};

// fp8 keys: tiles half the size, two workgroups per CU (two waves per SIMD,
// so that one wave's fp8 conversion and epilogue overlap the other's
// products) and a ring of two tiles; 2-byte keys: one workgroup per CU and a
// ring of four tiles
template <int KK> constexpr int stream_occupancy() { return KK == KK_FP8 ? 2 : 1; }

template <int KK, int QK, int RB, int NQ>
__global__ __launch_bounds__(256, stream_occupancy<KK>()) void score_stream_kernel(ScoreParams p) {
  static_assert(KK == KK_BF16 || KK == KK_F16 || KK == KK_FP8, "1- or 2-byte keys");
  using G = StreamGeom<KK>;
  constexpr bool F16OP = (KK == KK_F16 || KK == KK_FP8);
  extern __shared__ __align__(16) uint8_t s_raw[];
  uint32_t* s_hist = reinterpret_cast<uint32_t*>(s_raw);
  uint8_t* s_kt = s_raw + HIST_BINS * 4;                                  // [wave][2][TB]
  float* s_out = reinterpret_cast<float*>(s_kt + 4 * 2 * G::TB);         // [wave][chunk_tiles * 32]

  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 31, h2 = lane >> 5;
  const int ncg = (p.n_chunks + 3) >> 2;
  const int row32 = static_cast<int>(blockIdx.x) / ncg;   // rows * ncg < 2^31 (grid size)
  const int64_t row = row32;
  const int chunk = (static_cast<int>(blockIdx.x) - row32 * ncg) * 4 + wid;
  const int s = row32 / p.n_q;
  const bool active = chunk < p.n_chunks;
  const int tiles_row = static_cast<int>((p.n_units + 31) >> 5);
  // local tile j of this wave is tile chunk + j * n_chunks of the row
  auto tile_of = [&](int j) -> int64_t { return static_cast<int64_t>(chunk) + static_cast<int64_t>(j) * p.n_chunks; };

  // load i of a tile covers the 1 KB of rows 1024 i / ROW ..; lane L takes
  // the 16 bytes that belong at byte 16 L of it: row r = (1024 i + 16 L) / ROW,
  // slot (16 L % ROW) / 16, holding chunk slot ^ swz(r)
  const char* kbase = static_cast<const char*>(p.k) + static_cast<int64_t>(s) * p.n_units * G::ROW;
  const float* sbase = KK == KK_FP8 ? p.k_scale + static_cast<int64_t>(s) * p.n_units : nullptr;
  uint32_t loff[G::NLD];
#pragma unroll
  for (int i = 0; i < G::NLD; ++i) {
    if constexpr (G::ROW == 256) {
      const int r = 4 * i + (lane >> 4);
      loff[i] = static_cast<uint32_t>(r) * 256u + 16u * ((lane & 15) ^ (r & 15));
    } else {
      const int r = 8 * i + (lane >> 3);
      loff[i] = static_cast<uint32_t>(r) * 128u + 16u * ((lane & 7) ^ ((r >> 1) & 7));
    }
  }
  // Every load is unconditional, at an in-range address: rows past the cache
  // reload the tile's last stored row (their scores are never written), and
  // the caller clamps the tile index.  With no predicate on any load, the
  // compiler counts the ring's loads exactly (a wait for the oldest tile
  // only) instead of draining all of them before each LDS store.  The keys
  // are streamed once, so the loads are non-temporal.
  auto load_tile = [&](StreamTile<KK>& tt, int j) __attribute__((always_inline)) {
    const int64_t ut = tile_of(j) * 32;
    const char* tb = kbase + ut * G::ROW;
    const int64_t lim = (p.n_units - ut) * G::ROW;   // bytes of the tile inside the cache (>= one row)
#pragma unroll
    for (int i = 0; i < G::NLD; ++i) {
      const uint32_t o = static_cast<int64_t>(loff[i]) < lim
                             ? loff[i]
                             : static_cast<uint32_t>(lim - G::ROW) + (loff[i] & (G::ROW - 1));
      tt.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(tb + o));
    }
    if constexpr (KK == KK_FP8) tt.sc = sbase[ut + n < p.n_units ? ut + n : p.n_units - 1];
  };
  // The prepared query operands and head weights are loaded first, then the
  // first NR tiles of the chunk (the visible length is not known yet: tiles
  // past it are loaded, never used).  Loads complete in issue order, so the
  // products wait for the query alone while the keys stream.
  u32x4_t qa[RB][8][NQ];
  float wv[RB][16];
  {
    const u32x4_t* qo = reinterpret_cast<const u32x4_t*>(p.qop) + row * (RB * 8 * NQ * 64) + lane;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) qa[rb][ks][nq] = qo[((rb * 8 + ks) * NQ + nq) * 64];
    const u32x4_t* wo = reinterpret_cast<const u32x4_t*>(p.qw) + row * (RB * 4 * 64) + lane;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const u32x4_t t = wo[(rb * 4 + jq) * 64];
        wv[rb][4 * jq] = __uint_as_float(t.x);
        wv[rb][4 * jq + 1] = __uint_as_float(t.y);
        wv[rb][4 * jq + 2] = __uint_as_float(t.z);
        wv[rb][4 * jq + 3] = __uint_as_float(t.w);
      }
  }
  __builtin_amdgcn_sched_barrier(0);
  constexpr int NR = stream_occupancy<KK>() == 2 ? 2 : 4;
  StreamTile<KK> rr[NR];
  const int n_pre = active && chunk < tiles_row ? (tiles_row - chunk + p.n_chunks - 1) / p.n_chunks : 0;
  if (n_pre > 0) {
#pragma unroll
    for (int k = 0; k < NR; ++k) load_tile(rr[k], k < n_pre ? k : n_pre - 1);
  }

  const int32_t qpos = p.q_pos[row];
  const int64_t kl = p.kv_len ? p.kv_len[s] : p.n_units * p.c;
  for (int b = threadIdx.x; b < HIST_BINS; b += 256) s_hist[b] = 0;

  const int64_t n_vis = visible_tokens(qpos, kl, p.n_units * p.c) / p.c;
  const bool do_hist = n_vis > p.k_out;
  const int64_t nf = (p.c == 1 && p.n_sink < n_vis) ? p.n_sink : (p.c == 1 ? n_vis : 0);
  const int t_vis = static_cast<int>((n_vis + 31) >> 5);   // tiles with a visible unit
  const int n_t = active && chunk < t_vis ? (t_vis - chunk + p.n_chunks - 1) / p.n_chunks : 0;

  const uint32_t wbase = static_cast<uint32_t>(wid) * (2 * G::TB);
  auto store_tile = [&](const StreamTile<KK>& tt, int buf) __attribute__((always_inline)) {
    uint8_t* d = s_kt + wbase + buf * G::TB + 16 * lane;
#pragma unroll
    for (int i = 0; i < G::NLD; ++i) *reinterpret_cast<u32x4_t*>(d + 1024 * i) = tt.v[i];
  };
  float* so = s_out + wid * (p.chunk_tiles * 32);
  auto compute = [&](int j, float sc) __attribute__((always_inline)) {
    const uint8_t* kt = s_kt + wbase + (j & 1) * G::TB;
    f32x16_t acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x16_t{};
    if constexpr (G::ROW == 256) {
      uint32_t hx = 8u * h2;
      asm volatile("" : "+v"(hx));
      const uint8_t* kr = kt + n * 256;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4_t bh = *reinterpret_cast<const u32x4_t*>(kr + 16u * ((hx + ks) ^ (n & 15)));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if constexpr (F16OP) {
            acc[rb] = mfma32x32x16_f16(qa[rb][ks][0], bh, acc[rb]);
          } else {
            acc[rb] = mfma32x32x16_bf16(qa[rb][ks][0], bh, acc[rb]);
            if constexpr (NQ == 2) acc[rb] = mfma32x32x16_bf16(qa[rb][ks][NQ - 1], bh, acc[rb]);
          }
        }
      }
    } else {
      uint32_t hx = 4u * h2;
      asm volatile("" : "+v"(hx));
      const uint8_t* kr = kt + n * 128;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(kr + 16u * ((hx + kk) ^ ((n >> 1) & 7)));
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const u32x2_t ca = fp8x4_to_f16x4_scaled(half ? v.z : v.x);
          const u32x2_t cb = fp8x4_to_f16x4_scaled(half ? v.w : v.y);
          const u32x4_t bh = u32x4_t{ca.x, ca.y, cb.x, cb.y};
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) acc[rb] = mfma32x32x16_f16(qa[rb][2 * kk + half][0], bh, acc[rb]);
        }
      }
    }
    // epilogue: ReLU, head weight, head sum
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) part[jj & 3] = fmaf(wv[rb][jj], relu(acc[rb][jj]), part[jj & 3]);
    float tot = half_sum((part[0] + part[1]) + (part[2] + part[3]));
    if constexpr (KK == KK_FP8) tot *= sc;
    const int64_t u = tile_of(j) * 32 + n;
    const float val = u < n_vis ? tot : NEG_INF;
    if (h2 == 0) {
      so[j * 32 + n] = val;
      if (do_hist && u >= nf && u < n_vis) atomicAdd(&s_hist[order_key(val) >> 20], 1u);
    }
  };

  // Tile t sits in ring slot t % NR until it is written into LDS buffer
  // t & 1; step j writes tile j + 1 (loaded NR - 1 steps earlier), refills
  // its slot with tile j + 1 + NR (clamped to the last tile), then computes
  // tile j.  The steps run in whole rounds of NR: past the last tile a step
  // only stores and reloads (the compute is skipped by a uniform branch), so
  // every round issues the same loads and the wait before a store is always
  // for the oldest tile in flight alone.
  float scb[2] = {0.f, 0.f};   // fp8 scales of the tiles in the LDS buffers
  __syncthreads();   // the histogram is clear
  if (n_t > 0) {
    const int last = n_t - 1;
    store_tile(rr[0], 0);
    scb[0] = rr[0].sc;
    load_tile(rr[0], NR < last ? NR : last);
    auto step = [&](auto kc, int j) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr int k1 = (k + 1) % NR;
      store_tile(rr[k1], (k + 1) & 1);   // tile j + 1, over tile j - 1 (read by the previous step)
      scb[(k + 1) & 1] = rr[k1].sc;
      const int jn = j + 1 + NR;
      load_tile(rr[k1], jn < last ? jn : last);
      if (j < n_t) compute(j, scb[k & 1]);
    };
    for (int j = 0; j < n_t; j += NR) {
      step(std::integral_constant<int, 0>{}, j);
      step(std::integral_constant<int, 1>{}, j + 1);
      if constexpr (NR == 4) {
        step(std::integral_constant<int, 2>{}, j + 2);
        step(std::integral_constant<int, 3>{}, j + 3);
      }
    }
  }
  // write-out of the wave's tiles: computed ones, then -inf for the
  // invisible rest when asked
  if (active) {
    float* orow = p.scores + row * p.n_units;
    for (int i = lane; i < n_pre * 32; i += 64) {
      const int j = i >> 5;
      const int64_t u = tile_of(j) * 32 + (i & 31);
      if (u < p.n_units && (j < n_t || p.fill_invisible)) orow[u] = j < n_t ? so[i] : NEG_INF;
    }
  }
  __syncthreads();
  uint32_t* g = p.hist + row * HIST_BINS;
  for (int b = threadIdx.x; b < HIST_BINS; b += 256) {
    const uint32_t v = s_hist[b];
    if (v) atomicAdd(g + b, v);
  }
}

// Generic path: any element types, H <= 128, D <= 256.  One thread per
// (row, unit); the row's (rotated) query and weights sit in LDS.  The key is
// read once per group of 8 heads, in runs of 8 elements (16-byte loads when
// D is a multiple of 8), and each run goes into every head of the group
// before the next is read; each head's dot product still adds its terms in
// dim order.
template <int KD>
__device__ __forceinline__ float key_elem(const void* k, int64_t i) {
  return load_elem(k, i, KD);
}
template <int KD, bool VEC>
__device__ __forceinline__ void key_run8(const void* k, int64_t i, float (&x)[8]) {
  if constexpr (VEC && KD == DSA_F32) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(k) + i);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(k) + i + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = a[j];
      x[4 + j] = b[j];
    }
  } else if constexpr (VEC && (KD == DSA_BF16 || KD == DSA_F16)) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(k) + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t lo = v[j] & 0xffffu, hi = v[j] >> 16;
      x[2 * j] = KD == DSA_BF16 ? bf16_to_f32(lo) : f16_to_f32(lo);
      x[2 * j + 1] = KD == DSA_BF16 ? bf16_to_f32(hi) : f16_to_f32(hi);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = key_elem<KD>(k, i + j);
  }
}

template <int KD, bool VEC>
__global__ __launch_bounds__(256) void score_valu_kernel(ScoreParams p) {
  extern __shared__ __align__(16) float s_q[];   // [H * D] then w[H]
  const int64_t n_ub = (p.n_units + 255) / 256;
  const int64_t row = blockIdx.x / n_ub;
  const int64_t ublk = blockIdx.x % n_ub;
  const int s = static_cast<int>(row / p.n_q);
  const int H = p.H, D = p.D;
  float* s_w = s_q + H * D;
  for (int i = threadIdx.x; i < H * D; i += 256) s_q[i] = load_elem(p.q, row * H * D + i, p.q_dtype);
  for (int i = threadIdx.x; i < H; i += 256) s_w[i] = p.w[row * H + i];
  __syncthreads();
  if (p.hadamard) {   // D == 128: butterflies over the 7 index bits, then 1/sqrt(128)
    for (int b = 1; b < D; b <<= 1) {
      for (int i = threadIdx.x; i < H * D / 2; i += 256) {
        const int h = i / (D / 2), r = i % (D / 2);
        const int lo = (r / b) * 2 * b + (r % b), hi = lo + b;
        const float u = s_q[h * D + lo], v = s_q[h * D + hi];
        s_q[h * D + lo] = u + v;
        s_q[h * D + hi] = u - v;
      }
      __syncthreads();
    }
    for (int i = threadIdx.x; i < H * D; i += 256) s_q[i] *= 0.088388347648318440550f;
    __syncthreads();
  }
  const int64_t kl = p.kv_len ? p.kv_len[s] : p.n_units * p.c;
  const int64_t n_vis = visible_tokens(p.q_pos[row], kl, p.n_units * p.c) / p.c;
  const int64_t u = ublk * 256 + threadIdx.x;
  if (u >= p.n_units) return;
  float val = NEG_INF;
  if (u < n_vis) {
    const int64_t kb = (static_cast<int64_t>(s) * p.n_units + u) * D;
    const int D8 = D & ~7;
    float tot = 0.f;
    for (int h0 = 0; h0 < H; h0 += 8) {
      const int hn = H - h0 < 8 ? H - h0 : 8;   // heads of this group
      float dot[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int d0 = 0; d0 < D8; d0 += 8) {
        float x[8];
        key_run8<KD, VEC>(p.k, kb + d0, x);
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
          if (hh < hn) {
            const float* qh = s_q + (h0 + hh) * D + d0;
#pragma unroll
            for (int j = 0; j < 8; ++j) dot[hh] = fmaf(qh[j], x[j], dot[hh]);
          }
        }
      }
      for (int d = D8; d < D; ++d) {
        const float xk = key_elem<KD>(p.k, kb + d);
#pragma unroll
        for (int hh = 0; hh < 8; ++hh)
          if (hh < hn) dot[hh] = fmaf(s_q[(h0 + hh) * D + d], xk, dot[hh]);
      }
#pragma unroll
      for (int hh = 0; hh < 8; ++hh)
        if (hh < hn) tot = fmaf(s_w[h0 + hh], fmaxf(dot[hh], 0.f), tot);
    }
    if (KD == DSA_FP8_E4M3) tot *= p.k_scale[static_cast<int64_t>(s) * p.n_units + u];
    val = tot;
  }
  p.scores[row * p.n_units + u] = val;
}

bool scores_use_mfma(int q_dtype, int k_dtype, int H, int D) {
  return D == 128 && H <= 64 && (q_dtype == DSA_BF16 || q_dtype == DSA_F16);
}

template <int KK, int QK, int NQ>
static hipError_t launch_mfma_rb(const ScoreParams& p, dim3 grid, size_t lds, hipStream_t st) {
  if (p.H <= 32)
    hipLaunchKernelGGL((score_mfma_kernel<KK, QK, 1, NQ>), grid, dim3(256), lds, st, p);
  else
    hipLaunchKernelGGL((score_mfma_kernel<KK, QK, 2, NQ>), grid, dim3(256), lds, st, p);
  return hipGetLastError();
}

// the tiled prefill kernel covers 2-byte keys, n_q a multiple of 4, no histogram
static bool scores_use_tiled(const ScoreParams& p) {
  return (p.k_dtype == DSA_BF16 || p.k_dtype == DSA_F16 || p.k_dtype == DSA_F32) && p.n_q % 4 == 0 &&
         p.hist == nullptr && p.chunk_tiles <= SC_MAX_TILES &&
         p.n_units * (p.k_dtype == DSA_F32 ? 512 : 256) < (int64_t(1) << 32);   // 32-bit row offsets
}

// the decode stream kernel covers 1- and 2-byte keys on rows with the histogram
bool scores_use_prep(int q_dtype, int k_dtype, int H, int D, int64_t n_units) {
  return scores_use_mfma(q_dtype, k_dtype, H, D) &&
         (k_dtype == DSA_BF16 || k_dtype == DSA_F16 || k_dtype == DSA_FP8_E4M3) &&
         n_units < (int64_t(1) << 24);   // 32-bit row offsets
}
static bool scores_use_stream(const ScoreParams& p) {
  return p.hist != nullptr && p.qop != nullptr && p.chunk_major && p.chunk_tiles <= 32 &&
         scores_use_prep(p.q_dtype, p.k_dtype, p.H, p.D, p.n_units);
}

// operand blocks of the stream kernel: RB head blocks, NQ operands per step
static int prep_rb(int H) { return H <= 32 ? 1 : 2; }
static int prep_nq(int q_dtype, int k_dtype, int hadamard) {
  const bool f16op = k_dtype == DSA_F16 || k_dtype == DSA_FP8_E4M3;
  return !f16op && (q_dtype != DSA_BF16 || hadamard) ? 2 : 1;
}

size_t score_prep_bytes(int64_t rows, int q_dtype, int k_dtype, int H, int hadamard) {
  const size_t per_row = static_cast<size_t>(prep_rb(H)) * (8 * prep_nq(q_dtype, k_dtype, hadamard) + 4) * 64 * 16;
  return (static_cast<size_t>(rows) * per_row + 255) / 256 * 256;
}

void score_prep_bind(ScoreParams& p, void* ws) {
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  const size_t ops = static_cast<size_t>(rows) * prep_rb(p.H) * 8 * prep_nq(p.q_dtype, p.k_dtype, p.hadamard) * 64 * 16;
  p.qop = static_cast<const uint32_t*>(ws);
  p.qw = reinterpret_cast<const float*>(static_cast<const char*>(ws) + ops);
}

template <int KK>
static hipError_t launch_prep_k(const ScoreParams& p, uint32_t* cand_cnt, dim3 grid, hipStream_t st) {
  const bool nq2 = prep_nq(p.q_dtype, p.k_dtype, p.hadamard) == 2;
  if (p.q_dtype == DSA_BF16) {
    if (nq2) hipLaunchKernelGGL((score_prep_kernel<KK, 0, 2>), grid, dim3(256), 0, st, p, cand_cnt);
    else hipLaunchKernelGGL((score_prep_kernel<KK, 0, 1>), grid, dim3(256), 0, st, p, cand_cnt);
  } else {
    if (nq2) hipLaunchKernelGGL((score_prep_kernel<KK, 1, 2>), grid, dim3(256), 0, st, p, cand_cnt);
    else hipLaunchKernelGGL((score_prep_kernel<KK, 1, 1>), grid, dim3(256), 0, st, p, cand_cnt);
  }
  return hipGetLastError();
}

hipError_t launch_score_prep(const ScoreParams& p, uint32_t* cand_cnt, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  int64_t blocks = (rows * HIST_BINS + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (p.qop != nullptr) {
    const int64_t head_blocks = rows * prep_rb(p.H) * 32 / 4;
    if (blocks < head_blocks) blocks = head_blocks;
  }
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (p.k_dtype) {
    case DSA_F16: return launch_prep_k<KK_F16>(p, cand_cnt, grid, st);
    case DSA_FP8_E4M3: return launch_prep_k<KK_FP8>(p, cand_cnt, grid, st);
    default: return launch_prep_k<KK_BF16>(p, cand_cnt, grid, st);
  }
}

template <int KK, int QK, int NQ>
static hipError_t launch_stream_rb(const ScoreParams& p, dim3 grid, hipStream_t st) {
  const size_t lds = stream_lds_bytes<KK>(p.chunk_tiles);
  // the kernel's dynamic LDS limit, set on every call to the largest size any
  // call uses (the same value each time: no state kept between calls, and
  // concurrent calls agree)
  const void* fn = p.H <= 32 ? reinterpret_cast<const void*>(score_stream_kernel<KK, QK, 1, NQ>)
                             : reinterpret_cast<const void*>(score_stream_kernel<KK, QK, 2, NQ>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(stream_lds_bytes<KK>(SC_MAX_TILES)));
  if (e != hipSuccess) return e;
  if (p.H <= 32)
    hipLaunchKernelGGL((score_stream_kernel<KK, QK, 1, NQ>), grid, dim3(256), lds, st, p);
  else
    hipLaunchKernelGGL((score_stream_kernel<KK, QK, 2, NQ>), grid, dim3(256), lds, st, p);
  return hipGetLastError();
}

template <int KK, int QK, int NQ>
static hipError_t launch_tiled_rb(const ScoreParams& p, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  const dim3 grid(static_cast<unsigned>((rows / 4 + 7) / 8 * 8 * p.n_chunks));
  constexpr size_t lds = TiledGeom<KK>::LDS;
  const void* fn = p.H <= 32 ? reinterpret_cast<const void*>(score_tiled_kernel<KK, QK, 1, NQ>)
                             : reinterpret_cast<const void*>(score_tiled_kernel<KK, QK, 2, NQ>);
  if (lds > 65536) {   // set on every call (the same value each time, no state kept between calls)
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  if (p.H <= 32)
    hipLaunchKernelGGL((score_tiled_kernel<KK, QK, 1, NQ>), grid, dim3(256), lds, st, p);
  else
    hipLaunchKernelGGL((score_tiled_kernel<KK, QK, 2, NQ>), grid, dim3(256), lds, st, p);
  return hipGetLastError();
}

// q enters the MFMA as one f16 operand (f16/fp8 keys, after a power-of-two
// prescale) or as bf16; a bf16 q that is not rotated is exact in one bf16
// operand, anything else is split into a bf16 high part and a bf16 residual.
template <int KK>
static hipError_t launch_mfma_q(const ScoreParams& p, dim3 grid, size_t lds, hipStream_t st) {
  constexpr bool F16OP = (KK == KK_F16 || KK == KK_FP8);
  const bool split = !F16OP && (p.q_dtype != DSA_BF16 || p.hadamard);
  if constexpr (KK == KK_BF16 || KK == KK_F16 || KK == KK_FP8) {
    if (scores_use_stream(p)) {
      if (p.q_dtype == DSA_BF16)
        return split ? launch_stream_rb<KK, 0, 2>(p, grid, st) : launch_stream_rb<KK, 0, 1>(p, grid, st);
      return split ? launch_stream_rb<KK, 1, 2>(p, grid, st) : launch_stream_rb<KK, 1, 1>(p, grid, st);
    }
  }
  if constexpr (KK == KK_BF16 || KK == KK_F16 || KK == KK_F32) {
    if (scores_use_tiled(p)) {
      if (p.q_dtype == DSA_BF16)
        return split ? launch_tiled_rb<KK, 0, 2>(p, st) : launch_tiled_rb<KK, 0, 1>(p, st);
      return split ? launch_tiled_rb<KK, 1, 2>(p, st) : launch_tiled_rb<KK, 1, 1>(p, st);
    }
  }
  if (p.q_dtype == DSA_BF16)
    return split ? launch_mfma_rb<KK, 0, 2>(p, grid, lds, st) : launch_mfma_rb<KK, 0, 1>(p, grid, lds, st);
  return split ? launch_mfma_rb<KK, 1, 2>(p, grid, lds, st) : launch_mfma_rb<KK, 1, 1>(p, grid, lds, st);
}

hipError_t launch_scores(ScoreParams p, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(p.S) * p.n_q;
  if (!scores_use_mfma(p.q_dtype, p.k_dtype, p.H, p.D)) {
    const size_t lds = (static_cast<size_t>(p.H) * p.D + p.H) * sizeof(float);
    dim3 grid(static_cast<unsigned>(((p.n_units + 255) / 256) * rows));
    // 16-byte runs when every key row starts 16-byte aligned
    const size_t esz = p.k_dtype == DSA_F32 ? 4 : (p.k_dtype == DSA_FP8_E4M3 ? 1 : 2);
    const bool vec = p.D % 8 == 0 && (reinterpret_cast<uintptr_t>(p.k) & 15) == 0 && (p.D * esz) % 16 == 0;
    switch (p.k_dtype) {
      case DSA_F32:
        if (vec) hipLaunchKernelGGL((score_valu_kernel<DSA_F32, true>), grid, dim3(256), lds, st, p);
        else hipLaunchKernelGGL((score_valu_kernel<DSA_F32, false>), grid, dim3(256), lds, st, p);
        break;
      case DSA_BF16:
        if (vec) hipLaunchKernelGGL((score_valu_kernel<DSA_BF16, true>), grid, dim3(256), lds, st, p);
        else hipLaunchKernelGGL((score_valu_kernel<DSA_BF16, false>), grid, dim3(256), lds, st, p);
        break;
      case DSA_F16:
        if (vec) hipLaunchKernelGGL((score_valu_kernel<DSA_F16, true>), grid, dim3(256), lds, st, p);
        else hipLaunchKernelGGL((score_valu_kernel<DSA_F16, false>), grid, dim3(256), lds, st, p);
        break;
      default: hipLaunchKernelGGL((score_valu_kernel<DSA_FP8_E4M3, false>), grid, dim3(256), lds, st, p);
    }
    return hipGetLastError();
  }
  const int64_t n_tiles = (p.n_units + 31) / 32;
  // Long rows: chunks of up to 32 tiles per wave; short rows spread over 4
  // waves, unless there are rows enough to fill the GPU with fewer (every
  // wave loads and converts its row's query first: chunks then grow until
  // about 2048 waves remain); fp8 decode rows (two waves per SIMD) in chunks
  // that give about 2048 waves.
  int64_t ct = (n_tiles + 3) / 4;
  const int64_t fill_rows = (rows * n_tiles + 2047) / 2048;
  if (ct < fill_rows) ct = fill_rows < n_tiles ? fill_rows : n_tiles;
  if (ct > 32) ct = 32;
  if (p.hist != nullptr && p.k_dtype == DSA_FP8_E4M3) {
    const int64_t fill = (rows * n_tiles + 2047) / 2048;
    if (ct > fill) ct = fill < 4 ? 4 : fill;
  }
  if (ct < 1) ct = 1;
  p.chunk_tiles = static_cast<int32_t>(ct);
  p.n_chunks = static_cast<int32_t>((n_tiles + ct - 1) / ct);
  p.chunk_major = p.hist != nullptr ? 1 : 0;
  dim3 grid;
  if (p.chunk_major) grid = dim3(static_cast<unsigned>(rows * ((p.n_chunks + 3) / 4)));
  else grid = dim3(static_cast<unsigned>(((rows + 3) / 4) * p.n_chunks));
  const size_t lds = p.hist ? HIST_BINS * sizeof(uint32_t) : 0;
  switch (p.k_dtype) {
    case DSA_BF16: return launch_mfma_q<KK_BF16>(p, grid, lds, st);
    case DSA_F16: return launch_mfma_q<KK_F16>(p, grid, lds, st);
    case DSA_FP8_E4M3: return launch_mfma_q<KK_FP8>(p, grid, lds, st);
    default: return launch_mfma_q<KK_F32>(p, grid, lds, st);
  }
}

}  // namespace dsa
