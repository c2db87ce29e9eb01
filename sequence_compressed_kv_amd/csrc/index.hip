// Lightning-indexer scoring: s_j = sum_h w_h * max(0, qI_h . kI_j) for every
// visible entry j (knightli.com DeepSeek-V4 KV-cache article, section "CSA":
// the indexer scores the compressed blocks before the top-k; the score form is
// fixed by the CSA decode workload definition).
//
// MFMA path (bf16 queries; bf16, e4m3 or MXFP4 keys dequantised exactly to bf16): the
// contraction is [H_I x D_I] . [D_I x 32 keys] per tile, heads as M, keys as N.
//   decode rows : (HBM-bound) v_mfma_f32_32x32x16_bf16; each lane owns one key
//                 column and 16 head rows per 32-head tile, so the ReLU . w head
//                 reduction is lane-local plus one exchange between the two
//                 half-waves; D_I is split between the half-waves as two
//                 contiguous halves (a lane streams 128 contiguous key bytes per
//                 tile).  A block takes one row and 4 waves x NT tiles of 32 keys,
//                 keys streamed from HBM straight into MFMA fragments.
//   causal rows : (MFMA-bound) v_mfma_f32_16x16x32_bf16; a block takes 8
//                 consecutive rows (one per wave) and walks every visible key
//                 tile through LDS (each tile fetched once per block), each wave
//                 overlapping one tile's products with the previous tile's
//                 reduction; blocks with the longest rows start first
#include "device_common.h"
#include "sckv_internal.h"

namespace sckv {

struct RowRef {
  int64_t seq;
  int64_t t;
};

__device__ __forceinline__ RowRef row_ref(int kind, const int32_t* pos, int32_t pos_max, int32_t seq0,
                                          int32_t pos0, int r) {
  if (kind == SCKV_ROWS_DECODE) {
    int32_t t = pos[r];
    t = t < 0 ? 0 : (t > pos_max ? pos_max : t);
    return {r, t};
  }
  return {seq0, (int64_t)pos0 + r};
}

__device__ __forceinline__ int64_t visible(int64_t t, int m, int W, int64_t E_cap) {
  const int64_t d = t - W;
  const int64_t e = d < 0 ? 0 : d / m;
  return e < E_cap ? e : E_cap;
}

// Element offset of dims 8 db .. 8 db + 7 of key j in a tiled key cache
// ([E_cap/32][DI/8][32][8] per sequence, sequence base seq_elem).
template <int DI>
__device__ __forceinline__ int64_t key_tile_elem(int64_t seq_elem, int64_t j, int db) {
  return seq_elem + (((j >> 5) * (DI / 8) + db) * 32 + (j & 31)) * 8;
}

// Keys of one 32-key tile as MFMA B fragments: lane (n = l%32, half hh = l/32)
// holds dims hh*DI/2 + 8 ks .. +7 of key n, for ks = 0 .. DI/16 - 1.  In the
// tiled layout the 32 lanes of a half-wave read one contiguous run of 32 x 8
// elements per ks (elem0: offset of key n's first dim block of its half).
template <int KEY, int DI>
__device__ __forceinline__ void load_key_tile(gbytes keys, int64_t elem0, bf16x8 (&b)[DI / 16]) {
  constexpr int KS = DI / 16;
  if constexpr (KEY == SCKV_BF16) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) b[ks] = bitcast<bf16x8>(gload<u32x4>(keys, (elem0 + 256 * ks) * 2));
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) b[ks] = bitcast<bf16x8>(e4m3x8_to_bf16x8(gload<u32x2>(keys, elem0 + 256 * ks)));
  }
}

// MXFP4 keys (tiles of 17 DI bytes per 32 keys: codes [DI/32][32][16 B], then
// scales [32][DI/32] B): the same fragments as load_key_tile, dequantised exactly
// to bf16 by the gfx950 scaled FP4 conversion (two codes per instruction, the
// low nibble first; the block scale byte s enters as the float 2^(s - 127)).
// Lane (n, hh) reads the 16-byte blocks DI/64 hh .. of key n and its scale bytes.
__device__ __forceinline__ float e8m0_scale(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);    // 2^(s - 127); s = 0: 2^-127
}

__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t v, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3));
  return bitcast<bf16x8>(r);
}

template <int DI>
__device__ __forceinline__ void load_fp4_tile(gbytes keys, int64_t tile_byte, int n, int hh, bf16x8 (&b)[DI / 16]) {
  constexpr int NB = DI / 64;                  // 32-channel blocks per half of a key
  uint32_t sc;
  if constexpr (DI == 128) sc = gload<uint32_t>(keys, tile_byte + 16 * DI + 4 * n);
  else sc = gload<uint16_t>(keys, tile_byte + 16 * DI + 2 * n);
  u32x4 c[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) c[i] = gload<u32x4>(keys, tile_byte + ((NB * hh + i) * 32 + n) * 16);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const float f = e8m0_scale((sc >> (8 * (NB * hh + i))) & 255u);
#pragma unroll
    for (int q = 0; q < 4; ++q) b[4 * i + q] = fp4x8_to_bf16x8(c[i][q], f);
  }
}

// Causal-row scoring of one wave on v_mfma_f32_16x16x32_bf16: heads as M in tiles
// of 16, keys as N in two 16-key halves of a 32-key tile, D_I as K in steps of
// 32.  (Under this load gfx950 holds a higher clock with this shape than with
// 32x32x16, which outweighs the extra instructions.)  Lane l
// holds key (l % 16) of each half and heads 16 mt + 4 (l / 16) + i, so the head
// reduction is lane-local over MT x 4 values per half, then across the four
// 16-lane groups: one half-wave swap that also separates the halves (lanes 0-31
// keep half 0, lanes 32-63 half 1), then one 16-lane swap.
template <int KEY, int HI, int DI>
struct ScoreWave {
  static constexpr int MT = HI / 16;
  static constexpr int KS = DI / 32;
  bf16x8 a[MT][KS];
  float w[MT][4];
  using Frag = bf16x8[2][KS];
  using Acc = f32x4[2][MT];

  __device__ __forceinline__ void load_query(gbytes q_row, const float* w_row) {
    const int l = lane_id(), c = l & 15, g = l >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t e0 = (int64_t)(16 * mt + c) * DI + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a[mt][ks] = bitcast<bf16x8>(gload<u32x4>(q_row, (e0 + 32 * ks) * 2));
#pragma unroll
      for (int i = 0; i < 4; ++i) w[mt][i] = w_row[16 * mt + 4 * g + i];
    }
  }

  // half nh, k-step ks: dims 32 ks + 8 (l / 16) .. +7 of key 16 nh + l % 16
  __device__ __forceinline__ static void frags(const uint8_t* tile, bf16x8 (&b)[2][KS]) {
    constexpr int ESZ = KEY == SCKV_BF16 ? 2 : 1;
    const int l = lane_id(), c = l & 15, g = l >> 4;
    if constexpr (KEY == SCKV_MXFP4) {
      // MXFP4 tile: k-step ks is 32-channel block ks; the lane's 8 codes are 4
      // bytes of the key's 16-byte block, its scale one of the key's scale bytes
#pragma unroll
      for (int nh = 0; nh < 2; ++nh) {
        const int key = 16 * nh + c;
        uint32_t sc;
        if constexpr (DI == 128) sc = *reinterpret_cast<const uint32_t*>(tile + 16 * DI + 4 * key);
        else sc = *reinterpret_cast<const uint16_t*>(tile + 16 * DI + 2 * key);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint32_t v = *reinterpret_cast<const uint32_t*>(tile + (ks * 32 + key) * 16 + 4 * g);
          b[nh][ks] = fp4x8_to_bf16x8(v, e8m0_scale((sc >> (8 * ks)) & 255u));
        }
      }
      return;
    }
#pragma unroll
    for (int nh = 0; nh < 2; ++nh)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = ((4 * ks + g) * 32 + 16 * nh + c) * 8 * ESZ;
        if constexpr (KEY == SCKV_BF16) b[nh][ks] = bitcast<bf16x8>(*reinterpret_cast<const u32x4*>(tile + off));
        else b[nh][ks] = bitcast<bf16x8>(e4m3x8_to_bf16x8(*reinterpret_cast<const u32x2*>(tile + off)));
      }
  }
  __device__ __forceinline__ static int lane_key() { const int l = lane_id(); return (l & 15) | ((l & 32) >> 1); }
  __device__ __forceinline__ static void zero(f32x4 (&acc)[2][MT]) {
#pragma unroll
    for (int nh = 0; nh < 2; ++nh)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nh][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ static bool lane_stores() { return !(lane_id() & 16); }

  __device__ __forceinline__ void mfmas(const bf16x8 (&b)[2][KS], f32x4 (&acc)[2][MT]) const {
#pragma unroll
    for (int nh = 0; nh < 2; ++nh)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nh][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nh = 0; nh < 2; ++nh) acc[nh][mt] = mfma16_bf16(a[mt][ks], b[nh][ks], acc[nh][mt]);
  }

  __device__ __forceinline__ float reduce(const f32x4 (&acc)[2][MT]) const {
    float part[2] = {0.f, 0.f};
#pragma unroll
    for (int nh = 0; nh < 2; ++nh)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[nh] += w[mt][i] * relu(acc[nh][mt][i]);
    const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]), false, false);
    const float s = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    const float tot = __uint_as_float(y[0]) + __uint_as_float(y[1]);
    return tot == 0.f ? 0.f : tot;
  }
};

// Decode rows: a block takes one row and 4 consecutive ranges of NT tiles of 32
// keys (one range per wave).  The row's query sits in LDS (shared by the four
// waves, rows padded against bank conflicts).  A wave's tile loop is unrolled
// completely, with two tiles in flight ahead of the one being multiplied: in
// straight-line code every wait covers exactly the tile it needs.  Loads past
// the row's last visible tile re-read it; their scores are not stored.
template <int KEY, int HI, int DI, int NT>
__global__ __launch_bounds__(256) void index_score_decode(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const void* __restrict__ keys,
    float* __restrict__ scores, int64_t stride, int64_t E_cap, int m, int W, const int32_t* __restrict__ pos,
    int32_t pos_max, uint32_t* __restrict__ zero_hist, int zero_words) {
  constexpr int MT = HI / 32, KS = DI / 16, QS = DI + 8;
  constexpr int64_t KPW = 32 * NT;
  __shared__ uint16_t qs[HI * QS];
  const int r = blockIdx.y;
  if (zero_hist != nullptr && blockIdx.x == 0) {                 // the row's top-k histogram, cleared
    uint32_t* h = zero_hist + (int64_t)r * zero_words;
    for (int i = 4 * threadIdx.x; i < zero_words; i += 4 * 256) *reinterpret_cast<u32x4*>(h + i) = u32x4{0u, 0u, 0u, 0u};
  }
  const RowRef rr = row_ref(SCKV_ROWS_DECODE, pos, pos_max, 0, 0, r);
  const int64_t e_vis = visible(rr.t, m, W, E_cap);
  if ((int64_t)blockIdx.x * 4 * KPW >= e_vis) return;           // whole block past the row
  const int l = lane_id(), n = l & 31, hh = l >> 5;
  // a wave past the row's last key re-reads its last tile and stores nothing
  const int64_t j_begin = ((int64_t)blockIdx.x * 4 + wave_id()) * KPW;
  const int64_t j_end = j_begin + KPW < e_vis ? j_begin + KPW : e_vis;
  const int64_t key_row0 = rr.seq * E_cap;
  float* srow = scores + (int64_t)r * stride;
  const gbytes gkeys = opaque_global(keys);

  auto load = [&](int t, bf16x8 (&b)[KS]) {
    int64_t key = j_begin + 32 * t + n;
    key = key < e_vis ? key : e_vis - 1;
    if constexpr (KEY == SCKV_MXFP4) load_fp4_tile<DI>(gkeys, (key_row0 + (key & ~(int64_t)31)) / 32 * (17 * DI), n, hh, b);
    else load_key_tile<KEY, DI>(gkeys, key_tile_elem<DI>(key_row0 * DI, key, hh * KS), b);
  };
  // the first two tiles' loads go out before the query is staged, so the
  // stream of keys starts one round trip earlier
  bf16x8 buf[3][KS];
  load(0, buf[0]);
  if constexpr (NT > 1) load(1, buf[1]);
  for (int i = threadIdx.x; i < HI * DI / 8; i += 256) {
    const int h = i / (DI / 8), c = i % (DI / 8);
    *reinterpret_cast<u32x4*>(&qs[h * QS + c * 8]) =
        *reinterpret_cast<const u32x4*>(q + ((int64_t)r * HI + h) * DI + c * 8);
  }
  float wr[MT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) wr[mt][i] = w[(int64_t)r * HI + 32 * mt + 8 * (i >> 2) + 4 * hh + (i & 3)];
  __syncthreads();
  if (j_begin >= e_vis) return;

  auto compute = [&](int t, const bf16x8 (&b)[KS]) {
    float part = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = bitcast<bf16x8>(*reinterpret_cast<const u32x4*>(&qs[(32 * mt + n) * QS + hh * (DI / 2) + 8 * ks]));
        acc = mfma32_bf16(a, b[ks], acc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) part += wr[mt][i] * relu(acc[i]);
    }
    const float tot = add_xor32(part);
    const int64_t j = j_begin + 32 * t + n;
    if (hh == 0 && j < j_end) srow[j] = tot == 0.f ? 0.f : tot;
  };

#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t + 2 < NT) load(t + 2, buf[(t + 2) % 3]);
    compute(t, buf[t % 3]);
  }
}

// Causal rows, keys shared through LDS: a block takes 8 consecutive rows (one
// per wave; their visible counts differ by at most two entries) and walks the
// key tiles of the widest of them.  Key tiles travel global -> LDS by
// asynchronous copies (1 KB per wavefront instruction, spread over the waves)
// into stages of 64 KB (pairs of tiles A, B; two or three stages), so each tile
// is fetched from L2 once per block instead of once per row; every wave reads it
// from LDS as its MFMA B operand.  The copy counts per wave are uniform (tiles past the row
// re-read the last one), so the explicit vector-memory waits count exactly the
// stages still in flight (later score stores only make them stricter).
//
// Each wave runs a two-tile software pipeline: the MFMAs of one tile are issued
// next to the ReLU . w reduction of the tile before it (independent work for
// the matrix core and the vector ALU), and the B fragments of the next tile are
// read from LDS one step ahead.
template <int KEY, int HI, int DI>
__global__ __launch_bounds__(512) void index_score_causal_lds(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const void* __restrict__ keys,
    float* __restrict__ scores, int64_t stride, int64_t E_cap, int m, int W, int32_t seq0, int32_t pos0, int R) {
  constexpr int NWR = 8;
  constexpr bool FP4 = KEY == SCKV_MXFP4;
  constexpr int ESZ = KEY == SCKV_BF16 ? 2 : 1;
  constexpr int TB = FP4 ? 17 * DI : 32 * DI * ESZ;                    // bytes per 32-key tile
  constexpr int PPS = 32768 / TB;                                      // tile pairs per stage (64 KB)
  // bytes per stage: whole tiles; MXFP4 tiles (17 DI bytes) are copied as one
  // linear run rounded up to 1 KB per wave (the bytes past the last tile are not read)
  constexpr int SB = FP4 ? (2 * PPS * TB + NWR * 1024 - 1) / (NWR * 1024) * (NWR * 1024) : 2 * PPS * TB;
  constexpr int NC = SB / 1024;                                        // 1 KB copies per stage
  constexpr int CPW = NC >= NWR ? NC / NWR : 1;                        // copies per copying wave
  constexpr int NSTG = 3 * SB <= 96 * 1024 ? 3 : 2;
  static_assert(NC >= 1 && (NC < NWR ? 1 : NC % NWR == 0), "stage must split evenly over the waves");
  __shared__ __attribute__((aligned(16))) uint8_t stg[NSTG * SB];

  const int grp = gridDim.x - 1 - blockIdx.x;                          // longest rows first
  const int r0 = grp * NWR;
  const int wv = wave_id(), l = lane_id();
  const int r_last = (r0 + NWR < R ? r0 + NWR : R) - 1;
  const int r = r0 + wv <= r_last ? r0 + wv : r_last;                  // surplus waves shadow the last row
  const bool own_row = r0 + wv <= r_last;
  const int64_t ev_max = visible((int64_t)pos0 + r_last, m, W, E_cap);
  if (ev_max == 0) return;                                             // whole block: nothing visible
  const int64_t ev = visible((int64_t)pos0 + r, m, W, E_cap);
  const int ntiles = (int)((ev_max + 31) / 32);
  const int npairs = (ntiles + 1) / 2;
  const int nst = (npairs + PPS - 1) / PPS;

  using SW = ScoreWave<KEY, HI, DI>;
  SW sw;
  sw.load_query(opaque_global(q) + (int64_t)r * HI * DI * 2, w + (int64_t)r * HI);
  float* srow = scores + (int64_t)r * stride;
  const gbytes gk = opaque_global(keys) + (int64_t)seq0 * (E_cap / 32) * TB;
  const int wu = __builtin_amdgcn_readfirstlane(wv);
  const bool copier = NC >= NWR || wu < NC;
  const int lkey = SW::lane_key();
  const bool lstore = own_row && SW::lane_stores();

  auto issue = [&](int st, int buf) __attribute__((always_inline)) {
    if (!copier) return;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int cb = (wu * CPW + c) * 1024;                            // byte offset within the stage
      if constexpr (FP4) {
        // the stage's tiles as one run; a lane whose 16 bytes would pass the end of
        // the sequence's cache re-reads its last 16 bytes (landing past every tile
        // the block scores)
        int64_t off = (int64_t)2 * PPS * st * TB + cb + l * 16;
        const int64_t last = (E_cap / 32) * TB - 16;
        off = off < last ? off : last;
        copy_to_lds16(gk + off, &stg[buf * SB + cb]);
      } else {
        int tile = 2 * PPS * st + cb / TB;
        tile = tile < ntiles ? tile : ntiles - 1;
        copy_to_lds16(gk + (int64_t)tile * TB + (cb % TB) + l * 16, &stg[buf * SB + cb]);
      }
    }
  };
  auto store = [&](int tile, float v) __attribute__((always_inline)) {
    const int64_t j = (int64_t)tile * 32 + lkey;
    if (lstore && j < ev) srow[j] = v;
  };

  for (int st = 0; st < NSTG && st < nst; ++st) issue(st, st);
  if (NSTG == 3 && nst > 2) wait_vm_lgkm<2 * CPW, 0>();
  else if (nst > 1) wait_vm_lgkm<CPW, 0>();
  else wait_vm_lgkm<0, 0>();
  block_barrier();                                                     // stage 0 visible

  typename SW::Frag bA, bB;
  typename SW::Acc accA, accB;
  SW::zero(accB);                                                      // reduced (unused) for the first pair
  SW::frags(&stg[0], bA);
  int cur = 0, st = 0, gi = 0;                                         // buffer, stage, pair within it
  for (int g = 0; g < npairs; ++g) {
    // tile A of pair g on the matrix core, tile B of pair g-1 reduced
    SW::frags(&stg[cur * SB + (2 * gi + 1) * TB], bB);
    sw.mfmas(bA, accA);
    const float sB = sw.reduce(accB);
    if (g > 0) store(2 * g - 1, sB);
    int ncur = cur, ngi = gi + 1;
    if (ngi == PPS) {                                                  // next pair in the next stage
      if (st + 1 < nst) {
        if (NSTG == 3 && st + 2 < nst) wait_vm_lgkm<CPW, 0>();
        else wait_vm_lgkm<0, 0>();
        block_barrier();                                               // stage st+1 visible; buffer cur free
        if (st + NSTG < nst) issue(st + NSTG, cur);
      }
      ncur = cur == NSTG - 1 ? 0 : cur + 1;
      ngi = 0;
      ++st;
    }
    // tile B on the matrix core, tile A reduced; tile A of the next pair read
    // ahead (after the last pair it reads a settled buffer and is unused)
    SW::frags(&stg[ncur * SB + 2 * ngi * TB], bA);
    sw.mfmas(bB, accB);
    const float sA = sw.reduce(accA);
    store(2 * g, sA);
    cur = ncur;
    gi = ngi;
  }
  store(2 * npairs - 1, sw.reduce(accB));
}

// fp32 path: one thread per key, query and weights staged in LDS.
__global__ __launch_bounds__(256) void index_score_f32(
    const float* __restrict__ q, const float* __restrict__ w, const float* __restrict__ keys,
    float* __restrict__ scores, int64_t stride, int64_t E_cap, int m, int W, int HI, int DI, int kind,
    const int32_t* __restrict__ pos, int32_t pos_max, int32_t seq0, int32_t pos0) {
  extern __shared__ float sq[];                       // [HI*DI] query, then [HI] weights
  const int r = blockIdx.y;
  const RowRef rr = row_ref(kind, pos, pos_max, seq0, pos0, r);
  const int64_t e_vis = visible(rr.t, m, W, E_cap);
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if ((int64_t)blockIdx.x * 256 >= e_vis) return;
  for (int i = threadIdx.x; i < HI * DI; i += 256) sq[i] = q[(int64_t)r * HI * DI + i];
  for (int i = threadIdx.x; i < HI; i += 256) sq[HI * DI + i] = w[(int64_t)r * HI + i];
  __syncthreads();
  if (j >= e_vis) return;
  // key j in the tiled layout: dims 8 db .. 8 db + 7 at tile_base + db * 256
  const float* kr = keys + rr.seq * E_cap * DI + ((j >> 5) * (DI / 8) * 32 + (j & 31)) * 8;
  float s = 0.f;
  for (int h = 0; h < HI; ++h) {
    float d = 0.f;
    for (int c = 0; c < DI; ++c) d = fmaf(sq[h * DI + c], kr[(c >> 3) * 256 + (c & 7)], d);
    s += sq[HI * DI + h] * fmaxf(d, 0.f);
  }
  scores[(int64_t)r * stride + j] = s == 0.f ? 0.f : s;
}

int64_t index_rows_cover(const sckv_index_args& a) {
  const int64_t t = a.rows.kind == SCKV_ROWS_DECODE ? a.rows.pos_max : (int64_t)a.rows.pos0 + a.rows.R - 1;
  const int64_t e = entries_visible(t, a.m, a.W);
  return e < a.E_cap ? e : a.E_cap;
}

template <int KEY, int HI, int DI>
static void launch_mfma(const sckv_index_args& a, float* scores, int64_t stride, int64_t cover,
                        hipStream_t stream, uint32_t* zero_hist, int zero_words, bool* zeroed) {
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  if (a.rows.kind == SCKV_ROWS_DECODE) {
    // Tiles per wave.  bf16 keys, bound by HBM: 4 (16 KB a wave).  At two waves
    // per SIMD a long grid runs in rounds, and short waves keep the last round's
    // tail short: 32 rows of 1023 tiles take 49-51 us with 4, 52-53.5 with 8,
    // 53-54 with 16 and 58-61 with 2 (the block's query staging then weighs on
    // too few keys).  MXFP4 keys (68 bytes a key) spend more per tile on their
    // conversion and do best in one round of long waves: 16 tiles once that
    // still gives 2048 waves (same rows: 20.1-20.2 us with 16, 21.4-22.5 with 8,
    // 25.5 with 4).  e4m3 keys: the largest of 16/8/4 that still gives about
    // 2048 waves.
    const int64_t tiles = (cover + 31) / 32 * a.rows.R;
    const int nt = KEY == SCKV_BF16    ? 4
                   : KEY == SCKV_MXFP4 ? (tiles >= 2048 * 8 ? 16 : 4)
                                       : (tiles >= 2048 * 16 ? 16 : (tiles >= 2048 * 8 ? 8 : 4));
    const int64_t kpb = 4 * 32 * (int64_t)nt;
    const dim3 grid((unsigned)((cover + kpb - 1) / kpb), (unsigned)a.rows.R);
#define SCKV_DEC(NTT)                                                                                          \
  hipLaunchKernelGGL((index_score_decode<KEY, HI, DI, NTT>), grid, dim3(256), 0, stream, q, a.w, a.keys, scores, \
                     stride, a.E_cap, a.m, a.W, a.rows.pos, a.rows.pos_max, zero_hist, zero_words)
    if (nt == 16) SCKV_DEC(16);
    else if (nt == 8) SCKV_DEC(8);
    else SCKV_DEC(4);
#undef SCKV_DEC
    if (zeroed) *zeroed = zero_hist != nullptr;
  } else {
    const dim3 grid((unsigned)((a.rows.R + 7) / 8));
    hipLaunchKernelGGL((index_score_causal_lds<KEY, HI, DI>), grid, dim3(512), 0, stream, q, a.w, a.keys, scores,
                       stride, a.E_cap, a.m, a.W, a.rows.seq0, a.rows.pos0, a.rows.R);
  }
}

template <int KEY>
static void launch_mfma_key(const sckv_index_args& a, float* scores, int64_t stride, int64_t cover,
                            hipStream_t stream, uint32_t* zh, int zw, bool* zeroed) {
  if (a.H_I == 64 && a.D_I == 128) launch_mfma<KEY, 64, 128>(a, scores, stride, cover, stream, zh, zw, zeroed);
  else if (a.H_I == 64 && a.D_I == 64) launch_mfma<KEY, 64, 64>(a, scores, stride, cover, stream, zh, zw, zeroed);
  else if (a.H_I == 32 && a.D_I == 128) launch_mfma<KEY, 32, 128>(a, scores, stride, cover, stream, zh, zw, zeroed);
  else launch_mfma<KEY, 32, 64>(a, scores, stride, cover, stream, zh, zw, zeroed);
}

hipError_t launch_index_score(const sckv_index_args& a, float* scores, int64_t stride, int64_t cover,
                              hipStream_t stream, uint32_t* zh, int zw, bool* zeroed) {
  if (zeroed) *zeroed = false;
  if (zw <= 0 || zw % 4) zh = nullptr;
  if (cover <= 0) return hipSuccess;
  if (a.key_dtype == SCKV_F32) {
    const dim3 grid((unsigned)((cover + 255) / 256), (unsigned)a.rows.R);
    const size_t lds = (size_t)(a.H_I * a.D_I + a.H_I) * sizeof(float);
    hipLaunchKernelGGL(index_score_f32, grid, dim3(256), lds, stream, static_cast<const float*>(a.q), a.w,
                       static_cast<const float*>(a.keys), scores, stride, a.E_cap, a.m, a.W, a.H_I, a.D_I,
                       a.rows.kind, a.rows.pos, a.rows.pos_max, a.rows.seq0, a.rows.pos0);
  } else if (a.key_dtype == SCKV_BF16) {
    launch_mfma_key<SCKV_BF16>(a, scores, stride, cover, stream, zh, zw, zeroed);
  } else if (a.key_dtype == SCKV_MXFP4) {
    launch_mfma_key<SCKV_MXFP4>(a, scores, stride, cover, stream, zh, zw, zeroed);
  } else {
    launch_mfma_key<SCKV_E4M3>(a, scores, stride, cover, stream, zh, zw, zeroed);
  }
  return hipGetLastError();
}

}  // namespace sckv
