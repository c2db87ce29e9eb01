// Sparse-plus-window (CSA) and dense-plus-window (HCA) attention over a shared
// latent K = V: o_h = sum_u softmax_u(scale * q_h . u) u, u over the kept entries
// and the raw tokens max(0, t-W+1) .. t, one softmax for both (knightli.com
// DeepSeek-V4 KV-cache article, sections "CSA", "HCA" and "Ventana deslizante").
//
// MFMA path (bf16 queries; bf16 or e4m3 entries; bf16 window):
//   block = (split, row); one wave per 16 heads.  Items are staged 32 or 64 at
//   a time into LDS twice, as bf16: row-major for Q.K^T and transposed for P.V.
//   S^T = items x heads on v_mfma_f32_16x16x32_bf16 (items as M), so each lane
//   holds one head column; the S accumulator registers become the A operand of
//   P.V directly (the K order of the item axis is chosen to match), with an
//   online softmax between the two.  P enters P.V as two bf16 parts (hi + lo).
//   fp8 entries keep their exact codes in the MFMA operands; the per-entry scale
//   multiplies the logit and the probability instead.
//   Split-K over the item list writes (m, l, unnormalised o) partials that a
//   second kernel merges in a fixed order.
// fp32 path: plain VALU, one block per row.
#include "device_common.h"
#include "sckv_internal.h"

namespace sckv {

constexpr int kPlanChunk = 64;    // split boundaries fall on multiples of this many items (32 in one case)
constexpr int kMaxSplits = 256;   // splits per row: about one block per CU when a single row is decoded
constexpr int kSegItems = 1024;   // item sources resolved per segment of a block's range

struct AttendParams {
  const uint16_t* q;
  const void* entries;
  const float* escale;
  const int32_t* idx;
  const void* win;
  void* out;
  float* lse;
  float* ws_o;
  float* ws_ml;
  const int32_t* pos;
  int64_t E_cap, R_w;
  int32_t kind, pos_max, seq0, pos0;
  int32_t H, m, W, k;
  int32_t csa, out_dtype, nsplit, per_split;
  int32_t rows_R;
  float scale;
};

struct RowItems {
  int64_t seq, t, e_vis, n_list, n_win, win_first, n_items;
};

__device__ __forceinline__ RowItems row_items(const AttendParams& p, int r) {
  RowItems ri;
  if (p.kind == SCKV_ROWS_DECODE) {
    int32_t t = p.pos[r];
    ri.t = t < 0 ? 0 : (t > p.pos_max ? p.pos_max : t);
    ri.seq = r;
  } else {
    ri.t = (int64_t)p.pos0 + r;
    ri.seq = p.seq0;
  }
  const int64_t d = ri.t - p.W;
  int64_t e = d < 0 ? 0 : d / p.m;
  ri.e_vis = e < p.E_cap ? e : p.E_cap;
  ri.n_list = p.csa ? p.k : ri.e_vis;
  ri.n_win = ri.t + 1 < p.W ? ri.t + 1 : p.W;
  ri.win_first = ri.t - ri.n_win + 1;
  ri.n_items = ri.n_list + ri.n_win;
  return ri;
}

// Where item q of a row lives: entry row (>= 0), window slot (encoded as
// -2 - slot) or nothing (-1).
__device__ __forceinline__ int64_t item_source(const AttendParams& p, const RowItems& ri, int r, int64_t q) {
  if (q >= ri.n_items) return -1;
  if (q < ri.n_list) {
    const int64_t j = p.csa ? (int64_t)p.idx[(int64_t)r * p.k + q] : q;
    return (j >= 0 && j < p.E_cap) ? j : -1;
  }
  const int64_t i = ri.win_first + (q - ri.n_list);
  return -2 - (i % p.R_w);
}

// Sources of items [q_begin, q_end) of a row, resolved into LDS ahead of the
// streaming loop (index-list reads and ring-slot arithmetic off its path).
__device__ __forceinline__ void block_sources(const AttendParams& p, const RowItems& ri, int r, int64_t q_begin,
                                              int64_t q_end, int nthreads, int32_t* srcs) {
  for (int64_t q = q_begin + threadIdx.x; q < q_end; q += nthreads)
    srcs[q - q_begin] = (int32_t)item_source(p, ri, r, q);
}

// Staging unit: 4 consecutive items x 8 consecutive dims ("pair" (a, p): items
// 4a .. 4a+3, dims 8p .. 8p+7).  A thread loads the four row segments into
// registers one chunk ahead; at store time it writes them row-major for Q.K^T
// and, transposed in registers, as eight 8-byte cells (one dim, four items) of
// the P.V operand.  Everything that needs the loaded values (masking, fp8
// decoding) happens at store time, so issuing the loads never waits on them.
template <int ENT, int D, int NW, int CH>
struct Stage {
  static constexpr int NT = NW * kWave;
  static constexpr int PARTS = D / 8;                 // 8-dim parts per item row
  static constexpr int NPAIR = (CH / 4) * PARTS;      // (item group, part) pairs per chunk
  static constexpr int PPT = (NPAIR + NT - 1) / NT;   // pairs per thread
  u32x4 v[PPT][4];                                   // bf16 x 8: entries (BF16) or window rows
  u32x2 c[ENT == SCKV_E4M3 ? PPT : 1][4];            // e4m3 x 8 entry codes
  float sc[ENT == SCKV_E4M3 ? PPT : 1][4];           // e4m3 entry scales
  int32_t src[PPT][4];                               // item sources (entry >= 0, window <= -2, none -1)
};

template <int ENT, int D, int NW, int CH>
__device__ __forceinline__ void stage_load(const AttendParams& p, gbytes ent, gbytes win, gbytes esc,
                                           const RowItems& ri, const int32_t* srcs, int64_t q_rel, bool has_ent,
                                           bool has_win, Stage<ENT, D, NW, CH>& st) {
  using S = Stage<ENT, D, NW, CH>;
#pragma unroll
  for (int s = 0; s < S::PPT; ++s) {
    const int pair = threadIdx.x + s * S::NT;
    const int pr = pair < S::NPAIR ? pair : 0;
    const int part = pr % S::PARTS, a = pr / S::PARTS;
    // the four item sources of this pair in one LDS read
    const int4 src4 = *reinterpret_cast<const int4*>(&srcs[q_rel + 4 * a]);
    st.src[s][0] = pair < S::NPAIR ? src4.x : -1;
    st.src[s][1] = pair < S::NPAIR ? src4.y : -1;
    st.src[s][2] = pair < S::NPAIR ? src4.z : -1;
    st.src[s][3] = pair < S::NPAIR ? src4.w : -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t sv = st.src[s][i];
      const int64_t erow = ri.seq * p.E_cap + (sv >= 0 ? sv : 0);         // masked: row 0, zeroed later
      const int64_t wrow = ri.seq * p.R_w + (sv <= -2 ? -2 - sv : 0);
      if constexpr (ENT == SCKV_E4M3) {
        if (has_ent) {
          st.c[s][i] = gload<u32x2>(ent, erow * D + part * 8);
          st.sc[s][i] = gload<float>(esc, erow * 4);
        }
        if (has_win) st.v[s][i] = gload<u32x4>(win, (wrow * D + part * 8) * 2);
      } else {
        const bool is_win = sv <= -2;
        st.v[s][i] = gload<u32x4>(is_win ? win : ent, ((is_win ? wrow : erow) * D + part * 8) * 2);
      }
    }
  }
}

template <int D, int CH>
struct Lds {
  static constexpr int KR_STRIDE = D + 8;   // bf16 elements per item row
  static constexpr int CELLS = CH / 4;      // 4-item cells per dim row
  uint16_t kr[CH * KR_STRIDE];
  u32x2 vt[D * CELLS];                      // [dim][cells of 4 items] bf16, cells XOR-swizzled
  float isc[CH];
};

// Cell position of items 4a .. 4a+3 in the row of dim d: spreads both the
// transposed writes (dims 8p + e over lanes p) and the operand reads (dims
// 16 nd + col over lanes col) over the LDS banks.
template <int CH>
__device__ __forceinline__ int vt_cell(int d, int a) {
  return d * (CH / 4) + (a ^ (((d >> 1) ^ (d >> 4)) & 7));
}

template <int ENT, int D, int NW, int CH>
__device__ __forceinline__ void stage_store(const Stage<ENT, D, NW, CH>& st, Lds<D, CH>& L) {
  using S = Stage<ENT, D, NW, CH>;
#pragma unroll
  for (int s = 0; s < S::PPT; ++s) {
    const int pair = threadIdx.x + s * S::NT;
    if (pair < S::NPAIR) {
      const int part = pair % S::PARTS, a = pair / S::PARTS;
      u32x4 v[4];
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t sv = st.src[s][i];
        if constexpr (ENT == SCKV_E4M3) {
          v[i] = sv >= 0 ? e4m3x8_to_bf16x8(st.c[s][i]) : st.v[s][i];
          sc[i] = sv >= 0 ? st.sc[s][i] : 1.f;
        } else {
          v[i] = st.v[s][i];
          sc[i] = 1.f;
        }
        if (sv == -1) {
          v[i] = u32x4{0u, 0u, 0u, 0u};
          sc[i] = 0.f;
        }
        *reinterpret_cast<u32x4*>(&L.kr[(4 * a + i) * Lds<D, CH>::KR_STRIDE + part * 8]) = v[i];
      }
      // the same bf16 values transposed: cell (dim 8 part + e, group a) = items
      // 4a .. 4a+3 of that dim
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = (v[i][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        L.vt[vt_cell<CH>(part * 8 + e, a)] = u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
      }
      if (part == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) L.isc[4 * a + i] = sc[i];
      }
    }
  }
}

template <int ENT, int D, int NW, int CH>
__global__ __launch_bounds__(NW * 64) void attend_mfma(AttendParams p) {
  constexpr int KSQ = D / 32;      // k-steps of Q.K^T
  constexpr int ND = D / 16;       // 16-dim output tiles
  constexpr int MT = CH / 16;      // 16-item tiles of a chunk
  constexpr int KK = CH / 32;      // 32-item k-steps of P.V
  __shared__ Lds<D, CH> L;
  __shared__ int32_t srcs[kSegItems];

  const int r = blockIdx.y, split = blockIdx.x;
  const RowItems ri = row_items(p, r);
  const int l = lane_id(), w = wave_id() + NW * blockIdx.z;  // 16-head group of this wave
  const int col = l & 15, g = l >> 4;
  const int head = 16 * w + col;

  const int64_t q_begin = (int64_t)split * p.per_split;     // per_split: items, a multiple of CH
  int64_t q_end = q_begin + p.per_split;
  q_end = q_end < ri.n_items ? q_end : ri.n_items;

  const gbytes gent = opaque_global(p.entries), gwin = opaque_global(p.win), gesc = opaque_global(p.escale);
  // query fragments (B operand of S^T = items x heads): dims g*D/4 + 8 ks .. +7
  // loads issued here, waited for once the first chunk's loads are also in flight
  bf16x8 bq[KSQ];
  {
    const gbytes gq = opaque_global(p.q);
    const int64_t e0 = ((int64_t)r * p.H + head) * D + g * (D / 4);
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) bq[ks] = bitcast<bf16x8>(gload<u32x4>(gq, (e0 + 8 * ks) * 2));
  }
  f32x4 o[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) o[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;       // running maximum (base-2 logits) and sum
  const float scale2 = p.scale * 1.4426950408889634f;

  // which kinds of item a chunk starting at q holds (uniform branches in stage_load)
  auto has_ent = [&](int64_t q) { return q < ri.n_list; };
  auto has_win = [&](int64_t q) { return q + CH > ri.n_list; };
  Stage<ENT, D, NW, CH> st;
  for (int64_t s0 = q_begin; s0 < q_end; s0 += kSegItems) {
    const int64_t s1 = s0 + kSegItems < q_end ? s0 + kSegItems : q_end;
    // sources of this segment's items, padded with "nothing" to whole chunks
    __syncthreads();
    block_sources(p, ri, r, s0, s0 + (s1 - s0 + CH - 1) / CH * CH, NW * kWave, srcs);
    __syncthreads();
    stage_load<ENT, D, NW, CH>(p, gent, gwin, gesc, ri, srcs, 0, has_ent(s0), has_win(s0), st);
    if (s0 == q_begin) {
      // the query fragments stay in registers for the whole block; redefine them
      // here (their loads were issued first) so no later instruction waits on them
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks) pin(bq[ks]);
    }
    for (int64_t q0 = s0; q0 < s1; q0 += CH) {
      __syncthreads();
      stage_store<ENT, D, NW, CH>(st, L);
      __syncthreads();
      if (q0 + CH < s1)
        stage_load<ENT, D, NW, CH>(p, gent, gwin, gesc, ri, srcs, q0 + CH - s0, has_ent(q0 + CH), has_win(q0 + CH),
                                   st);

      // S^T for the chunk: MT tiles of 16 items
      f32x4 sacc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* kr = &L.kr[(16 * mt + col) * Lds<D, CH>::KR_STRIDE + g * (D / 4)];
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks) {
          const bf16x8 a = bitcast<bf16x8>(*reinterpret_cast<const u32x4*>(kr + 8 * ks));
          acc = mfma16_bf16(a, bq[ks], acc);
        }
        sacc[mt] = acc;
      }
      // logits in the base-2 domain (scale * log2 e folded in), chunk maximum per head
      float x[4 * MT], isc[4 * MT];
      float cmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sc = L.isc[16 * mt + 4 * g + i];
          isc[4 * mt + i] = sc;
          const float v = sc != 0.f ? sacc[mt][i] * (scale2 * sc) : -INFINITY;
          x[4 * mt + i] = v;
          cmax = fmaxf(cmax, v);
        }
      cmax = group_max4(cmax);
      const float m_new = fmaxf(m_run, cmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const bool grows = m_new > m_run;                  // this head's running maximum moved
      const float alpha = grows ? (m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new)) : 1.f;
      m_run = m_new;
      // P as the A operand of P.V: k-step kk takes items 32kk + {4g..4g+3} (tile 2kk)
      // and 32kk + 16 + {4g..4g+3} (tile 2kk+1), the order of the S^T registers.
      // With fp8 entries the operand is p times the entry's scale.  It enters as
      // the sum of two bf16 parts (about 16 significant bits together, fp32's
      // exponent range): V stays in bf16, exact for decoded fp8 and bf16 values
      float psum = 0.f;
      bf16x8 ph[KK], pl[KK];
#pragma unroll
      for (int e = 0; e < 4 * MT; ++e) {
        const float pe = __builtin_amdgcn_exp2f(x[e] - m_use);
        psum += pe;
        const float pv = ENT == SCKV_E4M3 ? pe * isc[e] : pe;
        ph[e / 8][e % 8] = (__bf16)pv;
        pl[e / 8][e % 8] = (__bf16)(pv - (float)ph[e / 8][e % 8]);
      }
      l_run = l_run * alpha + psum;
      // rescale the output rows (heads 4g + i of this wave) only when some maximum moved
      if (__any(grows)) {
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
        for (int nd = 0; nd < ND; ++nd)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[nd][i] *= al[i];
      }
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        const int d = 16 * nd + col;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const u32x2 lo = L.vt[vt_cell<CH>(d, 8 * kk + g)];
          const u32x2 hi = L.vt[vt_cell<CH>(d, 8 * kk + 4 + g)];
          const bf16x8 bv = bitcast<bf16x8>(u32x4{lo[0], lo[1], hi[0], hi[1]});
          o[nd] = mfma16_bf16(ph[kk], bv, o[nd]);
          o[nd] = mfma16_bf16(pl[kk], bv, o[nd]);
        }
      }
    }
  }

  // per-head totals
  float l_tot = l_run;
  l_tot += shfl_xor_f(l_tot, 16);
  l_tot += shfl_xor_f(l_tot, 32);
  float lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lrow[i] = __shfl(l_tot, 4 * g + i, kWave);
  const int hbase = 16 * w + 4 * g;
  if (p.nsplit == 1) {
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = o[nd][i] / lrow[i];
        const int64_t off = ((int64_t)r * p.H + hbase + i) * D + 16 * nd + col;
        if (p.out_dtype == SCKV_BF16) static_cast<uint16_t*>(p.out)[off] = (uint16_t)f32_to_bf16_rne(v);
        else static_cast<float*>(p.out)[off] = v;
      }
    if (p.lse && g == 0) p.lse[(int64_t)r * p.H + head] = (m_run + log2f(l_tot)) * 0.6931471805599453f;
  } else {
    const int64_t sbase = ((int64_t)r * p.nsplit + split) * p.H;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
#pragma unroll
      for (int i = 0; i < 4; ++i) p.ws_o[(sbase + hbase + i) * D + 16 * nd + col] = o[nd][i];
    if (g == 0) {
      p.ws_ml[(sbase + head) * 2] = m_run;
      p.ws_ml[(sbase + head) * 2 + 1] = l_tot;
    }
  }
}

// Sources of items [q_begin, q_end) (at most PER * NT of them) into srcs: every
// index-list load is issued before any is used, so the whole table costs one
// memory round trip.  Positions and ring sizes fit 32 bits here.
template <int PER, int NT>
__device__ __forceinline__ void block_sources_batched(const AttendParams& p, const RowItems& ri, int r,
                                                      int64_t q_begin, int64_t q_end, int32_t* srcs) {
  int32_t j[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int64_t q = q_begin + threadIdx.x + u * NT;
    const bool listed = q < ri.n_list;
    j[u] = (int32_t)q;
    if (p.csa) j[u] = p.idx[(int64_t)r * p.k + (listed ? q : 0)];
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int64_t q = q_begin + threadIdx.x + u * NT;
    int32_t sv = -1;
    if (q < ri.n_list) {
      sv = (j[u] >= 0 && j[u] < p.E_cap) ? j[u] : -1;
    } else if (q < ri.n_items) {
      const uint32_t i = (uint32_t)(ri.win_first + (q - ri.n_list));
      sv = -2 - (int32_t)(i % (uint32_t)p.R_w);
    }
    if (q < q_end) srcs[q - q_begin] = sv;
  }
}

// Chunk permutation of a staged row (row index within the stage, low four
// bits): bits 0 and 1 of the row go to chunk bits 1 and 2, bit 2 to chunk bit 3,
// and bit 2 xor bit 3 to chunk bit 0.  It stays within aligned groups of 16
// chunks, so a row's copy still reads whole 256-byte segments.
__device__ __forceinline__ int chunk_swizzle(int r) {
  return (((r >> 2) ^ (r >> 3)) & 1) | ((r & 3) << 1) | (((r >> 2) & 1) << 3);
}

// bf16 entries and window with D = 512 (the MLA-style latent), 64 heads: items
// travel global -> LDS by asynchronous copies (one 1 KB row per wavefront
// instruction) into four 32-item stages, without staging registers.  Waits are
// explicit: before a chunk is used each wave waits until only the next chunk's
// copies are outstanding, then one barrier per chunk publishes it.
//
// Eight waves in two roles, one of each on every SIMD: wave w < 4 ("score
// wave") takes the 16 heads 16 w .. over all 512 dims for Q.K^T and the online
// softmax, and hands P (as two bf16 parts) and the rescale factors to wave w + 4
// ("output wave") through LDS; the output wave accumulates P.V for the same 16
// heads over all 512 dims.  Chunk i's scores and chunk i - 1's products run
// between the same two barriers, so on every SIMD one wave's LDS reads and
// softmax overlap the other's MFMAs, and no logits cross waves.
//
// Both products read the same staged rows.  Q.K^T takes row fragments (one item,
// eight dims per lane).  P.V needs the transpose (one dim, eight items per lane):
// the gfx950 transposing LDS read delivers it directly.  Within each 16-lane
// group, lane 4r + c receives element c of the 8-byte words addressed by lanes
// r, r + 4, r + 8 and r + 12 of the group.  So lane a of group g points at item
// 4g + a/4, dims 4(a%4) .. +3, and lane n of the group comes back holding dim n
// of items 4g .. 4g + 3, the k-group layout of the P operand, which is also the
// layout in which a score wave's lane holds its probabilities.  That product
// runs in bf16, so P enters as the sum of two bf16 parts (a second MFMA per dim
// tile): a single bf16 P would cost up to 2^-9 of max |v| in the output.  The
// normaliser (and the log-sum-exp) sums the unrounded fp32 probabilities.
__global__ __launch_bounds__(512) void attend_dma512(AttendParams p) {
  constexpr int NW = 8, D = 512, CH = 32, KSQ = D / 32, ND = D / 16;
  constexpr int KRS = D;                     // LDS row (bf16 elements), 16-byte chunks swizzled per row
  constexpr int NT = NW * kWave;
  constexpr int RPW = CH / NW;               // rows copied per wave per chunk
  constexpr int NSTG = 4;
  constexpr int STG = CH * KRS;              // stage size (bf16 elements)
  __shared__ __attribute__((aligned(16))) uint16_t stg[NSTG * STG];
  __shared__ int32_t srcs[kSegItems];
  __shared__ u32x4 pb[2][4][2][kWave];       // P (hi, lo) of each score wave, two chunks
  __shared__ __attribute__((aligned(16))) float al[2][4][16];   // rescale factor per head, two chunks
  __shared__ int32_t resc[2][4];             // whether a chunk's factors differ from 1
  __shared__ float xml[4][2][16];            // (m, l) per head at the end

  // one-dimensional grid; with rows in multiples of 8 the splits of a row share
  // an XCD (blocks are dealt to the 8 XCDs in turn), so its query and index
  // list are fetched into one L2
  int r, split;
  {
    const int n = blockIdx.x;
    if ((p.rows_R & 7) == 0) {
      const int k = n >> 3;
      r = (n & 7) + 8 * (k / p.nsplit);
      split = k % p.nsplit;
    } else {
      r = n / p.nsplit;
      split = n % p.nsplit;
    }
  }
  const RowItems ri = row_items(p, r);
  const int l = lane_id(), w = wave_id();
  const bool scorer = w < 4;                 // wave-uniform role
  const int hg = w & 3;                      // head group of both roles
  const int col = l & 15, g = l >> 4;
  const int head = 16 * hg + col;

  const int64_t q_begin = (int64_t)split * p.per_split;
  int64_t q_end = q_begin + p.per_split;
  q_end = q_end < ri.n_items ? q_end : ri.n_items;

  const gbytes gent = opaque_global(p.entries), gwin = opaque_global(p.win);
  // One register array serves both roles: an output wave's sums of its 16 heads
  // x 512 dims, a score wave's query fragments in its first KSQ entries (lane
  // group g holds dims 128 g + 8 ks .. +7 of k-step ks; loads issued here,
  // waited for after the first source table).
  f32x4 o[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) o[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (scorer) {
    const gbytes gq = opaque_global(p.q);
    const int64_t e0 = ((int64_t)r * p.H + head) * D + g * (D / 4);
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) o[ks] = bitcast<f32x4>(gload<u32x4>(gq, (e0 + 8 * ks) * 2));
  }
  float m_run = -INFINITY, l_run = 0.f;      // score waves
  const float scale2 = p.scale * 1.4426950408889634f;

  const int wu = __builtin_amdgcn_readfirstlane(w);
  // the sequence's first entry / window row, held in scalar registers
  gbytes gent_row = gent + ri.seq * p.E_cap * (D * 2), gwin_row = gwin + ri.seq * p.R_w * (D * 2);
  asm volatile("" : "+s"(gent_row));
  asm volatile("" : "+s"(gwin_row));
  // items without a source copy the row's own token (always present) so that
  // every staged value is finite; their logits are masked
  const int32_t t_slot = (int32_t)(ri.t % p.R_w);

  // Staged rows keep their 16-byte chunks permuted: logical chunk c of row r
  // sits at chunk c ^ chunk_swizzle(r).  Sixteen consecutive rows then start in
  // sixteen different bank groups (the Q.K^T reads, one chunk of 16 rows per
  // instruction) and the four or eight rows of a transposing read group take
  // disjoint 32-byte bank spans (P.V, two chunks per row), with 32 or 64 banks.
  // Per-lane LDS byte offsets within a stage:
  const int fq = chunk_swizzle(col);                                        // Q.K^T: row col (+16)
  const int qk_row = col * KRS * 2 + 16 * g * 16;
  const int pv_r = 4 * g + (col >> 2);                                      // P.V: item 4g + col/4 (+16)
  const int fv = chunk_swizzle(pv_r);
  const int pv_row = pv_r * KRS * 2 + 8 * (col & 1);
  const int pv_h = (col >> 1) & 1;                                          // second chunk of the 32-byte span
  const lds_ptr lds0 = (lds_ptr)stg;

  // copies of chunk q_rel (relative to the segment's sources) into stage st
  auto issue = [&](int64_t q_rel, int st) __attribute__((always_inline)) {
    const int32_t my_src = srcs[q_rel + wu * RPW + (l % RPW)];   // lane i holds row i's source
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int c = wu * RPW + i;
      const int32_t sv = __builtin_amdgcn_readlane(my_src, i);    // one row per instruction
      const gbytes src = sv >= 0 ? gent_row + (int64_t)sv * (D * 2)
                                 : gwin_row + (int64_t)(sv <= -2 ? -2 - sv : t_slot) * (D * 2);
      copy_to_lds16(src + ((l ^ chunk_swizzle(c)) << 4), &stg[st * STG + c * KRS]);
    }
  };

  bool q_ready = false;
  for (int64_t s0 = q_begin; s0 < q_end; s0 += kSegItems) {
    const int64_t s1 = s0 + kSegItems < q_end ? s0 + kSegItems : q_end;
    const int nch = (int)((s1 - s0 + CH - 1) / CH);
    __syncthreads();
    block_sources_batched<kSegItems / NT, NT>(p, ri, r, s0, s0 + (int64_t)nch * CH, srcs);
    __syncthreads();
    if (!q_ready) {
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks) pin(o[ks]);
      q_ready = true;
    }
    for (int c = 0; c < 2 && c < nch; ++c) issue((int64_t)c * CH, c);

    // pass i: the score waves take chunk i, the output waves chunk i - 1
    for (int i = 0; i <= nch; ++i) {
      // validity of chunk i's 32 items: bit j set when item j has a source
      const int32_t my_item = srcs[(int64_t)(i < nch ? i : 0) * CH + (l & 31)];
      const uint64_t valid = __ballot(l < 32 && my_item != -1);
      if (i + 1 < nch) wait_vm_lgkm<RPW, 0>();
      else wait_vm_lgkm<0, 0>();
      // chunk i visible, chunk i - 1's P visible; chunk i - 2's stage free
      block_barrier();
      if (i + 2 < nch) issue((int64_t)(i + 2) * CH, (i + 2) & (NSTG - 1));

      if (scorer) {
        if (i < nch) {
          const int st = i & (NSTG - 1);
          // S^T = K Q^T over all 512 dims: two item tiles x even/odd k-steps,
          // fragments read in batches of 4 k-steps, one batch ahead
          const uint8_t* sb = reinterpret_cast<const uint8_t*>(&stg[st * STG]) + qk_row;
          f32x4 sacc[2][2];
#pragma unroll
          for (int j = 0; j < 4; ++j) sacc[j >> 1][j & 1] = f32x4{0.f, 0.f, 0.f, 0.f};
          constexpr int KB = 2, NB = KSQ / KB;
          bf16x8 fa[2][2 * KB];
          auto read_batch = [&](int b, bf16x8 (&f)[2 * KB]) __attribute__((always_inline)) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int j = 0; j < KB; ++j)
                f[mt * KB + j] = bitcast<bf16x8>(
                    *reinterpret_cast<const u32x4*>(sb + mt * 16 * KRS * 2 + (((KB * b + j) ^ fq) << 4)));
          };
          read_batch(0, fa[0]);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int j = 0; j < 2 * KB; ++j) pin(fa[b & 1][j]);
            if (b + 1 < NB) read_batch(b + 1, fa[(b + 1) & 1]);
#pragma unroll
            for (int j = 0; j < KB; ++j)
#pragma unroll
              for (int mt = 0; mt < 2; ++mt)
                sacc[mt][j & 1] = mfma16_bf16(fa[b & 1][mt * KB + j], bitcast<bf16x8>(o[KB * b + j]), sacc[mt][j & 1]);
          }
          float x[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[j] = (sacc[0][0][j] + sacc[0][1][j]) * scale2;
            x[4 + j] = (sacc[1][0][j] + sacc[1][1][j]) * scale2;
          }
          if ((uint32_t)valid != 0xffffffffu) {            // padding in this chunk
            const uint32_t lo = (uint32_t)(valid >> (4 * g)), hi = (uint32_t)(valid >> (16 + 4 * g));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (!((lo >> j) & 1u)) x[j] = -INFINITY;
              if (!((hi >> j) & 1u)) x[4 + j] = -INFINITY;
            }
          }
          float cmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
          cmax = group_max4(cmax);
          // the reference maximum moves only when a logit exceeds it by more
          // than 2^8 (probabilities then stay below 256): rescales are rare
          const bool grows = cmax > m_run + 8.f;
          const bool had = m_run != -INFINITY;   // an earlier chunk contributed
          const float m_new = grows ? cmax : m_run;
          const float m_use = m_new == -INFINITY ? 0.f : m_new;
          const float alpha = grows ? (had ? __builtin_amdgcn_exp2f(m_run - m_new) : 0.f) : 1.f;
          m_run = m_new;
          // P = hi + lo, both bf16 (about 16 significant bits together)
          bf16x8 pa, pl;
          float psum = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pe = __builtin_amdgcn_exp2f(x[e] - m_use);
            psum += pe;
            pa[e] = (__bf16)pe;
            pl[e] = (__bf16)(pe - (float)pa[e]);
          }
          l_run = l_run * alpha + psum;
          pb[i & 1][hg][0][l] = bitcast<u32x4>(pa);
          pb[i & 1][hg][1][l] = bitcast<u32x4>(pl);
          if (g == 0) al[i & 1][hg][col] = alpha;
          const bool any = __any(grows && had);
          if (l == 0) resc[i & 1][hg] = any ? 1 : 0;
        }
      } else if (i >= 1) {
        // O = O * alpha + P V for chunk i - 1, from the score wave's P
        const int c = i - 1, st = c & (NSTG - 1);
        const bf16x8 pa = bitcast<bf16x8>(pb[c & 1][hg][0][l]);
        const bf16x8 pl = bitcast<bf16x8>(pb[c & 1][hg][1][l]);
        if (resc[c & 1][hg]) {                   // nothing to rescale before the first contribution
          const f32x4 a4 = *reinterpret_cast<const f32x4*>(&al[c & 1][hg][4 * g]);
#pragma unroll
          for (int nd = 0; nd < ND; ++nd)
#pragma unroll
            for (int j = 0; j < 4; ++j) o[nd][j] *= a4[j];
        }
        const int vb0 = st * STG * 2 + pv_row;
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          const int off = vb0 + ((16 * (nd >> 3) + ((2 * (nd & 7) + pv_h) ^ fv)) << 4);
          const u32x2 lo = lds_read_tr16(lds0, off);
          const u32x2 hi = lds_read_tr16(lds0, off + 16 * KRS * 2);
          const bf16x8 vb = bitcast<bf16x8>(u32x4{lo[0], lo[1], hi[0], hi[1]});
          o[nd] = mfma16_bf16(pa, vb, o[nd]);
          o[nd] = mfma16_bf16(pl, vb, o[nd]);
        }
      }
    }
  }

  // The score waves' (m, l) per head meet the output waves' sums, and each
  // score wave takes over the upper latent half of its head group's sums
  // (through the stage memory, free now) so that all eight waves store.
  if (scorer) {
    float l_tot = l_run;
    l_tot += shfl_xor_f(l_tot, 16);
    l_tot += shfl_xor_f(l_tot, 32);
    if (g == 0) {
      xml[hg][0][col] = m_run;
      xml[hg][1][col] = l_tot;
    }
  }
  f32x4* xo = reinterpret_cast<f32x4*>(stg);          // [head group][16 tiles][64 lanes]
  __syncthreads();                                     // every stage read
  if (!scorer) {
#pragma unroll
    for (int j = 0; j < ND / 2; ++j) xo[(hg * (ND / 2) + j) * kWave + l] = o[ND / 2 + j];
  }
  __syncthreads();
  if (scorer) {
#pragma unroll
    for (int j = 0; j < ND / 2; ++j) o[j] = xo[(hg * (ND / 2) + j) * kWave + l];
  }
  const int hbase = 16 * hg + 4 * g;
  const int dbase = (scorer ? D / 2 : 0) + col;        // this wave's latent half
  float lrow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) lrow[j] = xml[hg][1][4 * g + j];
  if (p.nsplit == 1) {
#pragma unroll
    for (int nd = 0; nd < ND / 2; ++nd)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = o[nd][j] / lrow[j];
        const int64_t off = ((int64_t)r * p.H + hbase + j) * D + dbase + 16 * nd;
        if (p.out_dtype == SCKV_BF16) static_cast<uint16_t*>(p.out)[off] = (uint16_t)f32_to_bf16_rne(v);
        else static_cast<float*>(p.out)[off] = v;
      }
    if (p.lse && g == 0 && !scorer)
      p.lse[(int64_t)r * p.H + head] = (xml[hg][0][col] + log2f(xml[hg][1][col])) * 0.6931471805599453f;
  } else {
    const int64_t sbase = ((int64_t)r * p.nsplit + split) * p.H;
#pragma unroll
    for (int nd = 0; nd < ND / 2; ++nd)
#pragma unroll
      for (int j = 0; j < 4; ++j) p.ws_o[(sbase + hbase + j) * D + dbase + 16 * nd] = o[nd][j];
    if (g == 0 && !scorer) {
      p.ws_ml[(sbase + head) * 2] = xml[hg][0][col];
      p.ws_ml[(sbase + head) * 2 + 1] = xml[hg][1][col];
    }
  }
}

// Merge of split partials (maxima m_s in base-2 logit units):
// o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One block per (head, row, latent slice of `dslice` dims); each thread takes
// four consecutive dims.
// - SG = 1 (many rows: the grid alone fills the chip): one thread per split
//   reads (m_s, l_s) and the block reduces them; the weights 2^(m_s - M) wait in
//   LDS, then each thread sums all the splits in split order, eight splits'
//   loads in flight.
// - SG > 1 (a few rows with many splits, about one block per CU): SG thread
//   groups take consecutive runs of at most kMaxSplits / SG splits, and their
//   sums are added in run order through LDS.  Nothing waits on the reductions
//   but the weighting, so every load is issued first: a thread's partials and,
//   one or two splits per thread, (m_s, l_s) as one 8-byte load.  The merge then
//   costs one memory round trip instead of one per reduction and per batch of
//   splits.
// The plan keeps the number of splits at or below kMaxSplits.
template <int SG>
__global__ __launch_bounds__(256) void attend_combine(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                                                      void* __restrict__ out, float* __restrict__ lse, int H, int D,
                                                      int nsplit, int out_dtype, int dslice) {
  __shared__ float wgt[kMaxSplits];
  __shared__ float red[2][4];
  __shared__ f32x4 part[SG][SG > 1 ? 64 : 1];
  const int r = blockIdx.y, h = blockIdx.x;
  const int nt = blockDim.x, nw = (nt + kWave - 1) / kWave;
  const int l = lane_id(), w = wave_id();
  const float* ml = ws_ml + ((int64_t)r * nsplit * H + h) * 2;           // split s at + s * 2 H
  if constexpr (SG > 1) {
    // dslice / 4 threads per group (dslice >= 64, so nt >= 2 * kWave and
    // nsplit <= 2 nt); one pass over the slice
    constexpr int MAXP = kMaxSplits / SG;
    const int td_n = nt / SG, td = threadIdx.x % td_n, sg = threadIdx.x / td_n;
    const int per = (nsplit + SG - 1) / SG;
    const int s_begin = sg * per;
    const int n = nsplit - s_begin < per ? nsplit - s_begin : per;         // may be <= 0 for the last groups
    const int dd = blockIdx.z * dslice + 4 * td;
    const float* src = ws_o + (((int64_t)r * nsplit + s_begin) * H + h) * D + dd;
    f32x4 v[MAXP];
#pragma unroll
    for (int u = 0; u < MAXP; ++u)
      if (u < n) v[u] = *reinterpret_cast<const f32x4*>(src + (int64_t)u * H * D);
    u32x2 mlv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int s = threadIdx.x + i * nt;
      mlv[i] = s < nsplit ? *reinterpret_cast<const u32x2*>(ml + (int64_t)s * 2 * H)
                          : u32x2{__float_as_uint(-INFINITY), 0u};
    }
    float mloc = fmaxf(__uint_as_float(mlv[0][0]), __uint_as_float(mlv[1][0]));
    for (int o = 32; o >= 1; o >>= 1) mloc = fmaxf(mloc, shfl_xor_f(mloc, o));
    if (l == 0) red[0][w] = mloc;
    __syncthreads();
    float M = red[0][0];
    for (int i = 1; i < nw; ++i) M = fmaxf(M, red[0][i]);
    float lloc = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int s = threadIdx.x + i * nt;
      if (s < nsplit) {
        const float ms = __uint_as_float(mlv[i][0]);
        const float e = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
        lloc += e * __uint_as_float(mlv[i][1]);
        wgt[s] = e;
      }
    }
    for (int o = 32; o >= 1; o >>= 1) lloc += shfl_xor_f(lloc, o);
    if (l == 0) red[1][w] = lloc;
    __syncthreads();
    float L = red[1][0];
    for (int i = 1; i < nw; ++i) L += red[1][i];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < MAXP; ++u)
      if (u < n) acc += wgt[s_begin + u] * v[u];
    part[sg][td] = acc;
    __syncthreads();
    if (sg == 0) {
      for (int g = 1; g < SG; ++g) acc += part[g][td];
      const float inv = 1.f / L;
      const int64_t off = ((int64_t)r * H + h) * D + dd;
      if (out_dtype == SCKV_BF16) {
        uint16_t* o = static_cast<uint16_t*>(out) + off;
        const uint32_t lo = f32_to_bf16_rne(acc[0] * inv) | (f32_to_bf16_rne(acc[1] * inv) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc[2] * inv) | (f32_to_bf16_rne(acc[3] * inv) << 16);
        *reinterpret_cast<u32x2*>(o) = u32x2{lo, hi};
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + off) = acc * inv;
      }
    }
    if (lse && threadIdx.x == 0 && blockIdx.z == 0) lse[(int64_t)r * H + h] = (M + log2f(L)) * 0.6931471805599453f;
  } else {
    float mloc = -INFINITY;
    for (int s = threadIdx.x; s < nsplit; s += nt) {
      wgt[s] = ml[(int64_t)s * 2 * H];
      mloc = fmaxf(mloc, wgt[s]);
    }
    for (int o = 32; o >= 1; o >>= 1) mloc = fmaxf(mloc, shfl_xor_f(mloc, o));
    if (l == 0) red[0][w] = mloc;
    __syncthreads();
    float M = red[0][0];
    for (int i = 1; i < nw; ++i) M = fmaxf(M, red[0][i]);
    float lloc = 0.f;
    for (int s = threadIdx.x; s < nsplit; s += nt) {
      const float ms = wgt[s];
      const float e = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
      lloc += e * ml[(int64_t)s * 2 * H + 1];
      wgt[s] = e;
    }
    for (int o = 32; o >= 1; o >>= 1) lloc += shfl_xor_f(lloc, o);
    if (l == 0) red[1][w] = lloc;
    __syncthreads();
    float L = red[1][0];
    for (int i = 1; i < nw; ++i) L += red[1][i];
    const float inv = 1.f / L;
    const int td_n = nt / SG, td = threadIdx.x % td_n, sg = threadIdx.x / td_n;
    const int per = (nsplit + SG - 1) / SG;
    const int s_begin = sg * per, s_end = s_begin + per < nsplit ? s_begin + per : nsplit;
    const int d_first = blockIdx.z * dslice;
    for (int d4 = td; d4 < dslice / 4; d4 += td_n) {
      const int dd = d_first + 4 * d4;
      const float* src = ws_o + ((int64_t)r * nsplit * H + h) * D + dd;      // split s at + s H D
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      int s = s_begin;
      for (; s + 8 <= s_end; s += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4*>(src + (int64_t)(s + u) * H * D);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += wgt[s + u] * v[u];
      }
      for (; s < s_end; ++s) acc += wgt[s] * *reinterpret_cast<const f32x4*>(src + (int64_t)s * H * D);
      const int64_t off = ((int64_t)r * H + h) * D + dd;
      if (out_dtype == SCKV_BF16) {
        uint16_t* o = static_cast<uint16_t*>(out) + off;
        const uint32_t lo = f32_to_bf16_rne(acc[0] * inv) | (f32_to_bf16_rne(acc[1] * inv) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc[2] * inv) | (f32_to_bf16_rne(acc[3] * inv) << 16);
        *reinterpret_cast<u32x2*>(o) = u32x2{lo, hi};
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + off) = acc * inv;
      }
    }
    if (lse && threadIdx.x == 0 && blockIdx.z == 0) lse[(int64_t)r * H + h] = (M + log2f(L)) * 0.6931471805599453f;
  }
}

// fp32 path: one block per row, items 64 at a time through LDS.
constexpr int kF32Chunk = 64;
__global__ __launch_bounds__(256) void attend_f32(AttendParams p, int D) {
  extern __shared__ float sm[];
  const int H = p.H;
  float* qs = sm;                              // [H][D]
  float* it = qs + H * D;                      // [64][D]
  float* lg = it + kF32Chunk * D;              // [H][64]
  float* mrun = lg + H * kF32Chunk;            // [H]
  float* lrun = mrun + H;                      // [H]
  float* alpha = lrun + H;                     // [H]
  float* ok = alpha + H;                       // [64]
  const int r = blockIdx.y;
  const RowItems ri = row_items(p, r);
  const float* qg = reinterpret_cast<const float*>(p.q) + (int64_t)r * H * D;
  for (int i = threadIdx.x; i < H * D; i += 256) qs[i] = qg[i];
  for (int h = threadIdx.x; h < H; h += 256) { mrun[h] = -INFINITY; lrun[h] = 0.f; }
  constexpr int MAXP = 16;                     // H * D <= 4096 = 16 * 256
  float o[MAXP];
#pragma unroll
  for (int k = 0; k < MAXP; ++k) o[k] = 0.f;
  __syncthreads();
  for (int64_t q0 = 0; q0 < ri.n_items; q0 += kF32Chunk) {
    for (int c = threadIdx.x; c < kF32Chunk; c += 256) {
      const int64_t src = item_source(p, ri, r, q0 + c);
      ok[c] = src == -1 ? 0.f : 1.f;
    }
    for (int i = threadIdx.x; i < kF32Chunk * D; i += 256) {
      const int c = i / D, d = i % D;
      const int64_t src = item_source(p, ri, r, q0 + c);
      float v = 0.f;
      if (src >= 0) v = static_cast<const float*>(p.entries)[(ri.seq * p.E_cap + src) * D + d];
      else if (src <= -2) v = static_cast<const float*>(p.win)[(ri.seq * p.R_w + (-2 - src)) * D + d];
      it[i] = v;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < H * kF32Chunk; i += 256) {
      const int h = i / kF32Chunk, c = i % kF32Chunk;
      float s = 0.f;
      for (int d = 0; d < D; ++d) s = fmaf(qs[h * D + d], it[c * D + d], s);
      lg[i] = ok[c] != 0.f ? s * p.scale : -INFINITY;
    }
    __syncthreads();
    for (int h = threadIdx.x; h < H; h += 256) {
      float cm = -INFINITY;
      for (int c = 0; c < kF32Chunk; ++c) cm = fmaxf(cm, lg[h * kF32Chunk + c]);
      const float mn = fmaxf(mrun[h], cm);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float a = mrun[h] == -INFINITY ? 0.f : expf(mrun[h] - mn);
      float ps = 0.f;
      for (int c = 0; c < kF32Chunk; ++c) {
        const float e = expf(lg[h * kF32Chunk + c] - mu);
        lg[h * kF32Chunk + c] = e;
        ps += e;
      }
      lrun[h] = lrun[h] * a + ps;
      mrun[h] = mn;
      alpha[h] = a;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
      const int i = threadIdx.x + 256 * k;
      if (i < H * D) {
        const int h = i / D, d = i % D;
        float acc = o[k] * alpha[h];
        for (int c = 0; c < kF32Chunk; ++c) acc = fmaf(lg[h * kF32Chunk + c], it[c * D + d], acc);
        o[k] = acc;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < MAXP; ++k) {
    const int i = threadIdx.x + 256 * k;
    if (i < H * D) {
      const int h = i / D;
      const float v = o[k] / lrun[h];
      const int64_t off = (int64_t)r * H * D + i;
      if (p.out_dtype == SCKV_BF16) static_cast<uint16_t*>(p.out)[off] = (uint16_t)f32_to_bf16_rne(v);
      else static_cast<float*>(p.out)[off] = v;
    }
  }
  if (p.lse)
    for (int h = threadIdx.x; h < H; h += 256) p.lse[(int64_t)r * H + h] = mrun[h] + logf(lrun[h]);
}

AttendPlan plan_attend(const sckv_attend_args& a, bool csa) {
  AttendPlan pl;
  const int64_t t = a.rows.kind == SCKV_ROWS_DECODE ? a.rows.pos_max : (int64_t)a.rows.pos0 + a.rows.R - 1;
  int64_t ev = entries_visible(t, a.m, a.W);
  ev = ev < a.E_cap ? ev : a.E_cap;
  pl.items = (csa ? a.k : ev) + a.W;
  // split granularity: 64 items, or for a few rows on the register-staged kernel
  // at D = 512 (which stages 32 items at a time) single 32-item chunks
  const bool dma = a.entry_dtype == SCKV_BF16 && a.D == 512 && a.H == 64;
  const int64_t unit = (!dma && a.D == 512 && a.rows.R <= 16) ? 32 : kPlanChunk;
  pl.chunks = (pl.items + unit - 1) / unit;
  pl.mfma = a.entry_dtype != SCKV_F32;
  if (!pl.mfma) {
    pl.nsplit = 1;
    pl.per_split = pl.chunks;
    pl.ok = true;
    return pl;
  }
  // about one block per CU (256): splits per row, each of at least two chunks,
  // or of single chunks when there are few rows (their partials are small)
  const int64_t target_blocks = kMaxSplits;
  const int waves = a.H / 16;
  // blocks of 1, 2, 4 or 8 waves: other head counts take one wave per 16-head group
  if ((waves & (waves - 1)) != 0) pl.hgroups = waves;
  const int64_t rows_x = (int64_t)a.rows.R * pl.hgroups;
  int64_t ns = (target_blocks + rows_x / 2) / rows_x;
  ns = ns < 1 ? 1 : (ns > pl.chunks ? pl.chunks : ns);
  int64_t per = (pl.chunks + ns - 1) / ns;
  const int64_t min_per = a.rows.R <= 16 ? 1 : (pl.chunks < 2 ? pl.chunks : 2);
  per = per < min_per ? min_per : per;
  per = per < 1 ? 1 : per;
  pl.per_split = per * unit;             // in items
  pl.nsplit = (int32_t)((pl.chunks + per - 1) / per);
  if (pl.nsplit < 1) pl.nsplit = 1;
  if (pl.nsplit > kMaxSplits) return pl;     // cannot happen: nsplit <= ns <= target_blocks
  if (pl.nsplit > 1)
    pl.ws_bytes = (size_t)a.rows.R * pl.nsplit * a.H * ((size_t)a.D + 2) * sizeof(float) + 256;
  pl.ok = true;
  return pl;
}

template <int ENT, int D>
static void launch_mfma_d(const AttendParams& p, int H, int hgroups, dim3 grid, hipStream_t s) {
  if (ENT == SCKV_BF16 && D == 512 && H == 64) {
    hipLaunchKernelGGL(attend_dma512, dim3(grid.x * grid.y), dim3(512), 0, s, p);
  } else {
    // register-staged chunks: 64 items when the latent is narrow, 32 at D = 512;
    // grid.z = head groups, each block takes H / 16 / hgroups waves of 16 heads
    constexpr int CH = D <= 256 ? 64 : 32;
    grid.z = (unsigned)hgroups;
    switch (H / 16 / hgroups) {    // the plan keeps this in {1, 2, 4, 8}
      case 1: hipLaunchKernelGGL((attend_mfma<ENT, D, 1, CH>), grid, dim3(64), 0, s, p); break;
      case 2: hipLaunchKernelGGL((attend_mfma<ENT, D, 2, CH>), grid, dim3(128), 0, s, p); break;
      case 4: hipLaunchKernelGGL((attend_mfma<ENT, D, 4, CH>), grid, dim3(256), 0, s, p); break;
      case 8: hipLaunchKernelGGL((attend_mfma<ENT, D, 8, CH>), grid, dim3(512), 0, s, p); break;
      default: break;
    }
  }
}

template <int ENT>
static void launch_mfma_e(const AttendParams& p, int H, int hgroups, int D, dim3 grid, hipStream_t s) {
  switch (D) {
    case 64: launch_mfma_d<ENT, 64>(p, H, hgroups, grid, s); break;
    case 128: launch_mfma_d<ENT, 128>(p, H, hgroups, grid, s); break;
    case 256: launch_mfma_d<ENT, 256>(p, H, hgroups, grid, s); break;
    default: launch_mfma_d<ENT, 512>(p, H, hgroups, grid, s); break;
  }
}

hipError_t launch_attend(const sckv_attend_args& a, bool csa, const AttendPlan& pl, void* ws, hipStream_t stream) {
  AttendParams p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.entries = a.entries;
  p.escale = a.entry_scale;
  p.idx = csa ? a.idx : nullptr;
  p.win = a.win;
  p.out = a.out;
  p.lse = a.lse;
  p.pos = a.rows.pos;
  p.E_cap = a.E_cap;
  p.R_w = a.R_w;
  p.kind = a.rows.kind;
  p.pos_max = a.rows.pos_max;
  p.seq0 = a.rows.seq0;
  p.pos0 = a.rows.pos0;
  p.H = a.H;
  p.m = a.m;
  p.W = a.W;
  p.k = a.k;
  p.csa = csa ? 1 : 0;
  p.out_dtype = a.out_dtype;
  p.nsplit = pl.nsplit;
  p.per_split = (int32_t)pl.per_split;   // items
  p.scale = a.softmax_scale;
  p.rows_R = a.rows.R;
  if (pl.nsplit > 1) {
    p.ws_o = static_cast<float*>(ws);
    p.ws_ml = p.ws_o + (size_t)a.rows.R * pl.nsplit * a.H * a.D;
  }
  if (!pl.mfma) {
    const size_t lds = ((size_t)a.H * a.D + (size_t)kF32Chunk * a.D + (size_t)a.H * kF32Chunk + 3 * (size_t)a.H +
                        kF32Chunk) * sizeof(float);
    hipLaunchKernelGGL(attend_f32, dim3(1, a.rows.R), dim3(256), lds, stream, p, a.D);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)pl.nsplit, (unsigned)a.rows.R);
  if (a.entry_dtype == SCKV_E4M3) launch_mfma_e<SCKV_E4M3>(p, a.H, pl.hgroups, a.D, grid, stream);
  else launch_mfma_e<SCKV_BF16>(p, a.H, pl.hgroups, a.D, grid, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nsplit == 1) return e;
  // a few rows with many splits: latent slices of 128 dims and 8 groups of splits
  // per block, so the merge runs on about one block per CU; otherwise one block per
  // (head, row) with each thread taking all the splits
  if ((int64_t)a.rows.R * a.H < 512 && pl.nsplit >= 16) {
    const int dslice = a.D < 128 ? a.D : 128;
    hipLaunchKernelGGL(attend_combine<8>, dim3(a.H, a.rows.R, a.D / dslice), dim3(dslice / 4 * 8), 0, stream,
                       p.ws_o, p.ws_ml, a.out, a.lse, a.H, a.D, pl.nsplit, a.out_dtype, dslice);
  } else {
    hipLaunchKernelGGL(attend_combine<1>, dim3(a.H, a.rows.R, 1), dim3(128), 0, stream, p.ws_o, p.ws_ml, a.out,
                       a.lse, a.H, a.D, pl.nsplit, a.out_dtype, a.D);
  }
  return hipGetLastError();
}

}  // namespace sckv
