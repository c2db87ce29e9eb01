// Gated per-channel softmax pooling of per-token streams into compressed entries.
//
// c_j[d] = sum_{i in P_j} softmax_i(g_i[d] + Bpos[i - m j + o][d]) v_i[d], with
// P_j = [m j - o, m j + m) cut to tokens i >= 0 (the CSA decode workload
// definition's compressor; knightli.com DeepSeek-V4 KV-cache article, sections
// "CSA" (4:1, learned pool, overlapping windows) and "HCA" (128:1)).
//
// HBM streaming: lane groups of D/8 lanes own one entry, each lane 8 channels,
// so every token row is read as one contiguous D-wide segment.
//  - 4:1 windows with overlap 4 (CSA): every 4-token block belongs to two
//    windows; a lane group walks a run of consecutive entries, reads each block
//    once and pools it once into two half-window sums with one exp per (token,
//    channel) (the softmax factored per block, below).
//  - Other windows: the softmax is taken online with one exp per (token,
//    channel), the larger of the running maximum and the new logit setting which
//    side is rescaled; a window of 64 tokens or more (HCA) is pooled in 4 parts
//    (on 4 waves) whose states are folded in order.
// In decode, one token per sequence is appended to small rings of recent tokens,
// and the entry it completes (one per m tokens) is pooled with the bulk kernel's
// arithmetic, so appends and bulk pooling store the same bits.
#include "device_common.h"
#include "sckv_internal.h"

// Every rounding in this file is written out: a product or sum is rounded on its
// own and fused multiply-adds are explicit fmaf calls.  Contraction is switched
// off for the file, and the rounded operations below are defined here (HIP's
// __fmul_rn / __fadd_rn are plain operators compiled under the header's own
// contraction setting), so the bulk and decode kernels round alike and store the
// same bits.
#pragma clang fp contract(off)

namespace sckv {

__device__ __forceinline__ float rmul(float a, float b) { return a * b; }
__device__ __forceinline__ float radd(float a, float b) { return a + b; }
__device__ __forceinline__ float rsub(float a, float b) { return a - b; }

template <int IN>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&x)[8]) {
  if constexpr (IN == SCKV_BF16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(v[i] << 16);
      x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + elem);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
  }
}

// Online-softmax state of one lane's 8 channels over some tokens: running maximum
// of the logits, sum of exp(logit - max) and the matching weighted sum of values.
struct PoolState {
  float mx[8], l[8], acc[8];
};

// Adds tokens [ia, ib) (ia >= 0) to st in token order; the bias row of token i is
// i - i0.  The loads of AHEAD tokens are issued before their updates (the
// arithmetic and its order do not depend on AHEAD).  The larger of the running
// maximum and the new logit decides which side is rescaled, so each
// (token, channel) costs one exp.
// exp(-|d|) as the hardware base-2 exponential of -|d| log2(e): relative error
// about |d| 2^-24 from rounding the product, below 1e-6 for every difference of
// logits that still weighs in the sum (exp(-|d|) underflows past |d| ~ 87)
__device__ __forceinline__ float pool_exp(float d) {
  return __builtin_amdgcn_exp2f(rmul(-fabsf(d), 1.4426950408889634f));
}

__device__ __forceinline__ void pool_init(PoolState& st) {
#pragma unroll
  for (int c = 0; c < 8; ++c) { st.mx[c] = -INFINITY; st.l[c] = 0.f; st.acc[c] = 0.f; }
}

// One token into the state: gate logits g (bias bp0, bp1 added) and values v.
__device__ __forceinline__ void pool_token(PoolState& st, const float (&g)[8], const float (&v)[8], f32x4 bp0,
                                           f32x4 bp1) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float a = radd(g[c], c < 4 ? bp0[c] : bp1[c - 4]);
    const float d = rsub(a, st.mx[c]);
    const float x = pool_exp(d);
    const bool up = d > 0.f;
    const float sc = up ? x : 1.f;
    const float p = up ? 1.f : x;
    st.l[c] = fmaf(st.l[c], sc, p);
    st.acc[c] = fmaf(st.acc[c], sc, rmul(p, v[c]));
    st.mx[c] = fmaxf(st.mx[c], a);
  }
}

template <int AHEAD, class Tok>
__device__ __forceinline__ void pool_range(Tok tok, const float* __restrict__ bpos, int64_t i0, int64_t ia,
                                           int64_t ib, int D, int ch, bool active, PoolState& st) {
  pool_init(st);
  for (int64_t i = ia; i < ib; i += AHEAD) {
    float g[AHEAD][8], v[AHEAD][8];
    f32x4 b0[AHEAD], b1[AHEAD];
#pragma unroll
    for (int u = 0; u < AHEAD; ++u) {
#pragma unroll
      for (int c = 0; c < 8; ++c) { g[u][c] = 0.f; v[u][c] = 0.f; }
      b0[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      b1[u] = b0[u];
      if (active && i + u < ib) {
        tok(i + u, g[u], v[u]);
        const f32x4* bp = reinterpret_cast<const f32x4*>(bpos + (i + u - i0) * D + ch);
        b0[u] = bp[0];
        b1[u] = bp[1];
      }
    }
#pragma unroll
    for (int u = 0; u < AHEAD; ++u)
      if (i + u < ib) pool_token(st, g[u], v[u], b0[u], b1[u]);
  }
}

// Folds the state of a later part of the window into r (an empty part, with a
// maximum of -inf, changes nothing).  Here and in the token update every rounding
// is spelled out (no contraction left to the compiler), so that the bulk and the
// decode kernels produce the same bits.
__device__ __forceinline__ void fold_state(PoolState& r, const PoolState& q) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const bool qe = q.mx[c] == -INFINITY, re = r.mx[c] == -INFINITY;
    const float M = fmaxf(r.mx[c], q.mx[c]);
    const float sa = re ? 0.f : pool_exp(rsub(r.mx[c], M));
    const float sb = qe ? 0.f : pool_exp(rsub(q.mx[c], M));
    const float l = qe ? r.l[c] : (re ? q.l[c] : fmaf(r.l[c], sa, rmul(q.l[c], sb)));
    const float acc = qe ? r.acc[c] : (re ? q.acc[c] : fmaf(r.acc[c], sa, rmul(q.acc[c], sb)));
    r.l[c] = l;
    r.acc[c] = acc;
    r.mx[c] = M;
  }
}

// A pooling window [i0, i1) of 64 tokens or more is cut into 4 parts of
// ceil((i1 - i0) / 4) tokens; each part is pooled on its own and the parts are
// folded in order.  The bulk compressor runs the parts one after another, the
// decode append on four waves, with identical arithmetic.  Shorter windows are
// pooled in one pass.
constexpr int kParts = 4;

__device__ __forceinline__ int window_parts(int64_t i0, int64_t i1) { return i1 - i0 >= 64 ? kParts : 1; }

__device__ __forceinline__ void part_range(int64_t i0, int64_t i1, int q, int64_t& ia, int64_t& ib) {
  const int np = window_parts(i0, i1);
  const int64_t len = (i1 - i0 + np - 1) / np;
  int64_t a = i0 + q * len, b = a + len;
  b = b < i1 ? b : i1;
  a = a < 0 ? 0 : a;
  ia = a;
  ib = b > a ? b : a;
}

// Stores entry e of sequence b from its pooled state.  This lane owns channels
// ch .. ch+7; the entry's G = D/8 lanes are G consecutive lanes of a G-aligned
// group (the e4m3 scale is reduced over them).  Lanes with active == false take
// part in the reduction but store nothing.
template <int OUT, bool SCALED>
__device__ __forceinline__ void store_values(const float (&cv)[8], int ch, int G, bool active, int sub, int64_t b,
                                             int64_t e, int D, int64_t E_cap, int key_tiles, void* __restrict__ out,
                                             float* __restrict__ out_scale) {

  // rows: [E_cap][D]; key tiles: [E_cap/32][D/8][32][8] (8 channels of 32 entries contiguous)
  const int64_t orow = key_tiles ? b * E_cap * D + (((e >> 5) * (D >> 3) + (ch >> 3)) * 32 + (e & 31)) * 8
                                 : (b * E_cap + e) * D + ch;
  if constexpr (OUT == SCKV_F32) {
    if (active) {
      f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(out) + orow);
      p[0] = f32x4{cv[0], cv[1], cv[2], cv[3]};
      p[1] = f32x4{cv[4], cv[5], cv[6], cv[7]};
    }
  } else if constexpr (OUT == SCKV_BF16) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = f32_to_bf16_rne(cv[2 * i]) | (f32_to_bf16_rne(cv[2 * i + 1]) << 16);
    if (active) *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + orow) = r;
  } else if constexpr (OUT == SCKV_MXFP4) {
    // OCP MX block of 32 channels = the 4 lanes sub = 4i .. 4i + 3 of this entry.
    // Shared scale 2^X with X = floor(log2 max|c|) - 2 clamped to [-127, 127]
    // (the biased fp32 exponent of the block maximum gives floor(log2); a zero or
    // subnormal maximum gives -127).
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(cv[c]));
    amax = fmaxf(amax, shfl_xor_f(amax, 1));
    amax = fmaxf(amax, shfl_xor_f(amax, 2));
    int X = (int)((__float_as_uint(amax) >> 23) & 255u) - 127 - 2;
    X = X < -127 ? -127 : (X > 127 ? 127 : X);
    // e2m1 code of c / 2^X (exact power-of-two scaling), to nearest with ties to
    // the even mantissa bit, saturating at 6: the count of rounding midpoints
    // 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 that |x| passes (a tie passes the
    // midpoints below the even neighbours 1, 2, 4 and not those below 0.5, 1.5, 3, 6)
    uint32_t word = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float a = fabsf(ldexpf(cv[c], -X));
      uint32_t code = (a > 0.25f ? 1u : 0u) + (a >= 0.75f ? 1u : 0u) + (a > 1.25f ? 1u : 0u) +
                      (a >= 1.75f ? 1u : 0u) + (a > 2.5f ? 1u : 0u) + (a >= 3.5f ? 1u : 0u) + (a > 5.0f ? 1u : 0u);
      code |= (__float_as_uint(cv[c]) >> 31) << 3;
      word |= code << (4 * c);
    }
    if (active) {
      // tile of 32 entries: codes [D/32][32][16 B], then scales [32][D/32] B
      uint8_t* tile = static_cast<uint8_t*>(out) + (b * (E_cap >> 5) + (e >> 5)) * (17 * (int64_t)D);
      *reinterpret_cast<uint32_t*>(tile + ((ch >> 5) * 32 + (e & 31)) * 16 + 4 * ((ch >> 3) & 3)) = word;
      if ((ch & 31) == 0) tile[16 * D + (e & 31) * (D >> 5) + (ch >> 5)] = (uint8_t)(X + 127);
    }
  } else {
    float scale = 1.f;
    if constexpr (SCALED) {
      float amax = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(cv[c]));
      for (int s = 1; s < G; s <<= 1) amax = fmaxf(amax, shfl_xor_f(amax, s));
      scale = amax > 0.f ? amax / 448.0f : 1.0f;
    }
    const float rscale = 1.0f / scale;
    u32x2 r = {0u, 0u};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t q = f32_to_e4m3_sat(SCALED ? rmul(cv[c], rscale) : cv[c]);
      r[c >> 2] |= q << ((c & 3) * 8);
    }
    if (active) {
      *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(out) + orow) = r;
      if (SCALED && sub == 0) out_scale[b * E_cap + e] = scale;
    }
  }
}

// Stores the entry of an online-softmax state (the pooled value of each channel is
// its weighted sum over its normaliser).
template <int OUT, bool SCALED>
__device__ __forceinline__ void store_entry(const PoolState& st, int ch, int G, bool active, int sub, int64_t b,
                                            int64_t e, int D, int64_t E_cap, int key_tiles, void* __restrict__ out,
                                            float* __restrict__ out_scale) {
  float cv[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) cv[c] = st.acc[c] / st.l[c];
  store_values<OUT, SCALED>(cv, ch, G, active, sub, b, e, D, E_cap, key_tiles, out, out_scale);
}

// ------------------------------------------------------------------ overlapping 4:1 windows
// CSA pooling (m = 4, overlap o = 4): entry e pools tokens [4e - 4, 4e + 4), token
// blocks e - 1 and e (block k = tokens 4k .. 4k+3), with the bias rows 0..3 on
// block e - 1 and 4..7 on block e, so every block belongs to two windows.  The
// softmax is factored per block: with s_k the block's largest gate logit (per
// channel) and u_p = exp(Bpos[p] - max_p Bpos[p]),
//   exp(g_i + Bpos[p] - const) = exp(g_i - s_k) u_p exp(s_k - S),  S = max(s_{e-1}, s_e),
// so one exp per (token, channel) serves both windows: each block keeps two
// half-window sums (sum of w and of w v, w = exp(g_i - s_k) u_p) for its two bias
// halves, and an entry joins the previous block's first-half sums to its own
// block's second-half sums with the factors exp(s_k - S), then divides.  The
// common factor cancels in the quotient.  Exact in real arithmetic; in fp32 a
// weight below 2^-126 of the window's largest is lost, which needs a spread of
// the bias rows of more than about 60 (the largest weight is at least
// exp(-spread)): such channels take the online path.  The bulk kernel and the
// decode append share these functions, so both store the same bits.
constexpr int kOvM = 4;                       // tokens per block (m = o = 4)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxBiasSpread = 60.0f;
constexpr int kOvMaxD = 512;                  // widest latent the bulk kernel's factor table holds

// Block maximum and per-token factors exp(g_t - s) (base 2, log2 e folded in).
__device__ __forceinline__ void ov_block(const float (&g)[kOvM][8], float (&s)[8], float (&E)[kOvM][8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    s[c] = fmaxf(fmaxf(g[0][c], g[1][c]), fmaxf(g[2][c], g[3][c]));
    const float sl = rmul(s[c], kLog2e);
#pragma unroll
    for (int t = 0; t < kOvM; ++t) E[t][c] = __builtin_amdgcn_exp2f(fmaf(g[t][c], kLog2e, -sl));
  }
}

// Half-window sums of one block for the bias rows u[0..3] (token order).
__device__ __forceinline__ void ov_half(const float (&E)[kOvM][8], const float (&v)[kOvM][8],
                                        const float (&u)[kOvM][8], float (&l)[8], float (&acc)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float w = rmul(E[0][c], u[0][c]);
    float ls = w, as = rmul(w, v[0][c]);
#pragma unroll
    for (int t = 1; t < kOvM; ++t) {
      w = rmul(E[t][c], u[t][c]);
      ls = radd(ls, w);
      as = fmaf(w, v[t][c], as);
    }
    l[c] = ls;
    acc[c] = as;
  }
}

// Entry from the first half (previous block: max sp, sums lp, ap) and the second
// half (this block: s, l, a).  A missing previous block has sp = -inf, lp = ap = 0.
__device__ __forceinline__ void ov_entry(const float (&sp)[8], const float (&lp)[8], const float (&ap)[8],
                                         const float (&s)[8], const float (&l)[8], const float (&a)[8],
                                         float (&cv)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    // the half with the larger maximum keeps factor 1, the other exp(-|difference|)
    // (a missing previous block: exp2(-inf) = 0)
    const float d = rsub(sp[c], s[c]);
    const float f = __builtin_amdgcn_exp2f(rmul(-fabsf(d), kLog2e));
    const bool prev_up = d > 0.f;
    const float f1 = prev_up ? 1.f : f;
    const float f2 = prev_up ? f : 1.f;
    const float lt = fmaf(lp[c], f1, rmul(l[c], f2));
    const float at = fmaf(ap[c], f1, rmul(a[c], f2));
    cv[c] = rmul(at, __builtin_amdgcn_rcpf(lt));
  }
}

// Bias factors u[p] = exp(Bpos[p][c] - max_p Bpos[p][c]) of one channel c (rows
// 0 .. 7), and whether the rows spread by at most kMaxBiasSpread.
__device__ __forceinline__ bool ov_bias_channel(const float* __restrict__ bpos, int D, int c, float (&u)[2 * kOvM]) {
  float b[2 * kOvM];
#pragma unroll
  for (int p = 0; p < 2 * kOvM; ++p) b[p] = bpos[(int64_t)p * D + c];
  float hi = b[0], lo = b[0];
#pragma unroll
  for (int p = 1; p < 2 * kOvM; ++p) { hi = fmaxf(hi, b[p]); lo = fminf(lo, b[p]); }
  const float hl = rmul(hi, kLog2e);
#pragma unroll
  for (int p = 0; p < 2 * kOvM; ++p) u[p] = __builtin_amdgcn_exp2f(fmaf(b[p], kLog2e, -hl));
  return rsub(hi, lo) <= kMaxBiasSpread;
}

// The factors of this lane's channels ch .. ch+7, and whether every one of the
// entry's D channels (G lanes from group lane 0) stays within the spread.
__device__ __forceinline__ bool ov_bias(const float* __restrict__ bpos, int D, int ch, int G,
                                        float (&u)[2 * kOvM][8]) {
  bool ok = true;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float uc[2 * kOvM];
    ok = ov_bias_channel(bpos, D, ch + c, uc) && ok;
#pragma unroll
    for (int p = 0; p < 2 * kOvM; ++p) u[p][c] = uc[p];
  }
  // all lanes of the entry's group agree (G is a power of two, the group G-aligned)
  int okall = ok ? 1 : 0;
  for (int sft = 1; sft < G; sft <<= 1) okall &= __shfl_xor(okall, sft, kWave);
  return okall != 0;
}

// A block's gate and value rows for one lane's 8 channels as loaded (bf16 pairs
// or fp32), unpacked only when used, so a prefetched block costs few registers.
template <int IN>
struct RawBlock {
  static constexpr int W = IN == SCKV_BF16 ? 1 : 2;   // 16-byte words per 8 channels
  u32x4 g[kOvM][W], v[kOvM][W];
};

template <int IN>
__device__ __forceinline__ void raw_load(const void* base, int64_t elem, u32x4 (&w)[RawBlock<IN>::W]) {
  if constexpr (IN == SCKV_BF16) {
    w[0] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem);
  } else {
    const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + elem);
    w[0] = q[0];
    w[1] = q[1];
  }
}

template <int IN>
__device__ __forceinline__ void raw_unpack(const u32x4 (&w)[RawBlock<IN>::W], float (&x)[8]) {
  if constexpr (IN == SCKV_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[0][i] << 16);
      x[2 * i + 1] = __uint_as_float(w[0][i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = __uint_as_float(w[0][i]); x[4 + i] = __uint_as_float(w[1][i]); }
  }
}

template <int IN>
__device__ __forceinline__ void raw_block_load(const void* gate, const void* val, int64_t row0, int D,
                                               RawBlock<IN>& rb) {
#pragma unroll
  for (int t = 0; t < kOvM; ++t) {
    raw_load<IN>(gate, row0 + (int64_t)t * D, rb.g[t]);
    raw_load<IN>(val, row0 + (int64_t)t * D, rb.v[t]);
  }
}

template <int IN>
__device__ __forceinline__ void raw_block_unpack(const RawBlock<IN>& rb, float (&g)[kOvM][8], float (&v)[kOvM][8]) {
#pragma unroll
  for (int t = 0; t < kOvM; ++t) {
    raw_unpack<IN>(rb.g[t], g[t]);
    raw_unpack<IN>(rb.v[t], v[t]);
  }
}

__device__ __forceinline__ const float (&ov_rows(const float (&u)[2 * kOvM][8], int half))[kOvM][8] {
  return *reinterpret_cast<const float(*)[kOvM][8]>(&u[kOvM * half]);
}

// Windows shorter than 64 tokens, pooled in one pass by D/8 lanes per entry, the
// loads of two tokens in flight (windows of 64 or more: compress_parts_kernel).
template <int IN, int OUT, bool SCALED>
__global__ __launch_bounds__(256) void compress_kernel(
    const void* __restrict__ val, const void* __restrict__ gate, const float* __restrict__ bpos,
    void* __restrict__ out, float* __restrict__ out_scale, int64_t N, int D, int m, int o,
    int64_t e_begin, int64_t e_count, int64_t E_cap, int G, int key_tiles) {
  const int lane = lane_id();
  const int epw = kWave / G;
  const int slot = lane / G, sub = lane % G;
  const int64_t e_local = (int64_t)blockIdx.x * (4 * epw) + wave_id() * epw + slot;
  const bool active = e_local < e_count;
  const int64_t e = e_begin + (active ? e_local : 0);
  const int64_t b = blockIdx.y;
  const int ch = sub * 8;
  auto tok = [&](int64_t i, float (&g)[8], float (&v)[8]) __attribute__((always_inline)) {
    const int64_t row = (b * N + i) * D + ch;
    load8<IN>(gate, row, g);
    load8<IN>(val, row, v);
  };
  const int64_t i0 = (int64_t)m * e - o, i1 = (int64_t)m * e + m;
  PoolState r;
  int64_t ia, ib;
  part_range(i0, i1, 0, ia, ib);
  pool_range<2>(tok, bpos, i0, ia, ib, D, ch, active, r);
  store_entry<OUT, SCALED>(r, ch, G, active, sub, b, e, D, E_cap, key_tiles, out, out_scale);
}

// Bias-factor table in LDS: row p, channel c at [p][c mod 8 >= 4][c / 8][c mod 4],
// so the 16-byte reads of a wave's lanes (channels 8 l .. 8 l + 3, then + 4 .. + 7)
// are contiguous and free of bank conflicts.
__device__ __forceinline__ int ov_u_index(int p, int c, int ch, int D) {
  const int cc = ch + c;
  return (2 * p + ((cc >> 2) & 1)) * (D >> 1) + (cc >> 3) * 4 + (cc & 3);
}

// Both half-window sums of one block straight from its loaded rows: the block
// maximum first, then token by token the factor exp(g - s) and its two weighted
// terms, with the bias factors of rows 4..7 (second half: la, aa) and rows 0..3
// (first half of the next entry: lb, ab) read from the table in LDS.  The same
// operations in the same order as ov_block and ov_half, so the same bits, with
// far fewer values live at once.
template <int IN>
__device__ __forceinline__ void ov_block_sums(const RawBlock<IN>& rb, const float* u_sh, int D, int ch,
                                              float (&s)[8], float (&la)[8], float (&aa)[8], float (&lb)[8],
                                              float (&ab)[8]) {
  {
    float x[8];
    raw_unpack<IN>(rb.g[0], x);
#pragma unroll
    for (int c = 0; c < 8; ++c) s[c] = x[c];
#pragma unroll
    for (int t = 1; t < kOvM; ++t) {
      raw_unpack<IN>(rb.g[t], x);
#pragma unroll
      for (int c = 0; c < 8; ++c) s[c] = fmaxf(s[c], x[c]);
    }
  }
  float sl[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) sl[c] = rmul(s[c], kLog2e);
#pragma unroll
  for (int t = 0; t < kOvM; ++t) {
    float g[8], v[8], ua[8], ub[8];
    raw_unpack<IN>(rb.g[t], g);
    raw_unpack<IN>(rb.v[t], v);
    {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(&u_sh[ov_u_index(kOvM + t, 0, ch, D)]);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(&u_sh[ov_u_index(kOvM + t, 4, ch, D)]);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(&u_sh[ov_u_index(t, 0, ch, D)]);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(&u_sh[ov_u_index(t, 4, ch, D)]);
#pragma unroll
      for (int c = 0; c < 4; ++c) { ua[c] = a0[c]; ua[4 + c] = a1[c]; ub[c] = b0[c]; ub[4 + c] = b1[c]; }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float E = __builtin_amdgcn_exp2f(fmaf(g[c], kLog2e, -sl[c]));
      const float wa = rmul(E, ua[c]), wb = rmul(E, ub[c]);
      if (t == 0) {
        la[c] = wa;
        aa[c] = rmul(wa, v[c]);
        lb[c] = wb;
        ab[c] = rmul(wb, v[c]);
      } else {
        la[c] = radd(la[c], wa);
        aa[c] = fmaf(wa, v[c], aa[c]);
        lb[c] = radd(lb[c], wb);
        ab[c] = fmaf(wb, v[c], ab[c]);
      }
    }
  }
}

// Arguments of one stream of the overlapping-window compressor.
struct OvArgs {
  const void* val;
  const void* gate;
  const float* bpos;
  void* out;
  float* out_scale;
  int64_t N, e_begin, e_count, E_cap;
  int D, G, key_tiles, J;
};

// Overlapping 4:1 windows (m = o = 4) by the factored softmax.  The S = 4 * 64/G
// lane groups ("slots", G = D/8 lanes each) of a block take S consecutive entries
// per step, J steps in turn, so a block pools a run of S * J consecutive entries.
// Each slot loads and pools one 4-token block per step (the next step's block in
// flight meanwhile) into its two half-window sums; an entry needs the first-half
// sums of the block before its own, which the neighbouring slot computed in the
// same step (slot 0: slot S-1 in the step before), passed through LDS.  Only the
// block before the run is pooled twice.  Channels whose bias rows spread too far
// take the online path entry by entry.
// The block (bx, b) of one stream's grid (block-uniform: every barrier inside is
// reached by the whole block).
// LDS of an overlap block: the bias factors of all D channels ([row][channel],
// shared by the block's slots) and the first-half state (block max, sums) of
// each slot's block, two steps' worth.
struct OvLds {
  __attribute__((aligned(16))) float u_sh[2 * kOvM * kOvMaxD];
  float carry[2][3 * 8][256];
};

template <int IN, int OUT, bool SCALED>
__device__ __forceinline__ void overlap_run(const OvArgs& a, int64_t bx, int64_t by, OvLds& L) {
  const void* __restrict__ val = a.val;
  const void* __restrict__ gate = a.gate;
  const float* __restrict__ bpos = a.bpos;
  void* __restrict__ out = a.out;
  float* __restrict__ out_scale = a.out_scale;
  const int64_t N = a.N, e_begin = a.e_begin, e_count = a.e_count, E_cap = a.E_cap;
  const int D = a.D, G = a.G, key_tiles = a.key_tiles, J = a.J;
  const int lane = lane_id();
  const int epw = kWave / G;
  const int S = 4 * epw;
  const int gs = wave_id() * epw + lane / G, sub = lane % G;    // slot in the block; threadIdx.x = gs * G + sub
  const int64_t R0 = bx * S * J;                                // the block's first local entry
  const int64_t b = by;
  const int ch = sub * 8;
  float* u_sh = L.u_sh;
  float (*carry)[3 * 8][256] = L.carry;
  bool ok = true;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float uc[2 * kOvM];
    ok = ov_bias_channel(bpos, D, c, uc) && ok;
#pragma unroll
    for (int p = 0; p < 2 * kOvM; ++p) u_sh[ov_u_index(p, 0, c, D)] = uc[p];
  }
  const bool fast = __syncthreads_and(ok ? 1 : 0) != 0;
  if (R0 >= e_count) return;                                     // whole block
  if (!fast) {
    auto tok = [&](int64_t i, float (&g)[8], float (&v)[8]) __attribute__((always_inline)) {
      const int64_t row = (b * N + i) * D + ch;
      load8<IN>(gate, row, g);
      load8<IN>(val, row, v);
    };
    for (int j = 0; j < J; ++j) {
      const int64_t el = R0 + (int64_t)j * S + gs;
      if (el >= e_count) break;
      const int64_t e = e_begin + el;
      const int64_t i0 = (int64_t)kOvM * e - kOvM, i1 = (int64_t)kOvM * e + kOvM;
      PoolState r;
      int64_t ia, ib;
      part_range(i0, i1, 0, ia, ib);
      pool_range<2>(tok, bpos, i0, ia, ib, D, ch, true, r);
      store_entry<OUT, SCALED>(r, ch, G, true, sub, b, e, D, E_cap, key_tiles, out, out_scale);
    }
    return;
  }
  const int64_t row_b = b * N * D + ch;            // token i's channels at row_b + i * D
  const int64_t last = e_count - 1;                // loads of entries past the range re-read the last one
  float sp[8], lp[8], ap[8];                       // slot 0: the state of the block before its entry
  if (gs == 0) {
    const int64_t e_prev = e_begin + R0 - 1;
    if (e_prev >= 0) {
      RawBlock<IN> pb;
      raw_block_load<IN>(gate, val, row_b + e_prev * kOvM * D, D, pb);
      float la[8], aa[8];
      ov_block_sums<IN>(pb, u_sh, D, ch, sp, la, aa, lp, ap);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) { sp[c] = -INFINITY; lp[c] = 0.f; ap[c] = 0.f; }
    }
  }
  auto entry_of = [&](int j) { const int64_t el = R0 + (int64_t)j * S + gs; return el < last ? el : last; };
  RawBlock<IN> rb;
  raw_block_load<IN>(gate, val, row_b + (e_begin + entry_of(0)) * kOvM * D, D, rb);
  for (int j = 0; j < J; ++j) {
    if (R0 + (int64_t)j * S >= e_count) break;                  // uniform over the block
    const int64_t el = R0 + (int64_t)j * S + gs;
    const int64_t e = e_begin + (el < last ? el : last);
    RawBlock<IN> cur = rb;
    if (j + 1 < J) raw_block_load<IN>(gate, val, row_b + (e_begin + entry_of(j + 1)) * kOvM * D, D, rb);
    float s[8], la[8], aa[8], lb[8], ab[8], cv[8];
    ov_block_sums<IN>(cur, u_sh, D, ch, s, la, aa, lb, ab);
    float (&cw)[3 * 8][256] = carry[j & 1];
#pragma unroll
    for (int c = 0; c < 8; ++c) { cw[c][threadIdx.x] = s[c]; cw[8 + c][threadIdx.x] = lb[c]; cw[16 + c][threadIdx.x] = ab[c]; }
    __syncthreads();
    if (gs != 0) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        sp[c] = cw[c][threadIdx.x - G];
        lp[c] = cw[8 + c][threadIdx.x - G];
        ap[c] = cw[16 + c][threadIdx.x - G];
      }
    }
    ov_entry(sp, lp, ap, s, la, aa, cv);
    if (el < e_count) store_values<OUT, SCALED>(cv, ch, G, true, sub, b, e, D, E_cap, key_tiles, out, out_scale);
    if (gs == 0) {                                               // slot S-1's block precedes slot 0's next entry
      const int src = threadIdx.x + (S - 1) * G;
#pragma unroll
      for (int c = 0; c < 8; ++c) { sp[c] = cw[c][src]; lp[c] = cw[8 + c][src]; ap[c] = cw[16 + c][src]; }
    }
  }
}

template <int IN, int OUT, bool SCALED>
__global__ __launch_bounds__(256) void compress_overlap_kernel(OvArgs a) {
  __shared__ OvLds L;
  overlap_run<IN, OUT, SCALED>(a, blockIdx.x, blockIdx.y, L);
}

// Two streams of one input type in one grid (the latent and the indexer keys of
// a CSA layer; each with its own output type): blocks 0 .. nb0 - 1 take the
// first, the rest the second, so the second stream's blocks fill the first one's
// tail instead of a launch of their own.
template <int IN, int OUT0, bool SC0, int OUT1, bool SC1>
__global__ __launch_bounds__(256) void compress_overlap_pair(OvArgs a0, OvArgs a1, unsigned nb0) {
  __shared__ OvLds L;
  if (blockIdx.x < nb0) overlap_run<IN, OUT0, SC0>(a0, blockIdx.x, blockIdx.y, L);
  else overlap_run<IN, OUT1, SC1>(a1, blockIdx.x - nb0, blockIdx.y, L);
}

// Windows of 64 tokens or more (HCA): the 4 parts of each window on the 4 waves
// of a block (wave q pools part q of the block's entries), folded in order by
// wave 0 through LDS, the arithmetic of the decode append, with two tokens'
// loads in flight per wave.
template <int IN, int OUT, bool SCALED>
__global__ __launch_bounds__(256) void compress_parts_kernel(
    const void* __restrict__ val, const void* __restrict__ gate, const float* __restrict__ bpos,
    void* __restrict__ out, float* __restrict__ out_scale, int64_t N, int D, int m, int o,
    int64_t e_begin, int64_t e_count, int64_t E_cap, int G, int key_tiles) {
  __shared__ PoolState parts[kParts - 1][kWave];
  const int lane = lane_id(), w = wave_id();
  const int epw = kWave / G;
  const int slot = lane / G, sub = lane % G;
  const int64_t e_local = (int64_t)blockIdx.x * epw + slot;
  const bool active = e_local < e_count;
  const int64_t e = e_begin + (active ? e_local : 0);
  const int64_t b = blockIdx.y;
  const int ch = sub * 8;
  auto tok = [&](int64_t i, float (&g)[8], float (&v)[8]) __attribute__((always_inline)) {
    const int64_t row = (b * N + i) * D + ch;
    load8<IN>(gate, row, g);
    load8<IN>(val, row, v);
  };
  const int64_t i0 = (int64_t)m * e - o, i1 = (int64_t)m * e + m;
  PoolState st;
  int64_t ia, ib;
  part_range(i0, i1, w, ia, ib);
  pool_range<2>(tok, bpos, i0, ia, ib, D, ch, active, st);
  if (w > 0) parts[w - 1][lane] = st;
  __syncthreads();
  if (w != 0) return;
#pragma unroll 1
  for (int p = 1; p < kParts; ++p) fold_state(st, parts[p - 1][lane]);
  store_entry<OUT, SCALED>(st, ch, G, active, sub, b, e, D, E_cap, key_tiles, out, out_scale);
}

// One stream of a decode append, as the kernel sees it.
struct AppendK {
  const int32_t* pos;
  const void* val;
  const void* gate;
  void* val_ring;
  void* gate_ring;
  const float* bpos;
  void* out;
  float* out_scale;
  int64_t E_cap;
  int D, P, key_tiles;
};

// Decode append: one new token per sequence (one block of 4 waves per sequence;
// blockIdx.y picks one of up to two streams that share the pool and the dtypes).
// The token goes into the value and gate rings at slot t mod P; when it completes
// entry e = (t + 1) / m - 1, the entry is pooled from the rings (tokens before t)
// and the new token: wave q pools part q of the window (wave 0 alone for a short
// window), and wave 0 folds the parts in order and stores the entry (the bulk
// compressor's arithmetic, bit for bit).
template <int IN, int OUT, bool SCALED>
__global__ __launch_bounds__(256) void append_kernel(AppendK s0, AppendK s1, int m, int o) {
  constexpr int ES = IN == SCKV_BF16 ? 2 : 4;
  __shared__ PoolState parts[kParts - 1][kWave];
  const AppendK& s = blockIdx.y == 0 ? s0 : s1;
  const int64_t b = blockIdx.x;
  const int D = s.D, P = s.P;
  const int G = D / 8, lane = lane_id(), w = wave_id();
  const bool active = lane < G;
  const int ch = active ? lane * 8 : 0;
  const int32_t t = s.pos[b];
  if (t < 0) return;                                       // whole block: nothing to append
  const int64_t slot_t = t % P;
  if (w == 0 && active) {
    const uint8_t* sv = static_cast<const uint8_t*>(s.val) + (b * D + ch) * ES;
    const uint8_t* sg = static_cast<const uint8_t*>(s.gate) + (b * D + ch) * ES;
    uint8_t* dv = static_cast<uint8_t*>(s.val_ring) + ((b * P + slot_t) * D + ch) * ES;
    uint8_t* dg = static_cast<uint8_t*>(s.gate_ring) + ((b * P + slot_t) * D + ch) * ES;
#pragma unroll
    for (int k = 0; k < ES / 2; ++k) {
      reinterpret_cast<u32x4*>(dv)[k] = reinterpret_cast<const u32x4*>(sv)[k];
      reinterpret_cast<u32x4*>(dg)[k] = reinterpret_cast<const u32x4*>(sg)[k];
    }
  }
  if ((t + 1) % m != 0) return;                            // uniform: no entry completes
  const int64_t e = (int64_t)(t + 1) / m - 1;
  if (e >= s.E_cap) return;
  auto tok = [&](int64_t i, float (&g)[8], float (&v)[8]) __attribute__((always_inline)) {
    if (i == t) {
      load8<IN>(s.gate, b * D + ch, g);
      load8<IN>(s.val, b * D + ch, v);
    } else {
      const int64_t row = (b * P + i % P) * D + ch;
      load8<IN>(s.gate_ring, row, g);
      load8<IN>(s.val_ring, row, v);
    }
  };
  if (m == kOvM && o == kOvM) {
    // overlapping 4:1 windows: the bulk kernel's factored softmax on wave 0, with
    // the bulk kernel's choice of path (the same bits either way)
    if (w != 0) return;
    float u[2 * kOvM][8];
    if (ov_bias(s.bpos, D, ch, G, u)) {
      float sp[8], lp[8], ap[8], g[kOvM][8], v[kOvM][8], E[kOvM][8];
      if (e > 0) {
#pragma unroll
        for (int q = 0; q < kOvM; ++q) tok(kOvM * (e - 1) + q, g[q], v[q]);
        ov_block(g, sp, E);
        ov_half(E, v, ov_rows(u, 0), lp, ap);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) { sp[c] = -INFINITY; lp[c] = 0.f; ap[c] = 0.f; }
      }
#pragma unroll
      for (int q = 0; q < kOvM; ++q) tok(kOvM * e + q, g[q], v[q]);
      float sb[8], la[8], aa[8], cv[8];
      ov_block(g, sb, E);
      ov_half(E, v, ov_rows(u, 1), la, aa);
      ov_entry(sp, lp, ap, sb, la, aa, cv);
      store_values<OUT, SCALED>(cv, ch, G, active, lane, b, e, D, s.E_cap, s.key_tiles, s.out, s.out_scale);
      return;
    }
  }
  const int64_t i0 = (int64_t)m * e - o, i1 = (int64_t)m * e + m;
  const int np = window_parts(i0, i1);                     // uniform
  PoolState st;
  if (w < np) {
    int64_t ia, ib;
    part_range(i0, i1, w, ia, ib);
    pool_range<2>(tok, s.bpos, i0, ia, ib, D, ch, active, st);
    if (w > 0) parts[w - 1][lane] = st;
  }
  __syncthreads();
  if (w != 0) return;
#pragma unroll 1
  for (int p = 1; p < np; ++p) fold_state(st, parts[p - 1][lane]);
  store_entry<OUT, SCALED>(st, ch, G, active, lane, b, e, D, s.E_cap, s.key_tiles, s.out, s.out_scale);
}

// Overlapping 4:1 windows: a block pools 4 * epw * J consecutive entries (and the
// block before them), J as large as keeps 1024 blocks in the stream's grid
// (*nbx blocks along x, B along y).
static OvArgs ov_args(const sckv_pool_stream& s, int32_t B, int64_t N, int64_t e_begin, int64_t e_count,
                      unsigned* nbx) {
  const int G = s.D / 8;
  const int epw = kWave / G;
  int J = 16;
  auto ov_blocks = [&](int j) { return ((e_count + (int64_t)j * 4 * epw - 1) / ((int64_t)j * 4 * epw)) * B; };
  while (J > 1 && ov_blocks(J) < 1024) J /= 2;
  *nbx = (unsigned)((e_count + (int64_t)J * 4 * epw - 1) / ((int64_t)J * 4 * epw));
  const int tiles = s.out_layout == SCKV_LAYOUT_KEY_TILES ? 1 : 0;
  return OvArgs{s.val, s.gate, s.bpos, s.out, s.out_scale, N, e_begin, e_count, s.E_cap, s.D, G, tiles, J};
}

template <int IN>
static hipError_t launch_in(const sckv_pool_stream& s, int32_t B, int64_t N, int32_t m, int32_t o,
                            int64_t e_begin, int64_t e_count, hipStream_t stream) {
  const int G = s.D / 8;
  const int epw = kWave / G;
  const dim3 grid((unsigned)((e_count + 4 * epw - 1) / (4 * epw)), (unsigned)B);
  const dim3 block(256);
  const int tiles = s.out_layout == SCKV_LAYOUT_KEY_TILES ? 1 : 0;
  const dim3 grid_parts((unsigned)((e_count + epw - 1) / epw), (unsigned)B);
  unsigned nb_ov;
  const OvArgs ov = ov_args(s, B, N, e_begin, e_count, &nb_ov);
  const dim3 grid_ov(nb_ov, (unsigned)B);
#define SCKV_LAUNCH(OUT, SC)                                                                                   \
  if (m == kOvM && o == kOvM)                                                                                  \
    hipLaunchKernelGGL((compress_overlap_kernel<IN, OUT, SC>), grid_ov, block, 0, stream, ov);                 \
  else if (m + o >= 64)                                                                                        \
    hipLaunchKernelGGL((compress_parts_kernel<IN, OUT, SC>), grid_parts, block, 0, stream, s.val, s.gate,      \
                       s.bpos, s.out, s.out_scale, N, s.D, m, o, e_begin, e_count, s.E_cap, G, tiles);          \
  else                                                                                                         \
    hipLaunchKernelGGL((compress_kernel<IN, OUT, SC>), grid, block, 0, stream, s.val, s.gate, s.bpos,          \
                       s.out, s.out_scale, N, s.D, m, o, e_begin, e_count, s.E_cap, G, tiles)
  switch (s.out_dtype) {
    case SCKV_F32: SCKV_LAUNCH(SCKV_F32, false); break;
    case SCKV_BF16: SCKV_LAUNCH(SCKV_BF16, false); break;
    case SCKV_MXFP4: SCKV_LAUNCH(SCKV_MXFP4, false); break;
    default:
      if (s.out_scale) SCKV_LAUNCH(SCKV_E4M3, true);
      else SCKV_LAUNCH(SCKV_E4M3, false);
  }
#undef SCKV_LAUNCH
  return hipGetLastError();
}

static AppendK append_k(const sckv_append_stream& s) {
  return AppendK{s.pos,       s.val, s.gate, s.val_ring, s.gate_ring, s.bpos, s.out, s.out_scale,
                 s.E_cap,     s.D,   s.P,    s.out_layout == SCKV_LAYOUT_KEY_TILES ? 1 : 0};
}

template <int IN>
static hipError_t launch_append_in(const AppendK& k0, const AppendK& k1, int nstreams, int out_dtype, bool scaled,
                                   int32_t B, int32_t m, int32_t o, hipStream_t stream) {
  const dim3 grid((unsigned)B, (unsigned)nstreams);
#define SCKV_LAUNCH(OUT, SC) \
  hipLaunchKernelGGL((append_kernel<IN, OUT, SC>), grid, dim3(kParts * kWave), 0, stream, k0, k1, m, o)
  switch (out_dtype) {
    case SCKV_F32: SCKV_LAUNCH(SCKV_F32, false); break;
    case SCKV_BF16: SCKV_LAUNCH(SCKV_BF16, false); break;
    case SCKV_MXFP4: SCKV_LAUNCH(SCKV_MXFP4, false); break;
    default:
      if (scaled) SCKV_LAUNCH(SCKV_E4M3, true);
      else SCKV_LAUNCH(SCKV_E4M3, false);
  }
#undef SCKV_LAUNCH
  return hipGetLastError();
}

static hipError_t launch_append_group(const sckv_append_stream& s, const sckv_append_stream* s2, int32_t B,
                                      int32_t m, int32_t o, hipStream_t stream) {
  const AppendK k0 = append_k(s), k1 = s2 ? append_k(*s2) : k0;
  const int n = s2 ? 2 : 1;
  if (s.in_dtype == SCKV_BF16)
    return launch_append_in<SCKV_BF16>(k0, k1, n, s.out_dtype, s.out_scale != nullptr, B, m, o, stream);
  return launch_append_in<SCKV_F32>(k0, k1, n, s.out_dtype, s.out_scale != nullptr, B, m, o, stream);
}

// Streams with the same input dtype, output dtype and scaling share one launch.
hipError_t launch_append(const sckv_append_stream& s, const sckv_append_stream* s2, int32_t B, int32_t m, int32_t o,
                         hipStream_t stream) {
  if (s2 && s2->in_dtype == s.in_dtype && s2->out_dtype == s.out_dtype &&
      (s2->out_scale != nullptr) == (s.out_scale != nullptr))
    return launch_append_group(s, s2, B, m, o, stream);
  hipError_t e = launch_append_group(s, nullptr, B, m, o, stream);
  if (e == hipSuccess && s2) e = launch_append_group(*s2, nullptr, B, m, o, stream);
  return e;
}

hipError_t launch_compress(const sckv_pool_stream& s, int32_t B, int64_t N, int32_t m, int32_t o,
                           int64_t e_begin, int64_t e_count, hipStream_t stream) {
  if (e_count == 0) return hipSuccess;
  if (s.in_dtype == SCKV_BF16) return launch_in<SCKV_BF16>(s, B, N, m, o, e_begin, e_count, stream);
  return launch_in<SCKV_F32>(s, B, N, m, o, e_begin, e_count, stream);
}

// Output kinds of a pair launch: bf16 / e4m3 scaled / e4m3 / MXFP4 (one
// template instance per supported combination).
enum OvKind { OV_BF16, OV_E4M3_SCALED, OV_E4M3, OV_MXFP4, OV_OTHER };
static OvKind ov_kind(const sckv_pool_stream& s) {
  switch (s.out_dtype) {
    case SCKV_BF16: return OV_BF16;
    case SCKV_E4M3: return s.out_scale ? OV_E4M3_SCALED : OV_E4M3;
    case SCKV_MXFP4: return OV_MXFP4;
    default: return OV_OTHER;
  }
}

// A CSA layer's two streams: with bf16 input and overlapping 4:1 windows, the
// combinations below share one launch (the latent in bf16 or scaled e4m3, the
// indexer keys in the same type, unscaled e4m3 or MXFP4); otherwise each stream
// takes its own.
hipError_t launch_compress_pair(const sckv_pool_stream& s0, const sckv_pool_stream& s1, int32_t B, int64_t N,
                                int32_t m, int32_t o, int64_t e_begin, int64_t e_count, hipStream_t stream) {
  if (e_count == 0) return hipSuccess;
  const OvKind k0 = ov_kind(s0), k1 = ov_kind(s1);
  const bool ov = m == kOvM && o == kOvM && s0.in_dtype == SCKV_BF16 && s1.in_dtype == SCKV_BF16;
  unsigned nb0 = 0, nb1 = 0;
  const OvArgs a0 = ov_args(s0, B, N, e_begin, e_count, &nb0);
  const OvArgs a1 = ov_args(s1, B, N, e_begin, e_count, &nb1);
  const dim3 grid(nb0 + nb1, (unsigned)B), block(256);
#define SCKV_PAIR(O0, S0, O1, S1) \
  hipLaunchKernelGGL((compress_overlap_pair<SCKV_BF16, O0, S0, O1, S1>), grid, block, 0, stream, a0, a1, nb0)
  bool launched = ov;
  if (ov) {
    if (k0 == OV_BF16 && k1 == OV_BF16) SCKV_PAIR(SCKV_BF16, false, SCKV_BF16, false);
    else if (k0 == OV_BF16 && k1 == OV_MXFP4) SCKV_PAIR(SCKV_BF16, false, SCKV_MXFP4, false);
    else if (k0 == OV_E4M3_SCALED && k1 == OV_E4M3) SCKV_PAIR(SCKV_E4M3, true, SCKV_E4M3, false);
    else if (k0 == OV_E4M3_SCALED && k1 == OV_E4M3_SCALED) SCKV_PAIR(SCKV_E4M3, true, SCKV_E4M3, true);
    else if (k0 == OV_E4M3_SCALED && k1 == OV_MXFP4) SCKV_PAIR(SCKV_E4M3, true, SCKV_MXFP4, false);
    else launched = false;
  }
#undef SCKV_PAIR
  if (launched) return hipGetLastError();
  hipError_t e = launch_compress(s0, B, N, m, o, e_begin, e_count, stream);
  if (e == hipSuccess) e = launch_compress(s1, B, N, m, o, e_begin, e_count, stream);
  return e;
}

}  // namespace sckv
