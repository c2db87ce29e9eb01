// Gated per-channel softmax pooling of per-token streams into compressed entries.
//
// c_j[d] = sum_{i in P_j} softmax_i(g_i[d] + Bpos[i - m j + o][d]) v_i[d], with
// P_j = [m j - o, m j + m) cut to tokens i >= 0 (the CSA decode workload
// definition's compressor; knightli.com DeepSeek-V4 KV-cache article, sections
// "CSA" (4:1, learned pool, overlapping windows) and "HCA" (128:1)).
//
// HBM streaming: lane groups of D/8 lanes own one entry, each lane 8 channels,
// so every token row is read as one contiguous D-wide segment.  The softmax is
// taken online with one exp per (token, channel): the larger of the running
// maximum and the new logit sets which side is rescaled.  An entry's window is
// pooled in 4 parts whose states are folded in order.  In decode, one token per
// sequence is appended to small rings of recent tokens, and the entry it
// completes (one per m tokens) is pooled with the same arithmetic, its 4 parts on
// 4 waves.
#include "device_common.h"
#include "sckv_internal.h"

namespace sckv {

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
// i - i0.  With AHEAD == 2 the loads of two tokens are issued before their
// updates (for few waves in flight; the arithmetic is the same).  The larger of
// the running maximum and the new logit decides which side is rescaled, so each
// (token, channel) costs one exp.
template <int AHEAD, class Tok>
__device__ __forceinline__ void pool_range(Tok tok, const float* __restrict__ bpos, int64_t i0, int64_t ia,
                                           int64_t ib, int D, int ch, bool active, PoolState& st) {
#pragma unroll
  for (int c = 0; c < 8; ++c) { st.mx[c] = -INFINITY; st.l[c] = 0.f; st.acc[c] = 0.f; }
  auto update = [&](const float (&g)[8], const float (&v)[8], f32x4 bp0, f32x4 bp1) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float a = __fadd_rn(g[c], c < 4 ? bp0[c] : bp1[c - 4]);
      const float d = __fsub_rn(a, st.mx[c]);
      const float x = expf(-fabsf(d));
      const bool up = d > 0.f;
      const float sc = up ? x : 1.f;
      const float p = up ? 1.f : x;
      st.l[c] = fmaf(st.l[c], sc, p);
      st.acc[c] = fmaf(st.acc[c], sc, __fmul_rn(p, v[c]));
      st.mx[c] = fmaxf(st.mx[c], a);
    }
  };
  for (int64_t i = ia; i < ib; i += AHEAD) {
    const bool two = AHEAD == 2 && i + 1 < ib;
    float g0[8] = {}, v0[8] = {}, g1[8] = {}, v1[8] = {};
    f32x4 b00 = {}, b01 = {}, b10 = {}, b11 = {};
    if (active) {
      tok(i, g0, v0);
      const f32x4* bp = reinterpret_cast<const f32x4*>(bpos + (i - i0) * D + ch);
      b00 = bp[0];
      b01 = bp[1];
      if (two) {
        tok(i + 1, g1, v1);
        b10 = bp[D / 4];
        b11 = bp[D / 4 + 1];
      }
    }
    update(g0, v0, b00, b01);
    if (two) update(g1, v1, b10, b11);
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
    const float sa = re ? 0.f : expf(__fsub_rn(r.mx[c], M));
    const float sb = qe ? 0.f : expf(__fsub_rn(q.mx[c], M));
    const float l = qe ? r.l[c] : (re ? q.l[c] : fmaf(r.l[c], sa, __fmul_rn(q.l[c], sb)));
    const float acc = qe ? r.acc[c] : (re ? q.acc[c] : fmaf(r.acc[c], sa, __fmul_rn(q.acc[c], sb)));
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
__device__ __forceinline__ void store_entry(const PoolState& st, int ch, int G, bool active, int sub, int64_t b,
                                            int64_t e, int D, int64_t E_cap, int key_tiles, void* __restrict__ out,
                                            float* __restrict__ out_scale) {
  float cv[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) cv[c] = st.acc[c] / st.l[c];

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
    u32x2 r = {0u, 0u};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t q = f32_to_e4m3_sat(SCALED ? cv[c] / scale : cv[c]);
      r[c >> 2] |= q << ((c & 3) * 8);
    }
    if (active) {
      *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(out) + orow) = r;
      if (SCALED && sub == 0) out_scale[b * E_cap + e] = scale;
    }
  }
}

// MULTI: the window has 64 tokens or more (pooled in parts; chosen on the host by
// the same rule as window_parts).
template <int IN, int OUT, bool SCALED, bool MULTI>
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
  pool_range<1>(tok, bpos, i0, ia, ib, D, ch, active, r);
  if constexpr (MULTI) {
    PoolState q;
#pragma unroll 1
    for (int p = 1; p < kParts; ++p) {
      part_range(i0, i1, p, ia, ib);
      pool_range<1>(tok, bpos, i0, ia, ib, D, ch, active, q);
      fold_state(r, q);
    }
  }
  store_entry<OUT, SCALED>(r, ch, G, active, sub, b, e, D, E_cap, key_tiles, out, out_scale);
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

template <int IN>
static hipError_t launch_in(const sckv_pool_stream& s, int32_t B, int64_t N, int32_t m, int32_t o,
                            int64_t e_begin, int64_t e_count, hipStream_t stream) {
  const int G = s.D / 8;
  const int epw = kWave / G;
  const dim3 grid((unsigned)((e_count + 4 * epw - 1) / (4 * epw)), (unsigned)B);
  const dim3 block(256);
#define SCKV_LAUNCH(OUT, SC)                                                                                   \
  if (m + o >= 64)                                                                                             \
    hipLaunchKernelGGL((compress_kernel<IN, OUT, SC, true>), grid, block, 0, stream, s.val, s.gate, s.bpos,    \
                       s.out, s.out_scale, N, s.D, m, o, e_begin, e_count, s.E_cap, G,                         \
                       s.out_layout == SCKV_LAYOUT_KEY_TILES ? 1 : 0);                                         \
  else                                                                                                         \
    hipLaunchKernelGGL((compress_kernel<IN, OUT, SC, false>), grid, block, 0, stream, s.val, s.gate, s.bpos,   \
                       s.out, s.out_scale, N, s.D, m, o, e_begin, e_count, s.E_cap, G,                         \
                       s.out_layout == SCKV_LAYOUT_KEY_TILES ? 1 : 0)
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

}  // namespace sckv
