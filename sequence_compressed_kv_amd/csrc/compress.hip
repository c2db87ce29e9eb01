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
// maximum and the new logit sets which side is rescaled.  In decode, one token
// per sequence is appended to small rings of recent tokens, and the entry it
// completes (one per m tokens) is pooled by the same code.
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

// Pools entry e of sequence b from tokens [i0, i1) (cut to i >= 0) and stores it.
// This lane owns channels ch .. ch+7 of the entry; the entry's G = D/8 lanes are
// G consecutive lanes of a G-aligned group (the e4m3 scale is reduced over them).
// tok(i, g, v) loads token i's 8 gate logits and values of this lane's channels.
// Lanes with active == false take part in the reduction but load and store nothing.
template <int IN, int OUT, bool SCALED, class Tok>
__device__ __forceinline__ void pool_and_store(Tok tok, const float* __restrict__ bpos, int64_t i0, int64_t i1,
                                               int D, int ch, int G, bool active, int sub, int64_t b, int64_t e,
                                               int64_t E_cap, int key_tiles, void* __restrict__ out,
                                               float* __restrict__ out_scale) {
  float mx[8], l[8], acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) { mx[c] = -INFINITY; l[c] = 0.f; acc[c] = 0.f; }

  for (int64_t i = i0 < 0 ? 0 : i0; i < i1; ++i) {
    float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    f32x4 bp0 = {0.f, 0.f, 0.f, 0.f}, bp1 = {0.f, 0.f, 0.f, 0.f};
    if (active) {
      tok(i, g, v);
      const f32x4* bp = reinterpret_cast<const f32x4*>(bpos + (i - i0) * D + ch);
      bp0 = bp[0];
      bp1 = bp[1];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float a = g[c] + (c < 4 ? bp0[c] : bp1[c - 4]);
      const float d = a - mx[c];
      const float x = expf(-fabsf(d));
      const bool up = d > 0.f;
      const float sc = up ? x : 1.f;
      const float p = up ? 1.f : x;
      l[c] = l[c] * sc + p;
      acc[c] = acc[c] * sc + p * v[c];
      mx[c] = fmaxf(mx[c], a);
    }
  }
  float cv[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) cv[c] = acc[c] / l[c];

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
  pool_and_store<IN, OUT, SCALED>(tok, bpos, (int64_t)m * e - o, (int64_t)m * e + m, D, ch, G, active, sub, b, e,
                                  E_cap, key_tiles, out, out_scale);
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

// Decode append: one new token per sequence (one wave per sequence; blockIdx.y
// picks one of up to two streams that share the pool and the dtypes).  The token
// goes into the value and gate rings at slot t mod P; when it completes entry
// e = (t + 1) / m - 1, the entry is pooled from the rings (tokens before t) and
// the new token, by the same code as the bulk compressor.
template <int IN, int OUT, bool SCALED>
__global__ __launch_bounds__(64) void append_kernel(AppendK s0, AppendK s1, int m, int o) {
  constexpr int ES = IN == SCKV_BF16 ? 2 : 4;
  const AppendK& s = blockIdx.y == 0 ? s0 : s1;
  const int64_t b = blockIdx.x;
  const int D = s.D, P = s.P;
  const int G = D / 8, lane = lane_id();
  const bool active = lane < G;
  const int ch = active ? lane * 8 : 0;
  const int32_t t = s.pos[b];
  if (t < 0) return;                                       // whole wave: nothing to append
  const int64_t slot_t = t % P;
  if (active) {
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
  pool_and_store<IN, OUT, SCALED>(tok, s.bpos, (int64_t)m * e - o, (int64_t)m * e + m, D, ch, G, active, lane, b, e,
                                  s.E_cap, s.key_tiles, s.out, s.out_scale);
}

template <int IN>
static hipError_t launch_in(const sckv_pool_stream& s, int32_t B, int64_t N, int32_t m, int32_t o,
                            int64_t e_begin, int64_t e_count, hipStream_t stream) {
  const int G = s.D / 8;
  const int epw = kWave / G;
  const dim3 grid((unsigned)((e_count + 4 * epw - 1) / (4 * epw)), (unsigned)B);
  const dim3 block(256);
#define SCKV_LAUNCH(OUT, SC)                                                                    \
  hipLaunchKernelGGL((compress_kernel<IN, OUT, SC>), grid, block, 0, stream, s.val, s.gate,     \
                     s.bpos, s.out, s.out_scale, N, s.D, m, o, e_begin, e_count, s.E_cap, G,           \
                     s.out_layout == SCKV_LAYOUT_KEY_TILES ? 1 : 0)
  switch (s.out_dtype) {
    case SCKV_F32: SCKV_LAUNCH(SCKV_F32, false); break;
    case SCKV_BF16: SCKV_LAUNCH(SCKV_BF16, false); break;
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
  hipLaunchKernelGGL((append_kernel<IN, OUT, SC>), grid, dim3(64), 0, stream, k0, k1, m, o)
  switch (out_dtype) {
    case SCKV_F32: SCKV_LAUNCH(SCKV_F32, false); break;
    case SCKV_BF16: SCKV_LAUNCH(SCKV_BF16, false); break;
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
