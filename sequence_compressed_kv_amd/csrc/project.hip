// Projections of decode rows between the model width and the attention path:
// the head queries q_h = W_q x, the indexer query qI = W_iq x and head weights
// w = W_w x, the per-token streams (v, g and the indexer's vI, gI) the
// compressor pools, the absorption of the head queries into the shared latent
// (q~_h = W_UK^h^T q_h), and the way back: heads o_h = W_UV^h o~_h, then
// y = W_o [o_1 .. o_H] (the CSA decode workload definition: per-head queries,
// attention, then W_o; knightli.com DeepSeek-V4 KV-cache article, "Varias
// generaciones de optimizacion de KV Cache": MLA keeps a compressed latent that
// the head queries are absorbed into).
//
// Decode has few rows, so every product streams its weights once: linear_rows
// takes up to 64 rows against a weight matrix W [N][K] (bf16 MFMA 16x16x32,
// fp32 accumulation).  A block owns 32 output columns; its 4 waves split K in
// quarters and their partial sums are added in a fixed order through LDS.  The
// absorption runs in fp32 on the VALU (the head queries stay fp32 on chip).
#include "device_common.h"
#include "sckv_internal.h"

namespace sckv {

// One product of a grouped launch: y = x W^T over N columns, tiles of the launch
// numbered from tile0.  Batch item b (blockIdx.y) adds b * w_bs to W and b * y_bs to y.
struct LinearSeg {
  const uint16_t* W;  // [N][K]
  void* y;            // row r, column n at y + r * y_rs + n
  int64_t w_bs, y_bs, y_rs;
  int N, tile0, out;  // out: SCKV_F32 or SCKV_BF16
  int pad;
};

constexpr int kMaxSegs = 4;

struct LinearParams {
  const uint16_t* x;  // batch item b, row r at x + b * x_bs + r * x_rs (K contiguous)
  int64_t x_bs, x_rs;
  LinearSeg seg[kMaxSegs];
  int nseg, R, K, pad;
};

// Up to 16 MT rows against 16 NT columns per block; the block's NW = blockDim / 64
// waves split K evenly and walk their share U k-steps of 32 at a time, the loads
// of the next U steps issued before the products of the current ones.  The
// waves' partial sums meet in LDS (dynamic, NW * MT * NT * 1 KiB) and are added
// in wave order.  Eight tiles per wave (MT * NT == 8) allow at most 8 waves.
template <int MT, int NT, int U>
__global__ __launch_bounds__(MT * NT >= 8 ? 512 : 1024) void linear_rows(LinearParams p) {
  extern __shared__ f32x4 red[];
  const int NW = blockDim.x / kWave;
  int s = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i)
    if (i < p.nseg && (int)blockIdx.x >= p.seg[i].tile0) s = i;
  const LinearSeg& sg = p.seg[s];
  const int64_t b = blockIdx.y;
  const int N = sg.N, n0 = ((int)blockIdx.x - sg.tile0) * 16 * NT;
  const int l = lane_id(), w = wave_id(), c = l & 15, g = l >> 4;
  const int KW = p.K / NW, k0 = w * KW;
  const gbytes xb = opaque_global(p.x + b * p.x_bs), wb = opaque_global(sg.W + b * sg.w_bs);
  int64_t xr[MT], wr[NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = 16 * mt + c;
    xr[mt] = ((int64_t)(row < p.R ? row : 0) * p.x_rs + k0 + 8 * g) * 2;   // rows past R read row 0 (not stored)
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = n0 + 16 * nt + c;
    wr[nt] = ((int64_t)(n < N ? n : N - 1) * p.K + k0 + 8 * g) * 2;        // columns past N read the last (not stored)
  }
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 a0[U][MT], w0[U][NT], a1[U][MT], w1[U][NT];
  auto load = [&](bf16x8(&a)[U][MT], bf16x8(&bw)[U][NT], int kk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = (int64_t)(kk + 32 * u) * 2;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bw[u][nt] = bitcast<bf16x8>(gload<u32x4>(wb, wr[nt] + off));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[u][mt] = bitcast<bf16x8>(gload<u32x4>(xb, xr[mt] + off));
    }
  };
  auto mma = [&](bf16x8(&a)[U][MT], bf16x8(&bw)[U][NT]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma16_bf16(a[u][mt], bw[u][nt], acc[mt][nt]);
  };
  const int trips = KW / (32 * U);
  load(a0, w0, 0);
  int t = 0;
  for (; t + 2 <= trips; t += 2) {
    load(a1, w1, (t + 1) * 32 * U);
    mma(a0, w0);
    if (t + 2 < trips) load(a0, w0, (t + 2) * 32 * U);
    mma(a1, w1);
  }
  if (t < trips) mma(a0, w0);
  // the waves' K shares meet: tile i is summed by wave i % NW in wave order
  constexpr int T = MT * NT;
#pragma unroll
  for (int i = 0; i < T; ++i) red[(w * T + i) * kWave + l] = acc[i / NT][i % NT];
  __syncthreads();
  for (int i = w; i < T; i += NW) {
    f32x4 v = red[i * kWave + l];
    for (int j = 1; j < NW; ++j) v += red[(j * T + i) * kWave + l];
    const int mt = i / NT, nt = i % NT;
    const int n = n0 + 16 * nt + c;
    if (n >= N) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * mt + 4 * g + e;
      if (row >= p.R) continue;
      const int64_t off = b * sg.y_bs + (int64_t)row * sg.y_rs + n;
      if (sg.out == SCKV_BF16) static_cast<uint16_t*>(sg.y)[off] = (uint16_t)f32_to_bf16_rne(v[e]);
      else static_cast<float*>(sg.y)[off] = v[e];
    }
  }
}

template <int MT, int NT>
static void launch_lr(const LinearParams& p, dim3 grid, int nw, hipStream_t s) {
  const int kw = p.K / nw;
  const size_t lds = (size_t)nw * MT * NT * kWave * sizeof(f32x4);
  if (kw % 64 == 0) hipLaunchKernelGGL((linear_rows<MT, NT, 2>), grid, dim3(nw * kWave), lds, s, p);
  else hipLaunchKernelGGL((linear_rows<MT, NT, 1>), grid, dim3(nw * kWave), lds, s, p);
}

struct Product {
  const void* W;
  void* y;
  int64_t w_bs, y_bs, y_rs;
  int N, out;
};

// Products sharing the rows x [R][K] (R <= 64, K % 128 == 0), one launch.  Small
// launches take 16-column tiles and 16 waves per block so that the K stream is
// cut into more, shorter pieces.
static hipError_t linear(const void* x, int64_t x_bs, int64_t x_rs, int R, int K, const Product* pr, int np,
                         int nbatch, hipStream_t s) {
  int64_t cols32 = 0;
  for (int i = 0; i < np; ++i) cols32 += (pr[i].N + 31) / 32;
  const int nt = cols32 * nbatch >= 256 ? 2 : 1;
  const int mt = R <= 16 ? 1 : (R <= 32 ? 2 : 4);
  int nw = (nt == 2 && cols32 * nbatch >= 512) ? 8 : 16;
  while (nw > 4 && (K % (nw * 32) != 0 || (size_t)nw * mt * nt * 1024 > 65536)) nw /= 2;
  LinearParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.x_bs = x_bs;
  p.x_rs = x_rs;
  p.nseg = np;
  p.R = R;
  p.K = K;
  int tiles = 0;
  for (int i = 0; i < np; ++i) {
    LinearSeg& g = p.seg[i];
    g.W = static_cast<const uint16_t*>(pr[i].W);
    g.y = pr[i].y;
    g.w_bs = pr[i].w_bs;
    g.y_bs = pr[i].y_bs;
    g.y_rs = pr[i].y_rs;
    g.N = pr[i].N;
    g.out = pr[i].out;
    g.tile0 = tiles;
    tiles += (pr[i].N + 16 * nt - 1) / (16 * nt);
  }
  const dim3 grid((unsigned)tiles, (unsigned)nbatch);
  if (nt == 2) {
    if (mt == 1) launch_lr<1, 2>(p, grid, nw, s);
    else if (mt == 2) launch_lr<2, 2>(p, grid, nw, s);
    else launch_lr<4, 2>(p, grid, nw, s);
  } else {
    if (mt == 1) launch_lr<1, 1>(p, grid, nw, s);
    else if (mt == 2) launch_lr<2, 1>(p, grid, nw, s);
    else launch_lr<4, 1>(p, grid, nw, s);
  }
  return hipGetLastError();
}

// q[r][h][d] = sum_k qh[r][h][k] W_UK[h][k][d] in fp32.  Block (head, 128 latent
// columns, 16 rows), 4 waves taking a quarter of k each; a lane owns two adjacent
// columns and keeps its W_UK values in registers; the rows' head queries sit in
// LDS; the quarters are added in wave order.
template <int OUT>
__global__ __launch_bounds__(256) void absorb_kernel(const float* __restrict__ qh, const uint16_t* __restrict__ WUK,
                                                     void* __restrict__ q, int R, int H, int dh, int D) {
  __shared__ float qs[16][256];
  __shared__ float part[4][16][128];
  const int h = blockIdx.x, c0 = blockIdx.y * 128, r0 = blockIdx.z * 16;
  const int l = lane_id(), w = wave_id();
  const int nr = R - r0 < 16 ? R - r0 : 16;
  for (int i = threadIdx.x; i < 16 * dh; i += blockDim.x) {
    const int rr = i / dh, k = i % dh;
    qs[rr][k] = rr < nr ? qh[((int64_t)(r0 + rr) * H + h) * dh + k] : 0.f;
  }
  __syncthreads();
  const int KQ = dh / 4, k0 = w * KQ;
  const uint32_t* wp = reinterpret_cast<const uint32_t*>(WUK + ((int64_t)h * dh + k0) * D + c0) + l;
  float acc[16][2];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i][0] = acc[i][1] = 0.f;
  for (int k = 0; k < KQ; k += 4) {
    uint32_t wv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wv[j] = wp[(int64_t)(k + j) * (D / 2)];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float wa = bf16_to_f32(wv[j] & 0xffffu), wb = bf16_to_f32(wv[j] >> 16);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float qv = qs[i][k0 + k + j];
        acc[i][0] = fmaf(qv, wa, acc[i][0]);
        acc[i][1] = fmaf(qv, wb, acc[i][1]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    part[w][i][2 * l] = acc[i][0];
    part[w][i][2 * l + 1] = acc[i][1];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * 128; i += blockDim.x) {
    const int rr = i / 128, col = i % 128;
    if (rr >= nr) break;
    const float v = ((part[0][rr][col] + part[1][rr][col]) + part[2][rr][col]) + part[3][rr][col];
    const int64_t off = ((int64_t)(r0 + rr) * H + h) * D + c0 + col;
    if constexpr (OUT == SCKV_BF16) static_cast<uint16_t*>(q)[off] = (uint16_t)f32_to_bf16_rne(v);
    else static_cast<float*>(q)[off] = v;
  }
}

hipError_t launch_layer_queries(const sckv_query_args& a, void* ws, hipStream_t s) {
  const int HD = a.H * a.d_h;
  const bool absorb = a.W_UK != nullptr;
  Product pr[3];
  int np = 0;
  // head queries: into the workspace (fp32) when they are absorbed, else straight to q
  pr[np++] = Product{a.W_q, absorb ? ws : a.q, 0, 0, HD, HD, absorb ? SCKV_F32 : a.q_dtype};
  if (a.W_iq) pr[np++] = Product{a.W_iq, a.qI, 0, 0, (int64_t)a.H_I * a.D_I, a.H_I * a.D_I, a.q_dtype};
  if (a.W_w) pr[np++] = Product{a.W_w, a.w, 0, 0, a.H_I, a.H_I, SCKV_F32};
  hipError_t e = linear(a.x, 0, a.d_model, a.R, a.d_model, pr, np, 1, s);
  if (e != hipSuccess || !absorb) return e;
  const dim3 grid((unsigned)a.H, (unsigned)(a.D / 128), (unsigned)((a.R + 15) / 16));
  if (a.q_dtype == SCKV_BF16)
    hipLaunchKernelGGL(absorb_kernel<SCKV_BF16>, grid, dim3(256), 0, s, static_cast<const float*>(ws),
                       static_cast<const uint16_t*>(a.W_UK), a.q, a.R, a.H, a.d_h, a.D);
  else
    hipLaunchKernelGGL(absorb_kernel<SCKV_F32>, grid, dim3(256), 0, s, static_cast<const float*>(ws),
                       static_cast<const uint16_t*>(a.W_UK), a.q, a.R, a.H, a.d_h, a.D);
  return hipGetLastError();
}

hipError_t launch_layer_streams(const sckv_stream_args& a, hipStream_t s) {
  const void* W[4] = {a.W_c, a.W_g, a.W_cI, a.W_gI};
  void* out[4] = {a.v, a.g, a.vI, a.gI};
  const int N[4] = {a.D, a.D, a.D_I, a.D_I};
  Product pr[4];
  int np = 0;
  for (int i = 0; i < 4; ++i)
    if (W[i]) pr[np++] = Product{W[i], out[i], 0, 0, N[i], N[i], a.out_dtype};
  if (np == 0) return hipSuccess;
  return linear(a.x, 0, a.d_model, a.R, a.d_model, pr, np, 1, s);
}

hipError_t launch_layer_output(const sckv_output_args& a, void* ws, hipStream_t s) {
  const int HD = a.H * a.d_h;
  const void* heads = a.o;
  if (a.W_UV) {
    // o_h = W_UV^h o~_h for every head (a batch of H products), rounded to bf16
    const Product pr{a.W_UV, ws, (int64_t)a.d_h * a.D, a.d_h, HD, a.d_h, SCKV_BF16};
    hipError_t e = linear(a.o, a.D, (int64_t)a.H * a.D, a.R, a.D, &pr, 1, a.H, s);
    if (e != hipSuccess) return e;
    heads = ws;
  }
  const Product pr{a.W_o, a.y, 0, 0, a.d_model, a.d_model, a.y_dtype};
  return linear(heads, 0, HD, a.R, HD, &pr, 1, 1, s);
}

}  // namespace sckv
