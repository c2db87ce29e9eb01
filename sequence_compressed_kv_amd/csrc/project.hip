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

// One product of a grouped launch: y = x W^T over N columns.  Its blocks are
// numbered from blk0: tiles of 16 NT columns times `splits` equal parts of K.  A
// product with several parts writes fp32 partial sums [splits][nbatch][R][N] at
// part_off (floats) of the launch's partial buffer; its results are elements
// e0 .. e0 + nbatch R N - 1 of the sum kernel.  Batch item b (blockIdx.y) adds
// b * w_bs to W and b * y_bs to y.
struct LinearSeg {
  const uint16_t* W;  // [N][K]
  void* y;            // row r, column n at y + r * y_rs + n
  int64_t w_bs, y_bs, y_rs;
  int64_t part_off, e0;
  int N, blk0, splits, out;  // out: SCKV_F32 or SCKV_BF16
};

constexpr int kMaxSegs = 8;
constexpr int kGemmRows = 512;  // from this many rows on, products run as tiled GEMMs

struct LinearParams {
  const uint16_t* x;  // batch item b, row r at x + b * x_bs + r * x_rs (K contiguous)
  int64_t x_bs, x_rs;
  LinearSeg seg[kMaxSegs];
  float* part;
  int nseg, R, K, nbatch;
};

__device__ __forceinline__ void store_out(const LinearSeg& sg, int64_t off, float v) {
  if (sg.out == SCKV_BF16) static_cast<uint16_t*>(sg.y)[off] = (uint16_t)f32_to_bf16_rne(v);
  else static_cast<float*>(sg.y)[off] = v;
}

// Rows r0 .. r0 + 16 MT - 1 (r0 = blockIdx.z * 16 MT) against 16 NT columns per
// block, over one part of K.  The
// block's NW = blockDim / 64 waves split that part evenly and walk their share U
// k-steps of 32 at a time, the loads of the next U steps issued before the
// products of the current ones.  The waves' partial sums meet in LDS (dynamic,
// NW * MT * NT KiB) and are added in wave order.
template <int MT, int NT, int U>
__global__ __launch_bounds__(MT * NT >= 8 ? 256 : 512) void linear_rows(LinearParams p) {
  extern __shared__ f32x4 red[];
  const int NW = blockDim.x / kWave;
  int si = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i)
    if (i < p.nseg && (int)blockIdx.x >= p.seg[i].blk0) si = i;
  const LinearSeg& sg = p.seg[si];
  const int j = (int)blockIdx.x - sg.blk0, ntile = (sg.N + 16 * NT - 1) / (16 * NT);
  const int tile = j % ntile, part = j / ntile;
  const int64_t b = blockIdx.y;
  const int r0 = (int)blockIdx.z * 16 * MT;  // row block
  const int N = sg.N, n0 = tile * 16 * NT;
  const int l = lane_id(), w = wave_id(), c = l & 15, g = l >> 4;
  const int KS = p.K / sg.splits, KW = KS / NW, k0 = part * KS + w * KW;
  const gbytes xb = opaque_global(p.x + b * p.x_bs), wb = opaque_global(sg.W + b * sg.w_bs);
  int64_t xr[MT], wr[NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = r0 + 16 * mt + c;
    xr[mt] = ((int64_t)(row < p.R ? row : r0) * p.x_rs + k0 + 8 * g) * 2;  // rows past R read row r0 (not stored)
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
  const bool split = sg.splits > 1;
  for (int i = w; i < T; i += NW) {
    f32x4 v = red[i * kWave + l];
    for (int jw = 1; jw < NW; ++jw) v += red[(jw * T + i) * kWave + l];
    const int mt = i / NT, nt = i % NT;
    const int n = n0 + 16 * nt + c;
    if (n >= N) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = r0 + 16 * mt + 4 * g + e;
      if (row >= p.R) continue;
      if (split)
        p.part[sg.part_off + (((int64_t)part * p.nbatch + b) * p.R + row) * N + n] = v[e];
      else
        store_out(sg, b * sg.y_bs + (int64_t)row * sg.y_rs + n, v[e]);
    }
  }
}

// Sum, in part order, of the partial results of the products whose K was split.
__global__ __launch_bounds__(256) void linear_reduce(LinearParams p, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  int si = 0;
#pragma unroll
  for (int j = 1; j < kMaxSegs; ++j)
    if (j < p.nseg && p.seg[j].splits > 1 && i >= p.seg[j].e0) si = j;
  const LinearSeg& sg = p.seg[si];
  const int64_t e = i - sg.e0, count = (int64_t)p.nbatch * p.R * sg.N;
  const int n = (int)(e % sg.N);
  const int64_t br = e / sg.N;
  const int r = (int)(br % p.R);
  const int64_t b = br / p.R;
  const float* src = p.part + sg.part_off + e;
  // the loads of 8 parts are issued before their sums (the parts sit in other
  // XCDs' caches or in HBM: one wait instead of eight)
  float v = 0.f;
  for (int k0 = 0; k0 < sg.splits; k0 += 8) {
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = k0 + j < sg.splits ? src[(k0 + j) * count] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < sg.splits) v = k0 + j == 0 ? t[j] : v + t[j];
  }
  store_out(sg, b * sg.y_bs + (int64_t)r * sg.y_rs + n, v);
}

// ---------------------------------------------------------------- many rows
// y = x W^T for many rows (prefill): block tiles of 256 rows x 256 columns over
// K chunks of 32.  Both operand tiles of a chunk go global -> LDS by direct
// copies (16 bytes per lane) into 4 stages (three chunks in flight while one is
// multiplied).  A tile row is 64 bytes = 4 chunks of 8 elements; chunk j of row r
// sits at position j ^ ((r >> 2) & 3), so the 16 lanes of a fragment read hit 16
// different 4-bank groups.  8 waves, each 128 rows x 64 columns: MFMA 32x32x16
// bf16, 4 x 2 tiles of fp32 accumulators.
struct GemmParams {
  const uint16_t* x;  // batch item b (blockIdx.z): rows at x + b * x_bs + r * x_rs
  int64_t x_bs, x_rs;
  const uint16_t* W;  // [N][K] at W + b * w_bs
  int64_t w_bs;
  void* y;            // row r, column n at y + b * y_bs + r * y_rs + n
  int64_t y_bs, y_rs;
  int R, N, K, out;
  int split;          // > 0: column n = h split + k goes to y as two bf16 parts, hi = bf16(v) at
                      // h 2 split + k and lo = bf16(v - hi) at h 2 split + split + k
};

constexpr int kGM = 256, kGN = 256, kGK = 32, kGStg = 4;
constexpr int kGTile = kGM * kGK * 2;  // bytes of one operand's chunk tile
constexpr int kGCopies = 4;            // copy instructions per wave per chunk

__global__ __launch_bounds__(512) void gemm_rows(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t stg[kGStg][2][kGTile];
  const int l = lane_id(), w = wave_id();
  const int bn = (int)blockIdx.x * kGN, bm = (int)blockIdx.y * kGM;
  const int64_t b = blockIdx.z;
  const gbytes xa = opaque_global(p.x + b * p.x_bs), wa = opaque_global(p.W + b * p.w_bs);
  // copies: wave w fills tile rows 32 w .. 32 w + 31 of both operands, 16 rows per
  // instruction; lane l writes row 32 w + 16 i + l / 4, position l % 4
  int64_t asrc[2], bsrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 32 * w + 16 * i + (l >> 2);
    const int j = (l & 3) ^ ((r >> 2) & 3);
    const int ar = bm + r < p.R ? bm + r : p.R - 1;  // rows past R repeat the last (not stored)
    const int br = bn + r < p.N ? bn + r : p.N - 1;  // columns past N likewise
    asrc[i] = ((int64_t)ar * p.x_rs + 8 * j) * 2;
    bsrc[i] = ((int64_t)br * p.K + 8 * j) * 2;
  }
  auto issue = [&](int kc, int buf) {
    const int64_t koff = (int64_t)kc * kGK * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) copy_to_lds16(xa + asrc[i] + koff, &stg[buf][0][(32 * w + 16 * i) * 64]);
#pragma unroll
    for (int i = 0; i < 2; ++i) copy_to_lds16(wa + bsrc[i] + koff, &stg[buf][1][(32 * w + 16 * i) * 64]);
  };
  const int wm = w & 1, wn = w >> 1, c = l & 31, g = l >> 5;
  const int swz = (c >> 2) & 3;
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][jn][e] = 0.f;
  const int nk = p.K / kGK;
  for (int s0 = 0; s0 < kGStg - 1 && s0 < nk; ++s0) issue(s0, s0);
  for (int kc = 0; kc < nk; ++kc) {
    const int ahead = nk - 1 - kc < kGStg - 2 ? nk - 1 - kc : kGStg - 2;  // chunks issued after kc
    if (ahead >= 2) wait_vm_lgkm<2 * kGCopies, 0>();
    else if (ahead == 1) wait_vm_lgkm<kGCopies, 0>();
    else wait_vm_lgkm<0, 0>();
    block_barrier();  // chunk kc visible to all waves; buffer (kc - 1) % kGStg read by all
    if (kc + kGStg - 1 < nk) issue(kc + kGStg - 1, (kc + kGStg - 1) % kGStg);
    const uint8_t* at = stg[kc % kGStg][0];
    const uint8_t* bt = stg[kc % kGStg][1];
#pragma unroll
    for (int st = 0; st < kGK / 16; ++st) {
      const int pos = (2 * st + g) ^ swz;
      bf16x8 af[4], bf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(at + (wm * 128 + 32 * i + c) * 64 + pos * 16);
#pragma unroll
      for (int jn = 0; jn < 2; ++jn)
        bf[jn] = *reinterpret_cast<const bf16x8*>(bt + (wn * 64 + 32 * jn + c) * 64 + pos * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) acc[i][jn] = mfma32_bf16(af[i], bf[jn], acc[i][jn]);
    }
  }
  // D lane l: column l % 32, rows 8 (e / 4) + 4 (l / 32) + e % 4
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
      const int col = bn + wn * 64 + 32 * jn + c;
      if (col >= p.N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = bm + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
        if (row >= p.R) continue;
        const float v = acc[i][jn][e];
        if (p.split) {
          const int64_t off = b * p.y_bs + (int64_t)row * p.y_rs + (col / p.split) * 2 * p.split + col % p.split;
          const uint32_t hi = f32_to_bf16_rne(v);
          static_cast<uint16_t*>(p.y)[off] = (uint16_t)hi;
          static_cast<uint16_t*>(p.y)[off + p.split] = (uint16_t)f32_to_bf16_rne(v - bf16_to_f32(hi));
          continue;
        }
        const int64_t off = b * p.y_bs + (int64_t)row * p.y_rs + col;
        if (p.out == SCKV_BF16) static_cast<uint16_t*>(p.y)[off] = (uint16_t)f32_to_bf16_rne(v);
        else static_cast<float*>(p.y)[off] = v;
      }
    }
}

template <int MT, int NT>
static void launch_lr(const LinearParams& p, const LinearPlan& pl, dim3 grid, hipStream_t s) {
  const size_t lds = (size_t)pl.nw * MT * NT * kWave * sizeof(f32x4);
  if (pl.u == 2) hipLaunchKernelGGL((linear_rows<MT, NT, 2>), grid, dim3(pl.nw * kWave), lds, s, p);
  else hipLaunchKernelGGL((linear_rows<MT, NT, 1>), grid, dim3(pl.nw * kWave), lds, s, p);
}

// One block per CU streams weights at what the CU's memory path sustains, so the
// plan aims at blocks that fill all 256 CUs once, none doubled up:
//  - column tiles of 64 (each x fragment serves four weight fragments); tiles of
//    32 when that alone reaches 256 blocks and 64 would not;
//  - with fewer blocks than that, every product's K is cut into equal parts;
//  - with enough, a product much smaller than the launch is cut into 16 parts, so
//    that its blocks are short wherever they land.
LinearPlan plan_linear(int R, int K, const int* N, int np, int nbatch) {
  LinearPlan pl;
  pl.np = np;
  if (R >= kGemmRows) {  // one tiled GEMM per product, no partial sums
    pl.gemm = true;
    return pl;
  }
  pl.mt = R <= 16 ? 1 : (R <= 32 ? 2 : 4);
  pl.row_blocks = (R + 16 * pl.mt - 1) / (16 * pl.mt);
  auto count_tiles = [&](int nt) {
    int64_t t = 0;
    for (int i = 0; i < np; ++i) t += (N[i] + 16 * nt - 1) / (16 * nt);
    return t * nbatch * pl.row_blocks;
  };
  pl.nt = (count_tiles(4) < 256 && count_tiles(2) >= 256) ? 2 : 4;
  pl.nw = pl.mt * pl.nt >= 8 ? 4 : 8;
  if (K % (pl.nw * 32)) pl.nw = 4;
  const int64_t tiles = count_tiles(pl.nt);
  auto fits = [&](int s) { return K % s == 0 && (K / s) % (pl.nw * 32) == 0; };
  int uniform = 1;
  if (tiles < 256)
    while (tiles * uniform < 256 && fits(2 * uniform)) uniform *= 2;
  int64_t blocks = 0, part = 0, elems = 0;
  bool u2 = pl.mt * pl.nt < 16;
  for (int i = 0; i < np; ++i) {
    const int64_t ti = (N[i] + 16 * pl.nt - 1) / (16 * pl.nt);
    int s = uniform;
    if (tiles >= 256 && ti * nbatch * pl.row_blocks * 16 <= tiles)  // keep two k-steps per wave trip
      while (s < 16 && fits(2 * s) && (K / (2 * s) / pl.nw) % 64 == 0) s *= 2;
    pl.splits[i] = s;
    pl.blk0[i] = (int)blocks;
    blocks += ti * s;
    if (s > 1) {
      const int64_t count = (int64_t)nbatch * R * N[i];
      pl.part_off[i] = part;
      pl.e0[i] = elems;
      part += count * s;
      elems += count;
    }
    if ((K / s / pl.nw) % 64) u2 = false;
  }
  pl.u = u2 ? 2 : 1;
  pl.blocks = (int)blocks;
  pl.reduce_elems = elems;
  pl.part_bytes = (size_t)part * sizeof(float);
  return pl;
}

struct Product {
  const void* W;
  void* y;
  int64_t w_bs, y_bs, y_rs;
  int N, out;
  int split;  // tiled GEMM only: write bf16 hi and lo parts per block of `split` columns
};

static LinearPlan plan_products(int R, int K, const Product* pr, int np, int nbatch) {
  int N[kMaxSegs];
  for (int i = 0; i < np; ++i) N[i] = pr[i].N;
  return plan_linear(R, K, N, np, nbatch);
}

// Products sharing the rows x [R][K] (K % 128 == 0) in one launch; `part`
// holds the plan's partial sums when it splits K.
static hipError_t linear(const void* x, int64_t x_bs, int64_t x_rs, int R, int K, const Product* pr, int np,
                         int nbatch, float* part, hipStream_t s) {
  const LinearPlan pl = plan_products(R, K, pr, np, nbatch);
  if (pl.gemm) {
    for (int i = 0; i < np; ++i) {
      GemmParams g{};
      g.x = static_cast<const uint16_t*>(x);
      g.x_bs = x_bs;
      g.x_rs = x_rs;
      g.W = static_cast<const uint16_t*>(pr[i].W);
      g.w_bs = pr[i].w_bs;
      g.y = pr[i].y;
      g.y_bs = pr[i].y_bs;
      g.y_rs = pr[i].y_rs;
      g.R = R;
      g.N = pr[i].N;
      g.K = K;
      g.out = pr[i].out;
      g.split = pr[i].split;
      const dim3 grid((unsigned)((pr[i].N + kGN - 1) / kGN), (unsigned)((R + kGM - 1) / kGM), (unsigned)nbatch);
      hipLaunchKernelGGL(gemm_rows, grid, dim3(512), 0, s, g);
    }
    return hipGetLastError();
  }
  LinearParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.x_bs = x_bs;
  p.x_rs = x_rs;
  p.part = part;
  p.nseg = np;
  p.R = R;
  p.K = K;
  p.nbatch = nbatch;
  for (int i = 0; i < np; ++i) {
    LinearSeg& g = p.seg[i];
    g.W = static_cast<const uint16_t*>(pr[i].W);
    g.y = pr[i].y;
    g.w_bs = pr[i].w_bs;
    g.y_bs = pr[i].y_bs;
    g.y_rs = pr[i].y_rs;
    g.N = pr[i].N;
    g.out = pr[i].out;
    g.blk0 = pl.blk0[i];
    g.splits = pl.splits[i];
    g.part_off = pl.part_off[i];
    g.e0 = pl.e0[i];
  }
  const dim3 grid((unsigned)pl.blocks, (unsigned)nbatch, (unsigned)pl.row_blocks);
  if (pl.nt == 2) {
    if (pl.mt == 1) launch_lr<1, 2>(p, pl, grid, s);
    else if (pl.mt == 2) launch_lr<2, 2>(p, pl, grid, s);
    else launch_lr<4, 2>(p, pl, grid, s);
  } else {
    if (pl.mt == 1) launch_lr<1, 4>(p, pl, grid, s);
    else if (pl.mt == 2) launch_lr<2, 4>(p, pl, grid, s);
    else launch_lr<4, 4>(p, pl, grid, s);
  }
  if (pl.reduce_elems)
    hipLaunchKernelGGL(linear_reduce, dim3((unsigned)((pl.reduce_elems + 255) / 256)), dim3(256), 0, s, p,
                       pl.reduce_elems);
  return hipGetLastError();
}

// q[r][h][d] = sum_k qh[r][h][k] W_UK[h][k][d], fp32 products on the matrix
// cores (16x16x4 fp32).  Block (128 latent columns, head, 16 MT rows); its NWV
// waves take equal shares of k (KG groups of 16 each) and add up in LDS in wave
// order.
// A lane loads 8 adjacent columns of one W_UK row (16 bytes), which serve as the
// B operands of 8 products whose 16 output columns are 8 apart: product e of
// lane column c holds latent column 8 c + e.  Within a group of 16 k, step ss
// (0..3) gives K slot g the value k = 16 q + 4 g + ss, so a lane's four A values
// of a group are 4 adjacent head-query elements (one 16-byte load).
template <int OUT, int MT, int KG, int NWV>
__global__ __launch_bounds__(NWV * 64) void absorb_kernel(const float* __restrict__ qh,
                                                          const uint16_t* __restrict__ WUK, void* __restrict__ q, int R,
                                                          int H, int D) {
  constexpr int dh = 16 * KG * NWV;
  __shared__ f32x4 red[NWV][8 * MT][kWave];
  const int nb = blockIdx.x * 128, h = blockIdx.y, r0 = blockIdx.z * 16 * MT;
  const int l = lane_id(), w = wave_id(), c = l & 15, g = l >> 4;
  const int kw0 = w * 16 * KG;  // first k of the wave
  const gbytes qb = opaque_global(qh), wb = opaque_global(WUK + (int64_t)h * dh * D + nb);
  f32x4 a[KG][MT];
  u32x4 bw[KG][4];
#pragma unroll
  for (int kg = 0; kg < KG; ++kg) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      int row = r0 + 16 * mt + c;
      row = row < R ? row : R - 1;  // rows past R repeat the last (not stored)
      a[kg][mt] = gload<f32x4>(qb, (((int64_t)row * H + h) * dh + kw0 + 16 * kg + 4 * g) * 4);
    }
#pragma unroll
    for (int ss = 0; ss < 4; ++ss)
      bw[kg][ss] = gload<u32x4>(wb, ((int64_t)(kw0 + 16 * kg + 4 * g + ss) * D + 8 * c) * 2);
  }
  f32x4 acc[MT][8];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[mt][e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kg = 0; kg < KG; ++kg)
#pragma unroll
    for (int ss = 0; ss < 4; ++ss)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t word = bw[kg][ss][e >> 1];
        const float b = bf16_to_f32((e & 1) ? word >> 16 : word & 0xffffu);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][e] = mfma16_f32(a[kg][mt][ss], b, acc[mt][e]);
      }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[w][mt * 8 + e][l] = acc[mt][e];
  __syncthreads();
  for (int t = w; t < 8 * MT; t += NWV) {
    f32x4 v = red[0][t][l];
#pragma unroll
    for (int j = 1; j < NWV; ++j) v += red[j][t][l];
    const int mt = t / 8, e = t % 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r0 + 16 * mt + 4 * g + i;
      if (row >= R) continue;
      const int64_t off = ((int64_t)row * H + h) * D + nb + 8 * c + e;
      if constexpr (OUT == SCKV_BF16) static_cast<uint16_t*>(q)[off] = (uint16_t)f32_to_bf16_rne(v[i]);
      else static_cast<float*>(q)[off] = v[i];
    }
  }
}

// Blocks of 16 rows; d_h = 64 on 4 waves, 128 and 256 on 8 (one or two groups of
// 16 k per wave).
template <int OUT>
static void launch_absorb(const sckv_query_args& a, const float* qh, hipStream_t s) {
  const dim3 grid((unsigned)(a.D / 128), (unsigned)a.H, (unsigned)((a.R + 15) / 16));
  const uint16_t* W = static_cast<const uint16_t*>(a.W_UK);
  if (a.d_h == 64)
    hipLaunchKernelGGL((absorb_kernel<OUT, 1, 1, 4>), grid, dim3(256), 0, s, qh, W, a.q, a.R, a.H, a.D);
  else if (a.d_h == 128)
    hipLaunchKernelGGL((absorb_kernel<OUT, 1, 1, 8>), grid, dim3(512), 0, s, qh, W, a.q, a.R, a.H, a.D);
  else
    hipLaunchKernelGGL((absorb_kernel<OUT, 1, 2, 8>), grid, dim3(512), 0, s, qh, W, a.q, a.R, a.H, a.D);
}

// W_UK [H][dh][D] -> T [H][D][2 dh] with T[h][n][k] = T[h][n][dh + k] = W_UK[h][k][n]:
// the absorption's weights as a GEMM operand over the two bf16 parts of the head
// queries.  64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void dup_transpose(const uint16_t* __restrict__ WUK, uint16_t* __restrict__ T,
                                                     int dh, int D) {
  __shared__ uint16_t t[64][65];
  const int h = blockIdx.z, n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  const uint16_t* src = WUK + (int64_t)h * dh * D;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int kk = i / 64, nn = i % 64;
    t[kk][nn] = src[(int64_t)(k0 + kk) * D + n0 + nn];
  }
  __syncthreads();
  uint16_t* dst = T + (int64_t)h * D * 2 * dh;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int nn = i / 64, kk = i % 64;
    const uint16_t v = t[kk][nn];
    dst[(int64_t)(n0 + nn) * 2 * dh + k0 + kk] = v;
    dst[(int64_t)(n0 + nn) * 2 * dh + dh + k0 + kk] = v;
  }
}

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Absorption of many rows runs on the bf16 GEMM: W_q writes each head query as two
// bf16 parts (hi, lo: the same bytes as fp32) and the GEMM multiplies [hi | lo]
// by [W_UK^T | W_UK^T] (the duplicated transpose, after the head queries).
static bool absorb_by_gemm(const sckv_query_args& a) { return a.W_UK && a.R >= kGemmRows; }

static int query_products(const sckv_query_args& a, void* ws, Product* pr) {
  const int HD = a.H * a.d_h;
  const bool absorb = a.W_UK != nullptr;
  int np = 0;
  // head queries: into the workspace when they are absorbed (fp32, or two bf16
  // parts for the GEMM absorption), else straight to q
  if (absorb_by_gemm(a)) pr[np++] = Product{a.W_q, ws, 0, 0, 2 * (int64_t)HD, HD, SCKV_BF16, a.d_h};
  else pr[np++] = Product{a.W_q, absorb ? ws : a.q, 0, 0, HD, HD, absorb ? SCKV_F32 : a.q_dtype, 0};
  if (a.W_iq) pr[np++] = Product{a.W_iq, a.qI, 0, 0, (int64_t)a.H_I * a.D_I, a.H_I * a.D_I, a.q_dtype, 0};
  if (a.W_w) pr[np++] = Product{a.W_w, a.w, 0, 0, a.H_I, a.H_I, SCKV_F32, 0};
  return np;
}

static size_t query_heads_bytes(const sckv_query_args& a) {
  if (!a.W_UK) return 0;
  const size_t heads = align256((size_t)a.R * a.H * a.d_h * sizeof(float));
  return absorb_by_gemm(a) ? heads + align256((size_t)a.H * a.D * 2 * a.d_h * sizeof(uint16_t)) : heads;
}

static hipError_t absorb(const sckv_query_args& a, void* ws, hipStream_t s) {
  if (absorb_by_gemm(a)) {
    uint16_t* T = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) +
                                              align256((size_t)a.R * a.H * a.d_h * sizeof(float)));
    hipLaunchKernelGGL(dup_transpose, dim3((unsigned)(a.D / 64), (unsigned)(a.d_h / 64), (unsigned)a.H), dim3(256), 0,
                       s, static_cast<const uint16_t*>(a.W_UK), T, a.d_h, a.D);
    // batch item h: x = [hi | lo] of head h (2 d_h columns), W = T[h] [D][2 d_h], y = q[:, h, :]
    const Product pr{T, a.q, (int64_t)a.D * 2 * a.d_h, a.D, (int64_t)a.H * a.D, a.D, a.q_dtype, 0};
    return linear(ws, 2 * a.d_h, (int64_t)a.H * 2 * a.d_h, a.R, 2 * a.d_h, &pr, 1, a.H, nullptr, s);
  }
  if (a.q_dtype == SCKV_BF16) launch_absorb<SCKV_BF16>(a, static_cast<const float*>(ws), s);
  else launch_absorb<SCKV_F32>(a, static_cast<const float*>(ws), s);
  return hipGetLastError();
}

size_t queries_workspace(const sckv_query_args& a) {
  Product pr[3];
  const int np = query_products(a, nullptr, pr);
  return query_heads_bytes(a) + plan_products(a.R, a.d_model, pr, np, 1).part_bytes;
}

hipError_t launch_layer_queries(const sckv_query_args& a, void* ws, hipStream_t s) {
  Product pr[3];
  const int np = query_products(a, ws, pr);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + query_heads_bytes(a));
  hipError_t e = linear(a.x, 0, a.d_model, a.R, a.d_model, pr, np, 1, part, s);
  if (e != hipSuccess || !a.W_UK) return e;
  return absorb(a, ws, s);
}

static int stream_products(const sckv_stream_args& a, Product* pr) {
  const void* W[4] = {a.W_c, a.W_g, a.W_cI, a.W_gI};
  void* out[4] = {a.v, a.g, a.vI, a.gI};
  const int N[4] = {a.D, a.D, a.D_I, a.D_I};
  int np = 0;
  for (int i = 0; i < 4; ++i)
    if (W[i]) pr[np++] = Product{W[i], out[i], 0, 0, N[i], N[i], a.out_dtype, 0};
  return np;
}

size_t streams_workspace(const sckv_stream_args& a) {
  Product pr[4];
  const int np = stream_products(a, pr);
  return np ? plan_products(a.R, a.d_model, pr, np, 1).part_bytes : 0;
}

hipError_t launch_layer_streams(const sckv_stream_args& a, void* ws, hipStream_t s) {
  Product pr[4];
  const int np = stream_products(a, pr);
  if (np == 0) return hipSuccess;
  return linear(a.x, 0, a.d_model, a.R, a.d_model, pr, np, 1, static_cast<float*>(ws), s);
}

// Queries and streams of the same rows in one launch.
size_t inputs_workspace(const sckv_query_args& a, const sckv_stream_args& st) {
  Product pr[kMaxSegs];
  int np = query_products(a, nullptr, pr);
  np += stream_products(st, pr + np);
  return query_heads_bytes(a) + plan_products(a.R, a.d_model, pr, np, 1).part_bytes;
}

hipError_t launch_layer_inputs(const sckv_query_args& a, const sckv_stream_args& st, void* ws, hipStream_t s) {
  Product pr[kMaxSegs];
  int np = query_products(a, ws, pr);
  np += stream_products(st, pr + np);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + query_heads_bytes(a));
  hipError_t e = linear(a.x, 0, a.d_model, a.R, a.d_model, pr, np, 1, part, s);
  if (e != hipSuccess || !a.W_UK) return e;
  return absorb(a, ws, s);
}

// o_h = W_UV^h o~_h for every head (a batch of H products), rounded to bf16 into
// the workspace; then y = W_o [o_1 .. o_H].
static Product heads_product(const sckv_output_args& a, void* ws) {
  return Product{a.W_UV, ws, (int64_t)a.d_h * a.D, a.d_h, (int64_t)a.H * a.d_h, a.d_h, SCKV_BF16, 0};
}

static Product out_product(const sckv_output_args& a) {
  return Product{a.W_o, a.y, 0, 0, a.d_model, a.d_model, a.y_dtype, 0};
}

static size_t output_heads_bytes(const sckv_output_args& a) {
  return a.W_UV ? align256((size_t)a.R * a.H * a.d_h * sizeof(uint16_t)) : 0;
}

size_t output_workspace(const sckv_output_args& a) {
  const Product po = out_product(a);
  size_t part = plan_products(a.R, a.H * a.d_h, &po, 1, 1).part_bytes;
  if (a.W_UV) {
    const Product ph = heads_product(a, nullptr);
    const size_t p1 = plan_products(a.R, a.D, &ph, 1, a.H).part_bytes;
    part = p1 > part ? p1 : part;
  }
  return output_heads_bytes(a) + part;
}

hipError_t launch_layer_output(const sckv_output_args& a, void* ws, hipStream_t s) {
  const int HD = a.H * a.d_h;
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + output_heads_bytes(a));
  const void* heads = a.o;
  if (a.W_UV) {
    const Product ph = heads_product(a, ws);
    hipError_t e = linear(a.o, a.D, (int64_t)a.H * a.D, a.R, a.D, &ph, 1, a.H, part, s);
    if (e != hipSuccess) return e;
    heads = ws;
  }
  const Product po = out_product(a);
  return linear(heads, 0, HD, a.R, HD, &po, 1, 1, part, s);
}

}  // namespace sckv
