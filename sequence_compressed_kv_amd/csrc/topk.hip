// Per-row top-k selection: the min(k, n) best entries by (score descending,
// index ascending), emitted as ascending indices padded with -1 (knightli.com
// DeepSeek-V4 KV-cache article, section "CSA": keep the top-k scored blocks;
// ties to the lower index as the workload definition states).
//
// Radix select held in registers and LDS: each thread keeps V consecutive
// scores as order-preserving 32-bit keys; three LDS histogram passes over key
// digits [31:20], [19:8], [7:0] find the exact k-th key T and how many keys
// equal to T to take; an ordered compaction (block prefix sums built from
// wavefront scans) then writes the kept indices in ascending order, taking the
// lowest-indexed ties.  Rows too long for one block are cut into slices whose
// local top-k are merged by a second pass over the slices' candidates.
#include <climits>

#include "device_common.h"
#include "sckv_internal.h"

namespace sckv {

constexpr int kBins = 4096;

enum { TOPK_ROW = 0, TOPK_SLICE = 1, TOPK_MERGE = 2 };

struct TopkRows {
  int kind;
  const int32_t* pos;
  int32_t pos_max, seq0, pos0;
  int m, W;
  int64_t E_cap;
};

__device__ __forceinline__ int64_t row_visible(const TopkRows& rr, int r) {
  int64_t t;
  if (rr.kind == SCKV_ROWS_DECODE) {
    int32_t p = rr.pos[r];
    t = p < 0 ? 0 : (p > rr.pos_max ? rr.pos_max : p);
  } else {
    t = (int64_t)rr.pos0 + r;
  }
  const int64_t d = t - rr.W;
  const int64_t e = d < 0 ? 0 : d / rr.m;
  return e < rr.E_cap ? e : rr.E_cap;
}

// Finds the kk-th largest key among valid elements: returns T and, in *need, how
// many elements equal to T belong to the selection.  Every thread must call it.
template <int NT, int V>
__device__ __forceinline__ uint32_t radix_threshold(const uint32_t (&key)[V], const bool (&valid)[V],
                                                    uint32_t kk, uint32_t* hist, uint32_t* scan_sh,
                                                    uint32_t* ctl, uint32_t* need) {
  constexpr int BPT = kBins / NT;
  uint32_t prefix = 0, kk_rem = kk;
  const int shifts[3] = {20, 8, 0};
  const uint32_t hmasks[3] = {0u, 0xFFF00000u, 0xFFFFFF00u};
  const uint32_t dmasks[3] = {0xFFFu, 0xFFFu, 0xFFu};
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (valid[v] && (key[v] & hmasks[p]) == prefix) atomicAdd(&hist[(key[v] >> shifts[p]) & dmasks[p]], 1u);
    __syncthreads();
    uint32_t tsum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) tsum += hist[threadIdx.x * BPT + i];
    uint32_t total;
    const uint32_t below = block_excl_scan<NT>(tsum, scan_sh, &total);
    const uint32_t above = total - below - tsum;      // elements in higher bins than this chunk
    if (above < kk_rem && kk_rem <= above + tsum) {
      uint32_t run = above;
      for (int i = BPT - 1; i >= 0; --i) {
        const uint32_t h = hist[threadIdx.x * BPT + i];
        if (run + h >= kk_rem) {
          ctl[0] = (uint32_t)(threadIdx.x * BPT + i);
          ctl[1] = kk_rem - run;
          break;
        }
        run += h;
      }
    }
    __syncthreads();
    prefix |= ctl[0] << shifts[p];
    kk_rem = ctl[1];
    __syncthreads();
  }
  *need = kk_rem;
  return prefix;
}

// Exclusive prefix of per-thread counts c[i] in element order, where a thread
// holds groups i = 0 .. NI-1 of 4 consecutive elements and element order is
// (wave, group, lane, element).  Returns per-group offsets and the block total.
template <int NT, int NI>
__device__ __forceinline__ void ordered_scan(const uint32_t (&c)[NI], uint32_t (&off)[NI], uint32_t* sh,
                                             uint32_t* total) {
  constexpr int NW = NT / kWave;
  const int w = wave_id(), l = lane_id();
  uint32_t run = 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t inc = wave_incl_scan(c[i]);
    off[i] = run + inc - c[i];
    run += last_lane(inc);
  }
  if (l == 0) sh[w] = run;
  __syncthreads();
  if (w == 0) {
    const uint32_t x = l < NW ? sh[l] : 0u;
    const uint32_t xi = wave_incl_scan(x);
    if (l < NW) sh[l] = xi - x;
    if (l == NW - 1) sh[NW] = xi;
  }
  __syncthreads();
  const uint32_t base = sh[w];
#pragma unroll
  for (int i = 0; i < NI; ++i) off[i] += base;
  *total = sh[NW];
  __syncthreads();
}

// MODE TOPK_ROW   : scores of row r, elements 0 .. n-1 (n = visible count), out to out_idx.
// MODE TOPK_SLICE : slice blockIdx.x of row r, local top-k written as candidates.
// MODE TOPK_MERGE : the candidates of row r (nslices x kc slots; unused slots hold index -1).
// Wave w owns elements [w*64*V, (w+1)*64*V); its group i is read as one coalesced
// 1 KB load: lane l takes elements w*64*V + (i*64 + l)*4 .. +3.
template <int NT, int V, int MODE>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ scores, int64_t stride,
                                                  TopkRows rows, int k, int64_t slice, int nslices, int kc,
                                                  int64_t cap, float* __restrict__ cand_s,
                                                  int32_t* __restrict__ cand_i,
                                                  int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  constexpr int NI = V / 4;
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scan_sh[NT / kWave + 1];
  __shared__ uint32_t ctl[2];
  const int r = blockIdx.y;
  const int w = wave_id(), l = lane_id();
  const int64_t n_row = row_visible(rows, r);

  int64_t base = 0, len = 0;
  if (MODE == TOPK_ROW) {
    len = n_row;
  } else if (MODE == TOPK_SLICE) {
    base = (int64_t)blockIdx.x * slice;
    len = n_row - base;
    len = len < 0 ? 0 : (len > slice ? slice : len);
  } else {
    len = (int64_t)nslices * kc;
  }

  uint32_t key[V];
  int32_t idx[V];
  bool valid[V];
  const float* src = MODE == TOPK_MERGE ? cand_s + (int64_t)r * cap : scores + (int64_t)r * stride + base;
  const bool vec = ((reinterpret_cast<uintptr_t>(src) & 15u) == 0);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int64_t e0 = (int64_t)w * 64 * V + ((int64_t)i * 64 + l) * 4;
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
    int32_t i4[4] = {-1, -1, -1, -1};
    if (vec && e0 + 3 < len) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + e0);
      s4[0] = v[0]; s4[1] = v[1]; s4[2] = v[2]; s4[3] = v[3];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (e0 + j < len) s4[j] = src[e0 + j];
    }
    if (MODE == TOPK_MERGE) {
      if (vec && e0 + 3 < len) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(cand_i + (int64_t)r * cap + e0);
        i4[0] = v[0]; i4[1] = v[1]; i4[2] = v[2]; i4[3] = v[3];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (e0 + j < len) i4[j] = cand_i[(int64_t)r * cap + e0 + j];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t e = e0 + j;
      bool ok = e < len;
      if (MODE == TOPK_MERGE) ok = ok && i4[j] >= 0;           // unused candidate slots hold -1
      valid[4 * i + j] = ok;
      key[4 * i + j] = ok ? score_key(s4[j]) : 0u;
      idx[4 * i + j] = MODE == TOPK_MERGE ? i4[j] : (int32_t)(base + e);
    }
  }

  // number of valid elements and how many to keep
  uint32_t nv = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) nv += valid[v] ? 1u : 0u;
  uint32_t n_valid;
  (void)block_excl_scan<NT>(nv, scan_sh, &n_valid);
  const uint32_t kk = n_valid < (uint32_t)k ? n_valid : (uint32_t)k;

  uint32_t T = 0, need = UINT_MAX;
  if (kk < n_valid) T = radix_threshold<NT, V>(key, valid, kk, hist, scan_sh, ctl, &need);

  // ordered compaction: keys above T, then the first `need` keys equal to T
  uint32_t ceq[NI], eq_off[NI], tot;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    ceq[i] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) ceq[i] += (valid[4 * i + j] && key[4 * i + j] == T) ? 1u : 0u;
  }
  ordered_scan<NT, NI>(ceq, eq_off, scan_sh, &tot);
  bool sel[V];
  uint32_t csel[NI], sel_off[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    uint32_t eq_rank = eq_off[i];
    csel[i] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = 4 * i + j;
      bool sv = valid[v] && key[v] > T;
      if (valid[v] && key[v] == T) sv = eq_rank++ < need;
      sel[v] = sv;
      csel[i] += sv ? 1u : 0u;
    }
  }
  ordered_scan<NT, NI>(csel, sel_off, scan_sh, &tot);

  int32_t* oi;
  float* os;
  if (MODE == TOPK_SLICE) {
    oi = cand_i + (int64_t)r * cap + (int64_t)blockIdx.x * kc;
    os = cand_s + (int64_t)r * cap + (int64_t)blockIdx.x * kc;
  } else {
    oi = out_idx + (int64_t)r * k;
    os = out_score ? out_score + (int64_t)r * k : nullptr;
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    uint32_t off = sel_off[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = 4 * i + j;
      if (sel[v]) {
        oi[off] = idx[v];
        if (os) os[off] = key_score(key[v]);
        ++off;
      }
    }
  }
  // pad to k (a slice pads its kc candidate slots: the merge skips index -1)
  const int kpad = MODE == TOPK_SLICE ? kc : k;
  for (int i = (int)kk + threadIdx.x; i < kpad; i += NT) {
    oi[i] = -1;
    if (os) os[i] = -INFINITY;
  }
}

static const int kCfg[][2] = {{256, 4}, {256, 16}, {256, 32}, {1024, 16}, {1024, 32}, {1024, 64}};

TopkPlan plan_topk(int64_t cover, int32_t k, int32_t R) {
  TopkPlan p;
  p.cover = cover;
  for (auto& c : kCfg) {
    if ((int64_t)c[0] * c[1] >= cover && c[1] <= 32) {
      p.single_nt = c[0];
      p.single_v = c[1];
      p.ok = true;
      return p;
    }
  }
  p.slice = 16384;
  p.nslices = (cover + p.slice - 1) / p.slice;
  const int64_t kc = k < p.slice ? k : p.slice;
  p.cand = (p.nslices * kc + 3) / 4 * 4;
  if (p.cand > 1024 * 64) return p;  // not ok
  p.ws_bytes = (size_t)R * (size_t)p.cand * 8 + 256;
  p.ok = true;
  return p;
}

template <int MODE>
static void launch_cfg(int nt, int v, dim3 grid, const float* scores, int64_t stride, const TopkRows& rr,
                       int k, int64_t slice, int nslices, int kc, int64_t cap, float* cs, int32_t* ci,
                       int32_t* oi, float* os, hipStream_t st) {
#define SCKV_TK(NT, VV)                                                                                  \
  if (nt == NT && v == VV) {                                                                             \
    hipLaunchKernelGGL((topk_kernel<NT, VV, MODE>), grid, dim3(NT), 0, st, scores, stride, rr, k, slice, \
                       nslices, kc, cap, cs, ci, oi, os);                                                \
    return;                                                                                              \
  }
  SCKV_TK(256, 4) SCKV_TK(256, 16) SCKV_TK(256, 32) SCKV_TK(1024, 16) SCKV_TK(1024, 32) SCKV_TK(1024, 64)
#undef SCKV_TK
}

hipError_t launch_topk(const sckv_index_args& a, const float* scores, int64_t stride, const TopkPlan& p,
                       void* ws, hipStream_t stream) {
  TopkRows rr{a.rows.kind, a.rows.pos, a.rows.pos_max, a.rows.seq0, a.rows.pos0, a.m, a.W, a.E_cap};
  const int R = a.rows.R;
  if (p.single_nt) {
    launch_cfg<TOPK_ROW>(p.single_nt, p.single_v, dim3(1, R), scores, stride, rr, a.k, 0, 1, 1, 0, nullptr,
                         nullptr, a.out_idx, a.out_score, stream);
    return hipGetLastError();
  }
  const int kc = (int)(a.k < p.slice ? a.k : p.slice);
  char* w = static_cast<char*>(ws);
  float* cs = reinterpret_cast<float*>(w);
  int32_t* ci = reinterpret_cast<int32_t*>(w + (size_t)R * p.cand * 4);
  launch_cfg<TOPK_SLICE>(1024, 16, dim3((unsigned)p.nslices, R), scores, stride, rr, a.k, p.slice,
                         (int)p.nslices, kc, p.cand, cs, ci, nullptr, nullptr, stream);
  int nt = 1024, v = 64;
  for (auto& c : kCfg)
    if ((int64_t)c[0] * c[1] >= p.cand) { nt = c[0]; v = c[1]; break; }
  launch_cfg<TOPK_MERGE>(nt, v, dim3(1, R), scores, stride, rr, a.k, p.slice, (int)p.nslices, kc, p.cand, cs,
                         ci, a.out_idx, a.out_score, stream);
  return hipGetLastError();
}

}  // namespace sckv
