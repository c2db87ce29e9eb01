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
#include <type_traits>

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

// Elements wbase + (i*64 + l)*4 + j (i < V/4, j < 4) of a row of len 32-bit
// values, for lane l of a wave; 0 past the end.  Every load is issued before any
// is used, so the wave's part costs one memory round trip: a wave whose elements
// all exist reads 16-byte vectors (wbase wave-uniform), a ragged wave reads each
// element from an address clamped into the row and masks it afterwards.
template <int V, typename T>
__device__ __forceinline__ void load_part(const T* src, int64_t len, int64_t wbase, T (&s)[V]) {
  static_assert(sizeof(T) == 4, "32-bit values");
  constexpr int NI = V / 4;
  typedef __attribute__((ext_vector_type(4))) T T4;
  const int l = lane_id();
  const bool vec = ((reinterpret_cast<uintptr_t>(src) & 15u) == 0);
  if (vec && wbase + 64 * V <= len) {
    T4 v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) v[i] = *reinterpret_cast<const T4*>(src + wbase + ((int64_t)i * 64 + l) * 4);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[4 * i + j] = v[i][j];
  } else if (len > 0) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int64_t e = wbase + ((int64_t)(v / 4) * 64 + l) * 4 + (v % 4);
      s[v] = src[e < len ? e : len - 1];
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int64_t e = wbase + ((int64_t)(v / 4) * 64 + l) * 4 + (v % 4);
      if (e >= len) s[v] = T(0);
    }
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) s[v] = T(0);
  }
}

// Bin of the kk_rem-th largest element of an LDS histogram (kBins bins, counted
// from the top): ctl[0] = bin, ctl[1] = kk_rem minus the elements in higher bins.
// A histogram of NC copies keeps bin b's counts at words NC b .. NC b + NC - 1.
// Every thread must call it (block scan, barriers).
template <int NT, int NC = 1>
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t kk_rem, uint32_t* scan_sh, uint32_t* ctl) {
  static_assert(NC == 1 || NC % 4 == 0, "copies are read four at a time");
  constexpr int BPT = kBins / NT;
  uint32_t hb[BPT];
  uint32_t tsum = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int b = threadIdx.x * BPT + i;
    uint32_t h = 0;
    if constexpr (NC == 1) {
      h = hist[b];
    } else {
#pragma unroll
      for (int c = 0; c < NC; c += 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(hist + b * NC + c);
        h += v[0] + v[1] + v[2] + v[3];
      }
    }
    hb[i] = h;
    tsum += h;
  }
  uint32_t total;
  const uint32_t below = block_excl_scan<NT>(tsum, scan_sh, &total);
  const uint32_t above = total - below - tsum;      // elements in higher bins than this chunk
  if (above < kk_rem && kk_rem <= above + tsum) {
    uint32_t run = above;
#pragma unroll
    for (int i = BPT - 1; i >= 0; --i) {
      const uint32_t h = hb[i];
      if (run + h >= kk_rem) {
        ctl[0] = (uint32_t)(threadIdx.x * BPT + i);
        ctl[1] = kk_rem - run;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
}

constexpr int kShift[3] = {20, 8, 0};
constexpr uint32_t kHMask[3] = {0u, 0xFFF00000u, 0xFFFFFF00u};
constexpr uint32_t kDMask[3] = {0xFFFu, 0xFFFu, 0xFFu};

// Finds the kk-th largest key among valid elements: returns T and, in *need, how
// many elements equal to T belong to the selection.  Every thread must call it.
// A caller that already knows the first digit passes it as prefix (with kk
// counted from that bin's top) and p0 = 1.
// The first digit's histogram has NC0 copies of each bin (kBins * NC0 words,
// 16-byte aligned when NC0 > 1), lane l counting into copy l % NC0: scores
// concentrate in a few dozen first-digit bins, and the atomics of a wave that
// hit one LDS word are serialised, so spreading a bin over NC0 words cuts that
// serialisation NC0-fold.  The later digits see only the keys of one bin,
// spread over many bins, and keep one copy.
template <int NT, int V, int NC0 = 1>
__device__ __forceinline__ uint32_t radix_threshold(const uint32_t (&key)[V], const bool (&valid)[V],
                                                    uint32_t kk, uint32_t* hist, uint32_t* scan_sh,
                                                    uint32_t* ctl, uint32_t* need, uint32_t prefix = 0,
                                                    int p0 = 0) {
  static_assert(NC0 == 1 || (NC0 % 4 == 0 && (NC0 & (NC0 - 1)) == 0), "copies: 1 or a power of two >= 4");
  uint32_t kk_rem = kk;
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    if (p < p0) continue;
    const int nc = p == 0 ? NC0 : 1;
    if (nc > 1) {
      for (int i = threadIdx.x * 4; i < kBins * nc; i += NT * 4)
        *reinterpret_cast<u32x4*>(hist + i) = u32x4{0u, 0u, 0u, 0u};
    } else {
      for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = 0;
    }
    __syncthreads();
    const uint32_t copy = p == 0 ? (uint32_t)(lane_id() & (NC0 - 1)) : 0u;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (valid[v] && (key[v] & kHMask[p]) == prefix)
        atomicAdd(&hist[((key[v] >> kShift[p]) & kDMask[p]) * nc + copy], 1u);
    __syncthreads();
    if (p == 0) find_bin<NT, NC0>(hist, kk_rem, scan_sh, ctl);
    else find_bin<NT>(hist, kk_rem, scan_sh, ctl);
    prefix |= ctl[0] << kShift[p];
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

// The kk best of a block's valid elements by (key descending, index ascending),
// written to oi (and os) in element order, which callers make ascending index
// order; slots kk .. kpad-1 get index -1.  Elements sit in element order
// (wave, group, lane, element).  Every thread must call it.
// A caller that knows the bin b of the first digit holding the kk-th key, and the
// count `above` of elements in higher bins, passes b1 = b + 1 and above.
template <int NT, int V, int NC0 = 1>
__device__ __forceinline__ void select_ordered(const uint32_t (&key)[V], const int32_t (&idx)[V],
                                               const bool (&valid)[V], uint32_t n_valid, uint32_t kk, int32_t* oi,
                                               float* os, int kpad, uint32_t* hist, uint32_t* scan_sh, uint32_t* ctl,
                                               uint32_t b1 = 0, uint32_t above = 0) {
  constexpr int NI = V / 4;
  uint32_t T = 0, need = UINT_MAX;
  bool all_eq = true;                    // every key equal to T is kept (no tie to break)
  if (kk < n_valid) {
    if (b1) T = radix_threshold<NT, V, NC0>(key, valid, kk - above, hist, scan_sh, ctl, &need, (b1 - 1) << 20, 1);
    else T = radix_threshold<NT, V, NC0>(key, valid, kk, hist, scan_sh, ctl, &need);
    // the last pass's histogram counts the keys equal to T (the same value in
    // every thread, read after that pass's final barrier)
    all_eq = hist[T & kDMask[2]] == need;
  }

  // ordered compaction: keys above T, then the first `need` keys equal to T; the
  // ranks among keys equal to T are only needed when some of them are left out
  uint32_t ceq[NI], eq_off[NI], tot;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    ceq[i] = 0;
    eq_off[i] = 0;
  }
  if (!all_eq) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) ceq[i] += (valid[4 * i + j] && key[4 * i + j] == T) ? 1u : 0u;
    ordered_scan<NT, NI>(ceq, eq_off, scan_sh, &tot);
  }
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
      if (valid[v] && key[v] == T) sv = all_eq || eq_rank++ < need;
      sel[v] = sv;
      csel[i] += sv ? 1u : 0u;
    }
  }
  ordered_scan<NT, NI>(csel, sel_off, scan_sh, &tot);
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
  for (int i = (int)kk + threadIdx.x; i < kpad; i += NT) {
    oi[i] = -1;
    if (os) os[i] = -INFINITY;
  }
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
  // one block per row of up to 32K scores: the first digit counted into four
  // copies per bin (64 KB); smaller blocks, several to a CU, keep one copy
  constexpr int NC0 = NT >= 1024 ? 4 : 1;
  __shared__ __attribute__((aligned(16))) uint32_t hist[kBins * NC0];
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
  const int64_t wbase = (int64_t)w * 64 * V;
  float sc[V];
  int32_t ci[V];
  load_part<V>(src, len, wbase, sc);
  if (MODE == TOPK_MERGE) load_part<V>(cand_i + (int64_t)r * cap, len, wbase, ci);
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t e = wbase + ((int64_t)(v / 4) * 64 + l) * 4 + (v % 4);
    bool ok = e < len;
    if (MODE == TOPK_MERGE) ok = ok && ci[v] >= 0;             // unused candidate slots hold -1
    valid[v] = ok;
    key[v] = ok ? score_key(sc[v]) : 0u;
    idx[v] = MODE == TOPK_MERGE ? ci[v] : (int32_t)(base + e);
  }

  // number of valid elements (a row or slice: its length; the merge counts the
  // used candidate slots) and how many to keep
  uint32_t n_valid;
  if (MODE == TOPK_MERGE) {
    uint32_t nv = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) nv += valid[v] ? 1u : 0u;
    (void)block_excl_scan<NT>(nv, scan_sh, &n_valid);
  } else {
    n_valid = (uint32_t)(len < (int64_t)NT * V ? len : (int64_t)NT * V);
  }
  const uint32_t kk = n_valid < (uint32_t)k ? n_valid : (uint32_t)k;

  int32_t* oi;
  float* os;
  int kpad;                              // a slice pads its kc candidate slots: the merge skips index -1
  if (MODE == TOPK_SLICE) {
    oi = cand_i + (int64_t)r * cap + (int64_t)blockIdx.x * kc;
    os = cand_s + (int64_t)r * cap + (int64_t)blockIdx.x * kc;
    kpad = kc;
  } else {
    oi = out_idx + (int64_t)r * k;
    os = out_score ? out_score + (int64_t)r * k : nullptr;
    kpad = k;
  }
  select_ordered<NT, V, NC0>(key, idx, valid, n_valid, kk, oi, os, kpad, hist, scan_sh, ctl);
}


// ------------------------------------------------------------------ many blocks per row
// For few rows longer than one block's registers hold (long-context decode):
// every row is cut into blocks of kMbS elements.
//   zero   : the rows' first-digit histograms are cleared
//   hist   : each block adds its elements' first-digit (key bits 31:20) counts
//            into the row's histogram
//   filter : each block finds, from the full histogram, the bin b holding the
//            row's kk-th largest key and writes its elements with digit >= b
//            (every member of the top-kk, plus the rest of bin b) in index order
//            to its own region of the workspace
//   final  : one block per row concatenates the regions in block order
//            (ascending index) and runs the exact selection on those survivors,
//            from the second digit on.
// When bin b is too full for one block (heavily tied or clustered scores), the
// filter writes nothing and the final block streams the whole row instead.
// (Handing the final step to the last filter block of each row instead would
// need a device-scope fence in every block, which writes back the L2.)
constexpr int kMbNT = 256, kMbV = 16, kMbS = kMbNT * kMbV;        // elements per filter block
constexpr int kFinNT = 1024, kFinV = 16, kFinCap = kFinNT * kFinV;  // survivors the final block holds
constexpr int kMbMaxBlocks = 1024;                                  // blocks per row

// Elements [base, base + NT*V) of a row (len of them exist) in element order
// (wave, group, lane, element): wave w owns elements w*64*V .. ; its group i is one
// coalesced 1 KB load, lane l taking elements (i*64 + l)*4 .. +3.
// Order-preserving keys, element indices and validity of a part loaded by
// load_part (wave w's elements w*64*V + (i*64 + l)*4 + j of a row part of len).
template <int V>
__device__ __forceinline__ void part_keys(const float (&sc)[V], int64_t len, int64_t base, uint32_t (&key)[V],
                                          int32_t (&idx)[V], bool (&valid)[V]) {
  const int64_t wbase = (int64_t)wave_id() * 64 * V;
  const int l = lane_id();
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t e = wbase + ((int64_t)(v / 4) * 64 + l) * 4 + (v % 4);
    const bool ok = e < len;
    valid[v] = ok;
    key[v] = ok ? score_key(sc[v]) : 0u;
    idx[v] = (int32_t)(base + e);
  }
}

template <int NT, int V>
__device__ __forceinline__ void load_row_part(const float* src, int64_t len, int64_t base, uint32_t (&key)[V],
                                              int32_t (&idx)[V], bool (&valid)[V]) {
  float sc[V];
  load_part<V>(src, len, (int64_t)wave_id() * 64 * V, sc);
  part_keys<V>(sc, len, base, key, idx, valid);
}

__global__ __launch_bounds__(256) void topk_zero_hist(uint32_t* __restrict__ hist, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) hist[i] = 0u;
}

__global__ __launch_bounds__(kMbNT) void topk_hist(const float* __restrict__ scores, int64_t stride, TopkRows rows,
                                                   uint32_t* __restrict__ ghist) {
  __shared__ uint32_t h[kBins];
  const int r = blockIdx.y;
  const int64_t base = (int64_t)blockIdx.x * kMbS;
  int64_t len = row_visible(rows, r) - base;
  if (len <= 0) return;
  len = len > kMbS ? kMbS : len;
  // the scores are in flight while the LDS histogram is cleared
  float sc[kMbV];
  load_part<kMbV>(scores + (int64_t)r * stride + base, len, (int64_t)wave_id() * 64 * kMbV, sc);
  for (int i = threadIdx.x; i < kBins; i += kMbNT) h[i] = 0u;
  __syncthreads();
  uint32_t key[kMbV];
  int32_t idx[kMbV];
  bool valid[kMbV];
  part_keys<kMbV>(sc, len, base, key, idx, valid);
#pragma unroll
  for (int v = 0; v < kMbV; ++v)
    if (valid[v]) atomicAdd(&h[key[v] >> 20], 1u);
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += kMbNT)
    if (h[i]) atomicAdd(&ghist[(int64_t)r * kBins + i], h[i]);
}

// From a row's first-digit histogram (global memory): ctl[3] = valid elements,
// kk = min(k, ctl[3]); ctl[0] = the bin of the kk-th largest key (kBins when kk
// is 0), ctl[1] = elements in higher bins, ctl[2] = elements in that bin.
template <int NT>
__device__ __forceinline__ void row_threshold_bin(const uint32_t* gh, int k, uint32_t* scan_sh, uint32_t* ctl) {
  constexpr int BPT = kBins / NT;
  static_assert(BPT % 4 == 0, "bins are read four at a time");
  uint32_t c[BPT];
#pragma unroll
  for (int i = 0; i < BPT; i += 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(gh + threadIdx.x * BPT + i);
    c[i] = v[0]; c[i + 1] = v[1]; c[i + 2] = v[2]; c[i + 3] = v[3];
  }
  uint32_t tsum = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) tsum += c[i];
  uint32_t total;
  const uint32_t below = block_excl_scan<NT>(tsum, scan_sh, &total);
  const uint32_t kk = total < (uint32_t)k ? total : (uint32_t)k;
  const uint32_t above = total - below - tsum;
  if (threadIdx.x == 0) {
    ctl[3] = total;
    if (kk == 0) { ctl[0] = kBins; ctl[1] = 0; ctl[2] = 0; }
  }
  if (kk > 0 && above < kk && kk <= above + tsum) {
    uint32_t run = above;
#pragma unroll
    for (int i = BPT - 1; i >= 0; --i) {
      if (run + c[i] >= kk) {
        ctl[0] = (uint32_t)(threadIdx.x * BPT + i);
        ctl[1] = run;
        ctl[2] = c[i];
        break;
      }
      run += c[i];
    }
  }
  __syncthreads();
}

// Exact top-kk of a whole row by one block, streamed in chunks of NT*V elements:
// three radix passes, then an ordered pass that writes the kept indices in order.
// (The rare path: kept out of line so it does not weigh on the common one.)
template <int NT, int V>
__device__ __noinline__ void topk_stream_row(const float* src, int64_t n, uint32_t kk, int32_t* oi, float* os, uint32_t* hist,
                                uint32_t* scan_sh, uint32_t* ctl) {
  constexpr int NI = V / 4, CH = NT * V;
  uint32_t prefix = 0, kk_rem = kk;
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = 0;
    __syncthreads();
    for (int64_t c0 = 0; c0 < n; c0 += CH) {
      uint32_t key[V];
      int32_t idx[V];
      bool valid[V];
      load_row_part<NT, V>(src + c0, n - c0, c0, key, idx, valid);
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (valid[v] && (key[v] & kHMask[p]) == prefix) atomicAdd(&hist[(key[v] >> kShift[p]) & kDMask[p]], 1u);
    }
    __syncthreads();
    find_bin<NT>(hist, kk_rem, scan_sh, ctl);
    prefix |= ctl[0] << kShift[p];
    kk_rem = ctl[1];
    __syncthreads();
  }
  const uint32_t T = prefix, need = kk_rem;
  uint32_t written = 0, eq_seen = 0;                   // block-uniform running totals
  for (int64_t c0 = 0; c0 < n && written < kk; c0 += CH) {
    uint32_t key[V];
    int32_t idx[V];
    bool valid[V];
    load_row_part<NT, V>(src + c0, n - c0, c0, key, idx, valid);
    uint32_t ceq[NI], eq_off[NI], tot_eq;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      ceq[i] = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) ceq[i] += (valid[4 * i + j] && key[4 * i + j] == T) ? 1u : 0u;
    }
    ordered_scan<NT, NI>(ceq, eq_off, scan_sh, &tot_eq);
    bool sel[V];
    uint32_t csel[NI], sel_off[NI], tot_sel;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      uint32_t eq_rank = eq_seen + eq_off[i];
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
    ordered_scan<NT, NI>(csel, sel_off, scan_sh, &tot_sel);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      uint32_t off = written + sel_off[i];
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
    written += tot_sel;
    eq_seen += tot_eq;
  }
}

// The final selection of row r (one block of kFinNT threads).
__device__ __forceinline__ void topk_row_final(const float* scores, int64_t stride, const TopkRows& rows, int r, int k,
                                            int nb, const int32_t* cnt, const uint32_t* rkey, const int32_t* ridx,
                                            uint32_t b, uint32_t above, uint32_t n_valid, int32_t* out_idx,
                                            float* out_score, uint32_t* hist, uint32_t* scan_sh, uint32_t* ctl,
                                            int32_t* pre, int32_t* flag, uint32_t* skey, int32_t* sidx,
                                            int32_t my) {
  static_assert(kMbMaxBlocks <= kFinNT, "one filter block's survivor count per thread");
  const int w = wave_id(), l = lane_id();
  int32_t* oi = out_idx + (int64_t)r * k;
  float* os = out_score ? out_score + (int64_t)r * k : nullptr;
  const uint32_t kk = n_valid < (uint32_t)k ? n_valid : (uint32_t)k;
  // survivors per filter block (my: block threadIdx.x's count, loaded by the
  // caller) -> exclusive prefix in block order
  if (threadIdx.x == 0) *flag = 0;
  __syncthreads();
  if (my < 0) *flag = 1;
  uint32_t run;
  const uint32_t ex = block_excl_scan<kFinNT>(my < 0 ? 0u : (uint32_t)my, scan_sh, &run);
  if (threadIdx.x < nb) pre[threadIdx.x] = (int32_t)ex;
  if (threadIdx.x == 0) pre[nb] = (int32_t)run;
  __syncthreads();
  if (*flag) {
    topk_stream_row<kFinNT, kFinV>(scores + (int64_t)r * stride, row_visible(rows, r), kk, oi, os, hist, scan_sh,
                                 ctl);
    for (int i = (int)kk + threadIdx.x; i < k; i += kFinNT) {
      oi[i] = -1;
      if (os) os[i] = -INFINITY;
    }
    return;
  }
  const int tot = pre[nb];
  // the survivors, region by region into LDS in concatenation (ascending index)
  // order: wave w copies regions w, w + 16, ..., each with coalesced reads.  The
  // first 64 survivors of four regions are loaded before any is stored (one
  // memory round trip for the usual region sizes); longer regions finish in a loop
  constexpr int NWF = kFinNT / kWave, RB = 4;
  for (int j0 = w; j0 < nb; j0 += RB * NWF) {
    int c0[RB], c[RB];
    uint32_t kv[RB];
    int32_t iv[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int j = j0 + i * NWF;
      c0[i] = j < nb ? pre[j] : 0;
      c[i] = j < nb ? pre[j + 1] - c0[i] : 0;
      const int64_t base = ((int64_t)r * nb + j) * kMbS;
      if (l < c[i]) {
        kv[i] = rkey[base + l];
        iv[i] = ridx[base + l];
      }
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (l < c[i]) {
        skey[c0[i] + l] = kv[i];
        sidx[c0[i] + l] = iv[i];
      }
      const int64_t base = ((int64_t)r * nb + j0 + i * NWF) * kMbS;
      for (int o = kWave + l; o < c[i]; o += kWave) {
        skey[c0[i] + o] = rkey[base + o];
        sidx[c0[i] + o] = ridx[base + o];
      }
    }
  }
  __syncthreads();
  // V survivors per thread in element order (wave, group, lane, element); up to
  // kFinNT * 4 of them (the common case) take the narrow form, whose passes touch
  // a quarter of the slots
  auto select = [&](auto vtag) __attribute__((always_inline)) {
    constexpr int V = decltype(vtag)::value, NV = V / 4;
    uint32_t key[V];
    int32_t idx[V];
    bool valid[V];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e0 = w * 64 * V + (i * 64 + l) * 4;
      const u32x4 kv = e0 < tot ? *reinterpret_cast<const u32x4*>(&skey[e0]) : u32x4{0u, 0u, 0u, 0u};
      const i32x4 iv = e0 < tot ? *reinterpret_cast<const i32x4*>(&sidx[e0]) : i32x4{-1, -1, -1, -1};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int v = 4 * i + jj;
        valid[v] = e0 + jj < tot;
        key[v] = valid[v] ? kv[jj] : 0u;
        idx[v] = valid[v] ? iv[jj] : -1;
      }
    }
    select_ordered<kFinNT, V>(key, idx, valid, (uint32_t)tot, kk, oi, os, k, hist, scan_sh, ctl, b + 1, above);
  };
  if (tot <= kFinNT * 4) select(std::integral_constant<int, 4>{});
  else select(std::integral_constant<int, kFinV>{});
}

__global__ __launch_bounds__(kMbNT) void topk_filter(const float* __restrict__ scores, int64_t stride,
                                                     TopkRows rows, int k, int nb,
                                                     const uint32_t* __restrict__ ghist, int32_t* __restrict__ cnt,
                                                     uint32_t* __restrict__ rkey, int32_t* __restrict__ ridx) {
  constexpr int NI = kMbV / 4;
  __shared__ uint32_t scan_sh[kMbNT / kWave + 1];
  __shared__ uint32_t ctl[4];
  const int r = blockIdx.y;
  const int64_t base = (int64_t)blockIdx.x * kMbS;
  const int64_t slot = (int64_t)r * nb + blockIdx.x;
  int64_t len = row_visible(rows, r) - base;
  len = len < 0 ? 0 : (len > kMbS ? kMbS : len);
  // the block's scores do not depend on the threshold bin: their loads and the
  // histogram's are in flight together
  float sc[kMbV];
  if (len > 0) load_part<kMbV>(scores + (int64_t)r * stride + base, len, (int64_t)wave_id() * 64 * kMbV, sc);
  row_threshold_bin<kMbNT>(ghist + (int64_t)r * kBins, k, scan_sh, ctl);
  const uint32_t b = ctl[0], above = ctl[1];
  if (len == 0) {
    if (threadIdx.x == 0) cnt[slot] = 0;
  } else if (above + ctl[2] > (uint32_t)kFinCap) {      // too many survivors: the final block streams the row
    if (threadIdx.x == 0) cnt[slot] = -1;
  } else {
    uint32_t key[kMbV];
    int32_t idx[kMbV];
    bool valid[kMbV];
    part_keys<kMbV>(sc, len, base, key, idx, valid);
    bool keep[kMbV];
    uint32_t c[NI], off[NI], tot;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      c[i] = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = 4 * i + j;
        keep[v] = valid[v] && (key[v] >> 20) >= b;
        c[i] += keep[v] ? 1u : 0u;
      }
    }
    ordered_scan<kMbNT, NI>(c, off, scan_sh, &tot);
    uint32_t* ok = rkey + slot * kMbS;
    int32_t* oi = ridx + slot * kMbS;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      uint32_t o = off[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = 4 * i + j;
        if (keep[v]) {
          ok[o] = key[v];
          oi[o] = idx[v];
          ++o;
        }
      }
    }
    if (threadIdx.x == 0) cnt[slot] = (int32_t)tot;
  }
}

__global__ __launch_bounds__(kFinNT) void topk_final(const float* __restrict__ scores, int64_t stride, TopkRows rows,
                                                    int k, int nb, const uint32_t* __restrict__ ghist,
                                                    const int32_t* __restrict__ cnt, const uint32_t* __restrict__ rkey,
                                                    const int32_t* __restrict__ ridx, int32_t* __restrict__ out_idx,
                                                    float* __restrict__ out_score) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scan_sh[kFinNT / kWave + 1];
  __shared__ uint32_t ctl[4];
  __shared__ int32_t pre[kMbMaxBlocks + 1];
  __shared__ int32_t flag;
  __shared__ __attribute__((aligned(16))) uint32_t skey[kFinCap];
  __shared__ __attribute__((aligned(16))) int32_t sidx[kFinCap];
  const int r = blockIdx.y;
  // the filter blocks' survivor counts, in flight with the histogram's loads
  const int32_t my = (int)threadIdx.x < nb ? cnt[(int64_t)r * nb + threadIdx.x] : 0;
  row_threshold_bin<kFinNT>(ghist + (int64_t)r * kBins, k, scan_sh, ctl);
  const uint32_t b = ctl[0], above = ctl[1], n_valid = ctl[3];
  topk_row_final(scores, stride, rows, r, k, nb, cnt, rkey, ridx, b, above, n_valid, out_idx, out_score, hist,
                 scan_sh, ctl, pre, &flag, skey, sidx, my);
}

static const int kCfg[][2] = {{256, 4}, {256, 16}, {256, 32}, {1024, 16}, {1024, 32}, {1024, 64}};

static size_t align16(size_t n) { return (n + 15) / 16 * 16; }
// many-block workspace: histograms [R][kBins], then block counts [R][nb], then
// survivor keys and indices [R][nb][kMbS] each
static size_t mb_cnt_offset(int R) { return align16((size_t)R * kBins * 4); }

TopkPlan plan_topk(int64_t cover, int32_t k, int32_t R) {
  TopkPlan p;
  p.cover = cover;
  // few rows too long for one block: spread each row over many blocks
  const int64_t nb = (cover + kMbS - 1) / kMbS;
  if (R <= 64 && cover > 1024 * 32 && nb <= kMbMaxBlocks && k <= kFinCap) {
    p.mb_blocks = (int)nb;
    p.ws_bytes = mb_cnt_offset(R) + align16((size_t)R * nb * 4) + (size_t)R * nb * kMbS * 8 + 256;
    p.ok = true;
    return p;
  }
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

int topk_hist_words(const TopkPlan& p) { return p.mb_blocks ? kBins : 0; }

hipError_t launch_topk(const sckv_index_args& a, const float* scores, int64_t stride, const TopkPlan& p,
                       void* ws, hipStream_t stream, bool hist_zeroed) {
  TopkRows rr{a.rows.kind, a.rows.pos, a.rows.pos_max, a.rows.seq0, a.rows.pos0, a.m, a.W, a.E_cap};
  const int R = a.rows.R;
  if (p.mb_blocks) {
    const int nb = p.mb_blocks;
    char* w = static_cast<char*>(ws);
    uint32_t* hist = reinterpret_cast<uint32_t*>(w);                    // [R][kBins]
    int32_t* cnt = reinterpret_cast<int32_t*>(w + mb_cnt_offset(R));
    uint32_t* rkey = reinterpret_cast<uint32_t*>(w + mb_cnt_offset(R) + align16((size_t)R * nb * 4));
    int32_t* ridx = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(rkey) + (size_t)R * nb * kMbS * 4);
    const int64_t nz = (int64_t)R * kBins;
    if (!hist_zeroed)
      hipLaunchKernelGGL(topk_zero_hist, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, stream, hist, nz);
    hipLaunchKernelGGL(topk_hist, dim3((unsigned)nb, R), dim3(kMbNT), 0, stream, scores, stride, rr, hist);
    hipLaunchKernelGGL(topk_filter, dim3((unsigned)nb, R), dim3(kMbNT), 0, stream, scores, stride, rr, a.k, nb, hist,
                       cnt, rkey, ridx);
    hipLaunchKernelGGL(topk_final, dim3(1, R), dim3(kFinNT), 0, stream, scores, stride, rr, a.k, nb, hist, cnt, rkey,
                       ridx, a.out_idx, a.out_score);
    return hipGetLastError();
  }
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
