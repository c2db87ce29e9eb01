// Host-side plans and kernel launchers behind the C ABI (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sckv.h"

namespace sckv {

// Entries visible to a query at position t: entry j is usable iff m (j + 1) <= t - W.
inline int64_t entries_visible(int64_t t, int64_t m, int64_t W) {
  const int64_t d = t - W;
  return d < 0 ? 0 : d / m;
}

// ---------------------------------------------------------------- compression
hipError_t launch_compress(const sckv_pool_stream& s, int32_t B, int64_t N, int32_t m, int32_t o,
                           int64_t e_begin, int64_t e_count, hipStream_t stream);
// Both streams of a CSA layer: one launch when they pool overlapping 4:1 windows
// of bf16 input into a supported pair of output types, else one launch each.
hipError_t launch_compress_pair(const sckv_pool_stream& s0, const sckv_pool_stream& s1, int32_t B, int64_t N,
                                int32_t m, int32_t o, int64_t e_begin, int64_t e_count, hipStream_t stream);
// Decode append of one stream, or of two streams (s2 non-NULL) over the same positions.
hipError_t launch_append(const sckv_append_stream& s, const sckv_append_stream* s2, int32_t B, int32_t m, int32_t o,
                         hipStream_t stream);

// ---------------------------------------------------------------- indexer
// Largest visible-entry count over the rows (the score matrix width needed).
int64_t index_rows_cover(const sckv_index_args& a);
// zero_hist (optional): per-row histograms [R][zero_words] that the decode scoring
// kernel clears before it scores (the first block of each row); *zeroed tells
// whether it did (other paths leave them to the top-k launch).
hipError_t launch_index_score(const sckv_index_args& a, float* scores, int64_t stride,
                              int64_t cover, hipStream_t stream, uint32_t* zero_hist = nullptr,
                              int zero_words = 0, bool* zeroed = nullptr);

// Top-k plan: one block per row when the visible count fits a block's registers;
// for a few longer rows, many blocks per row (histogram, filter, final selection
// over the survivors); else a first stage over fixed slices of each row followed
// by a final stage over the slices' candidates.
struct TopkPlan {
  int64_t cover = 0;        // widest row
  int mb_blocks = 0;        // many-block path: blocks per row (0 = not taken)
  int single_nt = 0;        // threads of the one-stage kernel (0 = two stages)
  int single_v = 0;         // values per thread of the one-stage kernel
  int64_t slice = 0;        // two stages: slice length
  int64_t nslices = 0;      // two stages: slices per row
  int64_t cand = 0;         // two stages: candidate capacity per row (nslices * min(k, slice))
  size_t ws_bytes = 0;      // workspace for the candidates
  bool ok = false;
};
TopkPlan plan_topk(int64_t cover, int32_t k, int32_t R);
// The many-block path's per-row histograms at the start of its workspace:
// words per row (0 when the plan does not take that path).
int topk_hist_words(const TopkPlan& p);
// hist_zeroed: the histograms were already cleared on the stream (by the scoring kernel)
hipError_t launch_topk(const sckv_index_args& a, const float* scores, int64_t stride,
                       const TopkPlan& p, void* ws, hipStream_t stream, bool hist_zeroed = false);

// ---------------------------------------------------------------- attention
struct AttendPlan {
  int64_t items = 0;        // widest row: listed/visible entries + window
  int64_t chunks = 0;       // items / split unit (64, or 32 for few rows at D = 512 off LDS-DMA) rounded up
  int64_t per_split = 0;    // items per split (a multiple of the unit)
  int32_t nsplit = 1;
  int32_t hgroups = 1;      // blocks per (row, split), each taking H / hgroups heads
  bool mfma = false;
  size_t ws_bytes = 0;      // split partials (0 when nsplit == 1)
  bool ok = false;
};
AttendPlan plan_attend(const sckv_attend_args& a, bool csa);
hipError_t launch_attend(const sckv_attend_args& a, bool csa, const AttendPlan& p, void* ws,
                         hipStream_t stream);

// ---------------------------------------------------------------- projections
// Plan of one grouped launch of up to 8 products sharing rows x [R][K]: row blocks
// of 16 mt rows, column tiles of 16 nt, nw waves per block; product i takes blocks
// blk0[i] .. and cuts K in splits[i] parts, whose fp32 partial sums (at part_off[i]
// floats of a buffer of part_bytes) a second kernel adds up.
struct LinearPlan {
  bool gemm = false;  // many rows: one tiled GEMM launch per product instead
  int np = 0, mt = 0, nt = 0, nw = 0, u = 1, blocks = 0, row_blocks = 1;
  int splits[8] = {1, 1, 1, 1, 1, 1, 1, 1};
  int blk0[8] = {};
  int64_t part_off[8] = {};
  int64_t e0[8] = {};
  int64_t reduce_elems = 0;
  size_t part_bytes = 0;
};
LinearPlan plan_linear(int R, int K, const int* N, int np, int nbatch);
// Arguments are validated.  Workspaces: the fp32 head queries before absorption
// (or the bf16 heads o_h on the output side) and the partial sums of split launches.
size_t queries_workspace(const sckv_query_args& a);
size_t streams_workspace(const sckv_stream_args& a);
size_t output_workspace(const sckv_output_args& a);
size_t inputs_workspace(const sckv_query_args& a, const sckv_stream_args& st);
hipError_t launch_layer_inputs(const sckv_query_args& a, const sckv_stream_args& st, void* ws, hipStream_t stream);
hipError_t launch_layer_queries(const sckv_query_args& a, void* ws, hipStream_t stream);
hipError_t launch_layer_streams(const sckv_stream_args& a, void* ws, hipStream_t stream);
hipError_t launch_layer_output(const sckv_output_args& a, void* ws, hipStream_t stream);

}  // namespace sckv
