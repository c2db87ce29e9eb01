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
// Decode append of one stream, or of two streams (s2 non-NULL) over the same positions.
hipError_t launch_append(const sckv_append_stream& s, const sckv_append_stream* s2, int32_t B, int32_t m, int32_t o,
                         hipStream_t stream);

// ---------------------------------------------------------------- indexer
// Largest visible-entry count over the rows (the score matrix width needed).
int64_t index_rows_cover(const sckv_index_args& a);
hipError_t launch_index_score(const sckv_index_args& a, float* scores, int64_t stride,
                              int64_t cover, hipStream_t stream);

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
hipError_t launch_topk(const sckv_index_args& a, const float* scores, int64_t stride,
                       const TopkPlan& p, void* ws, hipStream_t stream);

// ---------------------------------------------------------------- attention
struct AttendPlan {
  int64_t items = 0;        // widest row: listed/visible entries + window
  int64_t chunks = 0;       // items / 64 rounded up
  int64_t per_split = 0;    // items per split (a multiple of 64)
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
// Arguments are validated; ws holds R * H * d_h fp32 (queries, when absorbed) or
// bf16 (output heads, when W_UV is given).
hipError_t launch_layer_queries(const sckv_query_args& a, void* ws, hipStream_t stream);
hipError_t launch_layer_streams(const sckv_stream_args& a, hipStream_t stream);
hipError_t launch_layer_output(const sckv_output_args& a, void* ws, hipStream_t stream);

}  // namespace sckv
