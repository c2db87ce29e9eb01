// C ABI entry points: validation, workspace sizing and kernel dispatch.
// Every argument is checked before the first HIP call, so a failing status
// never leaves work enqueued (and the checks run on machines without a GPU).
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "sckv_internal.h"

// Scratch of csa_index_topk_noalloc: the score matrix and the top-k workspace of
// one call, held for the life of the process on every device the library runs
// on.  In host code `scratch` names a host-side stand-in, never the device
// memory: host code only uses the address hipGetSymbolAddress returns for the
// current device.
static __device__ __align__(256) uint8_t scratch[SCKV_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

sckv_status fail(sckv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

sckv_status ok() {
  g_err[0] = 0;
  return SCKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2_dim(int32_t D) {
  return D == 8 || D == 16 || D == 32 || D == 64 || D == 128 || D == 256 || D == 512;
}

const char* dtname(int32_t d) {
  switch (d) {
    case SCKV_F32: return "F32";
    case SCKV_BF16: return "BF16";
    case SCKV_E4M3: return "E4M3";
    case SCKV_MXFP4: return "MXFP4";
    default: return "?";
  }
}

sckv_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SCKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Device address of `scratch` on the current device, looked up once per device
// (each device holds its own copy of the array).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------- compression
sckv_status check_pool(const sckv_pool_stream* s, const char* name, int32_t B, int64_t N, int32_t m,
                       int32_t o, int64_t e_begin, int64_t e_count) {
  if (!s) return fail(SCKV_ERR_NULL, "%s: stream descriptor is NULL", name);
  if (!s->val || !s->gate || !s->bpos || !s->out) return fail(SCKV_ERR_NULL, "%s: val/gate/bpos/out must be set", name);
  if (s->in_dtype != SCKV_F32 && s->in_dtype != SCKV_BF16)
    return fail(SCKV_ERR_DTYPE, "%s: in_dtype %s not supported (F32, BF16)", name, dtname(s->in_dtype));
  if (s->out_dtype != SCKV_F32 && s->out_dtype != SCKV_BF16 && s->out_dtype != SCKV_E4M3 &&
      s->out_dtype != SCKV_MXFP4)
    return fail(SCKV_ERR_DTYPE, "%s: out_dtype %d not supported", name, s->out_dtype);
  if (!pow2_dim(s->D)) return fail(SCKV_ERR_UNSUPPORTED, "%s: D=%d not in {8,...,512} (powers of two)", name, s->D);
  if (s->out_layout != SCKV_LAYOUT_ROWS && s->out_layout != SCKV_LAYOUT_KEY_TILES)
    return fail(SCKV_ERR_SHAPE, "%s: unknown out_layout %d", name, s->out_layout);
  if (s->out_layout == SCKV_LAYOUT_KEY_TILES && s->E_cap % 32 != 0)
    return fail(SCKV_ERR_SHAPE, "%s: key-tile caches need E_cap %% 32 == 0 (E_cap=%lld)", name, (long long)s->E_cap);
  if (s->out_dtype == SCKV_MXFP4 && (s->out_layout != SCKV_LAYOUT_KEY_TILES || s->D < 32 || s->out_scale))
    return fail(SCKV_ERR_UNSUPPORTED, "%s: MXFP4 keys need the key-tile layout, D >= 32 and no out_scale", name);
  if (B < 1 || N < 1 || m < 1 || o < 0) return fail(SCKV_ERR_SHAPE, "%s: need B>=1, N>=1, m>=1, o>=0", name);
  if (e_begin < 0 || e_count < 0) return fail(SCKV_ERR_SHAPE, "%s: e_begin/e_count must be >= 0", name);
  if ((int64_t)m * (e_begin + e_count) > N)
    return fail(SCKV_ERR_SHAPE, "%s: entries up to %lld need %lld tokens, N=%lld", name,
                (long long)(e_begin + e_count), (long long)m * (e_begin + e_count), (long long)N);
  if (s->E_cap < e_begin + e_count)
    return fail(SCKV_ERR_SHAPE, "%s: E_cap=%lld < e_begin+e_count=%lld", name, (long long)s->E_cap,
                (long long)(e_begin + e_count));
  if (!aligned16(s->val) || !aligned16(s->gate) || !aligned16(s->bpos) || !aligned16(s->out) ||
      (s->out_scale && !aligned16(s->out_scale)))
    return fail(SCKV_ERR_ALIGN, "%s: tensors must be 16-byte aligned", name);
  return SCKV_OK;
}

// ---------------------------------------------------------------- decode append
sckv_status check_append(const sckv_append_stream* s, const char* name, int32_t B, int32_t m, int32_t o) {
  if (!s) return fail(SCKV_ERR_NULL, "%s: stream descriptor is NULL", name);
  if (!s->pos || !s->val || !s->gate || !s->val_ring || !s->gate_ring || !s->bpos || !s->out)
    return fail(SCKV_ERR_NULL, "%s: pos/val/gate/val_ring/gate_ring/bpos/out must be set", name);
  if (s->in_dtype != SCKV_F32 && s->in_dtype != SCKV_BF16)
    return fail(SCKV_ERR_DTYPE, "%s: in_dtype %s not supported (F32, BF16)", name, dtname(s->in_dtype));
  if (s->out_dtype != SCKV_F32 && s->out_dtype != SCKV_BF16 && s->out_dtype != SCKV_E4M3 &&
      s->out_dtype != SCKV_MXFP4)
    return fail(SCKV_ERR_DTYPE, "%s: out_dtype %d not supported", name, s->out_dtype);
  if (!pow2_dim(s->D)) return fail(SCKV_ERR_UNSUPPORTED, "%s: D=%d not in {8,...,512} (powers of two)", name, s->D);
  if (s->out_layout != SCKV_LAYOUT_ROWS && s->out_layout != SCKV_LAYOUT_KEY_TILES)
    return fail(SCKV_ERR_SHAPE, "%s: unknown out_layout %d", name, s->out_layout);
  if (s->out_layout == SCKV_LAYOUT_KEY_TILES && s->E_cap % 32 != 0)
    return fail(SCKV_ERR_SHAPE, "%s: key-tile caches need E_cap %% 32 == 0 (E_cap=%lld)", name, (long long)s->E_cap);
  if (s->out_dtype == SCKV_MXFP4 && (s->out_layout != SCKV_LAYOUT_KEY_TILES || s->D < 32 || s->out_scale))
    return fail(SCKV_ERR_UNSUPPORTED, "%s: MXFP4 keys need the key-tile layout, D >= 32 and no out_scale", name);
  if (B < 1 || m < 1 || o < 0 || s->E_cap < 1) return fail(SCKV_ERR_SHAPE, "%s: need B>=1, m>=1, o>=0, E_cap>=1", name);
  if ((int64_t)s->P < (int64_t)m + o)
    return fail(SCKV_ERR_SHAPE, "%s: P=%d ring slots < m+o=%d tokens of an entry", name, s->P, m + o);
  if (!aligned16(s->val) || !aligned16(s->gate) || !aligned16(s->val_ring) || !aligned16(s->gate_ring) ||
      !aligned16(s->bpos) || !aligned16(s->out) || (s->out_scale && !aligned16(s->out_scale)))
    return fail(SCKV_ERR_ALIGN, "%s: tensors must be 16-byte aligned", name);
  return SCKV_OK;
}

// ---------------------------------------------------------------- rows
sckv_status check_rows(const sckv_rows& r, int32_t B, const char* name) {
  if (r.R < 1) return fail(SCKV_ERR_SHAPE, "%s: rows.R=%d must be >= 1", name, r.R);
  if (r.kind == SCKV_ROWS_DECODE) {
    if (!r.pos) return fail(SCKV_ERR_NULL, "%s: decode rows need pos[]", name);
    if (r.R > B) return fail(SCKV_ERR_SHAPE, "%s: decode rows R=%d > B=%d", name, r.R, B);
    if (r.pos_max < 0) return fail(SCKV_ERR_SHAPE, "%s: pos_max must be >= 0", name);
  } else if (r.kind == SCKV_ROWS_CAUSAL) {
    if (r.seq0 < 0 || r.seq0 >= B) return fail(SCKV_ERR_SHAPE, "%s: seq0=%d outside [0,%d)", name, r.seq0, B);
    if (r.pos0 < 0 || (int64_t)r.pos0 + r.R - 1 > INT32_MAX) return fail(SCKV_ERR_SHAPE, "%s: bad pos0", name);
  } else {
    return fail(SCKV_ERR_SHAPE, "%s: unknown rows.kind %d", name, r.kind);
  }
  return SCKV_OK;
}

// ---------------------------------------------------------------- indexer
struct IndexPlan {
  int64_t cover = 0, stride = 0;
  sckv::TopkPlan topk;
  size_t ws_scores = 0, ws_total = 0;
};

sckv_status check_index(const sckv_index_args* a, IndexPlan* pl, bool need_out) {
  if (!a) return fail(SCKV_ERR_NULL, "index: args is NULL");
  if (a->B < 1) return fail(SCKV_ERR_SHAPE, "index: B must be >= 1");
  sckv_status s = check_rows(a->rows, a->B, "index");
  if (s != SCKV_OK) return s;
  if (!a->q || !a->w || !a->keys) return fail(SCKV_ERR_NULL, "index: q, w and keys must be set");
  if (need_out && !a->out_idx) return fail(SCKV_ERR_NULL, "index: out_idx must be set");
  if (a->k < 1) return fail(SCKV_ERR_SHAPE, "index: k=%d must be >= 1", a->k);
  if (a->m < 1 || a->W < 0 || a->E_cap < 1 || a->H_I < 1 || a->D_I < 1)
    return fail(SCKV_ERR_SHAPE, "index: need m>=1, W>=0, E_cap>=1, H_I>=1, D_I>=1");
  if (a->E_cap % 32 != 0 || a->D_I % 8 != 0)
    return fail(SCKV_ERR_SHAPE, "index: tiled keys need E_cap %% 32 == 0 and D_I %% 8 == 0 (got %lld, %d)",
                (long long)a->E_cap, a->D_I);
  if (a->q_dtype == SCKV_F32 && a->key_dtype == SCKV_F32) {
    if ((int64_t)a->H_I * a->D_I > 8192) return fail(SCKV_ERR_UNSUPPORTED, "index: F32 path needs H_I*D_I <= 8192");
  } else if (a->q_dtype == SCKV_BF16 &&
             (a->key_dtype == SCKV_BF16 || a->key_dtype == SCKV_E4M3 || a->key_dtype == SCKV_MXFP4)) {
    if (!(a->H_I == 32 || a->H_I == 64) || !(a->D_I == 64 || a->D_I == 128))
      return fail(SCKV_ERR_UNSUPPORTED, "index: MFMA path needs H_I in {32,64} and D_I in {64,128} (got %d, %d)",
                  a->H_I, a->D_I);
  } else {
    return fail(SCKV_ERR_DTYPE, "index: q %s with keys %s not supported (F32/F32, BF16/BF16, BF16/E4M3, BF16/MXFP4)",
                dtname(a->q_dtype), dtname(a->key_dtype));
  }
  if (!aligned16(a->q) || !aligned16(a->w) || !aligned16(a->keys) || (a->out_idx && !aligned16(a->out_idx)) ||
      (a->out_score && !aligned16(a->out_score)))
    return fail(SCKV_ERR_ALIGN, "index: tensors must be 16-byte aligned");
  pl->cover = sckv::index_rows_cover(*a);
  pl->stride = ((pl->cover > 0 ? pl->cover : 1) + 63) / 64 * 64;
  pl->topk = sckv::plan_topk(pl->cover, a->k, a->rows.R);
  if (!pl->topk.ok)
    return fail(SCKV_ERR_UNSUPPORTED, "index: top-%d over %lld entries exceeds the selection plan", a->k,
                (long long)pl->cover);
  pl->ws_scores = (size_t)a->rows.R * (size_t)pl->stride * sizeof(float);
  pl->ws_total = pl->ws_scores + pl->topk.ws_bytes;
  return SCKV_OK;
}

// ---------------------------------------------------------------- attention
sckv_status check_attend(const sckv_attend_args* a, bool csa, sckv::AttendPlan* pl) {
  const char* name = csa ? "csa_attend" : "hca_attend";
  if (!a) return fail(SCKV_ERR_NULL, "%s: args is NULL", name);
  if (a->B < 1) return fail(SCKV_ERR_SHAPE, "%s: B must be >= 1", name);
  sckv_status s = check_rows(a->rows, a->B, name);
  if (s != SCKV_OK) return s;
  if (!a->q || !a->entries || !a->win || !a->out) return fail(SCKV_ERR_NULL, "%s: q, entries, win, out must be set", name);
  if (csa && (!a->idx || a->k < 1)) return fail(SCKV_ERR_NULL, "%s: idx must be set and k >= 1", name);
  if (a->entry_dtype == SCKV_E4M3 && !a->entry_scale) return fail(SCKV_ERR_NULL, "%s: E4M3 entries need entry_scale", name);
  if (a->H < 1 || a->D < 1 || a->m < 1 || a->W < 1 || a->E_cap < 1 || a->R_w < a->W)
    return fail(SCKV_ERR_SHAPE, "%s: need H,D,m,W,E_cap >= 1 and R_w >= W", name);
  if (!std::isfinite(a->softmax_scale)) return fail(SCKV_ERR_SHAPE, "%s: softmax_scale must be finite", name);
  if (a->R_w > INT32_MAX || a->E_cap > INT32_MAX)
    return fail(SCKV_ERR_UNSUPPORTED, "%s: R_w and E_cap must fit 31 bits (got %lld, %lld)", name,
                (long long)a->R_w, (long long)a->E_cap);
  if (a->out_dtype != SCKV_F32 && a->out_dtype != SCKV_BF16)
    return fail(SCKV_ERR_DTYPE, "%s: out_dtype %s not supported", name, dtname(a->out_dtype));
  if (a->q_dtype == SCKV_F32 && a->entry_dtype == SCKV_F32 && a->win_dtype == SCKV_F32) {
    if ((int64_t)a->H * a->D > 4096 || a->D > 128)
      return fail(SCKV_ERR_UNSUPPORTED, "%s: F32 path needs H*D <= 4096 and D <= 128", name);
  } else if (a->q_dtype == SCKV_BF16 && (a->entry_dtype == SCKV_BF16 || a->entry_dtype == SCKV_E4M3) &&
             a->win_dtype == SCKV_BF16) {
    if (a->H % 16 != 0 || a->H > 128 || !(a->D == 64 || a->D == 128 || a->D == 256 || a->D == 512))
      return fail(SCKV_ERR_UNSUPPORTED, "%s: MFMA path needs H%%16==0, H<=128, D in {64,128,256,512} (got %d, %d)",
                  name, a->H, a->D);
  } else {
    return fail(SCKV_ERR_DTYPE, "%s: q %s / entries %s / window %s not supported", name, dtname(a->q_dtype),
                dtname(a->entry_dtype), dtname(a->win_dtype));
  }
  if (!aligned16(a->q) || !aligned16(a->entries) || !aligned16(a->win) || !aligned16(a->out) ||
      (a->idx && !aligned16(a->idx)) || (a->entry_scale && !aligned16(a->entry_scale)) ||
      (a->lse && !aligned16(a->lse)))
    return fail(SCKV_ERR_ALIGN, "%s: tensors must be 16-byte aligned", name);
  *pl = sckv::plan_attend(*a, csa);
  if (!pl->ok) return fail(SCKV_ERR_UNSUPPORTED, "%s: no plan", name);
  return SCKV_OK;
}

sckv_status attend_common(const sckv_attend_args* a, bool csa, void* ws, size_t ws_bytes, void* stream) {
  sckv::AttendPlan pl;
  sckv_status s = check_attend(a, csa, &pl);
  if (s != SCKV_OK) return s;
  if (pl.ws_bytes && (!ws || ws_bytes < pl.ws_bytes))
    return fail(SCKV_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", csa ? "csa_attend" : "hca_attend",
                pl.ws_bytes, ws ? ws_bytes : (size_t)0);
  if (ws && !aligned16(ws)) return fail(SCKV_ERR_ALIGN, "attend: workspace must be 16-byte aligned");
  return hip_status(sckv::launch_attend(*a, csa, pl, ws, static_cast<hipStream_t>(stream)),
                    csa ? "csa_attend" : "hca_attend");
}

// ---------------------------------------------------------------- projections
bool out_dtype_ok(int32_t d) { return d == SCKV_F32 || d == SCKV_BF16; }

sckv_status check_reduce_len(int64_t K, const char* name, const char* what) {
  if (K < 128 || K % 128) return fail(SCKV_ERR_UNSUPPORTED, "%s: %s=%lld must be a positive multiple of 128", name, what,
                                      (long long)K);
  if (K > (1 << 20)) return fail(SCKV_ERR_UNSUPPORTED, "%s: %s=%lld exceeds 2^20", name, what, (long long)K);
  return SCKV_OK;
}

sckv_status check_queries(const sckv_query_args* a, size_t* ws) {
  const char* name = "layer_queries";
  if (!a) return fail(SCKV_ERR_NULL, "%s: args is NULL", name);
  if (!a->x || !a->W_q || !a->q) return fail(SCKV_ERR_NULL, "%s: x, W_q and q must be set", name);
  if ((a->W_iq && !a->qI) || (a->W_w && !a->w)) return fail(SCKV_ERR_NULL, "%s: W_iq needs qI and W_w needs w", name);
  if (a->R < 1 || a->R > (1 << 21)) return fail(SCKV_ERR_SHAPE, "%s: R=%d outside [1,2^21]", name, a->R);
  if (a->H < 1 || a->d_h < 1 || a->D < 1) return fail(SCKV_ERR_SHAPE, "%s: need H, d_h, D >= 1", name);
  if ((int64_t)a->H * a->d_h > (1 << 20)) return fail(SCKV_ERR_UNSUPPORTED, "%s: H*d_h exceeds 2^20", name);
  if ((a->W_iq || a->W_w) && (a->H_I < 1 || a->D_I < 1 || (int64_t)a->H_I * a->D_I > (1 << 20)))
    return fail(SCKV_ERR_SHAPE, "%s: indexer needs 1 <= H_I, D_I and H_I*D_I <= 2^20", name);
  sckv_status s = check_reduce_len(a->d_model, name, "d_model");
  if (s != SCKV_OK) return s;
  if (!out_dtype_ok(a->q_dtype)) return fail(SCKV_ERR_DTYPE, "%s: q_dtype %s not supported (F32, BF16)", name,
                                             dtname(a->q_dtype));
  if (a->W_UK) {
    if (a->D % 128 || a->D > 4096 || (a->d_h != 64 && a->d_h != 128 && a->d_h != 256))
      return fail(SCKV_ERR_UNSUPPORTED,
                  "%s: absorption needs D %% 128 == 0 (D <= 4096) and d_h in {64, 128, 256} (got %d, %d)", name, a->D,
                  a->d_h);
  } else if (a->D != a->d_h) {
    return fail(SCKV_ERR_SHAPE, "%s: without W_UK the latent D=%d must equal d_h=%d", name, a->D, a->d_h);
  }
  if (!aligned16(a->x) || !aligned16(a->W_q) || !aligned16(a->q) || (a->W_UK && !aligned16(a->W_UK)) ||
      (a->W_iq && (!aligned16(a->W_iq) || !aligned16(a->qI))) || (a->W_w && (!aligned16(a->W_w) || !aligned16(a->w))))
    return fail(SCKV_ERR_ALIGN, "%s: tensors must be 16-byte aligned", name);
  *ws = sckv::queries_workspace(*a);
  return ok();
}

sckv_status check_streams(const sckv_stream_args* a, size_t* ws) {
  const char* name = "layer_streams";
  if (!a) return fail(SCKV_ERR_NULL, "%s: args is NULL", name);
  if (!a->x) return fail(SCKV_ERR_NULL, "%s: x must be set", name);
  if ((a->W_c && !a->v) || (a->W_g && !a->g) || (a->W_cI && !a->vI) || (a->W_gI && !a->gI))
    return fail(SCKV_ERR_NULL, "%s: every weight given needs its output", name);
  if (a->R < 1 || a->R > (1 << 21)) return fail(SCKV_ERR_SHAPE, "%s: R=%d outside [1,2^21]", name, a->R);
  if ((a->W_c || a->W_g) && (a->D < 1 || a->D > (1 << 20))) return fail(SCKV_ERR_SHAPE, "%s: D=%d", name, a->D);
  if ((a->W_cI || a->W_gI) && (a->D_I < 1 || a->D_I > (1 << 20)))
    return fail(SCKV_ERR_SHAPE, "%s: D_I=%d", name, a->D_I);
  sckv_status s = check_reduce_len(a->d_model, name, "d_model");
  if (s != SCKV_OK) return s;
  if (!out_dtype_ok(a->out_dtype))
    return fail(SCKV_ERR_DTYPE, "%s: out_dtype %s not supported (F32, BF16)", name, dtname(a->out_dtype));
  const void* p[9] = {a->x, a->W_c, a->W_g, a->W_cI, a->W_gI, a->v, a->g, a->vI, a->gI};
  for (const void* q : p)
    if (q && !aligned16(q)) return fail(SCKV_ERR_ALIGN, "%s: tensors must be 16-byte aligned", name);
  *ws = sckv::streams_workspace(*a);
  return ok();
}

sckv_status check_output(const sckv_output_args* a, size_t* ws) {
  const char* name = "layer_output";
  if (!a) return fail(SCKV_ERR_NULL, "%s: args is NULL", name);
  if (!a->o || !a->W_o || !a->y) return fail(SCKV_ERR_NULL, "%s: o, W_o and y must be set", name);
  if (a->R < 1 || a->R > (1 << 21)) return fail(SCKV_ERR_SHAPE, "%s: R=%d outside [1,2^21]", name, a->R);
  if (a->H < 1 || a->d_h < 1 || a->D < 1 || a->d_model < 1 || a->d_model > (1 << 20))
    return fail(SCKV_ERR_SHAPE, "%s: need H, d_h, D, d_model >= 1 (d_model <= 2^20)", name);
  sckv_status s = check_reduce_len((int64_t)a->H * a->d_h, name, "H*d_h");
  if (s != SCKV_OK) return s;
  if (a->W_UV) {
    s = check_reduce_len(a->D, name, "D");
    if (s != SCKV_OK) return s;
  } else if (a->D != a->d_h) {
    return fail(SCKV_ERR_SHAPE, "%s: without W_UV the latent D=%d must equal d_h=%d", name, a->D, a->d_h);
  }
  if (!out_dtype_ok(a->y_dtype))
    return fail(SCKV_ERR_DTYPE, "%s: y_dtype %s not supported (F32, BF16)", name, dtname(a->y_dtype));
  if (!aligned16(a->o) || !aligned16(a->W_o) || !aligned16(a->y) || (a->W_UV && !aligned16(a->W_UV)))
    return fail(SCKV_ERR_ALIGN, "%s: tensors must be 16-byte aligned", name);
  *ws = sckv::output_workspace(*a);
  return ok();
}

sckv_status check_inputs(const sckv_query_args* q, const sckv_stream_args* st, size_t* ws) {
  size_t w1 = 0, w2 = 0;
  sckv_status s = check_queries(q, &w1);
  if (s == SCKV_OK) s = check_streams(st, &w2);
  if (s != SCKV_OK) return s;
  if (q->x != st->x || q->R != st->R || q->d_model != st->d_model)
    return fail(SCKV_ERR_SHAPE, "layer_inputs: queries and streams must share x, R and d_model");
  *ws = sckv::inputs_workspace(*q, *st);
  return ok();
}

sckv_status check_ws(const char* name, size_t need, const void* ws, size_t ws_bytes) {
  if (need && (!ws || ws_bytes < need))
    return fail(SCKV_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", name, need,
                ws ? ws_bytes : (size_t)0);
  if (ws && !aligned16(ws)) return fail(SCKV_ERR_ALIGN, "%s: workspace must be 16-byte aligned", name);
  return SCKV_OK;
}

}  // namespace

extern "C" {

sckv_status csa_compress(int32_t B, int64_t N, int32_t m, int32_t o, int64_t e_begin, int64_t e_count,
                         const sckv_pool_stream* kv, const sckv_pool_stream* index_keys, void* stream) {
  sckv_status s = check_pool(kv, "csa_compress(kv)", B, N, m, o, e_begin, e_count);
  if (s != SCKV_OK) return s;
  if (index_keys) {
    s = check_pool(index_keys, "csa_compress(index_keys)", B, N, m, o, e_begin, e_count);
    if (s != SCKV_OK) return s;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = index_keys ? sckv::launch_compress_pair(*kv, *index_keys, B, N, m, o, e_begin, e_count, st)
                                   : sckv::launch_compress(*kv, B, N, m, o, e_begin, e_count, st);
  return hip_status(e, "csa_compress");
}

sckv_status hca_compress(int32_t B, int64_t N, int32_t m, int32_t o, int64_t e_begin, int64_t e_count,
                         const sckv_pool_stream* kv, void* stream) {
  sckv_status s = check_pool(kv, "hca_compress", B, N, m, o, e_begin, e_count);
  if (s != SCKV_OK) return s;
  return hip_status(sckv::launch_compress(*kv, B, N, m, o, e_begin, e_count, static_cast<hipStream_t>(stream)),
                    "hca_compress");
}

sckv_status csa_append(int32_t B, int32_t m, int32_t o, const sckv_append_stream* kv,
                       const sckv_append_stream* index_keys, void* stream) {
  sckv_status s = check_append(kv, "csa_append(kv)", B, m, o);
  if (s != SCKV_OK) return s;
  if (index_keys) {
    s = check_append(index_keys, "csa_append(index_keys)", B, m, o);
    if (s != SCKV_OK) return s;
  }
  return hip_status(sckv::launch_append(*kv, index_keys, B, m, o, static_cast<hipStream_t>(stream)), "csa_append");
}

sckv_status hca_append(int32_t B, int32_t m, int32_t o, const sckv_append_stream* kv, void* stream) {
  sckv_status s = check_append(kv, "hca_append", B, m, o);
  if (s != SCKV_OK) return s;
  return hip_status(sckv::launch_append(*kv, nullptr, B, m, o, static_cast<hipStream_t>(stream)), "hca_append");
}

size_t csa_index_topk_workspace_size(const sckv_index_args* a) {
  IndexPlan pl;
  if (check_index(a, &pl, false) != SCKV_OK) return 0;
  return pl.ws_total;
}

size_t csa_topk_select_workspace_size(const sckv_index_args* a) {
  IndexPlan pl;
  if (check_index(a, &pl, false) != SCKV_OK) return 0;
  return pl.topk.ws_bytes;
}

// Scores into the workspace, then the top-k; the scoring kernel clears the
// many-block top-k's histograms on its way (one launch fewer).
static hipError_t index_then_topk(const sckv_index_args& a, const IndexPlan& pl, void* ws, hipStream_t st) {
  float* scores = static_cast<float*>(ws);
  void* tws = static_cast<char*>(ws) + pl.ws_scores;
  bool zeroed = false;
  hipError_t e = sckv::launch_index_score(a, scores, pl.stride, pl.cover, st, static_cast<uint32_t*>(tws),
                                          sckv::topk_hist_words(pl.topk), &zeroed);
  if (e == hipSuccess) e = sckv::launch_topk(a, scores, pl.stride, pl.topk, tws, st, zeroed);
  return e;
}

sckv_status csa_index_topk(const sckv_index_args* a, void* ws, size_t ws_bytes, void* stream) {
  IndexPlan pl;
  sckv_status s = check_index(a, &pl, true);
  if (s != SCKV_OK) return s;
  if (!ws || ws_bytes < pl.ws_total)
    return fail(SCKV_ERR_WORKSPACE, "csa_index_topk: workspace of %zu bytes needed, %zu given", pl.ws_total,
                ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(SCKV_ERR_ALIGN, "csa_index_topk: workspace must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(index_then_topk(*a, pl, ws, st), "csa_index_topk");
}

sckv_status csa_index_topk_noalloc(const sckv_index_args* a, void* stream) {
  IndexPlan pl;
  sckv_status s = check_index(a, &pl, true);
  if (s != SCKV_OK) return s;
  if (pl.ws_total > (size_t)SCKV_NOALLOC_SCRATCH_BYTES)
    return fail(SCKV_ERR_WORKSPACE,
                "csa_index_topk_noalloc: these rows need %zu bytes of scratch, the static buffer holds %zu; "
                "call csa_index_topk with a workspace instead", pl.ws_total, (size_t)SCKV_NOALLOC_SCRATCH_BYTES);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "csa_index_topk_noalloc");
  if (st) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(st, &sdev);
    if (e != hipSuccess) return hip_status(e, "csa_index_topk_noalloc");
    if ((int)sdev != dev)
      return fail(SCKV_ERR_UNSUPPORTED, "csa_index_topk_noalloc: the stream belongs to device %d, current device is %d",
                  (int)sdev, dev);
  }
  void* ws = nullptr;
  e = scratch_address(dev, &ws);
  if (e != hipSuccess) return hip_status(e, "csa_index_topk_noalloc (scratch address)");
  return hip_status(index_then_topk(*a, pl, ws, st), "csa_index_topk_noalloc");
}

sckv_status csa_index_score(const sckv_index_args* a, float* scores, int64_t score_stride, void* stream) {
  IndexPlan pl;
  sckv_status s = check_index(a, &pl, false);
  if (s != SCKV_OK) return s;
  if (!scores) return fail(SCKV_ERR_NULL, "csa_index_score: scores must be set");
  if (score_stride < pl.cover)
    return fail(SCKV_ERR_SHAPE, "csa_index_score: score_stride %lld < %lld visible entries", (long long)score_stride,
                (long long)pl.cover);
  return hip_status(sckv::launch_index_score(*a, scores, score_stride, pl.cover, static_cast<hipStream_t>(stream)),
                    "csa_index_score");
}

sckv_status csa_topk_select(const sckv_index_args* a, const float* scores, int64_t score_stride, void* ws,
                            size_t ws_bytes, void* stream) {
  IndexPlan pl;
  sckv_status s = check_index(a, &pl, true);
  if (s != SCKV_OK) return s;
  if (!scores) return fail(SCKV_ERR_NULL, "csa_topk_select: scores must be set");
  if (score_stride < pl.cover)
    return fail(SCKV_ERR_SHAPE, "csa_topk_select: score_stride %lld < %lld visible entries", (long long)score_stride,
                (long long)pl.cover);
  if (pl.topk.ws_bytes && (!ws || ws_bytes < pl.topk.ws_bytes))
    return fail(SCKV_ERR_WORKSPACE, "csa_topk_select: workspace of %zu bytes needed, %zu given", pl.topk.ws_bytes,
                ws ? ws_bytes : (size_t)0);
  if (ws && !aligned16(ws)) return fail(SCKV_ERR_ALIGN, "csa_topk_select: workspace must be 16-byte aligned");
  return hip_status(sckv::launch_topk(*a, scores, score_stride, pl.topk, ws, static_cast<hipStream_t>(stream)),
                    "csa_topk_select");
}

size_t csa_attend_workspace_size(const sckv_attend_args* a) {
  sckv::AttendPlan pl;
  if (check_attend(a, true, &pl) != SCKV_OK) return 0;
  return pl.ws_bytes;
}

size_t hca_attend_workspace_size(const sckv_attend_args* a) {
  sckv::AttendPlan pl;
  if (check_attend(a, false, &pl) != SCKV_OK) return 0;
  return pl.ws_bytes;
}

sckv_status csa_attend(const sckv_attend_args* a, void* ws, size_t ws_bytes, void* stream) {
  return attend_common(a, true, ws, ws_bytes, stream);
}

sckv_status hca_attend(const sckv_attend_args* a, void* ws, size_t ws_bytes, void* stream) {
  return attend_common(a, false, ws, ws_bytes, stream);
}

size_t layer_queries_workspace_size(const sckv_query_args* a) {
  size_t ws = 0;
  return check_queries(a, &ws) == SCKV_OK ? ws : 0;
}

sckv_status layer_queries(const sckv_query_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  sckv_status s = check_queries(a, &need);
  if (s == SCKV_OK) s = check_ws("layer_queries", need, ws, ws_bytes);
  if (s != SCKV_OK) return s;
  return hip_status(sckv::launch_layer_queries(*a, ws, static_cast<hipStream_t>(stream)), "layer_queries");
}

size_t layer_streams_workspace_size(const sckv_stream_args* a) {
  size_t ws = 0;
  return check_streams(a, &ws) == SCKV_OK ? ws : 0;
}

sckv_status layer_streams(const sckv_stream_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  sckv_status s = check_streams(a, &need);
  if (s == SCKV_OK) s = check_ws("layer_streams", need, ws, ws_bytes);
  if (s != SCKV_OK) return s;
  return hip_status(sckv::launch_layer_streams(*a, ws, static_cast<hipStream_t>(stream)), "layer_streams");
}

size_t layer_inputs_workspace_size(const sckv_query_args* q, const sckv_stream_args* st) {
  size_t ws = 0;
  return check_inputs(q, st, &ws) == SCKV_OK ? ws : 0;
}

sckv_status layer_inputs(const sckv_query_args* q, const sckv_stream_args* st, void* ws, size_t ws_bytes,
                         void* stream) {
  size_t need = 0;
  sckv_status s = check_inputs(q, st, &need);
  if (s == SCKV_OK) s = check_ws("layer_inputs", need, ws, ws_bytes);
  if (s != SCKV_OK) return s;
  return hip_status(sckv::launch_layer_inputs(*q, *st, ws, static_cast<hipStream_t>(stream)), "layer_inputs");
}

size_t layer_output_workspace_size(const sckv_output_args* a) {
  size_t ws = 0;
  return check_output(a, &ws) == SCKV_OK ? ws : 0;
}

sckv_status layer_output(const sckv_output_args* a, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  sckv_status s = check_output(a, &need);
  if (s == SCKV_OK) s = check_ws("layer_output", need, ws, ws_bytes);
  if (s != SCKV_OK) return s;
  return hip_status(sckv::launch_layer_output(*a, ws, static_cast<hipStream_t>(stream)), "layer_output");
}

const char* sckv_last_error(void) { return g_err; }

int32_t sckv_abi_version(void) { return SCKV_ABI_VERSION; }

}  // extern "C"
