/*
 * sckv.h -- C ABI of the CSA / HCA compressed-attention hot path (gfx950).
 *
 * The method (DeepSeek-V4 hybrid compressed attention):
 *   - CSA pools the KV sequence about 4:1 with a learned gate over overlapping
 *     windows, scores the pooled entries with a lightning indexer, keeps a
 *     per-query top-k and attends to those entries plus a raw recent window
 *     (knightli.com DeepSeek-V4 KV-cache article, section "CSA: compresión 4x
 *     más recuperación dispersa"; kongchang.com "DeepSeek V4 Deep Dive",
 *     "Innovation 1: Hybrid Attention Architecture").
 *   - HCA pools 128:1 and attends densely to every pooled entry plus the window
 *     (same article, "HCA: compresión 128x más atención densa"; bayesiansapien
 *     "DeepSeek-V4: interleaved compressed attention ...", TL;DR).
 *   - Both concatenate the compressed branch with the sliding-window K/V of the
 *     most recent raw tokens in one softmax (same article, "Ventana deslizante").
 *
 * Formulas (the pages leave them open; the CSA decode workload definition fixes them):
 *   compressor  c_j[d] = sum_{i in P_j} softmax_i(g_i[d] + Bpos[i - m j + o][d]) * v_i[d],
 *               P_j = [m j - o, m j + m) restricted to tokens that exist (i >= 0)
 *   visibility  entry j is usable by the query at position t iff m (j + 1) <= t - W,
 *               so E_vis(t) = max(0, floor((t - W) / m)) entries are visible
 *   indexer     s_j = sum_h w_h * max(0, qI_h . kI_j)  over visible j
 *   top-k       the min(k, E_vis) best j by (s_j descending, j ascending)
 *   attention   o_h = sum_u softmax_u(scale * q_h . u) u over
 *               u in {entries kept} U {raw tokens max(0, t-W+1) .. t}; K = V = u
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE memory owned by the caller, dense row-major
 *     in the shapes given, 16-byte aligned.  Nothing is allocated, freed or
 *     synchronised by the library; work is enqueued on `stream` (a hipStream_t,
 *     NULL = the default stream) and the call returns at once.
 *   - Arguments are fully validated on the host before any HIP call; a non-OK
 *     status means nothing was enqueued, and sckv_last_error() (thread-local)
 *     describes the problem.  Faults inside kernels surface at the caller's
 *     next synchronisation.
 *   - Results are deterministic: identical inputs give bitwise identical
 *     outputs (fixed split counts, fixed reduction order, no float atomics).
 *   - Storage types: F32, BF16 (round-to-nearest-even), E4M3 (OCP 8-bit
 *     E4M3 "fn": max 448, saturating round-to-nearest-even).
 *   - Supported shapes: D in {8,16,32,64,128,256,512} for compression;
 *     the MFMA paths need bf16 queries, H % 16 == 0 (H <= 128), D in
 *     {64,128,256,512} for attention and H_I in {32,64}, D_I in {64,128} for
 *     the indexer; the F32 paths accept H*D <= 4096 and H_I*D_I <= 8192.
 *     Other shapes return SCKV_ERR_UNSUPPORTED.
 */
#ifndef SCKV_H
#define SCKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SCKV_ABI_VERSION 1

/* SCKV_MXFP4: FP4 indexer keys.  The pages say only that the CSA lightning
 * indexer uses FP4 (knightli.com DeepSeek-V4 KV-cache article, section "FP8 y FP4
 * reducen aun mas el costo de cache"); the format taken is OCP MXFP4: e2m1
 * elements (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives) in blocks of
 * 32 consecutive channels sharing one E8M0 scale byte s (scale 2^(s - 127)).
 * The compressor sets s - 127 = floor(log2 max|c|) - 2 over the block, clamped to
 * [-127, 127] (-127 for an all-zero block), and rounds c / 2^(s - 127) to e2m1 to
 * nearest, ties to even, saturating at 6.  Layout: see the key tiles below. */
typedef enum { SCKV_F32 = 0, SCKV_BF16 = 1, SCKV_E4M3 = 2, SCKV_MXFP4 = 3 } sckv_dtype;

typedef enum {
  SCKV_OK = 0,
  SCKV_ERR_NULL = 1,        /* a required pointer is NULL */
  SCKV_ERR_SHAPE = 2,       /* a size, count or index argument is out of range */
  SCKV_ERR_DTYPE = 3,       /* unsupported dtype or dtype combination */
  SCKV_ERR_UNSUPPORTED = 4, /* shape outside what the kernels implement */
  SCKV_ERR_ALIGN = 5,       /* a tensor pointer is not 16-byte aligned */
  SCKV_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the size query asks for */
  SCKV_ERR_HIP = 7          /* a kernel launch failed */
} sckv_status;

/* Query rows of an index or attend call.
 *   SCKV_ROWS_DECODE: row r belongs to sequence r (R <= B) and sits at position
 *     pos[r] (device int32 [R]).  pos_max (host) bounds every pos[r]; it sizes the
 *     grid.  Positions outside [0, pos_max] are clamped into it.
 *   SCKV_ROWS_CAUSAL: rows are the consecutive positions pos0 .. pos0 + R - 1 of
 *     sequence seq0 (causal prefill or a chunk of it); pos and pos_max are unused. */
typedef enum { SCKV_ROWS_DECODE = 0, SCKV_ROWS_CAUSAL = 1 } sckv_rows_kind;

typedef struct {
  const int32_t* pos; /* DECODE: device [R] positions; CAUSAL: unused (may be NULL) */
  int32_t kind;       /* sckv_rows_kind */
  int32_t R;          /* number of query rows, >= 1 */
  int32_t pos_max;    /* DECODE: host bound on pos[] */
  int32_t seq0;       /* CAUSAL: sequence of the rows */
  int32_t pos0;       /* CAUSAL: position of row 0 */
  int32_t reserved;
} sckv_rows;

/* ------------------------------------------------------------------ layouts
 * Entry caches (pooled KV entries, raw window) are row-major: [B][E_cap][D].
 * Indexer key caches use a tiled layout built for the MFMA scoring kernel, so
 * that one load instruction of a wavefront reads two contiguous runs of
 * 32 x 8 elements:  [B][E_cap / 32][D_I / 8][32][8], i.e. entry j, dim d of a
 * sequence sits at element ((j / 32 * (D_I / 8) + d / 8) * 32 + j % 32) * 8 + d % 8.
 * E_cap of a key cache must be a multiple of 32.
 * MXFP4 key caches (D_I a multiple of 32) use tiles of their own: per sequence
 * E_cap / 32 tiles of 17 * D_I bytes, each holding the codes [D_I/32][32][16]
 * (block b of key n as 16 bytes: its 32 codes two per byte, the even channel in
 * the low nibble) followed by the scales [32][D_I/32] (one byte per block), i.e.
 * code byte (j/32) * 17 D_I + ((d/32) * 32 + j%32) * 16 + (d%32)/2 and scale byte
 * (j/32) * 17 D_I + 16 D_I + (j%32) * (D_I/32) + d/32. */
typedef enum { SCKV_LAYOUT_ROWS = 0, SCKV_LAYOUT_KEY_TILES = 1 } sckv_layout;

/* ------------------------------------------------------------------ compression
 * One per-token stream pair pooled into entries (the compressor above).
 *   val, gate : [B][N][D] values v_i and gate logits g_i (in_dtype F32 or BF16)
 *   bpos      : [m+o][D] fp32 position bias
 *   out       : entries (out_dtype F32, BF16 or E4M3) in out_layout:
 *               SCKV_LAYOUT_ROWS [B][E_cap][D] or SCKV_LAYOUT_KEY_TILES (see above)
 *   out_scale : E4M3 only.  Non-NULL: [B][E_cap] fp32 per-entry scale, written as
 *               fp32(max_d |c_j[d]| / 448) (1 for an all-zero entry), codes are
 *               E4M3(c / scale).  NULL: unscaled E4M3(c) (indexer keys).
 *   out_dtype SCKV_MXFP4 (indexer keys) needs SCKV_LAYOUT_KEY_TILES, D >= 32 and
 *               out_scale NULL: the block scales sit inside the tiles. */
typedef struct {
  const void* val;
  const void* gate;
  const float* bpos;
  void* out;
  float* out_scale;
  int64_t E_cap;
  int32_t D;
  int32_t in_dtype;
  int32_t out_dtype;
  int32_t out_layout; /* sckv_layout */
} sckv_pool_stream;

/* csa_compress: pools entries e_begin .. e_begin + e_count - 1 of every sequence
 * from tokens of a stream holding N tokens per sequence (rows of val/gate are
 * strided by N).  Entry e needs tokens up to m (e + 1) - 1 < N, and
 * e_begin + e_count <= E_cap.  `kv` is the shared latent stream; `index_keys`
 * (may be NULL) is the lightning indexer's own stream, pooled over the same
 * windows (knightli.com article, CSA section: the indexer scores the pooled
 * blocks); give it out_layout SCKV_LAYOUT_KEY_TILES to feed csa_index_topk.
 * CSA uses m = 4, o = 4; the call accepts any m >= 1, 0 <= o. */
sckv_status csa_compress(int32_t B, int64_t N, int32_t m, int32_t o, int64_t e_begin,
                         int64_t e_count, const sckv_pool_stream* kv,
                         const sckv_pool_stream* index_keys, void* stream);

/* hca_compress: as csa_compress for the single HCA stream (128:1 pooling over
 * non-overlapping blocks: m = 128, o = 0; knightli.com article, HCA section). */
sckv_status hca_compress(int32_t B, int64_t N, int32_t m, int32_t o, int64_t e_begin,
                         int64_t e_count, const sckv_pool_stream* kv, void* stream);

/* ------------------------------------------------------------------ decode append
 * The compressor run incrementally in decode: one new token per sequence is
 * appended to rings of a stream's recent tokens, and where that token completes
 * an entry (one entry per m tokens; knightli.com article, CSA section: a
 * compressed entry stands for m tokens; HCA section for m = 128) the entry is
 * pooled into the cache.
 *   pos       : device [B] int32 position t of each sequence's new token; a
 *               sequence with t < 0 appends nothing
 *   val, gate : [B][D] the new tokens' values and gate logits (in_dtype F32 or BF16)
 *   val_ring, gate_ring : [B][P][D] (in_dtype) the stream's last P tokens, token i
 *               at slot i mod P; the call writes token t's slot.  For the shared
 *               latent stream val_ring may be the attention window ring (P = R_w).
 *   P         : ring slots, >= m + o (the tokens one entry pools)
 *   bpos, out, out_scale, E_cap, out_dtype, out_layout : as in sckv_pool_stream.
 * When (t + 1) % m == 0 and e = (t + 1) / m - 1 < E_cap, entry e is pooled over
 * tokens [m e - o, m e + m) from the rings and the new token (the rings must hold
 * the tokens before t), bit for bit as csa_compress / hca_compress would pool it.
 * Calls on one stream run in order; two calls that share rings must not overlap. */
typedef struct {
  const int32_t* pos;
  const void* val;
  const void* gate;
  void* val_ring;
  void* gate_ring;
  const float* bpos;
  void* out;
  float* out_scale;
  int64_t E_cap;
  int32_t D;
  int32_t P;
  int32_t in_dtype;
  int32_t out_dtype;
  int32_t out_layout; /* sckv_layout */
  int32_t reserved;
} sckv_append_stream;

/* csa_append: appends one token per sequence to the latent stream `kv` and to
 * the indexer stream `index_keys` (may be NULL), with the CSA pool (m = 4, o = 4;
 * any m >= 1, o >= 0 accepted).  Both streams take the same positions; pass the
 * same pos pointer in both descriptors. */
sckv_status csa_append(int32_t B, int32_t m, int32_t o, const sckv_append_stream* kv,
                       const sckv_append_stream* index_keys, void* stream);

/* hca_append: as csa_append for the single HCA stream (m = 128, o = 0). */
sckv_status hca_append(int32_t B, int32_t m, int32_t o, const sckv_append_stream* kv, void* stream);

/* ------------------------------------------------------------------ lightning indexer + top-k
 *   q         : [R][H_I][D_I] indexer queries (q_dtype F32 or BF16)
 *   w         : [R][H_I] fp32 head weights w_h
 *   keys      : indexer keys in SCKV_LAYOUT_KEY_TILES [B][E_cap/32][D_I/8][32][8]
 *               (key_dtype F32, BF16 or unscaled E4M3; E_cap a multiple of 32), or
 *               MXFP4 tiles (key_dtype SCKV_MXFP4 with BF16 queries: each key is
 *               dequantised exactly to bf16 and scored as bf16 keys are)
 *   out_idx   : [R][k] int32: the kept entries of each row in ascending order,
 *               then -1 padding (k' = min(k, E_vis) entries are kept; E_vis = 0
 *               gives an all -1 row)
 *   out_score : [R][k] fp32 scores of the kept entries (padding: -inf), or NULL
 * Only entries 0 .. min(E_vis(t), E_cap) - 1 of each row's sequence are read.
 * Scores of exactly zero are ranked as +0. */
typedef struct {
  sckv_rows rows;
  const void* q;
  const float* w;
  const void* keys;
  int32_t* out_idx;
  float* out_score;
  int64_t E_cap;
  int32_t B;
  int32_t H_I;
  int32_t D_I;
  int32_t q_dtype;
  int32_t key_dtype;
  int32_t m;
  int32_t W;
  int32_t k;
} sckv_index_args;

/* Workspace bytes csa_index_topk needs for these arguments (0 if they are invalid). */
size_t csa_index_topk_workspace_size(const sckv_index_args* a);

/* csa_index_topk: scores every visible entry of each row and keeps its top-k. */
sckv_status csa_index_topk(const sckv_index_args* a, void* workspace, size_t workspace_bytes,
                           void* stream);

/* csa_index_topk_noalloc: csa_index_topk without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The scores and the selection's
 * workspace live in a static device array of SCKV_NOALLOC_SCRATCH_BYTES that
 * the library holds on every device it runs on until the process ends; the
 * call allocates nothing.  Arguments, results and kernels are those of
 * csa_index_topk.  Returns SCKV_ERR_WORKSPACE (nothing enqueued) when the rows
 * need more scratch than the array holds (csa_index_topk_workspace_size above
 * it), SCKV_ERR_UNSUPPORTED when `stream` belongs to another device than the
 * current one.  Every call on a device shares that device's array: calls that
 * overlap on one device (two streams, two threads) race and may return wrong
 * indices; calls in order on one stream are safe.  The first call on a device
 * looks the array's address up (thread-safe). */
#define SCKV_NOALLOC_SCRATCH_BYTES (16u << 20)
sckv_status csa_index_topk_noalloc(const sckv_index_args* a, void* stream);

/* The two halves of csa_index_topk, for callers that want the scores themselves.
 * csa_index_score writes s_j for j < min(E_vis, E_cap) of row r to
 * scores[r * score_stride + j] (score_stride >= the visible count of every row;
 * entries beyond a row's visible count are left untouched).
 * csa_topk_select selects from such a score matrix; out_idx / out_score as above. */
sckv_status csa_index_score(const sckv_index_args* a, float* scores, int64_t score_stride,
                            void* stream);
size_t csa_topk_select_workspace_size(const sckv_index_args* a);
sckv_status csa_topk_select(const sckv_index_args* a, const float* scores, int64_t score_stride,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ attention
 *   q           : [R][H][D] queries in the shared latent (q_dtype F32 or BF16); with
 *                 a latent wider than the head dim the caller passes W_UK^h^T q_h
 *   entries     : [B][E_cap][D] pooled entries (entry_dtype F32, BF16 or E4M3)
 *   entry_scale : [B][E_cap] fp32 per-entry scale (E4M3 only, else ignored)
 *   idx         : csa_attend: [R][k] int32 kept entries (as out_idx above; -1 = none)
 *   win         : [B][R_w][D] raw per-token latents v_i (win_dtype F32 or BF16);
 *                 token i of a sequence lives in slot i % R_w (R_w >= W; pass the
 *                 whole stream with R_w = N for prefill)
 *   out         : [R][H][D] (out_dtype F32 or BF16), o_h of each row
 *   lse         : [R][H] fp32 natural-log sum of exp of the scaled logits, or NULL
 *   softmax_scale : multiplies every logit (1/sqrt(head dim))
 * csa_attend uses the k listed entries; hca_attend uses entries
 * 0 .. min(E_vis(t), E_cap) - 1 (dense).  Both add the raw tokens
 * max(0, t - W + 1) .. t.  The MFMA path computes P.V in fp16: entries and window
 * values must stay below 65504 in magnitude. */
typedef struct {
  sckv_rows rows;
  const void* q;
  const void* entries;
  const float* entry_scale;
  const int32_t* idx;
  const void* win;
  void* out;
  float* lse;
  int64_t E_cap;
  int64_t R_w;
  int32_t B;
  int32_t H;
  int32_t D;
  int32_t q_dtype;
  int32_t entry_dtype;
  int32_t win_dtype;
  int32_t out_dtype;
  int32_t m;
  int32_t W;
  int32_t k;
  float softmax_scale;
  int32_t reserved;
} sckv_attend_args;

size_t csa_attend_workspace_size(const sckv_attend_args* a);
size_t hca_attend_workspace_size(const sckv_attend_args* a);
sckv_status csa_attend(const sckv_attend_args* a, void* workspace, size_t workspace_bytes,
                       void* stream);
sckv_status hca_attend(const sckv_attend_args* a, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ------------------------------------------------------------------ projections
 * Decode rows enter and leave the attention path through dense projections of
 * their hidden state x (the CSA decode workload definition: per-head queries,
 * attention against the shared latent, then the output projection W_o; MLA keeps
 * one compressed latent per token and absorbs the head projections into the
 * queries: knightli.com DeepSeek-V4 KV-cache article, section on the successive
 * KV-cache optimisations).  Every weight is bf16, row-major [N][K] as a linear
 * layer stores it (y = x W^T), and every product accumulates in fp32 on the
 * matrix cores.  1 <= R <= 2^21 rows; up to 64 rows (decode) a call streams its
 * weights from HBM once, more rows are taken in blocks of 64.  Every reduction
 * length (d_model, and D or H * d_h on the output side) must be a multiple of 128.
 *
 * layer_queries -- the query side of one layer:
 *   x     : [R][d_model] bf16 hidden states of the query rows
 *   W_q   : [H * d_h][d_model]; q_h = rows h d_h .. (h+1) d_h - 1 of W_q x
 *   W_UK  : [H][d_h][D] or NULL.  Non-NULL: q = W_UK^h^T q_h (the head queries are
 *           kept in fp32 in the workspace and absorbed in fp32; D % 128 == 0,
 *           D <= 4096, d_h in {64, 128, 256}).  NULL: q = q_h, and D must equal d_h.
 *   q     : [R][H][D] (q_dtype F32 or BF16), the attention queries
 *   W_iq  : [H_I * D_I][d_model] or NULL; qI : [R][H_I][D_I] (q_dtype), indexer queries
 *   W_w   : [H_I][d_model] or NULL; w : [R][H_I] fp32, indexer head weights
 * layer_streams -- the per-token streams the compressors pool (rows may be the
 *   newest token of each sequence, as csa_append / hca_append take them):
 *   W_c, W_g : [D][d_model] -> v, g : [R][D]; W_cI, W_gI : [D_I][d_model] -> vI, gI :
 *   [R][D_I] (each pair member may be NULL, then its output is not written);
 *   outputs in out_dtype (F32 or BF16).
 * layer_inputs -- layer_queries and layer_streams of the same rows (one x, R and
 *   d_model) in one launch: the decode step's new token both queries and joins
 *   the streams.  Outputs and workspace as the two calls.
 * layer_output -- back to the model width:
 *   o     : [R][H][D] bf16 attention outputs against the latent
 *   W_UV  : [H][d_h][D] or NULL.  Non-NULL: o_h = W_UV^h o~_h (rounded to bf16 in
 *           the workspace; D % 128 == 0).  NULL: o_h = o~_h (D == d_h).
 *   W_o   : [d_model][H * d_h]; y = W_o [o_1 .. o_H] : [R][d_model] (y_dtype F32 or
 *           BF16); H * d_h % 128 == 0.
 * Workspaces hold the fp32 head queries before absorption, the bf16 heads o_h, and
 * the fp32 partial sums of launches that cut the reduction across blocks (small
 * products); the size queries return 0 when none is needed (or the arguments are
 * invalid). */
typedef struct {
  const void* x;
  const void* W_q;
  const void* W_UK;
  const void* W_iq;
  const void* W_w;
  void* q;
  void* qI;
  float* w;
  int32_t R;
  int32_t d_model;
  int32_t H;
  int32_t d_h;
  int32_t D;
  int32_t H_I;
  int32_t D_I;
  int32_t q_dtype;
} sckv_query_args;

typedef struct {
  const void* x;
  const void* W_c;
  const void* W_g;
  const void* W_cI;
  const void* W_gI;
  void* v;
  void* g;
  void* vI;
  void* gI;
  int32_t R;
  int32_t d_model;
  int32_t D;
  int32_t D_I;
  int32_t out_dtype;
  int32_t reserved;
} sckv_stream_args;

typedef struct {
  const void* o;
  const void* W_UV;
  const void* W_o;
  void* y;
  int32_t R;
  int32_t d_model;
  int32_t H;
  int32_t d_h;
  int32_t D;
  int32_t y_dtype;
} sckv_output_args;

size_t layer_queries_workspace_size(const sckv_query_args* a);
sckv_status layer_queries(const sckv_query_args* a, void* workspace, size_t workspace_bytes, void* stream);
size_t layer_streams_workspace_size(const sckv_stream_args* a);
sckv_status layer_streams(const sckv_stream_args* a, void* workspace, size_t workspace_bytes, void* stream);
size_t layer_inputs_workspace_size(const sckv_query_args* q, const sckv_stream_args* s);
sckv_status layer_inputs(const sckv_query_args* q, const sckv_stream_args* s, void* workspace, size_t workspace_bytes,
                         void* stream);
size_t layer_output_workspace_size(const sckv_output_args* a);
sckv_status layer_output(const sckv_output_args* a, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ misc */
const char* sckv_last_error(void); /* thread-local text of the last non-OK status */
int32_t sckv_abi_version(void);    /* SCKV_ABI_VERSION */

#ifdef __cplusplus
}
#endif
#endif /* SCKV_H */
