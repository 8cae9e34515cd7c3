/*
 * tileshare.h -- C ABI of the MI355X TileShare library (libtileshare.so).
 *
 * TileShare ("TileShare: Training-Free Acceleration of Overlapping Tiled ViT
 * Decoding", abstract and Figure 2 caption) runs a fixed-window ViT decoder
 * over overlapping tiles without duplicating per-token work: in a *shared
 * layer* normalisation, QKV projection, QK-normalisation, out-projection and
 * MLP run once per token of the union of all tiles, attention still runs per
 * tile window (the tile's tokens plus the tile's own global token, RoPE on
 * tile-local coordinates), and an overlap token's per-tile attention outputs
 * are blended into one state with fixed weights w-bar.  TileShare-k keeps the
 * first k layers per tile (abstract; Table 1 caption); k = n_layers is the
 * released overlapping-tile decoder.
 *
 * Conventions for every entry point
 *  - Plain C types only.  `stream` is a hipStream_t passed as void* (NULL =
 *    the default stream).  Device pointers are caller-owned and must stay
 *    valid until the work queued on `stream` has finished.
 *  - Arrays are row-major.  Grid row p of a (T, H, W) token grid is
 *    p = (tau*H + y)*W + x.  Linear weights are [out_features, in_features].
 *  - The residual stream (x, x_in, x_out, g, g_out) is fp32.  GEMM operands
 *    and attention run in the model's act_dtype (fp32 or bf16; fp8 e4m3 for
 *    the shared layers' GEMMs when gemm_dtype_shared = TS_FP8E4M3) with fp32
 *    accumulation.  1-D parameters (biases, norm gains) are fp32.
 *  - Argument and shape errors return synchronously with a negative status;
 *    the message is available from ts_last_error() on the calling thread.
 *    Launch failures map to TS_EHIP.  Forward calls are asynchronous on
 *    `stream`.  No forward call allocates device memory: the caller passes a
 *    workspace of at least ts_workspace_size() bytes (256-byte aligned).
 *  - Results are deterministic: no atomics take part in any floating-point
 *    sum, so repeated calls give bit-identical outputs.
 */
#ifndef TILESHARE_H
#define TILESHARE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TS_ABI_VERSION 6

typedef int32_t ts_status;
#define TS_OK 0
#define TS_EINVAL (-1)       /* null pointer or invalid value */
#define TS_ESHAPE (-2)       /* shape not supported by the kernels */
#define TS_EDTYPE (-3)       /* dtype combination not supported */
#define TS_EHIP (-4)         /* a HIP call or kernel launch failed */
#define TS_ENOMEM (-5)       /* host or plan-owned device allocation failed */
#define TS_EUNSUPPORTED (-6) /* valid request the library does not implement */
#define TS_EWORKSPACE (-7)   /* workspace missing, too small or misaligned */

typedef enum { TS_F32 = 0, TS_BF16 = 1, TS_FP8E4M3 = 2 } ts_dtype;

/* ---- tiling plan ------------------------------------------------------
 * Figure 2 caption: overlap tokens are stored once and attended in every
 * window that holds them; Figure 5: tiles per pixel and tile-start lines.
 * Per axis of length N with tile extent L and stride S the tiles start at
 * min(i*S, N-L), i = 0..ceil((N-L)/S) (last tile clamped to the grid end;
 * one tile of extent N when N <= L).  Tiles are numbered in raster order over
 * their (t, h, w) indices and a tile's tokens in raster order over local
 * (tau, y, x).  w-bar: per axis a linear ramp across every overlap with a
 * neighbour, (u+1)/(O+1) leading and (L-u)/(O+1) trailing, multiplied over the
 * axes and normalised to sum 1 per token, computed in float64 and rounded
 * once to fp32; global tokens have weight 1. */
typedef struct {
  int32_t ndim;       /* 2 or 3 (2: grid[0] = tile[0] = 1) */
  int32_t grid[3];    /* T, H, W token counts */
  int32_t tile[3];    /* tile extent per axis */
  int32_t stride[3];  /* tile stride per axis (>= 1) */
  int32_t n_global;   /* global tokens per tile; must be 1 */
  int32_t blend;      /* 0 = linear-ramp w-bar; 1 = hard stitching (Table 2,
                         Table S2): w-bar 1 on the covering tile with the largest
                         float64 ramp, 0 on the others, ties to the lowest tile */
} ts_tiling_desc;

typedef struct ts_plan ts_plan; /* opaque, library-owned */

typedef struct {
  int32_t n_tiles;     /* number of tiles */
  int32_t tile_tokens; /* tokens per tile, without the global token */
  int32_t n_union;     /* grid tokens = T*H*W */
  int32_t n_entries;   /* sum over tiles of tile_tokens = coverage entries */
  int32_t max_cover;   /* most tiles holding one token */
  int32_t extent[3];   /* tile extent per axis after clamping to the grid */
} ts_plan_info;

/* Build a plan on the host (deterministic; no device work).  *out receives
 * a plan that must be released with ts_plan_destroy. */
ts_status ts_plan_create(const ts_tiling_desc* desc, ts_plan** out);
ts_status ts_plan_get_info(const ts_plan* plan, ts_plan_info* out);
/* Copy the plan's maps into caller-owned host buffers (any may be NULL):
 * tile_start [n_tiles*3] (t, h, w start), tile_rows [n_tiles*tile_tokens]
 * (grid row of each tile token), cover_ptr [n_union+1], cover_tile and
 * cover_local [n_entries] (covering tiles of each grid row in ascending tile
 * order, and the token's local index in that tile), cover_w [n_entries]. */
ts_status ts_plan_export(const ts_plan* plan, int32_t* tile_start, int32_t* tile_rows,
                         int32_t* cover_ptr, int32_t* cover_tile, int32_t* cover_local,
                         float* cover_w);
/* Tile-local RoPE table (Table S1: RoPE per tile on tile coordinates) for a
 * head size: cos/sin [tile_tokens * head_dim/2] fp32, host buffers.  The
 * head_dim/2 rotation pairs (2k, 2k+1) are split over the axes (2D: h, w get
 * half each; 3D: t gets P - 2*floor(P/3), h and w floor(P/3) each, P =
 * head_dim/2); pair i of an axis chunk of m pairs turns by
 * pos * base^(-i/m), evaluated in float64 and rounded to fp32. */
ts_status ts_plan_export_rope(const ts_plan* plan, int32_t head_dim, float rope_base,
                              float* cos_out, float* sin_out);
/* The query blocks of the shared layers' attention (Figure 2 caption: the
 * blend of an overlap token's per-tile outputs): grid rows grouped by the set
 * of tiles holding them with a nonzero w-bar, groups ordered by decreasing set
 * size then by their ascending tile lists, rows ascending, cut into blocks of
 * 256 rows.  *nblk and *maxc receive the block count and the largest set;
 * the arrays (caller-owned host buffers, any may be NULL) receive blk_nt
 * [nblk] (tiles of each block), blk_tiles [nblk*maxc] (ascending, -1 padded),
 * blk_rows [nblk*256] (grid rows, -1 in empty slots) and blk_w
 * [nblk*maxc*256] (w-bar of (block, tile, slot), 0 in empty slots). */
ts_status ts_plan_export_blocks(const ts_plan* plan, int32_t* nblk, int32_t* maxc, int32_t* blk_nt,
                                int32_t* blk_tiles, int32_t* blk_rows, float* blk_w);
/* The order in which the bf16 blended attention takes its (block, head)
 * jobs; it decides speed only, never a value.  Each head's blocks are split
 * in two halves of equal work (windows): every class of blocks with the same
 * number of windows is cut at its middle, an odd block going to the half
 * with less work so far.  order [nblk] (caller-owned host buffer) lists half
 * A then half B, each class by class from the most windows down, blocks
 * ascending; cls [ncls*4] holds per class {count in A, offset of those in
 * order, count in B, offset}.  *ncls receives the class count; the arrays
 * may be NULL. */
ts_status ts_plan_export_job_order(const ts_plan* plan, int32_t* ncls, int32_t* order, int32_t* cls);
/* Upload the maps, the attention's query blocks (grid rows grouped by the
 * tiles that hold them with a nonzero w-bar) and the grid-coordinate RoPE
 * table for (head_dim, rope_base) to device memory owned by the plan (the
 * only device allocation the library makes).  Must be called before any
 * forward call that uses the plan; calling it again with another head size
 * replaces the table.  Synchronous. */
ts_status ts_plan_upload(ts_plan* plan, int32_t head_dim, float rope_base, void* stream);
void ts_plan_destroy(ts_plan* plan);

/* ---- model ------------------------------------------------------------- */
typedef struct {
  int32_t d;          /* model width */
  int32_t n_heads;
  int32_t head_dim;   /* d = n_heads * head_dim; 32, 64 or 128 */
  int32_t mlp_hidden; /* fc1 width */
  int32_t n_layers;
  int32_t norm;       /* 0 LayerNorm (gain + bias), 1 RMSNorm (gain) */
  int32_t qk_norm;    /* 1: per-head RMSNorm of q and k with gains [head_dim] */
  float eps;          /* norm epsilon */
  float rope_base;    /* RoPE base (10000) */
  int32_t act_dtype;  /* TS_F32 or TS_BF16: GEMM operands and attention */
  int32_t gemm_dtype_shared; /* act_dtype, or TS_FP8E4M3 (act_dtype bf16) for
                                the GEMMs of shared layers */
  /* FP8 scope (Table S2 "FP8 MLP layers only", "TileShare-4 + FP8"; Table S5
   * "V0 + FP8"), used when gemm_dtype_shared is TS_FP8E4M3: */
  int32_t fp8_gemms;    /* which GEMMs run in e4m3: TS_FP8_QKV | TS_FP8_OUT |
                           TS_FP8_FC1 | TS_FP8_FC2; 0 = all four */
  int32_t fp8_per_tile; /* 1: per-tile layers (and the tiled decoder) use the
                           same fp8 GEMMs; 0: only shared layers */
  int32_t layer0_dedup; /* 1: when layer 0 runs per tile (stack with k >= 1,
                           tiled decoder, merge-once, partial sharing with
                           k >= 1), its Norm1, QKV and QK-norm run once per
                           token on the rows every tile copied its states
                           from, and attention reads each window through the
                           tile map (Table S1, layer 0 column: exact); 0
                           (default): once per per-tile row */
} ts_model_desc;
#define TS_FP8_QKV 1
#define TS_FP8_OUT 2
#define TS_FP8_FC1 4
#define TS_FP8_FC2 8

/* Device pointers of one pre-norm block (Table S1 order):
 * x += W_o Attn(Norm1(x)) + b_o;  x += W_2 GELU(W_1 Norm2(x) + b_1) + b_2,
 * GELU the exact erf form.  Matrices are [out, in] in act_dtype; vectors fp32.
 * The fp8 fields are used only when gemm_dtype_shared = TS_FP8E4M3: e4m3
 * codes of the same matrices and w_scale_f8 [4] (device, fp32) their
 * per-tensor scales (qkv, o, 1, 2), e.g. from ts_fp8_quantize. */
typedef struct {
  const float* norm1_g; const float* norm1_b; /* [d]; norm1_b NULL for RMSNorm */
  const void* w_qkv;    const float* b_qkv;   /* [3d, d]; [3d]; rows q | k | v,
                                                  head h at rows h*hd .. */
  const float* q_g;     const float* k_g;     /* [head_dim] or NULL (no QK-norm) */
  const void* w_o;      const float* b_o;     /* [d, d]; [d] */
  const float* norm2_g; const float* norm2_b; /* [d]; NULL for RMSNorm */
  const void* w_1;      const float* b_1;     /* [mlp_hidden, d]; [mlp_hidden] */
  const void* w_2;      const float* b_2;     /* [d, mlp_hidden]; [d] */
  const uint8_t* w_qkv_f8; const uint8_t* w_o_f8;
  const uint8_t* w_1_f8;   const uint8_t* w_2_f8;
  const float* w_scale_f8;                    /* [4] */
} ts_layer_weights;

/* Bytes of workspace the forward calls below need for (model, plan, k);
 * k = -1 gives what ts_merge_once_forward needs (any l). */
ts_status ts_workspace_size(const ts_model_desc* model, const ts_plan* plan, int32_t k,
                            size_t* bytes);

/* One shared layer, in place (Figure 2; Table S1, layers >= k).
 * x: device fp32 [n_union + n_tiles, d]; rows 0..n_union-1 the shared
 * token states in grid order, row n_union + t the global token of tile t.
 * Norm1, QKV (+ QK-norm) run once per row; attention per tile over
 * its tile_rows plus its global row with tile-local RoPE; the per-tile
 * outputs of each grid row are blended with w-bar (global rows: their
 * tile's output); then out-projection + residual and Norm2 + MLP +
 * residual once per row. */
ts_status ts_shared_layer_forward(const ts_model_desc* model, const ts_layer_weights* w,
                                  const ts_plan* plan, float* x, void* ws, size_t ws_bytes,
                                  void* stream);

/* TileShare-k stack (abstract; Table 1 caption; Table S8 per-tile depth).
 * layers: HOST array of n_layers weight structs (device pointers inside).
 * x_in: device fp32 [n_union, d]; g: device fp32 [d], the global token, copied
 * into every tile.  Layers 0..k-1 run per tile on per-tile states
 * (gathered from x_in plus g); at layer k every grid row is merged as the
 * w-bar blend of its per-tile states (global rows stay per tile); layers
 * k..n_layers-1 are shared layers.  k = n_layers merges after the last layer
 * (the tiled baseline).  x_out: device fp32 [n_union, d]; g_out: device fp32
 * [n_tiles, d] final global rows, or NULL.  0 <= k <= n_layers. */
ts_status ts_stack_forward(const ts_model_desc* model, const ts_layer_weights* layers,
                           const ts_plan* plan, int32_t k, const float* x_in, const float* g,
                           float* x_out, float* g_out, void* ws, size_t ws_bytes, void* stream);

/* Released overlapping-tile decoding (abstract; Table S5 "V0"): every
 * tile runs the whole stack on its own window and the outputs are blended
 * with w-bar.  Same result and arguments as ts_stack_forward with
 * k = n_layers. */
ts_status ts_tiled_forward(const ts_model_desc* model, const ts_layer_weights* layers,
                           const ts_plan* plan, const float* x_in, const float* g, float* x_out,
                           float* g_out, void* ws, size_t ws_bytes, void* stream);

/* Merging once at layer l, then continuing per tile (Figure 3b): layers
 * 0 .. l-1 run per tile from the gathered input, the per-tile states are
 * merged with w-bar into one state (global rows stay per tile), every tile
 * is re-gathered from that state (with its own global row), layers l .. L-1
 * run per tile, and the outputs are merged as in ts_tiled_forward.  l in
 * 0..n_layers.  Arguments, layouts and errors as ts_stack_forward; the
 * workspace is ts_workspace_size(model, plan, -1, ...) bytes; the shared
 * GEMM dtype is not used (every layer runs per tile). */
ts_status ts_merge_once_forward(const ts_model_desc* model, const ts_layer_weights* layers,
                                const ts_plan* plan, int32_t l, const float* x_in, const float* g,
                                float* x_out, float* g_out, void* ws, size_t ws_bytes, void* stream);

/* Partial sharing with per-tile residual streams (Table 1 top, Table S7):
 * layers 0 .. k-1 run per tile; from layer k on every tile keeps its own
 * residual stream and only the operations in `share` run once per token,
 * attention always per tile.  A shared operation takes the w-bar blend of
 * the tiles' states as input (for TS_SHARE_O: the blend of their attention
 * outputs) and adds its result to every tile's stream; global rows stay
 * per tile.  The outputs are merged as in ts_tiled_forward.  share = 0 is the
 * tiled decoder; all three bits follow TileShare-k.  bf16 / fp32 GEMMs only
 * (TS_EUNSUPPORTED for fp8 models).  Arguments, layouts and errors as
 * ts_stack_forward; workspace ts_workspace_size(model, plan, -1, ...). */
#define TS_SHARE_Q 1 /* Norm1, QKV projection, QK-norm */
#define TS_SHARE_O 2 /* out-projection */
#define TS_SHARE_M 4 /* Norm2 and MLP */
ts_status ts_partial_share_forward(const ts_model_desc* model, const ts_layer_weights* layers,
                                   const ts_plan* plan, int32_t k, int32_t share, const float* x_in,
                                   const float* g, float* x_out, float* g_out, void* ws, size_t ws_bytes,
                                   void* stream);

/* Per-tensor e4m3 quantisation (Table S5 "V0 + FP8"; OCP e4m3, round to
 * nearest even, saturation at +-448): scale = max|src| / 448 (1 if all zero),
 * dst[i] = e4m3(clamp(src[i] / scale, -448, 448)).  src: device, n elements of
 * src_dtype (TS_F32 or TS_BF16), 16-byte aligned; dst: device uint8 [n],
 * 8-byte aligned (TS_EINVAL otherwise); scale: device fp32 [1].  ws: device
 * workspace of at least 256 bytes.  Asynchronous. */
ts_status ts_fp8_quantize(const void* src, int32_t src_dtype, int64_t n, uint8_t* dst,
                          float* scale, void* ws, size_t ws_bytes, void* stream);

/* ---- building blocks -----------------------------------------------------
 * The kernels the forward calls are made of, exposed for tests and timing. */

/* Projection GEMM (Table S6: QKV, out-projection and MLP GEMMs): with
 * v[i][j] = alpha * sum_k a[i][k] b[j][k] + bias[j] (bias may be NULL),
 *   TS_EPI_BIAS       c (dtype; bf16 for TS_FP8E4M3) = v
 *   TS_EPI_BIAS_GELU  c (same) = exact-erf GELU(v)
 *   TS_EPI_RESIDUAL   c (fp32) += v
 *   TS_EPI_F32        c (fp32) = v
 * a [m, k], b [n, k] row-major device arrays of `dtype`; c [m, n].  alpha = 1,
 * or *scale_a * *scale_b (device floats) for TS_FP8E4M3.  bf16 needs k % 64
 * == 0, fp8 k % 128 == 0, and n % 16 == 0 for both. */
#define TS_EPI_BIAS 0
#define TS_EPI_BIAS_GELU 1
#define TS_EPI_RESIDUAL 2
#define TS_EPI_F32 3
ts_status ts_op_gemm(int32_t dtype, int32_t epilogue, const void* a, const void* b, int32_t m,
                     int32_t n, int32_t k, const float* bias, void* c, const float* scale_a,
                     const float* scale_b, void* stream);
/* The same GEMM with a device workspace (ws, ws_bytes; 256-byte aligned, may
 * be NULL / 0): the 256x256 output tiles of a partial last round over the
 * compute units are split along k, their fp32 partial sums kept in ws and
 * added in part order (the result does not vary from run to run).  Long k
 * (>= 64 blocks of 128 bytes): up to 8 parts per tile, run after the full
 * tiles.  Short k with TS_EPI_RESIDUAL: two halves per tile, run first in the
 * same launch as the full tiles, so the residual epilogues of the later
 * tiles are staggered.  Uses at most ws_bytes; with less room it runs
 * unsplit.  8 x 256 KB per compute unit (64 MiB on MI355X) allows every
 * split.  The forward calls pass their workspace. */
#define TS_GEMM_SPLIT_WS_BYTES (64u << 20)
ts_status ts_op_gemm_ws(int32_t dtype, int32_t epilogue, const void* a, const void* b, int32_t m,
                        int32_t n, int32_t k, const float* bias, void* c, const float* scale_a,
                        const float* scale_b, void* ws, size_t ws_bytes, void* stream);

/* The attention step of one layer exactly as the forward calls run it
 * (Figure 2 caption; Table S1 "Attention (dense, per tile)" and "Blend of
 * attention outputs"): the q and k sections of qkv are normalised per head
 * (QK-RMSNorm with gains q_g, k_g [head_dim] fp32 when model->qk_norm) and
 * rotated, IN PLACE -- every row by its grid coordinate (a tile's global row
 * by the tile's start), which gives every window the scores of tile-local
 * RoPE -- then, for every tile t and head, dense softmax attention with scale
 * 1/sqrt(head_dim) over the tile's window (its tile_tokens rows plus its
 * global row).  qkv: device [rows, 3d] act_dtype, q | k | v as the QKV
 * projection writes them; with bf16 the q section is left multiplied by the
 * softmax scale in the log2 domain, log2(e)/sqrt(head_dim), before its bf16
 * rounding (the kernels' scores are then q.k), with fp32 it is left
 * unscaled.  With QK-norm the softmax subtracts the static bound on the
 * scores that the gains give (|q.k| <= head_dim max|q_g| max|k_g| times the
 * scale) instead of a running maximum when that bound is at most 32; in bf16
 * without QK-norm, the bound max|q| max|k| over the q and k heads of all rows
 * as stored (Cauchy-Schwarz), under the same limit.
 *  shared = 1: rows = n_union + n_tiles (grid rows, then the global row of
 *    tile t at n_union + t); out: device [n_union + n_tiles, d] act_dtype,
 *    row p < n_union the w-bar blend of the outputs of every window holding p
 *    (ascending tile order), row n_union + t tile t's global-token output --
 *    the out-projection's input of a shared layer;
 *  shared = 0: per-tile layout, rows = n_tiles*(tile_tokens+1) (tile t at
 *    t*(tile_tokens+1), its global token last); out in the same layout.
 * ws: device workspace of at least ts_workspace_size(model, plan, n_layers)
 * bytes, 256-byte aligned.  Asynchronous.  bf16: the qkv array of either
 * layout must stay below 4 GiB (rows * 6 * d bytes < 2^32; every forward call
 * returns TS_ESHAPE otherwise). */
ts_status ts_op_attention(const ts_model_desc* model, const ts_plan* plan, int32_t shared, void* qkv,
                          const float* q_g, const float* k_g, void* out, void* ws, size_t ws_bytes,
                          void* stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * serving loops, harnesses that forbid hipMalloc): ts_op_attention with no
 * workspace argument.  Its scratch -- 256 bytes of job counters and 256 of
 * the largest q and k head norms (both set by the call), the fp32 partial
 * blends of the shared layout (n_union * d * 4 bytes) and the global rows'
 * split states -- lives
 * in a file-scope device array of TS_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds until the process ends; the call allocates nothing.
 * A request whose counters and partial blends exceed the array returns TS_EWORKSPACE
 * (the per-tile layout, shared = 0, needs none).  All calls on one GPU share
 * its array: calls that overlap on one GPU (on different streams, or from
 * different threads) race and must be serialised by the caller.  Nothing in
 * the array needs to start at zero.  Arguments and results as
 * ts_op_attention. */
#define TS_NOALLOC_SCRATCH_BYTES (64u << 20)
ts_status ts_op_attention_noalloc(const ts_model_desc* model, const ts_plan* plan, int32_t shared, void* qkv,
                                  const float* q_g, const float* k_g, void* out, void* stream);

/* ---- diagnostics ------------------------------------------------------- */
/* Per-kernel timing of the calling thread's forward calls.  Between
 * ts_profile_begin and ts_profile_end every kernel the library launches is
 * bracketed by hipEvents on its stream; ts_profile_end synchronises them and
 * writes one record per kernel name (at most max_records) with the launch
 * count, total milliseconds and the algorithmic flops and HBM bytes of all
 * launches.  Profiling adds two event records per launch. */
typedef struct {
  char name[64];
  int32_t launches;
  double total_ms;
  double flops;    /* algorithmic floating-point operations, all launches */
  double bytes;    /* algorithmic HBM bytes (compulsory reads + writes) */
} ts_kernel_stat;
ts_status ts_profile_begin(void);
ts_status ts_profile_end(ts_kernel_stat* out, int32_t max_records, int32_t* n_records);

const char* ts_last_error(void);
int32_t ts_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TILESHARE_H */
