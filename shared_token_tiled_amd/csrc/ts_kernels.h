// Host-side launchers of the HIP kernels (internal to libtileshare).
// Every launcher validates nothing beyond what its kernel assumes; the
// C ABI (abi.hip) checks shapes before calling them.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsk {

enum Act { ACT_F32 = 0, ACT_BF16 = 1, ACT_FP8 = 2 };

// GEMM epilogues: C = A B^T (A [M,K], B [N,K], row-major), v = alpha*acc + bias[n]
enum Epi {
  EPI_BIAS = 0,      // C (act) = v
  EPI_BIAS_GELU = 1, // C (act) = GELU(v)
  EPI_RESID = 2,     // C (fp32) += v   (residual stream, in place)
  EPI_F32 = 3,       // C (fp32) = v
};

// ---- elementwise.hip ----
// y[M,d] (act) = Norm(x[M,d] fp32); rms: RMSNorm(g) else LayerNorm(g, b).
// amax (optional): atomic max of |y| as stored, in float bits (see fp8_quantize).
hipError_t norm(hipStream_t s, int act, bool rms, const float* x, int M, int d, const float* g,
                const float* b, float eps, void* y, unsigned* amax = nullptr);
// In place per-head RMSNorm of the q and k sections of qkv [M, 3d] (act).
// RoPE coordinates of the rows of a qkv array for qk_prep.  Shared layout
// (shared = true): row r < n_union is grid row r (coordinates (r / (gh*gw),
// (r / gw) % gh, r % gw) for grid = {gt, gh, gw}), row n_union + t is tile
// t's global token at the tile's start.  Per-tile layout: row t*(n+1) + i is
// tile t's start plus the local position of window token i (i = n: the
// global token, the start itself).
struct RopeRows {
  bool shared;
  int n_union, n, n_tiles;
  int grid[3];
  const int* tile_start;   // [n_tiles*3] (t, h, w)
  const int* local_pos;    // [n] packed tau | y<<10 | x<<20
  const float* tab;        // (cos, sin) of pair i of axis a at coordinate c: tab[off[a] + 2*(c*pairs[a] + i)]
  int off[3], pairs[3];
};
// In place on the q and k heads of qkv [M, 3d]: QK-RMSNorm with gains qg, kg
// (skipped when qg is null), then RoPE by the rows' coordinates.  qkn
// (optional, bf16, without QK-norm; QKN_BYTES): set to the largest norm of a
// q head and of a k head over all M rows as stored (float bits in qkn[0],
// qkn[1]), zeroed first by qk_prep itself.
constexpr int QKN_BYTES = 256;
hipError_t qk_prep(hipStream_t s, int act, void* qkv, int M, int d, int H, int hd, const float* qg,
                   const float* kg, float eps, const RopeRows& rr, unsigned* qkn = nullptr);
// out_union[p] = sum_e w[e] * in[entry_row[e]] over cover_ptr[p]..cover_ptr[p+1];
// out_global[t] = in[t*(n+1)+n] (skipped when out_global is null).
// amax (optional): atomic max of |output| as stored, over both outputs.
hipError_t blend(hipStream_t s, int tin, int tout, const void* in, int d, int n_union, int n_tiles,
                 int n, const int* cover_ptr, const int* entry_row, const float* w, void* out_union,
                 void* out_global, unsigned* amax = nullptr);
// X[t*(n+1)+j] += delta[tile_rows[t*n+j]], X[t*(n+1)+n] += delta[n_union+t]  (fp32)
hipError_t add_to_tiles(hipStream_t s, float* X, const float* delta, const int* tile_rows, int n_union,
                        int n_tiles, int n, int d);
// X[t*(n+1)+j] = x_in[tile_rows[t*n+j]], X[t*(n+1)+n] = g + t*g_stride  (fp32;
// g_stride 0: one global row for every tile)
hipError_t gather(hipStream_t s, const float* x_in, const float* g, int64_t g_stride, const int* tile_rows,
                  int n_tiles, int n, int d, float* X);
// xs[p] = x_in[p] (p < n_union), xs[n_union+t] = g  (fp32)
hipError_t init_shared(hipStream_t s, const float* x_in, const float* g, int n_union, int n_tiles,
                       int d, float* xs);
// dst[i] = src[i], n multiple of 4 (fp32)
hipError_t copy_f32(hipStream_t s, const float* src, float* dst, int64_t n);
// Max |value| slots of an fp8 operand: producers (norm, blend, GEMM
// epilogues) take atomic maxima in float bits into AMAX_SLOTS slots of 4
// bytes, AMAX_STRIDE unsigned apart (256 bytes), spread over their
// wavefronts; the quantisation takes the max over the slots.
constexpr int AMAX_SLOTS = 64, AMAX_STRIDE = 64;
// e4m3 per-tensor quantisation; amax_slot: nslots (1..AMAX_SLOTS) slots of
// scratch device memory, AMAX_STRIDE unsigned apart.  amax_ready: the slots
// already hold max |src| (its producer took it), so only the codes and the
// scale are written; otherwise a separate pass takes it (into slot 0).
hipError_t fp8_quantize(hipStream_t s, int tin, const void* src, int64_t n, uint8_t* dst,
                        float* scale_out, unsigned* amax_slot, bool amax_ready = false, int nslots = 1);
// All AMAX_SLOTS slots at p set to 0 (a kernel, so that it can sit in a
// captured graph)
hipError_t zero_amax(hipStream_t s, unsigned* p);

// ---- gemm_*.hip ----
// act: ACT_F32 (fp32 operands), ACT_BF16, ACT_FP8 (e4m3 operands, alpha = *sa * *sb).
// ws (fp32, ws_bytes; may be null): scratch for the K-split parts of a
// partial last round of tiles (up to 8 x 256 KB per tile of that round).
// amax (optional, bf16-output epilogues): atomic max of |C| as stored.
// lda, ldc: row pitches of A and C in elements (0: K and N; lda a multiple of
// 8, ldc of 4); B is [N, K] contiguous.
hipError_t gemm(hipStream_t s, int act, int epi, const void* A, const void* B, int M, int N, int K,
                const float* bias, void* C, const float* sa, const float* sb, float* ws = nullptr,
                size_t ws_bytes = 0, unsigned* amax = nullptr, int lda = 0, int ldc = 0);

// ---- attn.hip ----
// Query rows per attention workgroup, and per query block of the plan.
constexpr int QBLOCK = 256;
// bytes of the blended attention's job counters: 8 XCDs, 32 bytes apart
constexpr int JOB_COUNTERS_BYTES = 256;
// q and k of qkv are as qk_prep left them (normalised, rotated by grid
// coordinates).  Window token j of tile t is qkv row rows[t*n + j], its global
// token row g0 + gstep*t.  Layouts (see attn.hip):
//  - per tile: rows[t*n + j] = t*(n+1)+j, g0 = n, gstep = n+1; outputs in
//    the same rows;
//  - shared rows (blk_nt == null): the tile map into [n_union + n_tiles]
//    rows, g0 = n_union, gstep = 1; outputs per tile, t*(n+1)+i;
//  - blended (blk_nt != null): shared rows; every grid row's outputs of the
//    windows of its query block blended with the block's weights, written to
//    out row p (global rows: out row n_union + t).
struct AttnArgs {
  const void* qkv;          // [rows, 3d] act
  void* out;                // act, rows as above
  float* part = nullptr;    // blended: fp32 [n_union, d] partial sums between windows
  const int* rows = nullptr;       // [n_tiles*n] qkv row of each tile's tokens
  int g0 = 0, gstep = 0;           // qkv row of tile t's global token: g0 + gstep*t
  const int* blk_nt = nullptr;     // [nblk] windows of each query block
  const int* blk_tiles = nullptr;  // [nblk*maxc] their tiles, ascending
  const int* blk_rows = nullptr;   // [nblk*QBLOCK] grid row of each query slot (-1: empty)
  const float* blk_w = nullptr;    // [nblk*maxc*QBLOCK] w-bar of (block, window, slot)
  int nblk = 0, maxc = 0;
  const int* blk_order = nullptr;  // [nblk] blocks of the halves A, B of a head (bf16 job order)
  const int* blk_cls = nullptr;    // [ncls*4] per class of equal windows: count, offset in A; in B
  int ncls = 0, half_a = 0;        // classes; blocks in half A (half B: nblk - half_a)
  unsigned* jobs = nullptr;        // bf16 blended: per-XCD job counters (JOB_COUNTERS_BYTES), zeroed by attention()
  int n_union, d, H, hd, n_tiles, n;
  unsigned* amax = nullptr;        // optional (bf16): max |out| as stored
  // QK-RMSNorm gains [hd] of q and k, or null: with them every score obeys
  // |q.k| <= hd max|q_g| max|k_g|, a fixed softmax offset (bf16 kernel)
  const float* qg = nullptr;
  const float* kg = nullptr;
  // without QK-norm (bf16): qk_prep's largest q and k head norms, or null:
  // every score obeys |q.k| <= max|q| max|k| (Cauchy-Schwarz), the same use
  const unsigned* qkn = nullptr;
};
// fp32: every query row, the global rows included.  bf16: the tile-token
// query rows; the global-token rows are attention_global's.
hipError_t attention(hipStream_t s, int act, const AttnArgs& a);
// bf16 only: the global-token query row of every (tile, head).  With
// scratch (fp32, scratch_floats long) the keys are split over several
// workgroups per row and merged by a second kernel; without, one workgroup
// per row.
hipError_t attention_global(hipStream_t s, const AttnArgs& a, float* scratch, int64_t scratch_floats);

}  // namespace tsk
