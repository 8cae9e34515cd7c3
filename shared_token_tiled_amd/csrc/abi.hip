// C ABI of libtileshare: argument checks, plan upload, workspace layout, and
// the launch schedule of the per-tile block, the shared layer (TileShare
// paper page, Figure 2 caption and Table S1) and the TileShare-k stack
// (abstract, Table 1 caption).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "plan_internal.h"
#include "ts_kernels.h"

namespace {

thread_local std::string g_err;

ts_status fail(ts_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

#define TS_HIP(call, what)                                                                  \
  do {                                                                                      \
    hipError_t e_ = (call);                                                                 \
    if (e_ != hipSuccess) return fail(TS_EHIP, std::string(what) + ": " + hipGetErrorString(e_)); \
  } while (0)

// ---------------------------------------------------------------- profiler
struct ProfRec {
  std::string name;
  hipEvent_t a, b;
  double flops, bytes;
};
struct Profiler {
  bool on = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
thread_local Profiler g_prof;

// Brackets one launch with events when profiling is on.
struct Scope {
  hipStream_t s;
  ProfRec rec;
  bool active = false;
  Scope(hipStream_t st, const char* name, double flops, double bytes) : s(st) {
    if (!g_prof.on) return;
    rec.name = name;
    rec.flops = flops;
    rec.bytes = bytes;
    rec.a = g_prof.take();
    rec.b = g_prof.take();
    if (rec.a && rec.b && hipEventRecord(rec.a, s) == hipSuccess) active = true;
  }
  ~Scope() {
    if (active && hipEventRecord(rec.b, s) == hipSuccess) g_prof.recs.push_back(rec);
  }
};

// ------------------------------------------------------------ validation
int act_bytes(int act) { return act == TS_F32 ? 4 : (act == TS_BF16 ? 2 : 1); }

ts_status check_model(const ts_model_desc* m) {
  if (!m) return fail(TS_EINVAL, "model is null");
  if (m->d <= 0 || m->n_heads <= 0 || m->head_dim <= 0 || m->mlp_hidden <= 0 || m->n_layers < 0)
    return fail(TS_EINVAL, "model sizes must be positive");
  if (m->d != m->n_heads * m->head_dim) return fail(TS_ESHAPE, "d must equal n_heads * head_dim");
  if (m->d % 64 != 0 || m->d > 4096) return fail(TS_ESHAPE, "d must be a multiple of 64 and <= 4096");
  if (m->mlp_hidden % 64 != 0) return fail(TS_ESHAPE, "mlp_hidden must be a multiple of 64");
  if (m->norm != 0 && m->norm != 1) return fail(TS_EINVAL, "norm must be 0 (LayerNorm) or 1 (RMSNorm)");
  if (!(m->eps > 0.f)) return fail(TS_EINVAL, "eps must be > 0");
  if (m->layer0_dedup != 0 && m->layer0_dedup != 1) return fail(TS_EINVAL, "layer0_dedup must be 0 or 1");
  if (m->act_dtype == TS_F32) {
    if (m->head_dim != 32 && m->head_dim != 64)
      return fail(TS_ESHAPE, "fp32 attention supports head_dim 32 or 64");
    if (m->gemm_dtype_shared != TS_F32) return fail(TS_EDTYPE, "fp32 models need fp32 shared GEMMs");
  } else if (m->act_dtype == TS_BF16) {
    if (m->head_dim != 64 && m->head_dim != 128)
      return fail(TS_ESHAPE, "bf16 attention supports head_dim 64 or 128");
    if (m->gemm_dtype_shared != TS_BF16 && m->gemm_dtype_shared != TS_FP8E4M3)
      return fail(TS_EDTYPE, "bf16 models need bf16 or fp8 shared GEMMs");
    if (m->fp8_gemms < 0 || m->fp8_gemms > 15) return fail(TS_EINVAL, "fp8_gemms must be a mask of TS_FP8_* bits");
    if (m->fp8_per_tile != 0 && m->fp8_per_tile != 1) return fail(TS_EINVAL, "fp8_per_tile must be 0 or 1");
    if (m->gemm_dtype_shared == TS_FP8E4M3 && (m->d % 128 != 0 || m->mlp_hidden % 128 != 0))
      return fail(TS_ESHAPE, "fp8 GEMMs need d and mlp_hidden multiples of 128");
  } else {
    return fail(TS_EDTYPE, "act_dtype must be TS_F32 or TS_BF16");
  }
  return TS_OK;
}

// fp8 scope: mask of the GEMMs that run in e4m3 in a shared (or per-tile) layer
int fp8_mask(const ts_model_desc* m, bool shared) {
  if (m->gemm_dtype_shared != TS_FP8E4M3 || !(shared || m->fp8_per_tile)) return 0;
  return m->fp8_gemms ? m->fp8_gemms : (TS_FP8_QKV | TS_FP8_OUT | TS_FP8_FC1 | TS_FP8_FC2);
}

ts_status check_weights(const ts_model_desc* m, const ts_layer_weights* w, bool shared) {
  if (!w) return fail(TS_EINVAL, "layer weights are null");
  if (!w->norm1_g || !w->norm2_g || !w->w_qkv || !w->b_qkv || !w->w_o || !w->b_o || !w->w_1 ||
      !w->b_1 || !w->w_2 || !w->b_2)
    return fail(TS_EINVAL, "a required weight pointer is null");
  if (m->norm == 0 && (!w->norm1_b || !w->norm2_b)) return fail(TS_EINVAL, "LayerNorm needs norm biases");
  if (m->qk_norm && (!w->q_g || !w->k_g)) return fail(TS_EINVAL, "QK-norm needs q_g and k_g");
  const int f8 = fp8_mask(m, shared);
  if (f8 && (!w->w_scale_f8 || ((f8 & TS_FP8_QKV) && !w->w_qkv_f8) || ((f8 & TS_FP8_OUT) && !w->w_o_f8) ||
             ((f8 & TS_FP8_FC1) && !w->w_1_f8) || ((f8 & TS_FP8_FC2) && !w->w_2_f8)))
    return fail(TS_EINVAL, "fp8 GEMMs need their e4m3 weights and the weight scales");
  return TS_OK;
}

ts_status check_plan(const ts_plan* p, const ts_model_desc* m) {
  if (!p) return fail(TS_EINVAL, "plan is null");
  if (!p->uploaded) return fail(TS_EINVAL, "plan not uploaded (call ts_plan_upload)");
  if (p->rope_hd != m->head_dim || p->rope_base != m->rope_base)
    return fail(TS_EINVAL, "plan RoPE table was uploaded for another head_dim or base");
  // the bf16 attention stages K and V with 32-bit byte offsets into qkv
  const int64_t rows = std::max(int64_t(p->n_tiles) * (p->n + 1), int64_t(p->n_union) + p->n_tiles);
  if (m->act_dtype == TS_BF16 && rows * 6 * int64_t(m->d) >= (int64_t(1) << 32))
    return fail(TS_ESHAPE, "the qkv array (" + std::to_string(rows) + " rows x 3d bf16) reaches 4 GiB; the "
                           "attention's K/V staging takes 32-bit offsets");
  return TS_OK;
}

// ------------------------------------------------------------ workspace
// Row pitch (elements) of the MLP hidden activations, written by fc1 and read
// as fc2's A operand.  A bf16 row of a multiple of 4 KB is padded by 128
// bytes: an isolated fc2-shaped GEMM (hidden 10240) runs 3-4 % faster with A
// rows 20608 bytes apart than 20480 (likely because the 128-byte slices that
// a K block takes from a panel's 256 rows then spread over more memory
// channels).  An fp8 fc2 quantises the hidden as one contiguous array, so it
// keeps the plain pitch.
int64_t mlp_pitch(const ts_model_desc* m, bool fc2_fp8) {
  const int64_t dm = m->mlp_hidden;
  if (m->act_dtype != TS_BF16 || fc2_fp8 || (dm * 2) % 4096 != 0) return dm;
  return dm + 64;
}

struct WS {
  unsigned* amax = nullptr;  // fp8 scratch: amax bits
  float* sa = nullptr;       // fp8 scratch: activation scale
  float* X = nullptr;        // fp32 [M_t, d] per-tile states
  float* xs = nullptr;       // fp32 [M_s, d] shared states
  void* h = nullptr;         // act [M_max, d] norm / blend output
  void* big = nullptr;       // act [M_max, max(3d, mlp)] qkv, then MLP hidden
  void* o = nullptr;         // act [M_t, d] attention output, per-tile layout; in shared
                             // layers fp32 [n_union, d] partial blends of the attention
  uint8_t* q8 = nullptr;     // e4m3 [M_s, max(d, mlp)] quantised GEMM operand
  float* gpart = nullptr;    // fp32 split states of the global-token attention rows
  int64_t gpart_floats = 0;
  float* gsplit = nullptr;   // fp32 K-split parts of a GEMM's partial last round of tiles
  unsigned* jobs = nullptr;  // job counters of the blended attention
  unsigned* qkn = nullptr;   // bf16 without QK-norm: qk_prep's largest q and k head norms
  size_t bytes = 0;
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

WS layout(const ts_model_desc* m, const ts_plan* p, bool states, bool per_tile, bool shared_xs,
          char* base) {
  const int64_t Mt = int64_t(p->n_tiles) * (p->n + 1);
  const int64_t Ms = int64_t(p->n_union) + p->n_tiles;
  const int64_t Mmax = per_tile ? std::max(Mt, Ms) : Ms;
  const int64_t d = m->d, wide = std::max<int64_t>(3 * d, mlp_pitch(m, false));
  const int ab = act_bytes(m->act_dtype);
  WS w;
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* r = base ? base + off : nullptr;
    off += align256(bytes);
    return r;
  };
  // fp8 scratch: the max slots (tsk::AMAX_SLOTS, 256 bytes apart), then the scale
  char* scratch = take(size_t(tsk::AMAX_SLOTS) * tsk::AMAX_STRIDE * 4 + 256);
  w.amax = (unsigned*)scratch;
  w.sa = (float*)(scratch + size_t(tsk::AMAX_SLOTS) * tsk::AMAX_STRIDE * 4);
  if (states && per_tile) w.X = (float*)take(size_t(Mt * d * 4));
  // shared states; with layer-0 dedup also the shared-layout input rows of per-tile layer 0
  if (shared_xs || (per_tile && m->layer0_dedup)) w.xs = (float*)take(size_t(Ms * d * 4));
  w.h = take(size_t(Mmax * d * ab));
  w.big = take(size_t(Mmax * wide * ab));
  // per-tile attention outputs, or (shared layers) the fp32 partial blends
  w.o = take(std::max(size_t(Mt * d * ab), size_t(p->n_union) * d * 4));
  if (m->gemm_dtype_shared == TS_FP8E4M3)
    w.q8 = (uint8_t*)take(size_t((m->fp8_per_tile ? Mmax : Ms) * std::max<int64_t>(d, m->mlp_hidden)));
  if (m->act_dtype == TS_BF16) {  // up to 64 splits of each global row's keys
    w.gpart_floats = int64_t(p->n_tiles) * m->n_heads * 64 * (m->head_dim + 2);
    w.gpart = (float*)take(size_t(w.gpart_floats * 4));
  }
  if (m->act_dtype != TS_F32) w.gsplit = (float*)take(TS_GEMM_SPLIT_WS_BYTES);
  if (m->act_dtype == TS_BF16) w.jobs = (unsigned*)take(tsk::JOB_COUNTERS_BYTES);
  if (m->act_dtype == TS_BF16 && !m->qk_norm) w.qkn = (unsigned*)take(tsk::QKN_BYTES);
  w.bytes = off;
  return w;
}

// ------------------------------------------------------------ one layer
struct Ctx {
  const ts_model_desc* m;
  const ts_plan* p;
  hipStream_t s;
};

double gemm_bytes(int64_t M, int64_t N, int64_t K, int ab, int ob, bool resid) {
  return double(M * K + N * K) * ab + double(M * N) * ob * (resid ? 2 : 1);
}

// The MFMA GEMM addresses each operand with 32-bit byte offsets (A with row
// pitch lda >= K).
bool gemm_offsets_fit(int64_t M, int64_t N, int64_t K, int esz, int64_t lda = 0) {
  return M * std::max(lda, K) * esz < (int64_t(1) << 32) && N * K * esz < (int64_t(1) << 32);
}

// The producer of an fp8 GEMM operand (a norm, the blend, a bf16-output
// GEMM epilogue) takes the operand's max |value| itself, so its fp8
// quantisation only encodes; TS_FP8_SEPARATE_AMAX=1 selects the separate max
// pass instead (the two give bit-identical results).
bool fused_amax() {
  const char* e = getenv("TS_FP8_SEPARATE_AMAX");
  return !(e && atoi(e) == 1);
}

// y = A W^T (+ epilogue) for one projection; fp8 quantises A first.
// amax_ready: ws.amax already holds max |A| (see fused_amax).  out_amax: the
// epilogue takes max |C| into it (for the next projection's quantisation).
// lda, ldc: row pitches of A and C in elements (0: K and N; fp8 takes A
// contiguous).
ts_status proj(const Ctx& c, const WS& ws, bool f8, const char* role, int epi, const void* A, int64_t M,
               int N, int K, const void* Wt, const uint8_t* W8, const float* w8scale, const float* bias,
               void* C, bool amax_ready = false, unsigned* out_amax = nullptr, int lda = 0, int ldc = 0) {
  const int act = c.m->act_dtype;
  if (f8 && lda != 0 && lda != K) return fail(TS_EINVAL, std::string("fp8 GEMM operand with a row pitch (") + role + ")");
  if (act != TS_F32 && !gemm_offsets_fit(M, N, K, f8 ? 1 : 2, lda))
    return fail(TS_ESHAPE, std::string("GEMM operand larger than 4 GiB (") + role + ")");
  const int ob = (epi == tsk::EPI_RESID || epi == tsk::EPI_F32) ? 4 : act_bytes(act);
  std::string name = std::string(f8 ? "gemm_fp8[" : (act == TS_F32 ? "gemm_f32[" : "gemm_bf16[")) + role + "]";
  if (f8) {
    {
      Scope sc(c.s, (std::string("fp8_quantize[") + role + "]").c_str(), 0.0,
               double(M * K) * (2.0 * act_bytes(act) + 1.0));
      TS_HIP(tsk::fp8_quantize(c.s, act, A, M * K, ws.q8, ws.sa, ws.amax, amax_ready, tsk::AMAX_SLOTS),
             "fp8 quantize");
    }
    if (out_amax) TS_HIP(tsk::zero_amax(c.s, out_amax), "amax reset");  // after the quantisation read it
    Scope sc(c.s, name.c_str(), 2.0 * M * N * K, gemm_bytes(M, N, K, 1, ob, epi == tsk::EPI_RESID));
    TS_HIP(tsk::gemm(c.s, tsk::ACT_FP8, epi, ws.q8, W8, int(M), N, K, bias, C, ws.sa, w8scale, ws.gsplit,
                   TS_GEMM_SPLIT_WS_BYTES, out_amax, 0, ldc),
         "fp8 gemm");
    return TS_OK;
  }
  if (out_amax) TS_HIP(tsk::zero_amax(c.s, out_amax), "amax reset");
  Scope sc(c.s, name.c_str(), 2.0 * M * N * K, gemm_bytes(M, N, K, act_bytes(act), ob, epi == tsk::EPI_RESID));
  TS_HIP(tsk::gemm(c.s, act, epi, A, Wt, int(M), N, K, bias, C, nullptr, nullptr, ws.gsplit, TS_GEMM_SPLIT_WS_BYTES,
                   out_amax, lda, ldc),
         "gemm");
  return TS_OK;
}

// RoPE coordinates of the rows of a shared-layout (n_union + n_tiles rows)
// or per-tile-layout (n_tiles*(n+1) rows) qkv array.
tsk::RopeRows rope_rows(const ts_plan* p, bool shared) {
  tsk::RopeRows r;
  r.shared = shared;
  r.n_union = p->n_union;
  r.n = p->n;
  r.n_tiles = p->n_tiles;
  r.tile_start = (const int*)p->d_tile_start;
  r.local_pos = (const int*)p->d_local_pos;
  r.tab = (const float*)p->d_rope_glob;
  for (int a = 0; a < 3; ++a) {
    r.grid[a] = p->desc.grid[a];
    r.off[a] = p->rope_glob_off[a];
    r.pairs[a] = p->rope_pairs[a];
  }
  return r;
}

// Window attention of every (tile, head) for one layer; q and k as qk_prep
// left them.  Layouts: ATT_TILED (per-tile qkv rows and outputs),
// ATT_SHARED_ROWS (shared qkv rows read through the tile map, per-tile
// outputs: layer 0 once per token), ATT_BLENDED (shared qkv rows, outputs
// blended with w-bar into [n_union + n_tiles] rows; `part` holds the fp32
// partial blends; `jobs`, bf16 only, the job counters).  amax (optional,
// bf16): max |output| as stored.
enum AttnLayout { ATT_TILED, ATT_SHARED_ROWS, ATT_BLENDED };
ts_status window_attention(const ts_model_desc* m, const ts_plan* p, AttnLayout lay, const void* qkv, void* out,
                           float* part, unsigned* jobs, unsigned* amax, hipStream_t s, float* gscratch,
                           int64_t gscratch_floats, const float* q_g, const float* k_g, const unsigned* qkn) {
  tsk::AttnArgs a;
  if (m->qk_norm) {
    a.qg = q_g;
    a.kg = k_g;
  } else {
    a.qkn = qkn;  // the score bound from qk_prep's largest norms (bf16)
  }
  a.qkv = qkv;
  a.out = out;
  a.part = part;
  // window rows through a map in every layout: the tile map into shared
  // rows, or t*(n+1)+j into per-tile rows; the global key row is g0 + gstep*t
  a.rows = lay != ATT_TILED ? (const int*)p->d_tile_rows : (const int*)p->d_tile_rows_local;
  a.g0 = lay != ATT_TILED ? p->n_union : p->n;
  a.gstep = lay != ATT_TILED ? 1 : p->n + 1;
  if (lay == ATT_BLENDED) {
    a.blk_nt = (const int*)p->d_blk_nt;
    a.blk_tiles = (const int*)p->d_blk_tiles;
    a.blk_rows = (const int*)p->d_blk_rows;
    a.blk_w = (const float*)p->d_blk_w;
    a.nblk = p->nblk;
    a.maxc = p->blk_maxc;
    a.blk_order = (const int*)p->d_blk_order;
    a.blk_cls = (const int*)p->d_blk_cls;
    a.ncls = p->blk_ncls;
    a.jobs = jobs;
    a.half_a = p->blk_ncls ? p->blk_cls[4 * (p->blk_ncls - 1)] + p->blk_cls[4 * (p->blk_ncls - 1) + 1] : 0;
  }
  a.n_union = p->n_union;
  a.d = m->d;
  a.H = m->n_heads;
  a.hd = m->head_dim;
  a.n_tiles = p->n_tiles;
  a.n = p->n;
  a.amax = m->act_dtype == TS_BF16 ? amax : nullptr;
  // algorithmic work: 4 (n+1) d FLOPs per query row and window (QK^T and PV
  // over the n+1 keys); bytes: the windows' q, k, v rows read once, each
  // output row written once
  const double nn = double(p->n + 1), ab = act_bytes(m->act_dtype);
  const double qrows = lay == ATT_BLENDED ? double(p->n_entries) : double(p->n_tiles) * p->n;
  const double orows = lay == ATT_BLENDED ? double(p->n_union) : double(p->n_tiles) * p->n;
  if (m->act_dtype == TS_F32) {
    Scope sc(s, "attn_f32", 4.0 * nn * (qrows + p->n_tiles) * m->d,
             (double(p->n_tiles) * nn * 3 * m->d + orows * m->d + double(p->n_tiles) * m->d) * ab);
    TS_HIP(tsk::attention(s, m->act_dtype, a), "attention");
    return TS_OK;
  }
  {
    Scope sc(s, lay == ATT_BLENDED ? "attn_blend_bf16" : "attn_bf16", 4.0 * nn * qrows * m->d,
             (double(p->n_tiles) * nn * 3 * m->d + orows * m->d) * ab);
    TS_HIP(tsk::attention(s, m->act_dtype, a), "attention");
  }
  {
    Scope sc(s, "attn_global_bf16", 4.0 * nn * m->d * p->n_tiles,
             double(p->n_tiles) * (nn * 2 * m->d + 2 * m->d) * ab);
    TS_HIP(tsk::attention_global(s, a, gscratch, gscratch_floats), "attention (global rows)");
  }
  return TS_OK;
}

// One pre-norm block on rows x [M, d] fp32.  shared: M = n_union + n_tiles and
// attention reads each tile through the plan's row map, then the w-bar blend
// forms one row per token; otherwise M = n_tiles*(n+1) per-tile rows.
// xq (per-tile layer only): shared-layout rows [n_union + n_tiles, d] of which
// every per-tile row of x is a copy (layer 0 of a stack); Norm1, QKV and
// QK-norm then run once per token on xq and attention reads each window
// through the row map (Table S1, layer 0: exact), while the out-projection,
// Norm2 and MLP run on the per-tile rows.
ts_status run_layer(const Ctx& c, const ts_layer_weights& w, float* x, bool shared, const WS& ws,
                    const float* xq = nullptr) {
  const ts_model_desc* m = c.m;
  const ts_plan* p = c.p;
  const int act = m->act_dtype;
  const int ab = act_bytes(act);
  const int64_t Mt = int64_t(p->n_tiles) * (p->n + 1);
  const int64_t Ms = int64_t(p->n_union) + p->n_tiles;
  const int64_t M = shared ? Ms : Mt;
  const bool qsh = shared || xq;        // Norm1 .. attention on shared-layout rows
  const int64_t Mq = qsh ? Ms : Mt;
  const float* xn = xq ? xq : x;
  const int d = m->d, H = m->n_heads, hd = m->head_dim, dm = m->mlp_hidden;
  const int f8 = fp8_mask(m, shared);
  const bool rms = m->norm == 1;
  ts_status st;
  // producers that take the max of an fp8 operand (see fused_amax)
  const bool fa = f8 != 0 && fused_amax();
  unsigned* am_qkv = fa && (f8 & TS_FP8_QKV) ? ws.amax : nullptr;
  unsigned* am_out = fa && (f8 & TS_FP8_OUT) ? ws.amax : nullptr;
  unsigned* am_fc1 = fa && (f8 & TS_FP8_FC1) ? ws.amax : nullptr;
  unsigned* am_fc2 = fa && (f8 & TS_FP8_FC2) ? ws.amax : nullptr;

  {
    if (am_qkv) TS_HIP(tsk::zero_amax(c.s, am_qkv), "amax reset");
    Scope sc(c.s, "norm", 0.0, double(Mq * d) * (4 + ab));
    TS_HIP(tsk::norm(c.s, act, rms, xn, int(Mq), d, w.norm1_g, w.norm1_b, m->eps, ws.h, am_qkv), "norm1");
  }
  if ((st = proj(c, ws, (f8 & TS_FP8_QKV) != 0, "qkv", tsk::EPI_BIAS, ws.h, Mq, 3 * d, d, w.w_qkv, w.w_qkv_f8,
                 w.w_scale_f8 ? w.w_scale_f8 + 0 : nullptr, w.b_qkv, ws.big, am_qkv != nullptr)) != TS_OK)
    return st;
  {
    Scope sc(c.s, "qk_prep", 0.0, double(Mq * 2 * d) * 2 * ab);
    TS_HIP(tsk::qk_prep(c.s, act, ws.big, int(Mq), d, H, hd, m->qk_norm ? w.q_g : nullptr, w.k_g, m->eps,
                        rope_rows(p, qsh), ws.qkn),
           "qk_prep");
  }
  // shared layers: the w-bar blend of the windows' outputs is formed by the
  // attention itself, straight into the out-projection's operand rows
  if (am_out) TS_HIP(tsk::zero_amax(c.s, am_out), "amax reset");
  const void* aout = shared ? ws.h : ws.o;
  if ((st = window_attention(m, p, shared ? ATT_BLENDED : (qsh ? ATT_SHARED_ROWS : ATT_TILED), ws.big,
                             const_cast<void*>(aout), (float*)ws.o, ws.jobs, am_out, c.s, ws.gpart,
                             ws.gpart_floats, w.q_g, w.k_g, ws.qkn)) != TS_OK)
    return st;
  if ((st = proj(c, ws, (f8 & TS_FP8_OUT) != 0, "out", tsk::EPI_RESID, aout, M, d, d, w.w_o, w.w_o_f8,
                 w.w_scale_f8 ? w.w_scale_f8 + 1 : nullptr, w.b_o, x, am_out != nullptr)) != TS_OK)
    return st;
  {
    if (am_fc1) TS_HIP(tsk::zero_amax(c.s, am_fc1), "amax reset");
    Scope sc(c.s, "norm", 0.0, double(M * d) * (4 + ab));
    TS_HIP(tsk::norm(c.s, act, rms, x, int(M), d, w.norm2_g, w.norm2_b, m->eps, ws.h, am_fc1), "norm2");
  }
  const int hp = int(mlp_pitch(m, (f8 & TS_FP8_FC2) != 0));
  if ((st = proj(c, ws, (f8 & TS_FP8_FC1) != 0, "fc1", tsk::EPI_BIAS_GELU, ws.h, M, dm, d, w.w_1, w.w_1_f8,
                 w.w_scale_f8 ? w.w_scale_f8 + 2 : nullptr, w.b_1, ws.big, am_fc1 != nullptr, am_fc2, 0, hp)) != TS_OK)
    return st;
  if ((st = proj(c, ws, (f8 & TS_FP8_FC2) != 0, "fc2", tsk::EPI_RESID, ws.big, M, d, dm, w.w_2, w.w_2_f8,
                 w.w_scale_f8 ? w.w_scale_f8 + 3 : nullptr, w.b_2, x, am_fc2 != nullptr, nullptr, hp)) != TS_OK)
    return st;
  return TS_OK;
}

// A layer on per-tile residual streams X [Mt, d] fp32 whose operations in
// `share` (TS_SHARE_Q: Norm1, QKV, QK-norm; TS_SHARE_O: out-projection;
// TS_SHARE_M: Norm2 and MLP) run once per token on the w-bar blend of the
// tiles' states (for the out-projection: of their attention outputs) and add
// their one result to every tile's stream (Table 1, Table S7).  Attention
// always runs per tile.
ts_status run_layer_partial(const Ctx& c, const ts_layer_weights& w, float* X, int share, const WS& ws) {
  const ts_model_desc* m = c.m;
  const ts_plan* p = c.p;
  const int act = m->act_dtype;
  const int ab = act_bytes(act);
  const int64_t Mt = int64_t(p->n_tiles) * (p->n + 1);
  const int64_t Ms = int64_t(p->n_union) + p->n_tiles;
  const int d = m->d, H = m->n_heads, hd = m->head_dim, dm = m->mlp_hidden;
  const bool rms = m->norm == 1;
  const bool sq = share & TS_SHARE_Q, so = share & TS_SHARE_O, sm = share & TS_SHARE_M;
  float* xg = ws.xs + size_t(p->n_union) * d;  // global rows of a blend into xs
  ts_status st;
  auto blend_states = [&]() -> ts_status {   // xs = w-bar blend of the streams
    Scope sc(c.s, "blend", 0.0, (double(p->n_entries + p->n_tiles) + double(Ms)) * d * 4);
    TS_HIP(tsk::blend(c.s, TS_F32, TS_F32, X, d, p->n_union, p->n_tiles, p->n, (const int*)p->d_cover_ptr,
                      (const int*)p->d_entry_row, (const float*)p->d_cover_w, ws.xs, xg),
           "blend");
    return TS_OK;
  };
  auto add_back = [&]() -> ts_status {        // every stream += its token's row of xs
    Scope sc(c.s, "add_to_tiles", 0.0, double(Mt) * d * 12);
    TS_HIP(tsk::add_to_tiles(c.s, X, ws.xs, (const int*)p->d_tile_rows, p->n_union, p->n_tiles, p->n, d),
           "add to tiles");
    return TS_OK;
  };

  // Norm1, QKV, QK-norm, attention
  const int64_t Mq = sq ? Ms : Mt;
  if (sq && (st = blend_states()) != TS_OK) return st;
  {
    Scope sc(c.s, "norm", 0.0, double(Mq * d) * (4 + ab));
    TS_HIP(tsk::norm(c.s, act, rms, sq ? ws.xs : X, int(Mq), d, w.norm1_g, w.norm1_b, m->eps, ws.h), "norm1");
  }
  if ((st = proj(c, ws, false, "qkv", tsk::EPI_BIAS, ws.h, Mq, 3 * d, d, w.w_qkv, nullptr, nullptr, w.b_qkv,
                 ws.big)) != TS_OK)
    return st;
  {
    Scope sc(c.s, "qk_prep", 0.0, double(Mq * 2 * d) * 2 * ab);
    TS_HIP(tsk::qk_prep(c.s, act, ws.big, int(Mq), d, H, hd, m->qk_norm ? w.q_g : nullptr, w.k_g, m->eps,
                        rope_rows(p, sq), ws.qkn),
           "qk_prep");
  }
  if ((st = window_attention(m, p, sq ? ATT_SHARED_ROWS : ATT_TILED, ws.big, ws.o, nullptr, nullptr, nullptr, c.s,
                             ws.gpart, ws.gpart_floats, w.q_g, w.k_g, ws.qkn)) != TS_OK)
    return st;
  // out-projection
  if (so) {
    {
      Scope sc(c.s, "blend", 0.0, (double(p->n_entries + p->n_tiles) + double(Ms)) * d * ab);
      TS_HIP(tsk::blend(c.s, act, act, ws.o, d, p->n_union, p->n_tiles, p->n, (const int*)p->d_cover_ptr,
                        (const int*)p->d_entry_row, (const float*)p->d_cover_w, ws.h,
                        (char*)ws.h + size_t(p->n_union) * d * ab),
             "blend");
    }
    if ((st = proj(c, ws, false, "out", tsk::EPI_F32, ws.h, Ms, d, d, w.w_o, nullptr, nullptr, w.b_o, ws.xs)) !=
        TS_OK)
      return st;
    if ((st = add_back()) != TS_OK) return st;
  } else if ((st = proj(c, ws, false, "out", tsk::EPI_RESID, ws.o, Mt, d, d, w.w_o, nullptr, nullptr, w.b_o, X)) !=
             TS_OK) {
    return st;
  }
  // Norm2 and MLP
  const int64_t Mm = sm ? Ms : Mt;
  if (sm && (st = blend_states()) != TS_OK) return st;
  {
    Scope sc(c.s, "norm", 0.0, double(Mm * d) * (4 + ab));
    TS_HIP(tsk::norm(c.s, act, rms, sm ? ws.xs : X, int(Mm), d, w.norm2_g, w.norm2_b, m->eps, ws.h), "norm2");
  }
  const int hp = int(mlp_pitch(m, false));
  if ((st = proj(c, ws, false, "fc1", tsk::EPI_BIAS_GELU, ws.h, Mm, dm, d, w.w_1, nullptr, nullptr, w.b_1,
                 ws.big, false, nullptr, 0, hp)) != TS_OK)
    return st;
  if (sm) {
    // the blended state in xs has been consumed by Norm2: xs takes the MLP result
    if ((st = proj(c, ws, false, "fc2", tsk::EPI_F32, ws.big, Ms, d, dm, w.w_2, nullptr, nullptr, w.b_2,
                   ws.xs, false, nullptr, hp)) != TS_OK)
      return st;
    return add_back();
  }
  return proj(c, ws, false, "fc2", tsk::EPI_RESID, ws.big, Mt, d, dm, w.w_2, nullptr, nullptr, w.b_2, X, false,
              nullptr, hp);
}

ts_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(TS_EWORKSPACE, "workspace is null");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(TS_EWORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(TS_EWORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes, got " +
                                   std::to_string(ws_bytes));
  return TS_OK;
}

ts_status stack_impl(const ts_model_desc* m, const ts_layer_weights* layers, const ts_plan* p, int32_t k,
                     const float* x_in, const float* g, float* x_out, float* g_out, void* ws,
                     size_t ws_bytes, void* stream) {
  ts_status st;
  if ((st = check_model(m)) != TS_OK) return st;
  if ((st = check_plan(p, m)) != TS_OK) return st;
  if (!layers && m->n_layers > 0) return fail(TS_EINVAL, "layers is null");
  if (k < 0 || k > m->n_layers) return fail(TS_EINVAL, "k must be in 0..n_layers");
  if (!x_in || !g || !x_out) return fail(TS_EINVAL, "x_in, g and x_out must be non-null");
  for (int l = 0; l < m->n_layers; ++l)
    if ((st = check_weights(m, &layers[l], l >= k)) != TS_OK) return st;
  const bool per_tile = k > 0;
  const bool shared_xs = k < m->n_layers;
  WS w0 = layout(m, p, true, per_tile, shared_xs, nullptr);
  if ((st = check_ws(ws, ws_bytes, w0.bytes)) != TS_OK) return st;
  WS w = layout(m, p, true, per_tile, shared_xs, (char*)ws);
  Ctx c{m, p, (hipStream_t)stream};
  const int d = m->d;
  const int64_t Mt = int64_t(p->n_tiles) * (p->n + 1);
  const int64_t Ms = int64_t(p->n_union) + p->n_tiles;
  if (per_tile) {
    {
      Scope sc(c.s, "gather", 0.0, double(Mt) * d * 8);
      TS_HIP(tsk::gather(c.s, x_in, g, 0, (const int*)p->d_tile_rows, p->n_tiles, p->n, d, w.X), "gather");
    }
    // layer-0 dedup: the shared-layout input rows (the tokens, then g once per tile)
    const float* x0 = nullptr;
    if (m->layer0_dedup) {
      Scope sc(c.s, "init_shared", 0.0, double(Ms) * d * 8);
      TS_HIP(tsk::init_shared(c.s, x_in, g, p->n_union, p->n_tiles, d, w.xs), "init");
      x0 = w.xs;
    }
    for (int l = 0; l < k; ++l)
      if ((st = run_layer(c, layers[l], w.X, false, w, l == 0 ? x0 : nullptr)) != TS_OK) return st;
    // merge into one shared state (or the output, for the tiled baseline)
    float* mu = shared_xs ? w.xs : x_out;
    float* mg = shared_xs ? w.xs + size_t(p->n_union) * d : g_out;
    Scope sc(c.s, "merge", 0.0, (double(p->n_entries + p->n_tiles) + double(Ms)) * d * 4);
    TS_HIP(tsk::blend(c.s, TS_F32, TS_F32, w.X, d, p->n_union, p->n_tiles, p->n, (const int*)p->d_cover_ptr,
                      (const int*)p->d_entry_row, (const float*)p->d_cover_w, mu, mg),
           "merge");
  } else {
    Scope sc(c.s, "init_shared", 0.0, double(Ms) * d * 8);
    TS_HIP(tsk::init_shared(c.s, x_in, g, p->n_union, p->n_tiles, d, w.xs), "init");
  }
  if (shared_xs) {
    for (int l = k; l < m->n_layers; ++l)
      if ((st = run_layer(c, layers[l], w.xs, true, w)) != TS_OK) return st;
    Scope sc(c.s, "copy_out", 0.0, double(Ms) * d * 8);
    TS_HIP(tsk::copy_f32(c.s, w.xs, x_out, int64_t(p->n_union) * d), "copy out");
    if (g_out) TS_HIP(tsk::copy_f32(c.s, w.xs + size_t(p->n_union) * d, g_out, int64_t(p->n_tiles) * d), "copy g");
  }
  return TS_OK;
}

// Figure 3b: per-tile layers 0 .. l-1, one merge of the per-tile states
// into one state (global rows kept per tile), every tile re-gathered from
// that state (its own global row included), per-tile layers l .. L-1, and
// the final merge.
ts_status merge_once_impl(const ts_model_desc* m, const ts_layer_weights* layers, const ts_plan* p, int32_t l,
                          const float* x_in, const float* g, float* x_out, float* g_out, void* ws,
                          size_t ws_bytes, void* stream) {
  ts_status st;
  if ((st = check_model(m)) != TS_OK) return st;
  if ((st = check_plan(p, m)) != TS_OK) return st;
  if (!layers && m->n_layers > 0) return fail(TS_EINVAL, "layers is null");
  if (l < 0 || l > m->n_layers) return fail(TS_EINVAL, "l must be in 0..n_layers");
  if (!x_in || !g || !x_out) return fail(TS_EINVAL, "x_in, g and x_out must be non-null");
  for (int i = 0; i < m->n_layers; ++i)
    if ((st = check_weights(m, &layers[i], false)) != TS_OK) return st;
  WS w0 = layout(m, p, true, true, true, nullptr);
  if ((st = check_ws(ws, ws_bytes, w0.bytes)) != TS_OK) return st;
  WS w = layout(m, p, true, true, true, (char*)ws);
  Ctx c{m, p, (hipStream_t)stream};
  const int d = m->d;
  const int64_t Mt = int64_t(p->n_tiles) * (p->n + 1);
  const int64_t Ms = int64_t(p->n_union) + p->n_tiles;
  const double merge_bytes = (double(p->n_entries + p->n_tiles) + double(Ms)) * d * 4;
  auto merge = [&](float* mu, float* mg) -> ts_status {
    Scope sc(c.s, "merge", 0.0, merge_bytes);
    TS_HIP(tsk::blend(c.s, TS_F32, TS_F32, w.X, d, p->n_union, p->n_tiles, p->n, (const int*)p->d_cover_ptr,
                      (const int*)p->d_entry_row, (const float*)p->d_cover_w, mu, mg),
           "merge");
    return TS_OK;
  };
  {
    Scope sc(c.s, "gather", 0.0, double(Mt) * d * 8);
    TS_HIP(tsk::gather(c.s, x_in, g, 0, (const int*)p->d_tile_rows, p->n_tiles, p->n, d, w.X), "gather");
  }
  // layer-0 dedup: layer 0's per-tile rows are copies of the input rows (l >= 1)
  // or, after a merge at l = 0, of the merged rows
  const float* x0 = nullptr;
  if (m->layer0_dedup && l > 0) {
    Scope sc(c.s, "init_shared", 0.0, double(Ms) * d * 8);
    TS_HIP(tsk::init_shared(c.s, x_in, g, p->n_union, p->n_tiles, d, w.xs), "init");
    x0 = w.xs;
  }
  for (int i = 0; i < l; ++i)
    if ((st = run_layer(c, layers[i], w.X, false, w, i == 0 ? x0 : nullptr)) != TS_OK) return st;
  if ((st = merge(w.xs, w.xs + size_t(p->n_union) * d)) != TS_OK) return st;
  {
    Scope sc(c.s, "gather", 0.0, double(Mt) * d * 8);
    TS_HIP(tsk::gather(c.s, w.xs, w.xs + size_t(p->n_union) * d, d, (const int*)p->d_tile_rows, p->n_tiles,
                       p->n, d, w.X),
           "re-gather");
  }
  for (int i = l; i < m->n_layers; ++i)
    if ((st = run_layer(c, layers[i], w.X, false, w, i == 0 && m->layer0_dedup ? w.xs : nullptr)) != TS_OK)
      return st;
  return merge(x_out, g_out);
}

// Table 1 (top) / Table S7: per-tile layers 0 .. k-1, then per-tile residual
// streams with the operations in `share` run once per token, then the merge.
ts_status partial_share_impl(const ts_model_desc* m, const ts_layer_weights* layers, const ts_plan* p, int32_t k,
                             int32_t share, const float* x_in, const float* g, float* x_out, float* g_out,
                             void* ws, size_t ws_bytes, void* stream) {
  ts_status st;
  if ((st = check_model(m)) != TS_OK) return st;
  if ((st = check_plan(p, m)) != TS_OK) return st;
  if (m->gemm_dtype_shared == TS_FP8E4M3) return fail(TS_EUNSUPPORTED, "partial sharing runs bf16 / fp32 GEMMs only");
  if (!layers && m->n_layers > 0) return fail(TS_EINVAL, "layers is null");
  if (k < 0 || k > m->n_layers) return fail(TS_EINVAL, "k must be in 0..n_layers");
  if (share < 0 || share > (TS_SHARE_Q | TS_SHARE_O | TS_SHARE_M))
    return fail(TS_EINVAL, "share must be a mask of TS_SHARE_* bits");
  if (!x_in || !g || !x_out) return fail(TS_EINVAL, "x_in, g and x_out must be non-null");
  for (int i = 0; i < m->n_layers; ++i)
    if ((st = check_weights(m, &layers[i], false)) != TS_OK) return st;
  WS w0 = layout(m, p, true, true, true, nullptr);
  if ((st = check_ws(ws, ws_bytes, w0.bytes)) != TS_OK) return st;
  WS w = layout(m, p, true, true, true, (char*)ws);
  Ctx c{m, p, (hipStream_t)stream};
  const int d = m->d;
  const int64_t Mt = int64_t(p->n_tiles) * (p->n + 1);
  const int64_t Ms = int64_t(p->n_union) + p->n_tiles;
  {
    Scope sc(c.s, "gather", 0.0, double(Mt) * d * 8);
    TS_HIP(tsk::gather(c.s, x_in, g, 0, (const int*)p->d_tile_rows, p->n_tiles, p->n, d, w.X), "gather");
  }
  const float* x0 = nullptr;   // layer-0 dedup (per-tile layer 0 only)
  if (m->layer0_dedup && k > 0) {
    Scope sc(c.s, "init_shared", 0.0, double(Ms) * d * 8);
    TS_HIP(tsk::init_shared(c.s, x_in, g, p->n_union, p->n_tiles, d, w.xs), "init");
    x0 = w.xs;
  }
  for (int i = 0; i < k; ++i)
    if ((st = run_layer(c, layers[i], w.X, false, w, i == 0 ? x0 : nullptr)) != TS_OK) return st;
  for (int i = k; i < m->n_layers; ++i)
    if ((st = run_layer_partial(c, layers[i], w.X, share, w)) != TS_OK) return st;
  Scope sc(c.s, "merge", 0.0, (double(p->n_entries + p->n_tiles) + double(Ms)) * d * 4);
  TS_HIP(tsk::blend(c.s, TS_F32, TS_F32, w.X, d, p->n_union, p->n_tiles, p->n, (const int*)p->d_cover_ptr,
                    (const int*)p->d_entry_row, (const float*)p->d_cover_w, x_out, g_out),
         "merge");
  return TS_OK;
}

ts_status check_op_attention(const ts_model_desc* m, const ts_plan* p, void* qkv, const float* q_g,
                             const float* k_g, void* out) {
  ts_status st;
  if ((st = check_model(m)) != TS_OK) return st;
  if ((st = check_plan(p, m)) != TS_OK) return st;
  if (!qkv || !out) return fail(TS_EINVAL, "qkv and out must be non-null");
  if (m->qk_norm && (!q_g || !k_g)) return fail(TS_EINVAL, "QK-norm needs q_g and k_g");
  return TS_OK;
}

// The attention step on caller rows: qk_prep in place, then the window
// attention (blended when shared), with the partial blends in `part` (fp32
// [n_union, d], shared only) and the global rows' split states in gpart.
ts_status op_attention_impl(const ts_model_desc* m, const ts_plan* p, bool shared, void* qkv, const float* q_g,
                            const float* k_g, void* out, float* part, unsigned* jobs, unsigned* qkn, float* gpart,
                            int64_t gpart_floats, hipStream_t s) {
  const int64_t M = shared ? int64_t(p->n_union) + p->n_tiles : int64_t(p->n_tiles) * (p->n + 1);
  {
    Scope sc(s, "qk_prep", 0.0, double(M * 2 * m->d) * 2 * act_bytes(m->act_dtype));
    TS_HIP(tsk::qk_prep(s, m->act_dtype, qkv, int(M), m->d, m->n_heads, m->head_dim, m->qk_norm ? q_g : nullptr, k_g,
                        m->eps, rope_rows(p, shared), qkn),
           "qk_prep");
  }
  return window_attention(m, p, shared ? ATT_BLENDED : ATT_TILED, qkv, out, part, jobs, nullptr, s, gpart,
                          gpart_floats, q_g, k_g, qkn);
}

// ---- scratch of the no-allocation entry point --------------------------
// A file-scope device array: every GPU the library runs on holds its own
// copy until the process ends.  In host code its name is not a device
// address; the address is taken once per device with hipGetSymbolAddress
// (with that device current) and kept.
__device__ __align__(256) unsigned char scratch[TS_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
std::map<int, char*> g_scratch_ptr;

ts_status noalloc_scratch(char** out) {
  int dev = 0;
  TS_HIP(hipGetDevice(&dev), "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    TS_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    it = g_scratch_ptr.emplace(dev, (char*)ptr).first;
  }
  *out = it->second;
  return TS_OK;
}

}  // namespace

extern "C" {

int32_t ts_abi_version(void) { return TS_ABI_VERSION; }
const char* ts_last_error(void) { return g_err.c_str(); }

ts_status ts_plan_create(const ts_tiling_desc* desc, ts_plan** out) {
  if (!desc || !out) return fail(TS_EINVAL, "desc and out must be non-null");
  *out = nullptr;
  ts_plan* p = new (std::nothrow) ts_plan();
  if (!p) return fail(TS_ENOMEM, "host allocation failed");
  std::string err;
  try {
    err = tsplan::build(*desc, *p);
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(TS_ENOMEM, "host allocation failed");
  }
  if (!err.empty()) {
    delete p;
    return fail(TS_EINVAL, err);
  }
  *out = p;
  return TS_OK;
}

ts_status ts_plan_get_info(const ts_plan* p, ts_plan_info* out) {
  if (!p || !out) return fail(TS_EINVAL, "plan and out must be non-null");
  out->n_tiles = p->n_tiles;
  out->tile_tokens = p->n;
  out->n_union = p->n_union;
  out->n_entries = p->n_entries;
  out->max_cover = p->max_cover;
  for (int a = 0; a < 3; ++a) out->extent[a] = p->ext[a];
  return TS_OK;
}

ts_status ts_plan_export(const ts_plan* p, int32_t* tile_start, int32_t* tile_rows, int32_t* cover_ptr,
                         int32_t* cover_tile, int32_t* cover_local, float* cover_w) {
  if (!p) return fail(TS_EINVAL, "plan is null");
  if (tile_start) std::memcpy(tile_start, p->tile_start.data(), p->tile_start.size() * 4);
  if (tile_rows) std::memcpy(tile_rows, p->tile_rows.data(), p->tile_rows.size() * 4);
  if (cover_ptr) std::memcpy(cover_ptr, p->cover_ptr.data(), p->cover_ptr.size() * 4);
  if (cover_tile) std::memcpy(cover_tile, p->cover_tile.data(), p->cover_tile.size() * 4);
  if (cover_local) std::memcpy(cover_local, p->cover_local.data(), p->cover_local.size() * 4);
  if (cover_w) std::memcpy(cover_w, p->cover_w.data(), p->cover_w.size() * 4);
  return TS_OK;
}

ts_status ts_plan_export_rope(const ts_plan* p, int32_t head_dim, float rope_base, float* cos_out,
                              float* sin_out) {
  if (!p || !cos_out || !sin_out) return fail(TS_EINVAL, "null argument");
  if (head_dim <= 0 || head_dim % 2 != 0) return fail(TS_EINVAL, "head_dim must be even and positive");
  tsplan::rope_local(*p, head_dim, rope_base, cos_out, sin_out);
  return TS_OK;
}

ts_status ts_plan_export_blocks(const ts_plan* p, int32_t* nblk, int32_t* maxc, int32_t* blk_nt, int32_t* blk_tiles,
                                int32_t* blk_rows, float* blk_w) {
  if (!p) return fail(TS_EINVAL, "plan is null");
  static_assert(TS_QBLOCK == tsk::QBLOCK, "plan and kernel query blocks");
  if (nblk) *nblk = p->nblk;
  if (maxc) *maxc = p->blk_maxc;
  if (blk_nt) std::memcpy(blk_nt, p->blk_nt.data(), p->blk_nt.size() * 4);
  if (blk_tiles) std::memcpy(blk_tiles, p->blk_tiles.data(), p->blk_tiles.size() * 4);
  if (blk_rows) std::memcpy(blk_rows, p->blk_rows.data(), p->blk_rows.size() * 4);
  if (blk_w) std::memcpy(blk_w, p->blk_w.data(), p->blk_w.size() * 4);
  return TS_OK;
}

ts_status ts_plan_export_job_order(const ts_plan* p, int32_t* ncls, int32_t* order, int32_t* cls) {
  if (!p) return fail(TS_EINVAL, "plan is null");
  if (ncls) *ncls = p->blk_ncls;
  if (order) std::memcpy(order, p->blk_order.data(), p->blk_order.size() * 4);
  if (cls) std::memcpy(cls, p->blk_cls.data(), p->blk_cls.size() * 4);
  return TS_OK;
}

static void free_device(ts_plan* p) {
  void** ptrs[] = {&p->d_tile_rows, &p->d_tile_rows_local, &p->d_cover_ptr, &p->d_entry_row, &p->d_cover_w, &p->d_local_pos,
                   &p->d_rope_glob, &p->d_tile_start, &p->d_blk_nt,    &p->d_blk_tiles, &p->d_blk_rows,
                   &p->d_blk_w,    &p->d_blk_order, &p->d_blk_cls};
  for (void** q : ptrs) {
    if (*q) (void)hipFree(*q);
    *q = nullptr;
  }
  p->uploaded = false;
}

ts_status ts_plan_upload(ts_plan* p, int32_t head_dim, float rope_base, void* stream) {
  if (!p) return fail(TS_EINVAL, "plan is null");
  if (head_dim <= 0 || head_dim % 2 != 0 || head_dim > 256) return fail(TS_EINVAL, "bad head_dim");
  int32_t pairs[3];
  tsplan::rope_pairs(p->desc.ndim, head_dim, pairs);
  std::vector<float> gtab;
  int32_t goff[3];
  tsplan::rope_table_global(*p, head_dim, rope_base, gtab, goff);
  std::vector<int32_t> entry_row(p->n_entries);
  for (int32_t e = 0; e < p->n_entries; ++e) entry_row[e] = p->cover_tile[e] * (p->n + 1) + p->cover_local[e];
  std::vector<int32_t> rows_local(size_t(p->n_tiles) * p->n);
  for (int32_t t = 0; t < p->n_tiles; ++t)
    for (int32_t j = 0; j < p->n; ++j) rows_local[size_t(t) * p->n + j] = t * (p->n + 1) + j;
  free_device(p);
  hipStream_t s = (hipStream_t)stream;
  struct Item {
    void** dst;
    const void* src;
    size_t bytes;
  } items[] = {
      {&p->d_tile_rows, p->tile_rows.data(), p->tile_rows.size() * 4},
      {&p->d_tile_rows_local, rows_local.data(), rows_local.size() * 4},
      {&p->d_cover_ptr, p->cover_ptr.data(), p->cover_ptr.size() * 4},
      {&p->d_entry_row, entry_row.data(), entry_row.size() * 4},
      {&p->d_cover_w, p->cover_w.data(), p->cover_w.size() * 4},
      {&p->d_local_pos, p->local_pos.data(), p->local_pos.size() * 4},
      {&p->d_rope_glob, gtab.data(), gtab.size() * 4},
      {&p->d_tile_start, p->tile_start.data(), p->tile_start.size() * 4},
      {&p->d_blk_nt, p->blk_nt.data(), p->blk_nt.size() * 4},
      {&p->d_blk_tiles, p->blk_tiles.data(), p->blk_tiles.size() * 4},
      {&p->d_blk_rows, p->blk_rows.data(), p->blk_rows.size() * 4},
      {&p->d_blk_w, p->blk_w.data(), p->blk_w.size() * 4},
      {&p->d_blk_order, p->blk_order.data(), p->blk_order.size() * 4},
      {&p->d_blk_cls, p->blk_cls.data(), p->blk_cls.size() * 4},
  };
  for (auto& it : items) {
    if (hipMalloc(it.dst, std::max<size_t>(it.bytes, 4)) != hipSuccess) {
      free_device(p);
      return fail(TS_ENOMEM, "device allocation for the plan failed");
    }
    hipError_t e = hipMemcpyAsync(*it.dst, it.src, it.bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) {
      free_device(p);
      return fail(TS_EHIP, std::string("plan upload: ") + hipGetErrorString(e));
    }
  }
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    free_device(p);
    return fail(TS_EHIP, std::string("plan upload sync: ") + hipGetErrorString(e));
  }
  for (int a = 0; a < 3; ++a) {
    p->rope_pairs[a] = pairs[a];
    p->rope_glob_off[a] = goff[a];
  }
  p->rope_hd = head_dim;
  p->rope_base = rope_base;
  p->uploaded = true;
  return TS_OK;
}

void ts_plan_destroy(ts_plan* p) {
  if (!p) return;
  free_device(p);
  delete p;
}

ts_status ts_workspace_size(const ts_model_desc* m, const ts_plan* p, int32_t k, size_t* bytes) {
  ts_status st;
  if ((st = check_model(m)) != TS_OK) return st;
  if (!p || !bytes) return fail(TS_EINVAL, "plan and bytes must be non-null");
  if (k < -1 || k > m->n_layers) return fail(TS_EINVAL, "k must be in -1..n_layers");
  // the larger of what the stack (with k; -1: ts_merge_once_forward, which
  // holds per-tile and merged states) and a single shared layer need
  WS a = k < 0 ? layout(m, p, true, true, true, nullptr) : layout(m, p, true, k > 0, k < m->n_layers, nullptr);
  WS b = layout(m, p, false, false, false, nullptr);
  *bytes = std::max(a.bytes, b.bytes);
  return TS_OK;
}

ts_status ts_shared_layer_forward(const ts_model_desc* m, const ts_layer_weights* w, const ts_plan* p,
                                  float* x, void* ws, size_t ws_bytes, void* stream) {
  ts_status st;
  if ((st = check_model(m)) != TS_OK) return st;
  if ((st = check_plan(p, m)) != TS_OK) return st;
  if ((st = check_weights(m, w, true)) != TS_OK) return st;
  if (!x) return fail(TS_EINVAL, "x is null");
  WS w0 = layout(m, p, false, false, false, nullptr);
  if ((st = check_ws(ws, ws_bytes, w0.bytes)) != TS_OK) return st;
  WS wl = layout(m, p, false, false, false, (char*)ws);
  Ctx c{m, p, (hipStream_t)stream};
  return run_layer(c, *w, x, true, wl);
}

ts_status ts_stack_forward(const ts_model_desc* m, const ts_layer_weights* layers, const ts_plan* p,
                           int32_t k, const float* x_in, const float* g, float* x_out, float* g_out,
                           void* ws, size_t ws_bytes, void* stream) {
  return stack_impl(m, layers, p, k, x_in, g, x_out, g_out, ws, ws_bytes, stream);
}

ts_status ts_merge_once_forward(const ts_model_desc* m, const ts_layer_weights* layers, const ts_plan* p,
                                int32_t l, const float* x_in, const float* g, float* x_out, float* g_out, void* ws,
                                size_t ws_bytes, void* stream) {
  return merge_once_impl(m, layers, p, l, x_in, g, x_out, g_out, ws, ws_bytes, stream);
}

ts_status ts_partial_share_forward(const ts_model_desc* m, const ts_layer_weights* layers, const ts_plan* p,
                                   int32_t k, int32_t share, const float* x_in, const float* g, float* x_out,
                                   float* g_out, void* ws, size_t ws_bytes, void* stream) {
  return partial_share_impl(m, layers, p, k, share, x_in, g, x_out, g_out, ws, ws_bytes, stream);
}

ts_status ts_tiled_forward(const ts_model_desc* m, const ts_layer_weights* layers, const ts_plan* p,
                           const float* x_in, const float* g, float* x_out, float* g_out, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!m) return fail(TS_EINVAL, "model is null");
  return stack_impl(m, layers, p, m->n_layers, x_in, g, x_out, g_out, ws, ws_bytes, stream);
}

ts_status ts_fp8_quantize(const void* src, int32_t src_dtype, int64_t n, uint8_t* dst, float* scale,
                          void* ws, size_t ws_bytes, void* stream) {
  if (!src || !dst || !scale) return fail(TS_EINVAL, "null argument");
  if (src_dtype != TS_F32 && src_dtype != TS_BF16) return fail(TS_EDTYPE, "src_dtype must be TS_F32 or TS_BF16");
  if (n <= 0) return fail(TS_EINVAL, "n must be positive");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 8 != 0)
    return fail(TS_EINVAL, "src must be 16-byte and dst 8-byte aligned");
  ts_status st;
  if ((st = check_ws(ws, ws_bytes, 256)) != TS_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  Scope sc(s, "fp8_quantize", 0.0, double(n) * (2.0 * act_bytes(src_dtype) + 1.0));
  TS_HIP(tsk::fp8_quantize(s, src_dtype, src, n, dst, scale, (unsigned*)ws), "fp8 quantize");
  return TS_OK;
}

ts_status ts_op_gemm(int32_t dtype, int32_t epilogue, const void* a, const void* b, int32_t m, int32_t n,
                     int32_t k, const float* bias, void* c, const float* scale_a, const float* scale_b,
                     void* stream) {
  return ts_op_gemm_ws(dtype, epilogue, a, b, m, n, k, bias, c, scale_a, scale_b, nullptr, 0, stream);
}

ts_status ts_op_gemm_ws(int32_t dtype, int32_t epilogue, const void* a, const void* b, int32_t m, int32_t n,
                        int32_t k, const float* bias, void* c, const float* scale_a, const float* scale_b,
                        void* ws, size_t ws_bytes, void* stream) {
  if (ws && reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(TS_EWORKSPACE, "workspace must be 256-byte aligned");
  if (!a || !b || !c) return fail(TS_EINVAL, "a, b and c must be non-null");
  if (m < 0 || n <= 0 || k <= 0) return fail(TS_EINVAL, "bad GEMM sizes");
  if (epilogue < 0 || epilogue > 3) return fail(TS_EINVAL, "bad epilogue");
  if (dtype == TS_BF16 && (k % 64 != 0 || n % 16 != 0)) return fail(TS_ESHAPE, "bf16 GEMM needs k % 64 == 0, n % 16 == 0");
  if (dtype == TS_FP8E4M3 && (k % 128 != 0 || n % 16 != 0)) return fail(TS_ESHAPE, "fp8 GEMM needs k % 128 == 0, n % 16 == 0");
  if (dtype == TS_FP8E4M3 && (!scale_a || !scale_b)) return fail(TS_EINVAL, "fp8 GEMM needs both scales");
  if (dtype != TS_F32 && !gemm_offsets_fit(m, n, k, dtype == TS_BF16 ? 2 : 1))
    return fail(TS_ESHAPE, "GEMM operand larger than 4 GiB");
  if (dtype != TS_F32 && dtype != TS_BF16 && dtype != TS_FP8E4M3) return fail(TS_EDTYPE, "bad dtype");
  hipStream_t s = (hipStream_t)stream;
  const int ab = act_bytes(dtype);
  const int ob = (epilogue >= 2 || dtype == TS_F32) ? 4 : 2;
  Scope sc(s, dtype == TS_F32 ? "gemm_f32" : (dtype == TS_BF16 ? "gemm_bf16" : "gemm_fp8"), 2.0 * m * n * k,
           gemm_bytes(m, n, k, ab, ob, epilogue == TS_EPI_RESIDUAL));
  TS_HIP(tsk::gemm(s, dtype == TS_F32 ? tsk::ACT_F32 : (dtype == TS_BF16 ? tsk::ACT_BF16 : tsk::ACT_FP8), epilogue,
                   a, b, m, n, k, bias, c, scale_a, scale_b, (float*)ws, ws ? ws_bytes : 0),
         "gemm");
  return TS_OK;
}

ts_status ts_op_attention(const ts_model_desc* m, const ts_plan* p, int32_t shared, void* qkv, const float* q_g,
                          const float* k_g, void* out, void* ws, size_t ws_bytes, void* stream) {
  ts_status st;
  if ((st = check_op_attention(m, p, qkv, q_g, k_g, out)) != TS_OK) return st;
  WS w0 = layout(m, p, false, false, false, nullptr);
  if ((st = check_ws(ws, ws_bytes, w0.bytes)) != TS_OK) return st;
  WS w = layout(m, p, false, false, false, (char*)ws);
  return op_attention_impl(m, p, shared != 0, qkv, q_g, k_g, out, (float*)w.o, w.jobs, w.qkn, w.gpart,
                           w.gpart_floats, (hipStream_t)stream);
}

ts_status ts_op_attention_noalloc(const ts_model_desc* m, const ts_plan* p, int32_t shared, void* qkv,
                                  const float* q_g, const float* k_g, void* out, void* stream) {
  ts_status st;
  if ((st = check_op_attention(m, p, qkv, q_g, k_g, out)) != TS_OK) return st;
  // the job counters and the two largest head norms, then the fp32 partial
  // blends of the shared layout, the global rows' split states in the rest
  // (the split count shrinks to what fits)
  const size_t jobs_bytes = tsk::JOB_COUNTERS_BYTES + tsk::QKN_BYTES;
  const size_t part_bytes = shared ? align256(size_t(p->n_union) * m->d * 4) : 0;
  if (jobs_bytes + part_bytes > TS_NOALLOC_SCRATCH_BYTES)
    return fail(TS_EWORKSPACE, "ts_op_attention_noalloc: the partial blends need " + std::to_string(part_bytes) +
                                   " bytes; its scratch holds " +
                                   std::to_string(TS_NOALLOC_SCRATCH_BYTES - jobs_bytes));
  char* base = nullptr;
  if ((st = noalloc_scratch(&base)) != TS_OK) return st;
  const int64_t gfloats = int64_t((TS_NOALLOC_SCRATCH_BYTES - jobs_bytes - part_bytes) / 4);
  unsigned* qkn =
      m->act_dtype == TS_BF16 && !m->qk_norm ? (unsigned*)(base + tsk::JOB_COUNTERS_BYTES) : nullptr;
  return op_attention_impl(m, p, shared != 0, qkv, q_g, k_g, out, (float*)(base + jobs_bytes), (unsigned*)base, qkn,
                           (float*)(base + jobs_bytes + part_bytes), gfloats, (hipStream_t)stream);
}

ts_status ts_profile_begin(void) {
  g_prof.on = true;
  return TS_OK;
}

ts_status ts_profile_end(ts_kernel_stat* out, int32_t max_records, int32_t* n_records) {
  g_prof.on = false;
  std::map<std::string, ts_kernel_stat> agg;
  std::vector<std::string> order;
  ts_status result = TS_OK;
  for (auto& r : g_prof.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      result = fail(TS_EHIP, "profile event query failed");
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      ts_kernel_stat z{};
      std::snprintf(z.name, sizeof(z.name), "%s", r.name.c_str());
      it = agg.emplace(r.name, z).first;
      order.push_back(r.name);
    }
    it->second.launches += 1;
    it->second.total_ms += ms;
    it->second.flops += r.flops;
    it->second.bytes += r.bytes;
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  int32_t nrec = 0;
  for (auto& name : order) {
    if (out && nrec < max_records) out[nrec] = agg[name];
    ++nrec;
  }
  if (n_records) *n_records = std::min<int32_t>(nrec, max_records);
  return result;
}

}  // extern "C"
