// Window attention of the TileShare layer (Figure 2 caption and Table S1:
// attention still runs per released tile, with the tile's own global token
// and coordinates; in shared layers keys and values come from the shared
// states, and an overlap token's per-tile outputs are blended with w-bar).
//
// q and k arrive normalised and rotated by qk_prep, which rotates every row
// once by its grid coordinate (a tile's global row by the tile's start): a
// score depends only on the two coordinates' difference, the same in every
// tile, so rows are read in place and no per-tile copies are made.  In bf16
// q also carries the softmax scale log2(e)/sqrt(hd), so q.k is a score in the
// log2 domain of the exponentials.
//
// Three layouts of the query rows and outputs:
//  - per tile: qkv rows and outputs t*(n+1)+i (tile t's window token i, its
//    global token i = n);
//  - shared, per-tile outputs: keys and queries read from the shared
//    [n_union + n_tiles] rows through the tile map, outputs per tile (layer 0
//    of a stack run once per token);
//  - shared, blended (shared layers): the plan's query blocks group rows by
//    the tiles that hold them; a block is attended in each of its windows in
//    turn and the per-window outputs are added with their w-bar weights in
//    ascending tile order, so the blended row a[p] = sum_t w_t o_t is written
//    once (global rows: their tile's output, weight 1).
//
// bf16 kernel (gfx950 MFMA 32x32x16): a workgroup of eight wavefronts owns
// 256 query rows of one head, 32 per wavefront, and streams every window it
// attends in blocks of 64 keys, each block staged once for all of them.
// Scores are formed transposed, S^T = K Q^T, so each lane holds one query's
// scores and the softmax max/sum stay in-lane (plus one exchange with the
// lane 32 apart); the output is accumulated transposed, O^T = V^T P^T, so the
// per-query rescale is in-lane too.  K rows are fed to the MFMA in an order
// that swaps bits 2 and 3 of the row index, which makes the score accumulator
// layout equal the P^T operand layout of the second MFMA (no shuffles).  K
// and V blocks go from the qkv rows straight into LDS ([key][hd], 16-byte
// chunks XOR-swizzled by key) with global_load_lds, three blocks in flight;
// V^T fragments are read with the transposing LDS load ds_read_b64_tr_b16,
// so V is never copied transposed.  The key rows of a window come through an
// eight-slot LDS ring filled five blocks ahead.  The windows of a query block
// form one stream of key blocks, so the staging runs on across windows.  The
// score MFMA chains start from the softmax offset (-m), so a weight is one
// exponential of an accumulator; under QK-norm that offset is a static bound
// on the scores and needs no running max.
#include <algorithm>
#include <cstdlib>
#include <map>
#include <tuple>
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "ts_kernels.h"

namespace {

struct AttnP {
  const void* qkv;
  void* out;
  float* part;
  const int* rows;
  int g0, gstep;
  const int* blk_nt;
  const int* blk_tiles;
  const int* blk_rows;
  const float* blk_w;
  int nblk, maxc;
  const int* blk_order;
  const int* blk_cls;
  int ncls, half_a;
  unsigned* jobs;
  int n_union, d, H, n_tiles, n;
  float scale_log2;  // log2(e) / sqrt(hd)
  unsigned* amax;
  const float* qg;   // QK-norm gains [hd] or null
  const float* kg;
  const unsigned* qkn;  // without QK-norm: largest q and k head norms (float bits) or null
};

constexpr int QB = 256;  // query rows per workgroup (both kernels)

// qkv row of window token j < n of tile t, and of tile t's global token
__device__ __forceinline__ int key_row(const AttnP& p, int t, int j) { return p.rows[int64_t(t) * p.n + j]; }
__device__ __forceinline__ int gkey_row(const AttnP& p, int t) { return p.g0 + p.gstep * t; }
// output row of tile t's global query
__device__ __forceinline__ int gout_row(const AttnP& p, int t) { return p.blk_nt ? p.n_union + t : t * (p.n + 1) + p.n; }

// Wavefront max of m (all 64 lanes), then one atomic max in float bits
// (values >= 0) into one of the tsk::AMAX_SLOTS slots.
__device__ __forceinline__ void wave_amax(unsigned* amax, float m, int slot_seed) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0)
    atomicMax(amax + (slot_seed & (tsk::AMAX_SLOTS - 1)) * tsk::AMAX_STRIDE, __float_as_uint(m));
}

// ------------------------------------------------------------- fp32 -----
// One thread per query row, 256 per workgroup, keys staged through LDS 64 at
// a time.  Workgroups [0, njob) take query blocks, the next n_tiles the
// global query rows (thread 0).  blockIdx.y is the head.
template <int HD, bool BLEND>
__global__ __launch_bounds__(QB) void k_attn_f32(AttnP p) {
  __shared__ float Ks[64][HD + 1];
  __shared__ float Vs[64][HD + 1];
  const int h = blockIdx.y, tid = threadIdx.x, n = p.n, b = blockIdx.x;
  const int nqb = (n + QB - 1) / QB;
  const int njob = BLEND ? p.nblk : p.n_tiles * nqb;
  const float* qkv = (const float*)p.qkv;
  const int64_t ld = 3 * int64_t(p.d);
  const bool tok = b < njob;
  int npass = 1, t0 = 0, qrow, orow;
  bool valid;
  if (!tok) {
    t0 = b - njob;
    valid = tid == 0;
    qrow = gkey_row(p, t0);
    orow = gout_row(p, t0);
  } else if (BLEND) {
    npass = p.blk_nt[b];
    const int r = p.blk_rows[b * QB + tid];
    valid = r >= 0;
    qrow = valid ? r : p.blk_rows[b * QB];
    orow = qrow;
  } else {
    t0 = b / nqb;
    const int qi = (b % nqb) * QB + tid;
    valid = qi < n;
    qrow = key_row(p, t0, min(qi, n - 1));
    orow = t0 * (n + 1) + qi;
  }
  float q[HD], o[HD], acc[HD];
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    q[e] = qkv[qrow * ld + h * HD + e];
    acc[e] = 0.f;
  }
  const float scale = 1.0f / sqrtf(float(HD));
  for (int ps = 0; ps < npass; ++ps) {
    const int t = (BLEND && tok) ? p.blk_tiles[b * p.maxc + ps] : t0;
    // the global key is the initial state: score, weight 1, value
    const int64_t gr = gkey_row(p, t);
    float sg = 0.f;
#pragma unroll
    for (int e = 0; e < HD; ++e) sg += q[e] * qkv[gr * ld + p.d + h * HD + e];
    float m = sg * scale, l = 1.f;
#pragma unroll
    for (int e = 0; e < HD; ++e) o[e] = qkv[gr * ld + 2 * p.d + h * HD + e];
    for (int j0 = 0; j0 < n; j0 += 64) {
      __syncthreads();
      {  // stage keys j0 .. j0+63, four threads per key
        const int kk = tid >> 2, part = tid & 3, j = j0 + kk;
        if (j < n) {
          const int64_t r = key_row(p, t, j);
          for (int e = part; e < HD; e += 4) {
            Ks[kk][e] = qkv[r * ld + p.d + h * HD + e];
            Vs[kk][e] = qkv[r * ld + 2 * p.d + h * HD + e];
          }
        }
      }
      __syncthreads();
      const int jn = min(64, n - j0);
      for (int jj = 0; jj < jn; ++jj) {
        float sc = 0.f;
#pragma unroll
        for (int e = 0; e < HD; ++e) sc += q[e] * Ks[jj][e];
        sc *= scale;
        const float mn = fmaxf(m, sc);
        const float al = expf(m - mn), pj = expf(sc - mn);
        l = l * al + pj;
#pragma unroll
        for (int e = 0; e < HD; ++e) o[e] = o[e] * al + pj * Vs[jj][e];
        m = mn;
      }
    }
    // blend: acc += w-bar(t) * o / l, tiles in ascending order
    const float coef = ((BLEND && tok) ? p.blk_w[(b * p.maxc + ps) * QB + tid] : 1.0f) / l;
#pragma unroll
    for (int e = 0; e < HD; ++e) acc[e] = fmaf(coef, o[e], acc[e]);
  }
  if (!valid) return;
  float* out = (float*)p.out + int64_t(orow) * p.d + h * HD;
#pragma unroll
  for (int e = 0; e < HD; ++e) out[e] = acc[e];
}

// ------------------------------------------------------------- bf16 -----
constexpr int NW = 8;                  // wavefronts per workgroup
constexpr int KB = 64;                 // keys per staged block
// Staging pipeline.  NST LDS stages of K and V: at key block gb the DMA of
// block gb + NST - 1 is issued, and a block's end waits only for block gb+1
// (the NST - 2 newer blocks stay in flight).  A wavefront's vector memory
// operations complete in issue order, so a key-row ring load issued at block
// j has landed by the end of block j + NST - 3 and is read (for the DMA of its
// block) NST - 1 blocks before that block: the ring runs AHEAD = 2 NST - 3
// blocks ahead, in NSL slots.
constexpr int NST = 4;                 // LDS stages of K and V
constexpr int DEPTH = NST - 1;         // blocks whose DMA is in flight ahead of the current one
constexpr int AHEAD = 2 * DEPTH - 1;   // blocks ahead the key rows are fetched
constexpr int NSL = 8;                 // slots of the key-row ring (>= AHEAD + 1)
static_assert(NSL >= AHEAD + 1 && DEPTH >= 2 && DEPTH <= 3, "staging pipeline");
constexpr float RESCALE_LOG2 = 8.0f;   // keep a stale running max until a block exceeds it by 2^8
// The bf16 kernel comes in three modes: 0 takes the fixed softmax offset or
// the running max as the launch's scores allow, 1 runs only against the fixed
// offset and 2 only with a running max (each returns at once otherwise, so
// that launching 1 and then 2 runs exactly one of them): one version of the
// job loop per kernel, so neither carries the other's registers.
// Wavefronts per SIMD: at head size 64 a workgroup's LDS (67.6 KB) lets two
// workgroups share a CU, so with the fixed offset four wavefronts per SIMD
// (at most 128 VGPRs, no spills); their phases drift apart, so one
// workgroup's MFMAs run beside the other's softmax.  The running max needs
// more registers (two wavefronts per SIMD), and at head size 128 (133 KB of
// LDS) one workgroup fills a CU.
template <int HD, int MODE>
constexpr int WPS = HD == 64 && MODE == 1 ? 4 : 2;
// Largest static score bound used as the softmax offset: weights >= 2^-64,
// and the fp32 argument score*C - bound of a weight that matters (|.| < 32)
// is rounded to 2^-20, about as finely as against a running max.
constexpr float FIXED_MAX_LIMIT = 32.f;
static_assert(QB == 32 * NW, "32 query rows per wavefront");
static_assert(QB == tsk::QBLOCK, "query blocks of the plan");

// Swap bits 2 and 3 of a row index in 0..31.
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// LDS swizzles: 16-byte chunk c of key row r is stored at chunk c ^ key(r).
// The LDS has 64 banks of 4 bytes.  K fragment reads (16 bytes per lane,
// served 16 lanes at a time) touch 16 rows at one chunk: head size 128 takes
// row & 15; head size 64 (128-byte rows, row parity already picks the half of
// the bank range) (row >> 1) & 7.  V^T fragment reads are transposing 8-byte
// reads; a half wavefront touches 4 consecutive rows x 4 consecutive chunks:
// 4 (row & 3) at head size 128, 4 ((row >> 1) & 1) at 64, so the 16 pieces
// fall in 16 different 16-byte bank groups.
template <int HD> __device__ __forceinline__ int kswz(int r) { return HD == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int HD> __device__ __forceinline__ int vswz(int r) { return HD == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// One V^T operand fragment (32 hd rows x 16 keys) of the MFMA from two
// transposing reads.  In each group of 16 lanes, ds_read_b64_tr_b16 gives lane
// j element j % 4 of the 8-byte pieces addressed by lanes j/4, j/4 + 4,
// j/4 + 8 and j/4 + 12.  Lane 16G + j addresses key row (4 keys apart per
// j/4 step) and hd dims dbase + 4 (j % 4) .. +3, so it receives hd dim
// dbase + j of four consecutive keys: the A-operand layout (row = lane % 32,
// k = 8 (lane / 32) + 0..7) after the two reads, keys 0-3 then 4-7.
__device__ __forceinline__ bf16x8 v_fragment(const char* lo, const char* hi) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TS_LDS s16x4*)lo);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TS_LDS s16x4*)hi);
  const s16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// Halves of heads dealt to XCD x: the 2H halves (u = 2 head + {0: A, 1: B})
// cut into 8 contiguous runs; na, nb count the A and B halves of the run.
struct HalfRange {
  int u0, nu, na, nb;
};
__host__ __device__ __forceinline__ HalfRange xcd_halves(int H, int x) {
  const int U = 2 * H, q8 = U >> 3, r8 = U & 7;
  HalfRange r;
  r.u0 = x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8;
  r.nu = q8 + (x < r8 ? 1 : 0);
  r.na = (r.nu + ((r.u0 & 1) ? 0 : 1)) >> 1;
  r.nb = r.nu - r.na;
  return r;
}

// Blended job (block, head) number b >> 3 of XCD b % 8 (false past the
// XCD's last job).  The XCD holds a contiguous run of half-heads (two halves
// of equal work per head, so the runs carry equal work), which keeps the keys
// and values it streams to a few heads: together the XCDs touch each head's
// K and V about once.  Within the run the jobs go class by class, most
// windows first, so the XCD's CUs finish together; within a class, half by
// half, blocks ascending (neighbouring rows, the same windows).  All values
// are uniform.
__device__ __forceinline__ bool blend_job(const AttnP& p, int b, int& blk, int& h) {
  const HalfRange r = xcd_halves(p.H, b & 7);
  int rem = b >> 3;
  for (int c = 0; c < p.ncls; ++c) {
    const int ca = p.blk_cls[4 * c], oa = p.blk_cls[4 * c + 1];
    const int cb = p.blk_cls[4 * c + 2], ob = p.blk_cls[4 * c + 3];
    const int m = r.na * ca + r.nb * cb;
    if (rem < m) {
      for (int u = r.u0;; ++u) {  // ends: the counts of the run's halves sum to m > rem
        const int cnt = (u & 1) ? cb : ca;
        if (rem < cnt) {
          blk = p.blk_order[((u & 1) ? ob : oa) + rem];
          h = u >> 1;
          return true;
        }
        rem -= cnt;
      }
    }
    rem -= m;
  }
  return false;
}

template <int HD, bool BLEND, int MODE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPS<HD, MODE>, WPS<HD, MODE>))) void k_attn_bf16(AttnP p) {
  constexpr int KROWB = HD * 2;       // bytes per staged key row
  constexpr int NHB = HD / 32;        // 32-row hd blocks of O^T
  constexpr int KSTEPS = HD / 16;     // MFMA k-steps of S^T
  // LDS fragment reads kept ahead of their MFMAs: K fragments (reads) in the
  // score phase, V^T fragments in the output phase; fewer at head size 64,
  // where four wavefronts share a SIMD and cover each other's reads
  constexpr int SRA = WPS<HD, MODE> == 4 ? 2 : 4;
  constexpr int VRA = WPS<HD, MODE> == 4 ? 2 : 4;
  // global_load_lds: lane l of a wavefront instruction writes 16 bytes at LDS
  // base + 16*l; instruction i of wavefront w fills bytes [(w*KDI + i) KB,
  // +1 KB) of a stage, i.e. key row b / KROWB, slot (b % KROWB) / 16 for lane
  // byte b, and the lane loads the logical chunk the swizzle puts in that slot
  constexpr int KDI = KB * KROWB / 1024 / NW;  // DMA instructions per wavefront, each of K and V
  static_assert(KDI >= 1, "whole 1 KB DMA rows per wavefront");
  __shared__ __attribute__((aligned(16))) char Ks[NST][KB * KROWB];
  __shared__ __attribute__((aligned(16))) char Vs[NST][KB * KROWB];
  __shared__ int idx_s[NSL][KB];
  __shared__ int job_s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int n = p.n;
  const int nkb = (n + KB - 1) / KB;
  const int nqb = (n + QB - 1) / QB;
  // Job order.  The hardware deals workgroup b to XCD b % 8.  Per tile: one
  // job per workgroup, each XCD a contiguous run of jobs, the query blocks of
  // one (tile, head), which stream the same keys and values through that
  // XCD's L2.  Blended: one workgroup per CU slot, each taking jobs from its
  // XCD's counter in the order blend_job gives until they run out.  Jobs
  // differ in length (one to maxc windows), and the hardware hands out
  // workgroups in order, each to a fixed shader engine of its XCD: a long
  // job on one engine would hold back the launch of every later workgroup.
  // Pulled jobs keep every CU busy until its XCD's list is done.
  const int xcd = blockIdx.x & 7;
  // With QK-RMSNorm a q or k head row has norm at most sqrt(hd) max|gain|
  // (the RMS-normalised vector has norm sqrt(hd), RoPE rotates it, bf16
  // rounding adds < 0.4 %), so every score, q carrying the factor
  // C = log2(e)/sqrt(hd), lies within +-bnd.  For
  // bnd <= FIXED_MAX_LIMIT the softmax subtracts bnd instead of a running
  // max: every weight is in [2^-2bnd, 1], and the per-block max and rescale
  // go away.  bnd is an integer, so a weight is
  // 2^score scaled exactly and rounds to bf16 as 2^score would.
  bool fixedm = false;
  float bnd = 0.f;
  if (p.qg) {
    float gq = 0.f, gk = 0.f;
    for (int e = lane; e < HD; e += 64) {
      gq = fmaxf(gq, fabsf(p.qg[e]));
      gk = fmaxf(gk, fabsf(p.kg[e]));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      gq = fmaxf(gq, __shfl_xor(gq, o, 64));
      gk = fmaxf(gk, __shfl_xor(gk, o, 64));
    }
    bnd = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(
                                         int, ceilf(1.01f * float(HD) * p.scale_log2 * gq * gk + 1e-3f))));
    fixedm = bnd <= FIXED_MAX_LIMIT;
  } else if (p.qkn) {
    // Without QK-norm, qk_prep's largest q and k head norms bound every score
    // the same way (Cauchy-Schwarz; q carries C): |q.k| <= max|q| max|k|
    const float qm = __uint_as_float(p.qkn[0]), km = __uint_as_float(p.qkn[1]);
    bnd = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                        __builtin_bit_cast(int, ceilf(1.01f * qm * km + 1e-3f))));
    fixedm = bnd <= FIXED_MAX_LIMIT;
  }
  int njx = 0;  // blended: the XCD's job count
  if constexpr (BLEND) {
    const HalfRange xr = xcd_halves(p.H, xcd);
    njx = xr.na * p.half_a + xr.nb * (p.nblk - p.half_a);
  }
  // The job loop in two versions, each with its registers to its own code:
  // against the fixed offset, and with a running max.
  auto job_loop = [&](auto fixed_tag) {
  constexpr bool FIXED = decltype(fixed_tag)::value;
  for (int it = 0;; ++it) {
    int tid_j = int(threadIdx.x);
    if constexpr (WPS<HD, MODE> == 4) asm volatile("" : "+v"(tid_j));
    const int tid = tid_j, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, g = lane >> 5;
    int h = 0, t0 = 0, qblk = 0, blk = 0, npass = 1;
    if constexpr (BLEND) {
      // take the XCD's next job; every thread has read job_s before the job's
      // first barrier, after which thread 0 may write it again
      if (tid == 0) job_s = int(atomicAdd(p.jobs + 8 * xcd, 1u));
      __syncthreads();
      const int i = __builtin_amdgcn_readfirstlane(job_s);
      if (i >= njx) break;
      blend_job(p, 8 * i + xcd, blk, h);
      npass = p.blk_nt[blk];
    } else {
      if (it > 0) break;
      const int total = nqb * p.n_tiles * p.H;
      const int loc = blockIdx.x >> 3;
      const int q8 = total >> 3, r8 = total & 7;
      const int id = xcd < r8 ? xcd * (q8 + 1) + loc : r8 * (q8 + 1) + (xcd - r8) * q8 + loc;
      {
        qblk = id % nqb;
        h = (id / nqb) % p.H;
        t0 = id / (nqb * p.H);
      }
    }
    const bf16* qkv = (const bf16*)p.qkv;
    const int64_t ld = 3 * int64_t(p.d);
    const bf16* kbase = qkv + p.d + h * HD;
    const bf16* vbase = qkv + 2 * p.d + h * HD;
    const int nblocks = npass * nkb;  // key blocks streamed over all windows
    // the job's window tiles: uniform plan data that no launch writes, read
    // through the scalar cache, so that reading one (when the key-row stream
    // enters the next window) waits on scalar loads only, not on the K / V
    // loads in flight
    auto tile_of = [&](int ps) -> int {
      if constexpr (BLEND)
        return ((const __attribute__((address_space(4))) int*)p.blk_tiles)[__builtin_amdgcn_readfirstlane(blk * p.maxc + ps)];
      else return t0;
    };

    // key rows of the first AHEAD blocks (row-map layouts)
    if (tid < KB) {
#pragma unroll
      for (int b = 0; b < AHEAD; ++b)
        if (b < nblocks) {
          const int ps = b / nkb, kb = b - ps * nkb;
          idx_s[b][tid] = p.rows[int64_t(tile_of(ps)) * n + min(kb * KB + tid, n - 1)];
        }
    }
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    // DMA staging in two steps: the key rows this lane's loads need (from the
    // ring), then the loads, so that the ring can be refilled in between
    auto dma_rows = [&](int gb, int (&rr)[KDI]) {
#pragma unroll
      for (int i = 0; i < KDI; ++i) {
        const int row = ((wv * KDI + i) * 1024 + 16 * lane) / KROWB;
        rr[i] = idx_s[gb % NSL][row];
      }
    };
    // DMA source offsets in bytes, 32-bit: a row index times the row pitch by
    // a 24-bit multiply (one full-rate instruction, where a 64-bit product
    // takes three quarter-rate ones; the launcher checks that the qkv array
    // is below 4 GiB), plus this lane's swizzled chunk
    const uint32_t ldb = uint32_t(ld) * 2u;
    const char* kb8 = (const char*)kbase;
    const char* vb8 = (const char*)vbase;
    uint32_t kch[KDI], vch[KDI];
#pragma unroll
    for (int i = 0; i < KDI; ++i) {
      const int b = (wv * KDI + i) * 1024 + 16 * lane;
      const int row = b / KROWB, slot = (b % KROWB) / 16;
      kch[i] = uint32_t((slot ^ kswz<HD>(row)) * 16);
      vch[i] = uint32_t((slot ^ vswz<HD>(row)) * 16);
    }
    auto dma = [&](int gb, const int (&rr)[KDI]) {
      const int st = gb % NST;
#pragma unroll
      for (int i = 0; i < KDI; ++i) {
        const uint32_t ro = __umul24(uint32_t(rr[i]), ldb);
        __builtin_amdgcn_global_load_lds((const void*)(kb8 + (ro + kch[i])), (TS_LDS void*)(&Ks[st][(wv * KDI + i) * 1024]),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vb8 + (ro + vch[i])), (TS_LDS void*)(&Vs[st][(wv * KDI + i) * 1024]),
                                         16, 0, 0);
      }
    };

    __syncthreads();  // ring slots ready
    {
      int rr[KDI];
#pragma unroll
      for (int b = 0; b < DEPTH; ++b)
        if (b < nblocks) {
          dma_rows(b, rr);
          dma(b, rr);
        }
    }

    // ---- this wavefront's 32 queries: B operand of S^T = K Q^T (hd 16s + 8g + e)
    const int slot = wave * 32 + l32;
    int qrow;
    if constexpr (BLEND) {
      const int r = p.blk_rows[blk * QB + slot];
      qrow = r >= 0 ? r : p.blk_rows[blk * QB];   // an empty slot runs the block's first row
    } else {
      const int qc = min(qblk * QB + slot, n - 1);
      qrow = p.rows[int64_t(t0) * n + qc];
    }
    bf16x8 qf[KSTEPS];
    {
      const bf16* qp = qkv + int64_t(qrow) * ld + h * HD;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s + 8 * g);
    }
    float m_run = 0.f, l_run = 0.f;
    // start of every score chain, -m: the accumulators hold s - m and a
    // weight is one exponential (-bnd against the fixed offset; with a
    // running max, set by each window's start and each rescale)
    f32x16 sinit;
#pragma unroll
    for (int r = 0; r < 16; ++r) sinit[r] = FIXED ? -bnd : 0.f;
    f32x16 oacc[NHB];
    // the window's global key is the softmax's initial state: score, weight 1, value
    auto window_init = [&](int t) {
      const int64_t gr = gkey_row(p, t);
      const bf16* kgp = kbase + gr * ld;
      const bf16* vgp = vbase + gr * ld;
      // four wavefronts per SIMD: this lane's column offsets anew (opaque), so
      // that no lane address is formed once per job and held across windows
      int gw = g;
      if constexpr (WPS<HD, MODE> == 4) asm volatile("" : "+v"(gw));
      float sg = 0.f;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8 kg = *reinterpret_cast<const bf16x8*>(kgp + 16 * s + 8 * gw);
        // q opaque here: its fp32 copy (64 registers) would otherwise be made
        // once and held across every window
        bf16x8 q = qf[s];
        asm volatile("" : "+v"(q));
#pragma unroll
        for (int e = 0; e < 8; ++e) sg += float(q[e]) * float(kg[e]);
      }
      sg += __shfl_xor(sg, 32, 64);
      // weight of the global key (q carries C, so sg is in the log2 domain):
      // 1 against a running max started at its score, or 2^(sg - bnd)
      // against the fixed offset
      m_run = FIXED ? bnd : sg;
      const float w0 = FIXED ? __builtin_amdgcn_exp2f(sg - bnd) : 1.f;
      if constexpr (!FIXED) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sinit[r] = -sg;
      }
      l_run = g == 0 ? w0 : 0.f;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const bf16x4 v = *reinterpret_cast<const bf16x4*>(vgp + hb * 32 + 8 * r4 + 4 * gw);
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[hb][4 * r4 + e] = float(v[e]) * w0;
        }
    };
    // the window's output o = O / l: written (per-tile layouts), or weighted by
    // w-bar and added to the row's blend, the partial sum kept in fp32 between
    // windows and the blend written after the last one
    auto window_finish = [&](int ps) {
      const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
      // the output row is read again here rather than kept from the start:
      // nothing but the softmax state stays in registers across the key loop
      int orw;
      bool valid;
      float coef;
      if constexpr (BLEND) {
        // four wavefronts per SIMD: the slot index anew (opaque), so that
        // nothing formed from it at the job's start is held across the key loop
        int sl = slot;
        if constexpr (WPS<HD, MODE> == 4) asm volatile("" : "+v"(sl));
        const int r = p.blk_rows[blk * QB + sl];
        valid = r >= 0;
        orw = valid ? r : p.blk_rows[blk * QB];
        coef = p.blk_w[(int64_t(blk) * p.maxc + ps) * QB + sl] / l_tot;
      } else {
        const int qi = qblk * QB + slot;
        valid = qi < n;
        orw = t0 * (n + 1) + qi;
        coef = 1.0f / l_tot;
      }
      const bool last = !BLEND || ps + 1 == npass;
      float* prow = p.part + int64_t(orw) * p.d + h * HD;
      bf16* op = (bf16*)p.out + int64_t(orw) * p.d + h * HD;
      // in place on the accumulators (the next window starts them afresh)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) oacc[hb] *= coef;
      if (BLEND && ps > 0) {
        // every lane reads (an empty slot's row is the block's first row); the
        // reads of half the head go out together before they are added
#pragma unroll
        for (int h0 = 0; h0 < NHB; h0 += (NHB + 1) / 2) {
          f32x4 prev[(NHB + 1) / 2][4];
#pragma unroll
          for (int hb = h0; hb < min(h0 + (NHB + 1) / 2, NHB); ++hb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) prev[hb - h0][r4] = load4(prow + hb * 32 + 8 * r4 + 4 * g);
#pragma unroll
          for (int hb = h0; hb < min(h0 + (NHB + 1) / 2, NHB); ++hb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
              for (int e = 0; e < 4; ++e) oacc[hb][4 * r4 + e] += prev[hb - h0][r4][e];
        }
      }
      float am = 0.f;
      if (valid) {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int col = hb * 32 + 8 * r4 + 4 * g;
            const f32x4 v = {oacc[hb][4 * r4], oacc[hb][4 * r4 + 1], oacc[hb][4 * r4 + 2], oacc[hb][4 * r4 + 3]};
            if (!last) {
              store4(prow + col, v);
            } else {
              const bf16x4 w = {bf16(v[0]), bf16(v[1]), bf16(v[2]), bf16(v[3])};
              *reinterpret_cast<bf16x4*>(op + col) = w;
#pragma unroll
              for (int e = 0; e < 4; ++e) am = fmaxf(am, fabsf(float(w[e])));
            }
          }
      }
      if (last && p.amax) wave_amax(p.amax, am, int(blockIdx.x) * NW + wave);
    };

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wavefront's DMA of the first blocks landed
    __syncthreads();
    const int krow_a = swap23(l32);  // key row this lane feeds as MFMA A row
    // V^T fragment addresses: lane 16G + j reads key row 8 (G / 2) + j / 4 (+16
    // per 16-key chunk, +4 for the second read) at hd dims hb*32 + 16 (G % 2) +
    // 4 (j % 4) .. +3; the swizzle depends only on the row's low bits, which
    // the chunk and read offsets keep
    int vaddr[NHB];
    {
      const int G = lane >> 4, j = lane & 15;
      const int row0 = 8 * (G >> 1) + (j >> 2);
      const int clow = 2 * (G & 1) + ((j & 3) >> 1);
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) vaddr[hb] = row0 * KROWB + (((hb * 4 + clow) ^ vswz<HD>(row0)) * 16) + 8 * (j & 1);
    }

    // window and block AHEAD blocks ahead in the stream, and that window's map
    int ps3 = AHEAD / nkb, kb3 = AHEAD % nkb;
    const int* map3 = p.rows + int64_t(tile_of(min(ps3, npass - 1))) * n;
    for (int ps = 0; ps < npass; ++ps) {
     window_init(tile_of(ps));
     for (int kb = 0; kb < nkb; ++kb) {
      const int gb = ps * nkb + kb;  // position in the stream of key blocks
      const int cur = gb % NST;
      {
        // key rows of block gb+AHEAD: wavefront 0 copies them from the row map
        // straight into the ring (no registers, so nothing waits on them before
        // the block-end wait), ahead of this block's K / V loads so that wait
        // covers them
        int rr[KDI];
        if (gb + DEPTH < nblocks) dma_rows(gb + DEPTH, rr);
        if (gb + AHEAD < nblocks) {
          if (wv == 0) {
            const int j = min(kb3 * KB + lane, n - 1);
            __builtin_amdgcn_global_load_lds((const void*)(map3 + j), (TS_LDS void*)(&idx_s[(gb + AHEAD) % NSL][0]),
                                             4, 0, 0);
          }
          // the stream position AHEAD blocks on: its window's map is read only
          // when it enters a new window
          if (++kb3 == nkb) {
            kb3 = 0;
            if (++ps3 < npass) map3 = p.rows + int64_t(tile_of(ps3)) * n;
          }
        }
        if (gb + DEPTH < nblocks) dma(gb + DEPTH, rr);
      }
      const char* ks = Ks[cur];
      const char* vs = Vs[cur];
      const int j0 = kb * KB;

      // ---- S^T = K Q^T for the 64 keys: two 32-key chains, K fragments read
      // ahead of the MFMAs that use them (four LDS reads kept in flight)
      f32x16 sacc[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) sacc[sb] = sinit;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const int kr = sb * 32 + krow_a;
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(ks + kr * KROWB + (((2 * s + g) ^ kswz<HD>(kr)) * 16));
          sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[sb], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, SRA, 0);  // SRA LDS reads
#pragma unroll
      for (int i = 0; i < 2 * KSTEPS - SRA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the next LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, SRA, 0);
      if (j0 + KB > n) {  // keys past the window end (last block of a window only)
        // accumulator row 8(r/4)+4g+(r%4) holds key swap23(that row) =
        // 16(r/8) + 4((r/4)%2) + r%4 + 8g: one per-lane limit, constant offsets
        const int lim = n - j0 - 8 * g;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (sb * 32 + 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3) >= lim) sacc[sb][r] = -INFINITY;
      }
      // ---- softmax over the block: against the fixed offset, or online
      // (one rescale check per block)
      bf16x8 pf[4];
      {
        if constexpr (!FIXED) {
          // the accumulators hold s - m: the block max past the running max
          float mx = -INFINITY;
#pragma unroll
          for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sb][r]);
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          // rescale only when some query's block max passes its running max
          // by 2^8: each query of the wavefront raises its max to its block
          // max (if larger), and its scores follow
          if (__builtin_amdgcn_ballot_w64(mx > RESCALE_LOG2) != 0) {
            const float up = fmaxf(mx, 0.f);
            const float alpha = __builtin_amdgcn_exp2f(-up);
            m_run += up;
            l_run *= alpha;
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) oacc[hb] *= alpha;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) sacc[sb] -= up;
#pragma unroll
            for (int r = 0; r < 16; ++r) sinit[r] = -m_run;
          }
        }
        // the scores already hold s - m (the chains start from -m), so a
        // weight is one exponential
        float lsum = 0.f;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(sacc[sb][r]);
            lsum += pv;
            pf[sb * 2 + (r >> 3)][r & 7] = bf16(pv);
          }
        l_run += lsum;
      }
      // ---- O^T += V^T P^T over four 16-key chunks (NHB independent chains).
      // The transposing reads take no immediate offset, so their 8*NHB
      // addresses would all be precomputed and held across the loop; the empty
      // asm makes the NHB per-lane bases opaque here, so each address is one
      // add from a base inside the block instead.
      int vb[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        vb[hb] = vaddr[hb];
        asm volatile("" : "+v"(vb[hb]));
      }
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          const char* a = vs + vb[hb] + 16 * cc * KROWB;
          const bf16x8 vf = v_fragment(a, a + 4 * KROWB);
          oacc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[cc], oacc[hb], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * VRA, 0);  // VRA fragments (2 VRA reads) ahead
#pragma unroll
      for (int i = 0; i < 4 * NHB - VRA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, VRA, 0);

      // this wavefront's loads of block gb+1 have landed (the newer blocks'
      // may still be in flight) and its LDS traffic is done; then a barrier
      // without the fence of __syncthreads, which would also wait for those.
      // Vector memory operations complete in issue order, so the count also
      // covers the previous window's output loads and stores.
      if (gb + DEPTH < nblocks) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((DEPTH - 1) * 2 * KDI) : "memory");
      else if (DEPTH == 3 && gb + 2 < nblocks) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * KDI) : "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
     }
     window_finish(ps);
    }
  }  // jobs
  };
  if constexpr (MODE == 0) {
    if (fixedm) job_loop(std::true_type{});
    else job_loop(std::false_type{});
  } else if constexpr (MODE == 1) {
    if (fixedm) job_loop(std::true_type{});
  } else {
    if (!fixedm) job_loop(std::false_type{});
  }
}

// Global-token query row of one (head, tile), over the window keys
// [j_begin, j_end) of split blockIdx.z (key n is the global key itself).
// Keys are taken in chunks of GCH.  Score pass: HD/16 threads per key, 16
// dims each, summed across those lanes; scores and row indices go to LDS.
// Value pass: each thread owns one 8-dim group of the output and a strided
// subset of the chunk's keys and keeps a running (max-shifted) weighted sum;
// the chunk max is shared by the workgroup, so every thread rescales by the
// same factor.  The partial sums are added in LDS at the end.  With one split
// the row is written; with several, each split leaves its state (max m,
// weight sum l, unnormalised output o[HD], in the exp2 domain) in `part` for
// k_attn_global_merge.
constexpr int GCH = 1024;
template <int HD, int NT>
__global__ __launch_bounds__(NT) void k_attn_global_bf16(AttnP p, int split_keys, float* part) {
  constexpr int TPK = HD / 16;    // threads per key, score pass
  constexpr int KPP = NT / TPK;   // keys per score pass
  constexpr int DG = HD / 8;      // 8-dim groups, value pass
  constexpr int KG = NT / DG;     // key groups, value pass
  __shared__ float s_s[GCH];
  __shared__ int r_s[GCH];
  __shared__ float red[NT / 64];
  __shared__ __attribute__((aligned(16))) float acc_s[KG][HD + 4];
  __shared__ float l_s[KG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, t = blockIdx.y, n = p.n;
  const int j_begin = blockIdx.z * split_keys, j_end = min(j_begin + split_keys, n + 1);
  const bf16* qkv = (const bf16*)p.qkv;
  const int64_t ld = 3 * int64_t(p.d);
  const int64_t grow = gkey_row(p, t);

  // score-pass role: dims [16*sub, 16*sub + 16) of key slot kk
  const int sub = tid % TPK, kk = tid / TPK;
  const bf16* qp = qkv + grow * ld + h * HD + 16 * sub;
  const bf16x8 q0 = *reinterpret_cast<const bf16x8*>(qp), q1 = *reinterpret_cast<const bf16x8*>(qp + 8);
  // value-pass role: dims [8*dg, 8*dg + 8), keys kg, kg + KG, ...
  const int dg = tid % DG, kg = tid / DG;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float l = 0.f, m_run = -INFINITY;

  for (int c0 = j_begin; c0 < j_end; c0 += GCH) {
    const int cnt = min(GCH, j_end - c0);
#pragma unroll 4
    for (int jj = kk; jj < cnt; jj += KPP) {
      const int j = c0 + jj;
      const int64_t r = j < n ? key_row(p, t, j) : grow;
      const bf16* kp = qkv + r * ld + p.d + h * HD + 16 * sub;
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kp), k1 = *reinterpret_cast<const bf16x8*>(kp + 8);
      float sc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sc += float(q0[e]) * float(k0[e]);
#pragma unroll
      for (int e = 0; e < 8; ++e) sc += float(q1[e]) * float(k1[e]);
#pragma unroll
      for (int o = 1; o < TPK; o <<= 1) sc += __shfl_xor(sc, o);
      if (sub == 0) {
        s_s[jj] = sc;  // q carries log2(e)/sqrt(hd): the log2 domain
        r_s[jj] = int(r);
      }
    }
    __syncthreads();
    float mx = -INFINITY;
    for (int jj = tid; jj < cnt; jj += NT) mx = fmaxf(mx, s_s[jj]);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    float cmax = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) cmax = fmaxf(cmax, red[w]);
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll 8
    for (int jj = kg; jj < cnt; jj += KG) {
      const float pj = __builtin_amdgcn_exp2f(s_s[jj] - m_new);
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qkv + int64_t(r_s[jj]) * ld + 2 * p.d + h * HD + 8 * dg);
      l += pj;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += pj * float(v[e]);
    }
    __syncthreads();   // s_s / r_s are rewritten by the next chunk
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) acc_s[kg][8 * dg + e] = acc[e];
  if (dg == 0) l_s[kg] = l;
  __syncthreads();
  if (tid < HD) {
    float o = 0.f, lt = 0.f;
    for (int g = 0; g < KG; ++g) {
      o += acc_s[g][tid];
      lt += l_s[g];
    }
    if (part) {
      float* st = part + ((int64_t(t) * p.H + h) * gridDim.z + blockIdx.z) * (HD + 2);
      if (tid == 0) {
        st[0] = m_run;
        st[1] = lt;
      }
      st[2 + tid] = o;
    } else {
      bf16* out = (bf16*)p.out + int64_t(gout_row(p, t)) * p.d + h * HD;
      const bf16 w = bf16(o / lt);
      out[tid] = w;
      if (p.amax) wave_amax(p.amax, fabsf(float(w)), t * p.H + h + wave);  // tid < HD: whole wavefronts
    }
  }
}

// Merge the splits' states of one (head, tile) global row: with M the largest
// split max, out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
template <int HD>
__global__ __launch_bounds__(HD) void k_attn_global_merge(AttnP p, int splits, const float* part) {
  const int h = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  const float* st = part + (int64_t(t) * p.H + h) * splits * (HD + 2);
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, st[s * (HD + 2)]);
  float o = 0.f, lt = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float w = __builtin_amdgcn_exp2f(st[s * (HD + 2)] - mx);
    lt += st[s * (HD + 2) + 1] * w;
    o += st[s * (HD + 2) + 2 + tid] * w;
  }
  bf16* out = (bf16*)p.out + int64_t(gout_row(p, t)) * p.d + h * HD;
  const bf16 w = bf16(o / lt);
  out[tid] = w;
  if (p.amax) wave_amax(p.amax, fabsf(float(w)), t * p.H + h + (tid >> 6));
}

}  // namespace

namespace tsk {

static AttnP make_params(const AttnArgs& a) {
  return AttnP{a.qkv,       a.out,       a.part, a.rows, a.g0, a.gstep, a.blk_nt, a.blk_tiles, a.blk_rows, a.blk_w, a.nblk, a.maxc,
               a.blk_order, a.blk_cls,   a.ncls,           a.half_a, a.jobs,
               a.n_union,   a.d,         a.H,    a.n_tiles,        a.n,
               1.4426950408889634f / sqrtf(float(a.hd)),           a.amax, a.qg, a.kg, a.qkn};
}

__global__ void k_zero_jobs(unsigned* jobs) {
  if (threadIdx.x < tsk::JOB_COUNTERS_BYTES / 4) jobs[threadIdx.x] = 0u;
}

// Workgroups of the blended bf16 kernel that the current device holds at
// once: CUs x resident workgroups per CU, rounded down to a multiple of 8
// (at least 8).  Cached per device.
hipError_t blend_slots(int hd, int mode, int* out) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int>, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({dev, hd, mode});
  if (it == cache.end()) {
    int cus = 0, per_cu = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if (hd == 64)
      e = mode == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_attn_bf16<64, true, 1>, NW * 64, 0)
                    : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_attn_bf16<64, true, 2>, NW * 64, 0);
    else
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_attn_bf16<128, true, 0>, NW * 64, 0);
    if (e != hipSuccess) return e;
    const int slots = std::max(8, (std::max(1, cus) * std::max(1, per_cu)) / 8 * 8);
    it = cache.emplace(std::make_tuple(dev, hd, mode), slots).first;
  }
  *out = it->second;
  return hipSuccess;
}

hipError_t attention(hipStream_t s, int act, const AttnArgs& a) {
  const AttnP p = make_params(a);
  const bool blend = a.blk_nt != nullptr;
  if (a.n < 1 || !a.rows || (blend && a.nblk < 1)) return hipErrorInvalidValue;
  const int nqb = (a.n + QB - 1) / QB;
  const int njob = blend ? a.nblk : nqb * a.n_tiles;
  if (act == ACT_F32) {
    const dim3 grid(njob + a.n_tiles, a.H), block(QB);
#define TS_F32A(HD)                                                                  \
  do {                                                                               \
    if (blend) hipLaunchKernelGGL((k_attn_f32<HD, true>), grid, block, 0, s, p);   \
    else hipLaunchKernelGGL((k_attn_f32<HD, false>), grid, block, 0, s, p);        \
  } while (0)
    if (a.hd == 32) TS_F32A(32);
    else if (a.hd == 64) TS_F32A(64);
    else return hipErrorInvalidValue;
#undef TS_F32A
    return hipGetLastError();
  }
  if (a.hd != 64 && a.hd != 128) return hipErrorInvalidValue;
  // the K / V staging takes 32-bit byte offsets into qkv: its rows (the last
  // is tile n_tiles-1's global row) must span less than 4 GiB
  const int64_t qkv_rows = int64_t(a.g0) + int64_t(a.gstep) * (a.n_tiles - 1) + 1;
  if (qkv_rows * 6 * int64_t(a.d) >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  const dim3 block(NW * 64);
  if (!blend) {
    const dim3 grid(njob * a.H);
    if (a.hd == 64) {  // the fixed-offset kernel, then the running-max one: one of them runs
      hipLaunchKernelGGL((k_attn_bf16<64, false, 1>), grid, block, 0, s, p);
      hipLaunchKernelGGL((k_attn_bf16<64, false, 2>), grid, block, 0, s, p);
    } else {
      hipLaunchKernelGGL((k_attn_bf16<128, false, 0>), grid, block, 0, s, p);
    }
    return hipGetLastError();
  }
  // blended: as many workgroups as the CUs hold at once (a multiple of 8, so
  // every XCD holds the same number), counters zeroed first
  if (!a.blk_order || !a.blk_cls || a.ncls < 1 || !a.jobs) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_zero_jobs, dim3(1), dim3(64), 0, s, a.jobs);
  if (a.hd == 64) {  // the fixed-offset kernel, then the running-max one: one of them takes the jobs
    int s1 = 0, s2 = 0;
    hipError_t e = blend_slots(64, 1, &s1);
    if (e == hipSuccess) e = blend_slots(64, 2, &s2);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_attn_bf16<64, true, 1>), dim3(s1), block, 0, s, p);
    hipLaunchKernelGGL((k_attn_bf16<64, true, 2>), dim3(s2), block, 0, s, p);
  } else {
    int slots = 0;
    hipError_t e = blend_slots(128, 0, &slots);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_attn_bf16<128, true, 0>), dim3(slots), block, 0, s, p);
  }
  return hipGetLastError();
}

int attention_global_splits(const AttnArgs& a, int64_t scratch_floats) {
  // about GLOBAL_WGS workgroups over the chip, splits of at least 128 keys
  static const int target = [] {
    const char* e = getenv("TS_GLOBAL_WGS");
    return e ? std::max(64, atoi(e)) : 2048;
  }();
  int splits = (target + a.H * a.n_tiles - 1) / (a.H * a.n_tiles);
  splits = std::min(splits, std::max(1, (a.n + 1) / 128));
  while (splits > 1 && int64_t(a.n_tiles) * a.H * splits * (a.hd + 2) > scratch_floats) --splits;
  return std::max(1, std::min(splits, 64));
}

hipError_t attention_global(hipStream_t s, const AttnArgs& a, float* scratch, int64_t scratch_floats) {
  const AttnP p = make_params(a);
  if (a.n < 1 || (a.hd != 64 && a.hd != 128)) return hipErrorInvalidValue;
  const int splits = scratch ? attention_global_splits(a, scratch_floats) : 1;
  if (splits == 1) {
    const dim3 grid(a.H, a.n_tiles, 1);
    if (a.hd == 64) hipLaunchKernelGGL((k_attn_global_bf16<64, 1024>), grid, dim3(1024), 0, s, p, a.n + 1, nullptr);
    else hipLaunchKernelGGL((k_attn_global_bf16<128, 1024>), grid, dim3(1024), 0, s, p, a.n + 1, nullptr);
    return hipGetLastError();
  }
  int split_keys = (a.n + 1 + splits - 1) / splits;
  split_keys = (split_keys + 63) / 64 * 64;
  const int used = (a.n + 1 + split_keys - 1) / split_keys;   // every split holds >= 1 key
  const dim3 grid(a.H, a.n_tiles, used);
  if (a.hd == 64) {
    hipLaunchKernelGGL((k_attn_global_bf16<64, 256>), grid, dim3(256), 0, s, p, split_keys, scratch);
    hipLaunchKernelGGL(k_attn_global_merge<64>, dim3(a.H, a.n_tiles), dim3(64), 0, s, p, used, scratch);
  } else {
    hipLaunchKernelGGL((k_attn_global_bf16<128, 256>), grid, dim3(256), 0, s, p, split_keys, scratch);
    hipLaunchKernelGGL(k_attn_global_merge<128>, dim3(a.H, a.n_tiles), dim3(128), 0, s, p, used, scratch);
  }
  return hipGetLastError();
}

}  // namespace tsk
