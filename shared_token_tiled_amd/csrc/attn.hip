// Per-tile window attention of the TileShare layer (Figure 2 caption and
// Table S1: attention still runs per released tile, with the tile's own
// global token and tile-local coordinates; in shared layers keys and values
// come from the shared states).  One launch covers every (tile, head):
// query / key / value rows of tile t are read in place from the row-major
// qkv array through the tile's row map (shared layers) or from the tile's own
// rows (per-tile layers), RoPE is applied while staging, and the global token
// enters the online softmax as its initial state (score, weight 1, value).
// Output rows are written in per-tile layout: row t*(n+1)+i for window token
// i (i = n is the global token).
//
// bf16 kernel (gfx950 MFMA 32x32x16): a workgroup of eight wavefronts owns
// 256 query rows of one (tile, head), 32 per wavefront, and stages each block
// of 64 keys once for all of them.  Scores are formed transposed, S^T = K Q^T,
// so each lane holds one query's scores and the softmax max/sum stay in-lane
// (plus one exchange with the lane 32 apart); the output is accumulated
// transposed, O^T = V^T P^T, so the per-query rescale is in-lane too.  K rows
// are fed to the MFMA in an order that swaps bits 2 and 3 of the row index,
// which makes the score accumulator layout equal the P^T operand layout of
// the second MFMA (no shuffles).  K is staged as [key][hd] (rotated) and V
// transposed as [hd][key], both with XOR-swizzled 16-byte chunks, double
// buffered; row indices and positions of the keys are prefetched two blocks
// ahead into an LDS ring, and the RoPE table sits in LDS.
#include <algorithm>
#include <cstdlib>

#include "device_common.h"
#include "ts_kernels.h"

namespace {

struct AttnP {
  const void* qkv;
  void* out;
  const int* rows;
  int n_union, d, H, n_tiles, n;
  const int* local_pos;
  const float* rope;   // compact per-axis (cos, sin) table (see rope_cs)
  int rope_floats;
  int pairs[3];
  int rope_off[3];
  int rope_wbase[3];
  int rope_wpairs[3];
  float scale_log2;  // log2(e) / sqrt(hd)
  const bf16* vt;    // [n_tiles][H][HD][n_pad] transposed window values (unrotated path)
};

__device__ __forceinline__ int window_row(const AttnP& p, int t, int i) {
  if (p.rows) return i < p.n ? p.rows[int64_t(t) * p.n + i] : p.n_union + t;
  return t * (p.n + 1) + i;
}

// Axis of rotation pair k (pairs are split over t, h, w in contiguous chunks).
__device__ __forceinline__ int pair_axis(const AttnP& p, int k) {
  return k < p.pairs[0] ? 0 : (k < p.pairs[0] + p.pairs[1] ? 1 : 2);
}
__device__ __forceinline__ int pick3(const int (&v)[3], int a) { return a == 0 ? v[0] : (a == 1 ? v[1] : v[2]); }

// (cos, sin) of rotation pair k of a head at the packed tile-local position
// pos (tau | y<<10 | x<<20).  Axis a's block of the compact table spans the
// pairs [rope_wbase[a], rope_wbase[a] + rope_wpairs[a]) per position.
__device__ __forceinline__ float2 rope_cs(const AttnP& p, const float* tab, int k, int pos) {
  const int ax = pair_axis(p, k);
  const int ps = (pos >> (10 * ax)) & 1023;
  return *reinterpret_cast<const float2*>(tab + pick3(p.rope_off, ax) +
                                          2 * (ps * pick3(p.rope_wpairs, ax) + k - pick3(p.rope_wbase, ax)));
}

// ------------------------------------------------------------- fp32 -----
// One thread per query row, keys staged through LDS 64 at a time.
template <int HD, bool ROPE>
__global__ __launch_bounds__(64) void k_attn_f32(AttnP p) {
  __shared__ float Ks[64][HD + 1];
  __shared__ float Vs[64][HD + 1];
  const int t = blockIdx.z, h = blockIdx.y;
  const int i = blockIdx.x * 64 + threadIdx.x;
  const int n = p.n;
  const float* qkv = (const float*)p.qkv;
  const int64_t ld = 3 * int64_t(p.d);
  const bool valid = i <= n;
  const int qrow = window_row(p, t, valid ? i : n);
  float q[HD];
  const float* qp = qkv + qrow * ld + h * HD;
  const int pos = (valid && i < n) ? p.local_pos[i] : -1;
#pragma unroll
  for (int k = 0; k < HD / 2; ++k) {
    float c = 1.f, s = 0.f;
    if (ROPE && pos >= 0) {
      const float2 cs = rope_cs(p, p.rope, k, pos);
      c = cs.x;
      s = cs.y;
    }
    const float a = qp[2 * k], b = qp[2 * k + 1];
    q[2 * k] = a * c - b * s;
    q[2 * k + 1] = a * s + b * c;
  }
  const float scale = 1.0f / sqrtf(float(HD));
  // global key: initial state
  const int grow = window_row(p, t, n);
  const float* kg = qkv + grow * ld + p.d + h * HD;
  const float* vg = qkv + grow * ld + 2 * p.d + h * HD;
  float sg = 0.f;
#pragma unroll
  for (int e = 0; e < HD; ++e) sg += q[e] * kg[e];
  float m = sg * scale, l = 1.f;
  float o[HD];
#pragma unroll
  for (int e = 0; e < HD; ++e) o[e] = vg[e];
  for (int j0 = 0; j0 < n; j0 += 64) {
    __syncthreads();
    {  // stage keys j0..j0+63 (this thread: key j0 + tid), RoPE applied
      const int j = j0 + threadIdx.x;
      if (j < n) {
        const int r = window_row(p, t, j);
        const float* kp = qkv + r * ld + p.d + h * HD;
        const float* vp = qkv + r * ld + 2 * p.d + h * HD;
        const int kpos = p.local_pos[j];
        for (int k = 0; k < HD / 2; ++k) {
          const float2 cs = ROPE ? rope_cs(p, p.rope, k, kpos) : make_float2(1.f, 0.f);
          const float a = kp[2 * k], b = kp[2 * k + 1];
          Ks[threadIdx.x][2 * k] = a * cs.x - b * cs.y;
          Ks[threadIdx.x][2 * k + 1] = a * cs.y + b * cs.x;
        }
        for (int e = 0; e < HD; ++e) Vs[threadIdx.x][e] = vp[e];
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
  if (!valid) return;
  float* out = (float*)p.out + (int64_t(t) * (n + 1) + i) * p.d + h * HD;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < HD; ++e) out[e] = o[e] * inv;
}

// ------------------------------------------------------------- bf16 -----
constexpr int NW = 8;              // wavefronts per workgroup
constexpr int QB = 32 * NW;        // query rows per workgroup
constexpr int KB = 64;             // keys per staged block
constexpr int ROPE_LDS_FLOATS = 4096;  // 16 KB
constexpr float RESCALE_LOG2 = 8.0f;   // keep a stale running max until a block exceeds it by 2^8

// Swap bits 2 and 3 of a row index in 0..31.
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// LDS swizzles (16-byte chunk c of row r is stored at chunk c ^ key(r)).  The
// LDS has 64 banks of 4 bytes; a 16-byte access is served 16 lanes at a time,
// so the 16 lanes of one phase must hit 16 different 16-byte bank groups.
// K rows (HD*2 bytes): the 16 rows one MFMA read phase touches (swap23(0..15)
// = 0..15) get 16 different keys (head size 128: row & 15; head size 64,
// 128-byte rows where row parity already selects the half: (row >> 1) & 7).
// V^T rows (128 bytes): hd ^ (hd >> 3), distinct over the even and over the
// odd rows of 16 consecutive hd rows (fragment reads) and over hd rows 8 apart
// (transposing writes).
template <int HD> __device__ __forceinline__ int kswz(int r) { return HD == 128 ? (r & 15) : ((r >> 1) & 7); }
__device__ __forceinline__ int vswz(int hd) { return (hd ^ (hd >> 3)) & 7; }

// Table lookup of one 8-dim group, rotation pairs 4c .. 4c+3.  Segment 0 is
// the table block of the axis of pair 4c, segment 1 that of pair 4c+3; the
// first `split` pairs take segment 0 (split = 4 when the group lies in one
// axis).  In each block the group's four (cos, sin) pairs are 32 contiguous,
// 32-byte aligned bytes, so a segment is two 16-byte reads.
struct GroupRope {
  int off0, step0, shift0;
  int off1, step1, shift1;
  int split;
};
__device__ __forceinline__ GroupRope group_rope(const AttnP& p, int c) {
  const int k = 4 * c;
  const int a0 = pair_axis(p, k), a1 = pair_axis(p, k + 3);
  GroupRope g;
  g.off0 = pick3(p.rope_off, a0) + 2 * (k - pick3(p.rope_wbase, a0));
  g.step0 = 2 * pick3(p.rope_wpairs, a0);
  g.shift0 = 10 * a0;
  g.off1 = pick3(p.rope_off, a1) + 2 * (k - pick3(p.rope_wbase, a1));
  g.step1 = 2 * pick3(p.rope_wpairs, a1);
  g.shift1 = 10 * a1;
  g.split = a0 == a1 ? 4 : (a0 == 0 ? p.pairs[0] : p.pairs[0] + p.pairs[1]) - k;
  return g;
}

// Rotate one 8-dim group (4 pairs, bf16) by position `pos`; each rotated
// value is rounded to bf16.
__device__ __forceinline__ bf16x8 rope_group(const float* tab, const GroupRope& gr, int pos, bf16x8 v) {
  const float* cs = tab + gr.off0 + ((pos >> gr.shift0) & 1023) * gr.step0;
  f32x4 c01 = *reinterpret_cast<const f32x4*>(cs);      // (cos, sin) of pairs 0, 1
  f32x4 c23 = *reinterpret_cast<const f32x4*>(cs + 4);  // pairs 2, 3
  if (gr.split < 4) {  // pairs split .. 3 belong to the next axis
    const float* cs1 = tab + gr.off1 + ((pos >> gr.shift1) & 1023) * gr.step1;
    const f32x4 d01 = *reinterpret_cast<const f32x4*>(cs1);
    const f32x4 d23 = *reinterpret_cast<const f32x4*>(cs1 + 4);
    if (gr.split == 1) c01 = f32x4{c01[0], c01[1], d01[2], d01[3]};
    if (gr.split <= 2) c23 = d23;
    else c23 = f32x4{c23[0], c23[1], d23[2], d23[3]};
  }
  bf16x8 o;
#pragma unroll
  for (int q2 = 0; q2 < 4; ++q2) {
    const float c = q2 < 2 ? c01[2 * q2] : c23[2 * q2 - 4];
    const float s = q2 < 2 ? c01[2 * q2 + 1] : c23[2 * q2 - 3];
    const float a = float(v[2 * q2]), b = float(v[2 * q2 + 1]);
    o[2 * q2] = bf16(a * c - b * s);
    o[2 * q2 + 1] = bf16(a * s + b * c);
  }
  return o;
}

template <int HD, bool ROPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_bf16(AttnP p) {
  constexpr int NT = NW * 64;         // threads
  constexpr int HC = HD / 8;          // 16-byte chunks per head row
  constexpr int KROWB = HD * 2;       // bytes per staged key row
  constexpr int KCPT = HC / 8;        // key chunks per thread (8 threads per key row)
  constexpr int VSB = KB / 2 * HC;    // V transpose units (2 keys x 8 hd)
  constexpr int NHB = HD / 32;        // 32-row hd blocks of O^T
  constexpr int KSTEPS = HD / 16;     // MFMA k-steps of S^T
  static_assert(VSB <= NT, "one V unit per thread");
  // LDS stages of K and V^T: two with in-kernel RoPE (registers carry the
  // next block), three when both are DMA-staged (block kb+2 is in flight
  // while kb is computed, so a block's loads have two blocks of time to land)
  constexpr int NST = ROPE ? 2 : 3;
  constexpr int AHEAD = ROPE ? 2 : 3;   // blocks ahead the key rows are fetched
  constexpr int NSL = ROPE ? 2 : 4;     // slots of the key-row ring
  __shared__ __attribute__((aligned(16))) char Ks[NST][KB * KROWB];
  __shared__ __attribute__((aligned(16))) char Vt[NST][HD * KB * 2];
  __shared__ __attribute__((aligned(16))) float rope_s[ROPE ? ROPE_LDS_FLOATS : 4];
  __shared__ int idx_s[NSL][2][KB];   // [slot][row | pos][key]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int n = p.n;
  // XCD-aware order: the hardware deals workgroup b to XCD b % 8; give each
  // XCD a contiguous run of (tile, head, query-block) jobs so the query blocks
  // that stream the same keys and values share one L2.
  const int nqb = (n + QB - 1) / QB;
  int qblk, h, t;
  {
    const int total = nqb * p.H * p.n_tiles;
    const int b = blockIdx.x, xcd = b & 7, loc = b >> 3;
    const int q8 = total >> 3, r8 = total & 7;
    const int id = xcd < r8 ? xcd * (q8 + 1) + loc : r8 * (q8 + 1) + (xcd - r8) * q8 + loc;
    qblk = id % nqb;
    h = (id / nqb) % p.H;
    t = id / (nqb * p.H);
  }
  const bf16* qkv = (const bf16*)p.qkv;
  const int64_t ld = 3 * int64_t(p.d);
  const bf16* kbase = qkv + p.d + h * HD;
  const bf16* vbase = qkv + 2 * p.d + h * HD;
  const int nkb = (n + KB - 1) / KB;

  if (ROPE)
    for (int e = tid; e < p.rope_floats; e += NT) rope_s[e] = p.rope[e];
  // row index and position of key j (clamped into the window)
  auto key_meta = [&](int j, int& row, int& pos) {
    j = min(j, n - 1);
    row = window_row(p, t, j);
    pos = ROPE ? p.local_pos[j] : 0;
  };
  if (tid < KB) {
#pragma unroll
    for (int b = 0; b < AHEAD; ++b) {
      int r0, p0;
      key_meta(b * KB + tid, r0, p0);
      idx_s[b][0][tid] = r0;
      idx_s[b][1][tid] = p0;
    }
  }

  // staging roles.  K: row kr_row, chunks kpart + 8*i, 8 threads per row; a
  // 16-lane write phase covers two rows, chosen 8 apart at head size 128 (so
  // their keys differ in bit 3) and adjacent at 64 (so their parity differs).
  // V: keys 2*v_k2, 2*v_k2+1 of hd chunk v_hc (one 4-byte write phase hits
  // 32 banks twice: a 2-way conflict on 8 small writes per block, cheaper than
  // the per-lane row reordering that would avoid it).
  const int lg = lane >> 3;
  const int kr_row = HD == 128 ? (wave >> 1) * 16 + (wave & 1) * 4 + (lg >> 1) + (lg & 1) * 8 : tid >> 3;
  const int kpart = tid & 7;
  GroupRope kgr[KCPT];
#pragma unroll
  for (int i = 0; i < KCPT; ++i) kgr[i] = group_rope(p, kpart + 8 * i);
  const bool v_on = tid < VSB;
  const int v_hc = (tid & 7) + 8 * (tid / 256), v_k2 = (tid >> 3) & 31;
  i32x4 kreg[KCPT], vreg[2];
  // without RoPE, K goes straight from global memory to LDS (global_load_lds:
  // lane l of a wavefront instruction writes 16 bytes at LDS base + 16*l):
  // instruction i of wavefront w fills bytes [(w*KDI + i) KB, +1 KB) of the
  // stage, i.e. row b / KROWB, slot (b % KROWB) / 16 for lane byte b, and the
  // lane loads the logical chunk the swizzle puts in that slot
  constexpr int KDI = KB * KROWB / 1024 / NW;  // K DMA instructions per wavefront
  constexpr int VDI = HD * KB * 2 / 1024 / NW;  // V^T DMA instructions per wavefront
  static_assert(KDI >= 1 && VDI >= 1, "whole 1 KB DMA rows per wavefront");
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int64_t n_pad = int64_t(nkb) * KB;
  const bf16* vtbase = ROPE ? nullptr : p.vt + (int64_t(t) * p.H + h) * HD * n_pad;
  // DMA staging in two steps: the key rows this lane's K loads need (from
  // the ring), then the loads, so that the ring can be refilled in between
  auto dma_rows = [&](int blk, int (&rr)[KDI]) {
#pragma unroll
    for (int i = 0; i < KDI; ++i) {
      const int row = ((wv * KDI + i) * 1024 + 16 * lane) / KROWB;
      rr[i] = p.rows ? idx_s[blk % NSL][0][row] : t * (n + 1) + min(blk * KB + row, n - 1);
    }
  };
  auto dma = [&](int blk, const int (&rr)[KDI]) {
    const int st = blk % NST;
#pragma unroll
    for (int i = 0; i < KDI; ++i) {
      const int b = (wv * KDI + i) * 1024 + 16 * lane;
      const int row = b / KROWB, c = ((b % KROWB) / 16) ^ kswz<HD>(row);
      __builtin_amdgcn_global_load_lds((const void*)(kbase + rr[i] * ld + c * 8),
                                       (TS_LDS void*)(&Ks[st][(wv * KDI + i) * 1024]), 16, 0, 0);
    }
    // V^T rows hd = 8*(wv*VDI + i) + lane/8, LDS slot lane%8 of the 128-byte
    // row holds logical key chunk slot ^ vswz(hd) of block blk
#pragma unroll
    for (int i = 0; i < VDI; ++i) {
      const int hdr = 8 * (wv * VDI + i) + (lane >> 3), c = (lane & 7) ^ vswz(hdr);
      __builtin_amdgcn_global_load_lds((const void*)(vtbase + int64_t(hdr) * n_pad + blk * KB + c * 8),
                                       (TS_LDS void*)(&Vt[st][(wv * VDI + i) * 1024]), 16, 0, 0);
    }
  };
  auto gload = [&](int blk) {
    const int slot = blk % NSL;
    if constexpr (!ROPE) {
      int rr[KDI];
      dma_rows(blk, rr);
      dma(blk, rr);
    } else {
      const int r = idx_s[slot][0][kr_row];
#pragma unroll
      for (int i = 0; i < KCPT; ++i)
        kreg[i] = *reinterpret_cast<const i32x4*>(kbase + r * ld + (kpart + 8 * i) * 8);
    }
    if (ROPE && v_on) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int rv = idx_s[slot][0][2 * v_k2 + e];
        vreg[e] = *reinterpret_cast<const i32x4*>(vbase + rv * ld + v_hc * 8);
      }
    }
  };
  auto lstore = [&](int blk, int st) {
    const int slot = blk % NSL;
    if constexpr (ROPE) {
      const int pos = idx_s[slot][1][kr_row];
#pragma unroll
      for (int i = 0; i < KCPT; ++i) {
        const int c = kpart + 8 * i;
        const bf16x8 o = rope_group(rope_s, kgr[i], pos, __builtin_bit_cast(bf16x8, kreg[i]));
        *reinterpret_cast<bf16x8*>(&Ks[st][kr_row * KROWB + ((c ^ kswz<HD>(kr_row)) * 16)]) = o;
      }
    }
    if (ROPE && v_on) {
      const bf16x8 v0 = __builtin_bit_cast(bf16x8, vreg[0]), v1 = __builtin_bit_cast(bf16x8, vreg[1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int hdr = v_hc * 8 + e;
        const bf16 w2[2] = {v0[e], v1[e]};
        const int chunk = (v_k2 >> 2) ^ vswz(hdr);
        *reinterpret_cast<uint32_t*>(&Vt[st][hdr * (KB * 2) + chunk * 16 + (v_k2 & 3) * 4]) =
            __builtin_bit_cast(uint32_t, w2);
      }
    }
  };

  __syncthreads();  // rope_s, idx_s ready
  gload(0);
  if (!ROPE && nkb > 1) gload(1);

  // ---- this wavefront's 32 queries: B operand of S^T = K Q^T (hd 16s + 8g + e)
  const int qi = qblk * QB + wave * 32 + l32;
  const int grow = window_row(p, t, n);
  const bf16* kgp = kbase + grow * ld;
  const bf16* vgp = vbase + grow * ld;
  const float C = p.scale_log2;
  bf16x8 qf[KSTEPS];
  float m_run, l_run;
  f32x16 oacc[NHB];
  {
    const int qc = min(qi, n - 1);
    const bf16* qp = qkv + window_row(p, t, qc) * ld + h * HD;
    const int qpos = p.local_pos[qc];
    float sg = 0.f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int hd0 = 16 * s + 8 * g;
      const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qp + hd0);
      const bf16x8 r = ROPE ? rope_group(rope_s, group_rope(p, hd0 / 8), qpos, qv) : qv;
      const bf16x8 kg = *reinterpret_cast<const bf16x8*>(kgp + hd0);
      qf[s] = r;
#pragma unroll
      for (int e = 0; e < 8; ++e) sg += float(r[e]) * float(kg[e]);
    }
    sg += __shfl_xor(sg, 32, 64);
    // online softmax state starts from the global key: score sg, weight 1, value v_g
    m_run = sg * C;
    l_run = g == 0 ? 1.f : 0.f;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[hb][r] = float(vgp[hb * 32 + 8 * (r >> 2) + 4 * g + (r & 3)]);
  }

  lstore(0, 0);
  if (!ROPE) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wavefront's K DMA landed
  __syncthreads();
  const int krow_a = swap23(l32);  // key row this lane feeds as MFMA A row
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb % NST;
    // key rows of block kb+AHEAD.  DMA-staged: wavefront 0 copies them from
    // the row map straight into the ring (no registers, so nothing waits on
    // them before the block-end wait), ahead of this block's K / V^T loads so
    // that wait covers them; per-tile rows need no map.  In-kernel RoPE: row
    // and position through registers, stored at the block end.
    int pre_r = 0, pre_p = 0;
    const bool pre = ROPE && tid < KB && kb + AHEAD < nkb;
    if (pre) key_meta((kb + AHEAD) * KB + tid, pre_r, pre_p);
    if constexpr (ROPE) {
      if (kb + 1 < nkb) gload(kb + 1);
    } else {
      int rr[KDI];
      if (kb + 2 < nkb) dma_rows(kb + 2, rr);
      if (p.rows && wave == 0 && kb + AHEAD < nkb) {
        const int j = min((kb + AHEAD) * KB + lane, n - 1);
        __builtin_amdgcn_global_load_lds((const void*)(p.rows + int64_t(t) * n + j),
                                         (TS_LDS void*)(&idx_s[(kb + AHEAD) % NSL][0][0]), 4, 0, 0);
      }
      if (kb + 2 < nkb) dma(kb + 2, rr);
    }
    const char* ks = Ks[cur];
    const char* vt = Vt[cur];
    const int j0 = kb * KB;

    // ---- S^T = K Q^T for the 64 keys: two 32-key chains, K fragments read
    // ahead of the MFMAs that use them (four LDS reads kept in flight)
    f32x16 sacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[sb][r] = 0.f;
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
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
#pragma unroll
    for (int i = 0; i < 2 * KSTEPS - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the next LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    if (j0 + KB > n) {  // keys past the window end (last block only)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // accumulator row 8(r/4)+4g+(r%4) holds key swap23(that row)
          const int key = j0 + sb * 32 + swap23(8 * (r >> 2) + 4 * g + (r & 3));
          if (key >= n) sacc[sb][r] = -INFINITY;
        }
    }
    // ---- online softmax over the block (one rescale check per block)
    bf16x8 pf[4];
    {
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * C;
      // rescale only when some query's block max passes its running max by 2^8
      if (__builtin_amdgcn_ballot_w64(mx > m_run + RESCALE_LOG2) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) oacc[hb] *= alpha;
      }
      const float mneg = -m_run;
      float lsum = 0.f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[sb][r], C, mneg));
          lsum += pv;
          pf[sb * 2 + (r >> 3)][r & 7] = bf16(pv);
        }
      l_run += lsum;
    }
    // ---- O^T += V^T P^T over four 16-key chunks (NHB independent chains)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const int hdr = hb * 32 + l32;
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
            vt + hdr * (KB * 2) + (((2 * cc + g) ^ vswz(hdr)) * 16));
        oacc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[cc], oacc[hb], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * NHB - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

    if (ROPE && kb + 1 < nkb) lstore(kb + 1, cur ^ 1);
    if (pre) {
      idx_s[(kb + AHEAD) % NSL][0][tid] = pre_r;
      idx_s[(kb + AHEAD) % NSL][1][tid] = pre_p;
    }
    if constexpr (ROPE) {
      __syncthreads();
    } else {
      // this wavefront's loads of block kb+1 have landed (kb+2's may still be
      // in flight) and its LDS traffic is done; then a barrier without the
      // fence of __syncthreads, which would also wait for block kb+2
      if (kb + 2 < nkb) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(KDI + VDI) : "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qi >= n) return;
  const float inv = 1.0f / l_tot;
  bf16* out = (bf16*)p.out + (int64_t(t) * (n + 1) + qi) * p.d + h * HD;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const bf16x4 w = {bf16(oacc[hb][4 * r4] * inv), bf16(oacc[hb][4 * r4 + 1] * inv),
                        bf16(oacc[hb][4 * r4 + 2] * inv), bf16(oacc[hb][4 * r4 + 3] * inv)};
      *reinterpret_cast<bf16x4*>(out + hb * 32 + 8 * r4 + 4 * g) = w;
    }
}

// Global-token query row of one (head, tile), over the window keys
// [j_begin, j_end) of split blockIdx.z (key n is the global key itself, not
// rotated).  Keys are taken in chunks of GCH.  Score pass: HD/16 threads per
// key, 16 dims each (two 8-dim RoPE groups, the rotated key rounded to bf16 as
// the MFMA kernel stages it), summed across those lanes; scores and row
// indices go to LDS.  Value pass: each thread owns one 8-dim group of the
// output and a strided subset of the chunk's keys and keeps a running
// (max-shifted) weighted sum; the chunk max is shared by the workgroup, so
// every thread rescales by the same factor.  The partial sums are added in
// LDS at the end.  With one split the row is written; with several, each
// split leaves its state (max m, weight sum l, unnormalised output o[HD], in
// the exp2 domain) in `part` for k_attn_global_merge.
constexpr int GCH = 1024;
template <int HD, int NT, bool ROPE>
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
  const int64_t grow = window_row(p, t, n);

  // score-pass role: dims [16*sub, 16*sub + 16) of key slot kk
  const int sub = tid % TPK, kk = tid / TPK;
  const bf16* qp = qkv + grow * ld + h * HD + 16 * sub;
  const bf16x8 q0 = *reinterpret_cast<const bf16x8*>(qp), q1 = *reinterpret_cast<const bf16x8*>(qp + 8);
  const GroupRope gr0 = group_rope(p, 2 * sub), gr1 = group_rope(p, 2 * sub + 1);
  // value-pass role: dims [8*dg, 8*dg + 8), keys kg, kg + KG, ...
  const int dg = tid % DG, kg = tid / DG;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float l = 0.f, m_run = -INFINITY;

  for (int c0 = j_begin; c0 < j_end; c0 += GCH) {
    const int cnt = min(GCH, j_end - c0);
#pragma unroll 4
    for (int jj = kk; jj < cnt; jj += KPP) {
      const int j = c0 + jj;
      const int64_t r = window_row(p, t, j);
      const bf16* kp = qkv + r * ld + p.d + h * HD + 16 * sub;
      bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kp), k1 = *reinterpret_cast<const bf16x8*>(kp + 8);
      if (ROPE && j < n) {
        const int pos = p.local_pos[j];
        k0 = rope_group(p.rope, gr0, pos, k0);
        k1 = rope_group(p.rope, gr1, pos, k1);
      }
      float sc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sc += float(q0[e]) * float(k0[e]);
#pragma unroll
      for (int e = 0; e < 8; ++e) sc += float(q1[e]) * float(k1[e]);
#pragma unroll
      for (int o = 1; o < TPK; o <<= 1) sc += __shfl_xor(sc, o);
      if (sub == 0) {
        s_s[jj] = sc * p.scale_log2;
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
      bf16* out = (bf16*)p.out + (int64_t(t) * (n + 1) + n) * p.d + h * HD;
      out[tid] = bf16(o / lt);
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
  bf16* out = (bf16*)p.out + (int64_t(t) * (p.n + 1) + p.n) * p.d + h * HD;
  out[tid] = bf16(o / lt);
}

// Window values of one (64-key block, head, tile) transposed into vt: the
// block's 64 V rows (gathered through the tile's row map, 16-byte loads) go
// into an LDS tile [key][hd] whose row stride is an odd number of 4-byte
// words, written as 4-byte words; then 8 consecutive lanes assemble one hd
// row's 64 keys (8 keys each, 2-byte LDS reads that are free of bank
// conflicts with that stride) and store its 128 contiguous bytes.  Keys past
// the window end are zero.
template <int HD>
__global__ __launch_bounds__(256) void k_vtrans(AttnP p) {
  constexpr int CPR = HD / 8;   // 16-byte chunks per key row
  constexpr int LD = HD + 2;    // LDS row stride (elements): HD/2 + 1 words, odd
  __shared__ __attribute__((aligned(16))) bf16 tile[64 * LD];
  const int jb = blockIdx.x, h = blockIdx.y, t = blockIdx.z, tid = threadIdx.x;
  const int n = p.n;
  const int64_t ld = 3 * int64_t(p.d);
  const bf16* qkv = (const bf16*)p.qkv;
  for (int c = tid; c < 64 * CPR; c += 256) {
    const int key = c / CPR, part = c % CPR, j = jb * 64 + key;
    i32x4 v = {0, 0, 0, 0};
    if (j < n) v = *reinterpret_cast<const i32x4*>(qkv + int64_t(window_row(p, t, j)) * ld + 2 * p.d + h * HD + part * 8);
    uint32_t* w = reinterpret_cast<uint32_t*>(&tile[key * LD + part * 8]);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = uint32_t(v[e]);
  }
  __syncthreads();
  const int64_t n_pad = int64_t((n + 63) / 64) * 64;
  bf16* dst = const_cast<bf16*>(p.vt) + (int64_t(t) * p.H + h) * HD * n_pad + jb * 64;
  for (int c = tid; c < HD * 8; c += 256) {
    const int row = c >> 3, kc = c & 7;
    bf16x8 w;
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = tile[(kc * 8 + e) * LD + row];
    *reinterpret_cast<bf16x8*>(dst + int64_t(row) * n_pad + kc * 8) = w;
  }
}

}  // namespace

namespace tsk {

static AttnP make_params(const AttnArgs& a) {
  return AttnP{a.qkv, a.out, a.rows, a.n_union, a.d, a.H, a.n_tiles, a.n, a.local_pos, a.rope, a.rope_floats,
               {a.pairs[0], a.pairs[1], a.pairs[2]}, {a.rope_off[0], a.rope_off[1], a.rope_off[2]},
               {a.rope_wbase[0], a.rope_wbase[1], a.rope_wbase[2]},
               {a.rope_wpairs[0], a.rope_wpairs[1], a.rope_wpairs[2]},
               1.4426950408889634f / sqrtf(float(a.hd)), (const bf16*)a.vt};
}

hipError_t attention(hipStream_t s, int act, const AttnArgs& a, bool rope) {
  const AttnP p = make_params(a);
  if (act == ACT_F32) {
    const dim3 grid((a.n + 1 + 63) / 64, a.H, a.n_tiles), block(64);
    if (a.hd == 32) {
      if (rope) hipLaunchKernelGGL((k_attn_f32<32, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((k_attn_f32<32, false>), grid, block, 0, s, p);
    } else if (a.hd == 64) {
      if (rope) hipLaunchKernelGGL((k_attn_f32<64, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((k_attn_f32<64, false>), grid, block, 0, s, p);
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (a.n < 1) return hipErrorInvalidValue;
  const dim3 grid(((a.n + QB - 1) / QB) * a.H * a.n_tiles), block(NW * 64);
  if (a.hd == 64) {
    if (rope) hipLaunchKernelGGL((k_attn_bf16<64, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_attn_bf16<64, false>), grid, block, 0, s, p);
  } else if (a.hd == 128) {
    if (rope) hipLaunchKernelGGL((k_attn_bf16<128, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_attn_bf16<128, false>), grid, block, 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t v_transpose(hipStream_t s, const AttnArgs& a, void* vt) {
  AttnArgs b = a;
  b.vt = vt;
  const AttnP p = make_params(b);
  if (a.n < 1) return hipErrorInvalidValue;
  const dim3 grid((a.n + 63) / 64, a.H, a.n_tiles), block(256);
  if (a.hd == 64) hipLaunchKernelGGL(k_vtrans<64>, grid, block, 0, s, p);
  else if (a.hd == 128) hipLaunchKernelGGL(k_vtrans<128>, grid, block, 0, s, p);
  else return hipErrorInvalidValue;
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

hipError_t attention_global(hipStream_t s, const AttnArgs& a, bool rope, float* scratch, int64_t scratch_floats) {
  const AttnP p = make_params(a);
  if (a.n < 1 || (a.hd != 64 && a.hd != 128)) return hipErrorInvalidValue;
  const int splits = scratch ? attention_global_splits(a, scratch_floats) : 1;
#define TS_GL(HD, NT, SK, PART)                                                                           \
  do {                                                                                                    \
    if (rope) hipLaunchKernelGGL((k_attn_global_bf16<HD, NT, true>), grid, dim3(NT), 0, s, p, SK, PART);  \
    else hipLaunchKernelGGL((k_attn_global_bf16<HD, NT, false>), grid, dim3(NT), 0, s, p, SK, PART);      \
  } while (0)
  if (splits == 1) {
    const dim3 grid(a.H, a.n_tiles, 1);
    if (a.hd == 64) TS_GL(64, 1024, a.n + 1, nullptr);
    else TS_GL(128, 1024, a.n + 1, nullptr);
    return hipGetLastError();
  }
  int split_keys = (a.n + 1 + splits - 1) / splits;
  split_keys = (split_keys + 63) / 64 * 64;
  const int used = (a.n + 1 + split_keys - 1) / split_keys;   // every split holds >= 1 key
  const dim3 grid(a.H, a.n_tiles, used);
  if (a.hd == 64) {
    TS_GL(64, 256, split_keys, scratch);
    hipLaunchKernelGGL(k_attn_global_merge<64>, dim3(a.H, a.n_tiles), dim3(64), 0, s, p, used, scratch);
  } else {
    TS_GL(128, 256, split_keys, scratch);
    hipLaunchKernelGGL(k_attn_global_merge<128>, dim3(a.H, a.n_tiles), dim3(128), 0, s, p, used, scratch);
  }
#undef TS_GL
  return hipGetLastError();
}

}  // namespace tsk
