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
// bf16 kernel (gfx950 MFMA 32x32x16): a workgroup of four wavefronts owns 128
// query rows of one (tile, head); each wavefront owns 32.  Scores are formed
// transposed, S^T = K Q^T, so each lane holds one query's scores and the
// softmax max/sum stay in-lane (plus one exchange with the lane 32 apart);
// the output is accumulated transposed, O^T = V^T P^T, so the per-query
// rescale is in-lane too.  K rows are fed to the MFMA in an order that swaps
// bits 2 and 3 of the row index, which makes the score accumulator layout
// equal the P^T operand layout of the second MFMA (no shuffles).  K is staged
// as [key][hd] and V transposed as [hd][key], both with XOR-swizzled 16-byte
// chunks, double buffered; the RoPE table sits in LDS.
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
  float scale_log2;  // log2(e) / sqrt(hd)
};

__device__ __forceinline__ int window_row(const AttnP& p, int t, int i) {
  if (p.rows) return i < p.n ? p.rows[int64_t(t) * p.n + i] : p.n_union + t;
  return t * (p.n + 1) + i;
}

// (cos, sin) of rotation pair k of a head at the packed tile-local position
// pos (tau | y<<10 | x<<20): pair k belongs to axis a with index i inside
// that axis' chunk, stored at tab[rope_off[a] + 2*(pos_a*pairs[a] + i)].
__device__ __forceinline__ float2 rope_cs(const AttnP& p, const float* tab, int k, int pos) {
  const int p0 = p.pairs[0], p01 = p.pairs[0] + p.pairs[1];
  const int ax = k < p0 ? 0 : (k < p01 ? 1 : 2);
  const int i = k - (ax == 0 ? 0 : (ax == 1 ? p0 : p01));
  const int np = ax == 0 ? p.pairs[0] : (ax == 1 ? p.pairs[1] : p.pairs[2]);
  const int off = ax == 0 ? p.rope_off[0] : (ax == 1 ? p.rope_off[1] : p.rope_off[2]);
  const int ps = (pos >> (10 * ax)) & 1023;
  return *reinterpret_cast<const float2*>(tab + off + 2 * (ps * np + i));
}

// Packed per-pair lookup descriptor: table offset of position 0 (bits 0..13),
// floats per position step (bits 14..22), axis (bits 24..25).
__device__ __forceinline__ int rope_desc(const AttnP& p, int k) {
  const int p0 = p.pairs[0], p01 = p.pairs[0] + p.pairs[1];
  const int ax = k < p0 ? 0 : (k < p01 ? 1 : 2);
  const int i = k - (ax == 0 ? 0 : (ax == 1 ? p0 : p01));
  const int np = ax == 0 ? p.pairs[0] : (ax == 1 ? p.pairs[1] : p.pairs[2]);
  const int off = ax == 0 ? p.rope_off[0] : (ax == 1 ? p.rope_off[1] : p.rope_off[2]);
  return (off + 2 * i) | ((2 * np) << 14) | (ax << 24);
}
__device__ __forceinline__ float2 rope_at(const float* tab, int desc, int pos) {
  const int ps = (pos >> (10 * (desc >> 24))) & 1023;
  return *reinterpret_cast<const float2*>(tab + (desc & 0x3fff) + ps * ((desc >> 14) & 0x1ff));
}

// ------------------------------------------------------------- fp32 -----
// One thread per query row, keys staged through LDS 64 at a time.
template <int HD>
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
    if (pos >= 0) {
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
          const float2 cs = rope_cs(p, p.rope, k, kpos);
          const float c = cs.x, s = cs.y;
          const float a = kp[2 * k], b = kp[2 * k + 1];
          Ks[threadIdx.x][2 * k] = a * c - b * s;
          Ks[threadIdx.x][2 * k + 1] = a * s + b * c;
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
constexpr int KB = 64;             // keys per staged block
// RoPE table floats kept in LDS: 14.75 KB at head_dim 128 (so two workgroups of
// 80 KB fit in a CU's 160 KB), 16 KB otherwise
template <int HD> constexpr int rope_lds_floats() { return HD == 128 ? 3776 : 4096; }
constexpr float RESCALE_LOG2 = 8.0f;   // keep a stale running max until a block exceeds it by 2^8

// Swap bits 2 and 3 of a row index in 0..31.
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// LDS swizzles (16-byte chunk c of row r is stored at chunk c ^ key(r)).
// Keys: bits 0, 1 and 3 of the key row, so the eight rows one MFMA read
// phase touches (rows swap23(0..7) = 0-3, 8-11) get eight different keys;
// for V^T rows, hd ^ (hd >> 3), distinct both for eight consecutive hd rows
// (fragment reads) and for eight hd rows 8 apart (transposing writes).
__device__ __forceinline__ int kswz(int r) { return (r & 3) | ((r >> 1) & 4); }
__device__ __forceinline__ int vswz(int hd) { return (hd ^ (hd >> 3)) & 7; }

// Rotate 4 pairs (8 bf16) by the tile-local position `pos` (packed tau|y<<10|x<<20),
// pairs 4*c .. 4*c+3 of the head, with their descriptors from desc_s.
__device__ __forceinline__ bf16x8 rope8(const float* rope_s, const int* desc_s, int c, int pos, bf16x8 v) {
  const i32x4 dsc = *reinterpret_cast<const i32x4*>(desc_s + 4 * c);
  bf16x8 o;
#pragma unroll
  for (int q2 = 0; q2 < 4; ++q2) {
    const float2 cs = rope_at(rope_s, dsc[q2], pos);
    const float a = float(v[2 * q2]), b = float(v[2 * q2 + 1]);
    o[2 * q2] = bf16(a * cs.x - b * cs.y);
    o[2 * q2 + 1] = bf16(a * cs.y + b * cs.x);
  }
  return o;
}

// Window attention for the tile tokens (query rows 0..n-1); the global
// token's own query row is done by k_attn_global_bf16.
// NQ 32-row query blocks per wavefront, four wavefronts per workgroup.
template <int HD, int NQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NQ == 1 ? 2 : 1, NQ == 1 ? 2 : 1))) void k_attn_bf16(AttnP p) {
  constexpr int QW = 32 * NQ;         // query rows per wavefront
  constexpr int QB = 4 * QW;          // query rows per workgroup
  constexpr int HC = HD / 8;          // 16-byte chunks per head row
  constexpr int KROWB = HD * 2;       // bytes per staged key row
  constexpr int KCPT = HC / 4;        // key chunks per thread (4 threads per key row)
  constexpr int VSB = KB / 4 * HC;    // V sub-blocks (4 keys x 8 hd), one per thread
  constexpr int NHB = HD / 32;        // 32-row hd blocks of O^T
  constexpr int KSTEPS = HD / 16;     // MFMA k-steps of S^T
  __shared__ __attribute__((aligned(16))) char Ks[2][KB * KROWB];
  __shared__ __attribute__((aligned(16))) char Vt[2][HD * KB * 2];
  __shared__ __attribute__((aligned(16))) float rope_s[rope_lds_floats<HD>()];
  __shared__ int idx_s[2][2][KB];     // [slot][row | pos][key]
  __shared__ __attribute__((aligned(16))) int desc_s[HD / 2];

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
  const int kcol = p.d + h * HD, vcol = 2 * p.d + h * HD;
  const int nkb = (n + KB - 1) / KB;

  for (int e = tid; e < p.rope_floats; e += 256) rope_s[e] = p.rope[e];
  if (tid < HD / 2) desc_s[tid] = rope_desc(p, tid);
  // row index and position of key j (clamped into the window)
  auto key_meta = [&](int j, int& row, int& pos) {
    j = min(j, n - 1);
    row = window_row(p, t, j);
    pos = p.local_pos[j];
  };
  if (tid < KB) {
    int r0, p0, r1, p1;
    key_meta(tid, r0, p0);
    key_meta(KB + tid, r1, p1);
    idx_s[0][0][tid] = r0;
    idx_s[0][1][tid] = p0;
    idx_s[1][0][tid] = r1;
    idx_s[1][1][tid] = p1;
  }

  // staging roles.  K: row kr_row, chunks kpart + 4*i; a wavefront's 64
  // lanes cover 16 rows, the 8 lanes of one LDS write phase rows m and m+8.
  // V: keys 4*v_k4 .. +3 of hd chunk v_hc, neighbouring lanes alternating
  // between two key groups so one 8-byte write phase hits 16 distinct slots.
  const int kr_row = 16 * wave + (((lane >> 2) & 1) << 3) + (lane >> 3), kpart = lane & 3;
  const bool v_on = tid < VSB;
  const int v_hc = (tid >> 1) % HC, v_k4 = (tid & 1) + 2 * (tid / (2 * HC));
  i32x4 kreg[KCPT], vreg[4];
  auto gload = [&](int slot) {
    const int r = idx_s[slot][0][kr_row];
#pragma unroll
    for (int i = 0; i < KCPT; ++i)
      kreg[i] = *reinterpret_cast<const i32x4*>(qkv + r * ld + kcol + (kpart + 4 * i) * 8);
    if (v_on) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rv = idx_s[slot][0][4 * v_k4 + e];
        vreg[e] = *reinterpret_cast<const i32x4*>(qkv + rv * ld + vcol + v_hc * 8);
      }
    }
  };
  auto lstore = [&](int slot, int st) {
    const int pos = idx_s[slot][1][kr_row];
#pragma unroll
    for (int i = 0; i < KCPT; ++i) {
      const int c = kpart + 4 * i;
      const bf16x8 o = rope8(rope_s, desc_s, c, pos, __builtin_bit_cast(bf16x8, kreg[i]));
      *reinterpret_cast<bf16x8*>(&Ks[st][kr_row * KROWB + ((c ^ kswz(kr_row)) * 16)]) = o;
    }
    if (v_on) {
      const bf16x8 v0 = __builtin_bit_cast(bf16x8, vreg[0]), v1 = __builtin_bit_cast(bf16x8, vreg[1]);
      const bf16x8 v2 = __builtin_bit_cast(bf16x8, vreg[2]), v3 = __builtin_bit_cast(bf16x8, vreg[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int hdr = v_hc * 8 + e;
        const bf16x4 w = {v0[e], v1[e], v2[e], v3[e]};
        const int chunk = (v_k4 >> 1) ^ vswz(hdr);
        *reinterpret_cast<bf16x4*>(&Vt[st][hdr * (KB * 2) + chunk * 16 + (v_k4 & 1) * 8]) = w;
      }
    }
  };

  __syncthreads();  // rope_s, idx_s ready
  gload(0);

  // ---- this wavefront's 64 queries: B operand of S^T = K Q^T (hd 16s + 8g + e)
  const int q0 = qblk * QB + wave * QW + l32;
  const int grow = window_row(p, t, n);
  const bf16* kgp = qkv + grow * ld + kcol;
  const bf16* vgp = qkv + grow * ld + vcol;
  const float C = p.scale_log2;
  bf16x8 qf[NQ][KSTEPS];
  float m_run[NQ], l_run[NQ];
  f32x16 oacc[NQ][NHB];
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    const int qi = min(q0 + 32 * qq, n - 1);
    const bf16* qp = qkv + window_row(p, t, qi) * ld + h * HD;
    const int qpos = p.local_pos[qi];
    float sg = 0.f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int hd0 = 16 * s + 8 * g;
      const bf16x8 r = rope8(rope_s, desc_s, hd0 / 8, qpos, *reinterpret_cast<const bf16x8*>(qp + hd0));
      const bf16x8 kg = *reinterpret_cast<const bf16x8*>(kgp + hd0);
      qf[qq][s] = r;
#pragma unroll
      for (int e = 0; e < 8; ++e) sg += float(r[e]) * float(kg[e]);
    }
    sg += __shfl_xor(sg, 32, 64);
    // online softmax state starts from the global key: score sg, weight 1, value v_g
    m_run[qq] = sg * C;
    l_run[qq] = g == 0 ? 1.f : 0.f;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qq][hb][r] = float(vgp[hb * 32 + 8 * (r >> 2) + 4 * g + (r & 3)]);
  }

  lstore(0, 0);
  __syncthreads();
  const int krow_a = swap23(l32);  // key row this lane feeds as MFMA A row
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) gload((kb + 1) & 1);
    int pre_r = 0, pre_p = 0;
    const bool pre = tid < KB && kb + 2 < nkb;
    if (pre) key_meta((kb + 2) * KB + tid, pre_r, pre_p);
    const char* ks = Ks[cur];
    const char* vt = Vt[cur];

    const int j0 = kb * KB;
    // ---- S^T = K Q^T for the 64 keys: two 32-key chains per query block.
    // K fragments are read ahead of the MFMAs that use them (the schedule
    // below keeps four LDS reads in flight).
    f32x16 sacc[NQ][2];
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qq][sb][r] = 0.f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int kr = sb * 32 + krow_a;
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(ks + kr * KROWB + (((2 * s + g) ^ kswz(kr)) * 16));
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq)
          sacc[qq][sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qq][s], sacc[qq][sb], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
#pragma unroll
    for (int i = 0; i < 2 * KSTEPS - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, NQ, 0);  // MFMA(s) of one fragment
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // next LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * NQ, 0);
    if (j0 + KB > n) {  // keys past the window end (last block only)
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            // accumulator row 8(r/4)+4g+(r%4) holds key swap23(that row)
            const int key = j0 + sb * 32 + swap23(8 * (r >> 2) + 4 * g + (r & 3));
            if (key >= n) sacc[qq][sb][r] = -INFINITY;
          }
    }
    // ---- online softmax over the block (one rescale check per block)
    bf16x8 pf[NQ][4];
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qq][sb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * C;
      // rescale only when some query's block max passes its running max by 2^8
      if (__builtin_amdgcn_ballot_w64(mx > m_run[qq] + RESCALE_LOG2) != 0) {
        const float m_new = fmaxf(m_run[qq], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qq] - m_new);
        m_run[qq] = m_new;
        l_run[qq] *= alpha;
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) oacc[qq][hb] *= alpha;
      }
      const float mneg = -m_run[qq];
      float lsum = 0.f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[qq][sb][r], C, mneg));
          lsum += pv;
          pf[qq][sb * 2 + (r >> 3)][r & 7] = bf16(pv);
        }
      l_run[qq] += lsum;
    }
    // ---- O^T += V^T P^T over four 16-key chunks (NHB independent chains)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const int hdr = hb * 32 + l32;
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
            vt + hdr * (KB * 2) + (((2 * cc + g) ^ vswz(hdr)) * 16));
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq)
          oacc[qq][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qq][cc], oacc[qq][hb], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * NHB - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, NQ, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * NQ, 0);
    if (kb + 1 < nkb) lstore((kb + 1) & 1, cur ^ 1);
    if (pre) {
      idx_s[cur][0][tid] = pre_r;
      idx_s[cur][1][tid] = pre_p;
    }
    __syncthreads();
  }

#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    const int qi = q0 + 32 * qq;
    const float l_tot = l_run[qq] + __shfl_xor(l_run[qq], 32, 64);
    if (qi >= n) continue;
    const float inv = 1.0f / l_tot;
    bf16* out = (bf16*)p.out + (int64_t(t) * (n + 1) + qi) * p.d + h * HD;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const bf16x4 w = {bf16(oacc[qq][hb][4 * r4] * inv), bf16(oacc[qq][hb][4 * r4 + 1] * inv),
                          bf16(oacc[qq][hb][4 * r4 + 2] * inv), bf16(oacc[qq][hb][4 * r4 + 3] * inv)};
        *reinterpret_cast<bf16x4*>(out + hb * 32 + 8 * r4 + 4 * g) = w;
      }
  }
}

// The global token's query row of every (tile, head): one workgroup per
// (head, tile); LPK lanes share one key (lane = rotation pair), each
// wavefront walks every 4th key group with its own online softmax, and the
// four partial states are merged through LDS at the end.
template <int HD>
__global__ __launch_bounds__(256) void k_attn_global_bf16(AttnP p) {
  constexpr int LPK = HD / 2;        // lanes per key: one rotation pair each
  constexpr int KPI = 64 / LPK;      // keys per wavefront step
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pr = lane % LPK, ksub = lane / LPK;
  const int h = blockIdx.x, t = blockIdx.y, n = p.n;
  const bf16* qkv = (const bf16*)p.qkv;
  const int64_t ld = 3 * int64_t(p.d);
  const int grow = window_row(p, t, n);
  const bf16* base = qkv + grow * ld + h * HD + 2 * pr;
  const float qa = float(base[0]), qb = float(base[1]);   // global query: no rotation
  const float C = p.scale_log2;
  // global key first (not rotated)
  float sg = qa * float(base[p.d]) + qb * float(base[p.d + 1]);
  sg = group_sum(sg, LPK);
  float m = sg * C, l = 0.f, a0 = 0.f, a1 = 0.f;
  if (wave == 0 && ksub == 0) {
    l = 1.f;
    a0 = float(base[2 * p.d]);
    a1 = float(base[2 * p.d + 1]);
  }
  const int dsc = rope_desc(p, pr);
  for (int j = wave * KPI + ksub; j < n; j += 4 * KPI) {
    const int r = window_row(p, t, j);
    const bf16* kp = qkv + r * ld + p.d + h * HD + 2 * pr;
    const float2 cs = rope_at(p.rope, dsc, p.local_pos[j]);
    const float c = cs.x, sn = cs.y;
    const float ka = float(kp[0]), kb = float(kp[1]);
    const float kra = float(bf16(ka * c - kb * sn)), krb = float(bf16(ka * sn + kb * c));
    float sc = group_sum(qa * kra + qb * krb, LPK) * C;
    const float mn = fmaxf(m, sc);
    const float al = __builtin_amdgcn_exp2f(m - mn), pj = __builtin_amdgcn_exp2f(sc - mn);
    l = l * al + pj;
    a0 = a0 * al + pj * float(kp[p.d]);
    a1 = a1 * al + pj * float(kp[p.d + 1]);
    m = mn;
  }
  // merge the 4 * KPI partial states
  __shared__ float ms[4 * KPI], ls[4 * KPI];
  __shared__ float acc_s[4 * KPI][HD];
  const int slot = wave * KPI + ksub;
  if (pr == 0) {
    ms[slot] = m;
    ls[slot] = l;
  }
  acc_s[slot][2 * pr] = a0;
  acc_s[slot][2 * pr + 1] = a1;
  __syncthreads();
  if (tid < HD) {
    float mm = -INFINITY;
    for (int s = 0; s < 4 * KPI; ++s) mm = fmaxf(mm, ms[s]);
    float lt = 0.f, at = 0.f;
    for (int s = 0; s < 4 * KPI; ++s) {
      const float w = __builtin_amdgcn_exp2f(ms[s] - mm);
      lt += ls[s] * w;
      at += acc_s[s][tid] * w;
    }
    bf16* out = (bf16*)p.out + (int64_t(t) * (n + 1) + n) * p.d + h * HD;
    out[tid] = bf16(at / lt);
  }
}

// Query rows per wavefront of the bf16 kernel: 32 (two workgroups per CU) or
// 64 (one); TS_ATTN_ROWS_PER_WAVE overrides the default for measurements.
int attn_rows_per_wave() {
  static int v = [] {
    const char* e = getenv("TS_ATTN_ROWS_PER_WAVE");
    return (e && atoi(e) == 64) ? 64 : 32;
  }();
  return v;
}

}  // namespace

namespace tsk {

hipError_t attention(hipStream_t s, int act, const AttnArgs& a) {
  AttnP p{a.qkv, a.out, a.rows, a.n_union, a.d, a.H, a.n_tiles, a.n, a.local_pos, a.rope, a.rope_floats,
          {a.pairs[0], a.pairs[1], a.pairs[2]}, {a.rope_off[0], a.rope_off[1], a.rope_off[2]},
          1.4426950408889634f / sqrtf(float(a.hd))};
  if (act == ACT_F32) {
    const dim3 grid((a.n + 1 + 63) / 64, a.H, a.n_tiles), block(64);
    if (a.hd == 32) hipLaunchKernelGGL(k_attn_f32<32>, grid, block, 0, s, p);
    else if (a.hd == 64) hipLaunchKernelGGL(k_attn_f32<64>, grid, block, 0, s, p);
    else hipLaunchKernelGGL(k_attn_f32<128>, grid, block, 0, s, p);
    return hipGetLastError();
  }
  if (a.n < 1) return hipErrorInvalidValue;
  const int nq = attn_rows_per_wave() / 32;
  const dim3 grid(((a.n + 128 * nq - 1) / (128 * nq)) * a.H * a.n_tiles), block(256);
  const dim3 ggrid(a.H, a.n_tiles);
  if (a.hd == 64) {
    if (nq == 1) hipLaunchKernelGGL((k_attn_bf16<64, 1>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_attn_bf16<64, 2>), grid, block, 0, s, p);
    hipLaunchKernelGGL(k_attn_global_bf16<64>, ggrid, block, 0, s, p);
  } else if (a.hd == 128) {
    if (nq == 1) hipLaunchKernelGGL((k_attn_bf16<128, 1>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_attn_bf16<128, 2>), grid, block, 0, s, p);
    hipLaunchKernelGGL(k_attn_global_bf16<128>, ggrid, block, 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tsk
