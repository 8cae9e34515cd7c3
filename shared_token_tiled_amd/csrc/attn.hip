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
#include "device_common.h"
#include "ts_kernels.h"

namespace {

struct AttnP {
  const void* qkv;
  void* out;
  const int* rows;
  int n_union, d, H, n_tiles, n;
  const int* local_pos;
  const float* rope;
  int maxl, pairs_t, pairs_h;
  float scale_log2;  // log2(e) / sqrt(hd)
};

__device__ __forceinline__ int window_row(const AttnP& p, int t, int i) {
  if (p.rows) return i < p.n ? p.rows[int64_t(t) * p.n + i] : p.n_union + t;
  return t * (p.n + 1) + i;
}

__device__ __forceinline__ int pair_axis(const AttnP& p, int k) {
  return k < p.pairs_t ? 0 : (k < p.pairs_t + p.pairs_h ? 1 : 2);
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
      const int ax = pair_axis(p, k);
      const int ps = (pos >> (10 * ax)) & 1023;
      c = p.rope[2 * (k * p.maxl + ps)];
      s = p.rope[2 * (k * p.maxl + ps) + 1];
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
          const int ax = pair_axis(p, k);
          const int ps = (kpos >> (10 * ax)) & 1023;
          const float c = p.rope[2 * (k * p.maxl + ps)], s = p.rope[2 * (k * p.maxl + ps) + 1];
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
constexpr int QB = 128;  // query rows per workgroup
constexpr int KB = 64;   // keys per staged block
constexpr int ROPE_LDS_FLOATS = 4096;  // 16 KB: pairs * maxl * (cos, sin)

// Swap bits 2 and 3 of a row index in 0..31.
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <int HD>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(AttnP p) {
  constexpr int HC = HD / 8;                 // 16-byte chunks per head row
  constexpr int KROWB = HD * 2;              // bytes per staged key row
  constexpr int KCH = KB * HC / 256;         // key chunks staged per thread
  constexpr int VSB = KB / 4 * HC;           // V sub-blocks (4 keys x 8 hd)
  constexpr int NHB = HD / 32;               // 32-row hd blocks of O^T
  constexpr int KSTEPS = HD / 16;            // MFMA k-steps of S^T
  __shared__ __attribute__((aligned(16))) char Ks[2][KB * KROWB];
  __shared__ __attribute__((aligned(16))) char Vt[2][HD * KB * 2];
  __shared__ float rope_s[ROPE_LDS_FLOATS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int t = blockIdx.z, h = blockIdx.y;
  const int n = p.n;
  const bf16* qkv = (const bf16*)p.qkv;
  const int64_t ld = 3 * int64_t(p.d);
  const int kcol = p.d + h * HD, vcol = 2 * p.d + h * HD;

  const int rope_n = (HD / 2) * p.maxl * 2;
  for (int e = tid; e < rope_n; e += 256) rope_s[e] = p.rope[e];

  // ---- staging roles ----
  // K: chunk c = tid + 256*i -> key row c / HC, hd chunk c % HC (fixed per thread)
  const int k_hc = tid % HC, k_r0 = tid / HC;
  constexpr int KRSTEP = 256 / HC;
  // V: sub-block sb = tid -> keys 4*(sb / HC) .. +3, hd chunk sb % HC
  const bool v_on = tid < VSB;
  const int v_hc = tid % HC, v_k4 = tid / HC;

  i32x4 kreg[KCH], vreg[4];
  int kpos[KCH];
  auto gload = [&](int kb) {
    const int j0 = kb * KB;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int j = min(j0 + k_r0 + KRSTEP * i, n - 1);
      const int r = window_row(p, t, j);
      kreg[i] = *reinterpret_cast<const i32x4*>(qkv + r * ld + kcol + k_hc * 8);
      kpos[i] = p.local_pos[j];
    }
    if (v_on) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = min(j0 + 4 * v_k4 + e, n - 1);
        const int r = window_row(p, t, j);
        vreg[e] = *reinterpret_cast<const i32x4*>(qkv + r * ld + vcol + v_hc * 8);
      }
    }
  };
  auto lstore = [&](int st) {
    // K with RoPE: pairs 4*k_hc .. 4*k_hc+3
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int r = k_r0 + KRSTEP * i;
      bf16x8 v = __builtin_bit_cast(bf16x8, kreg[i]);
      bf16x8 o;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const int k = 4 * k_hc + q2;
        const int ps = (kpos[i] >> (10 * pair_axis(p, k))) & 1023;
        const float c = rope_s[2 * (k * p.maxl + ps)], s = rope_s[2 * (k * p.maxl + ps) + 1];
        const float a = float(v[2 * q2]), b = float(v[2 * q2 + 1]);
        o[2 * q2] = bf16(a * c - b * s);
        o[2 * q2 + 1] = bf16(a * s + b * c);
      }
      *reinterpret_cast<bf16x8*>(&Ks[st][r * KROWB + ((k_hc ^ (r & 7)) * 16)]) = o;
    }
    if (v_on) {
      // transpose 4 keys x 8 hd into 8 rows (hd) x 4 keys
      bf16x8 v0 = __builtin_bit_cast(bf16x8, vreg[0]), v1 = __builtin_bit_cast(bf16x8, vreg[1]);
      bf16x8 v2 = __builtin_bit_cast(bf16x8, vreg[2]), v3 = __builtin_bit_cast(bf16x8, vreg[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int hdr = v_hc * 8 + e;
        bf16x4 w = {v0[e], v1[e], v2[e], v3[e]};
        const int chunk = (v_k4 >> 1) ^ (hdr & 7);
        *reinterpret_cast<bf16x4*>(&Vt[st][hdr * (KB * 2) + chunk * 16 + (v_k4 & 1) * 8]) = w;
      }
    }
  };

  // ---- this lane's query (B operand of S^T = K Q^T): hd 16s + 8g + e ----
  const int qi = blockIdx.x * QB + wave * 32 + l32;
  const bool qvalid = qi <= n;
  const int qrow = window_row(p, t, qvalid ? qi : n);
  const int qpos = (qvalid && qi < n) ? p.local_pos[qi] : -1;
  __syncthreads();  // rope_s ready
  bf16x8 qf[KSTEPS];
  float sg = 0.f;
  {
    const bf16* qp = qkv + qrow * ld + h * HD;
    const int grow = window_row(p, t, n);
    const bf16* kgp = qkv + grow * ld + kcol;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int hd0 = 16 * s + 8 * g;
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + hd0);
      const bf16x8 kg = *reinterpret_cast<const bf16x8*>(kgp + hd0);
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const int k = hd0 / 2 + q2;
        float c = 1.f, sn = 0.f;
        if (qpos >= 0) {
          const int ps = (qpos >> (10 * pair_axis(p, k))) & 1023;
          c = rope_s[2 * (k * p.maxl + ps)];
          sn = rope_s[2 * (k * p.maxl + ps) + 1];
        }
        const float a = float(v[2 * q2]), b = float(v[2 * q2 + 1]);
        const bf16 ra = bf16(a * c - b * sn), rb = bf16(a * sn + b * c);
        qf[s][2 * q2] = ra;
        qf[s][2 * q2 + 1] = rb;
        sg += float(ra) * float(kg[2 * q2]) + float(rb) * float(kg[2 * q2 + 1]);
      }
    }
  }
  sg += __shfl_xor(sg, 32, 64);

  // ---- online softmax state, initialised with the global key ----
  const float C = p.scale_log2;
  float m_run = sg * C;
  float l_run = g == 0 ? 1.f : 0.f;
  f32x16 oacc[NHB];
  {
    const int grow = window_row(p, t, n);
    const bf16* vgp = qkv + grow * ld + vcol;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[hb][r] = float(vgp[hb * 32 + 8 * (r >> 2) + 4 * g + (r & 3)]);
  }

  const int nkb = (n + KB - 1) / KB;
  gload(0);
  lstore(0);
  __syncthreads();
  const int krow_a = swap23(l32);  // key row this lane feeds as MFMA A row
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) gload(kb + 1);
    const char* ks = Ks[cur];
    const char* vt = Vt[cur];
    // S^T for two 32-key sub-blocks
    f32x16 sacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[sb][r] = 0.f;
      const int kr = sb * 32 + krow_a;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(ks + kr * KROWB + (((2 * s + g) ^ (kr & 7)) * 16));
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[sb], 0, 0, 0);
      }
    }
    // mask keys past the window end (last block only)
    const int j0 = kb * KB;
    if (j0 + KB > n) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // accumulator row 8(r/4)+4g+(r%4) holds key swap23(that row)
          const int key = j0 + sb * 32 + swap23(8 * (r >> 2) + 4 * g + (r & 3));
          if (key >= n) sacc[sb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * C);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2f(fmaf(sacc[sb][r], C, -m_new));
        lsum += pv;
        pf[sb * 2 + (r >> 3)][r & 7] = bf16(pv);
      }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) oacc[hb] *= alpha;
    // O^T += V^T P^T over four 16-key chunks
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int hdr = hb * 32 + l32;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
            vt + hdr * (KB * 2) + (((2 * cc + g) ^ (hdr & 7)) * 16));
        oacc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[cc], oacc[hb], 0, 0, 0);
      }
    }
    if (kb + 1 < nkb) lstore(cur ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!qvalid) return;
  const float inv = 1.0f / l_tot;
  bf16* out = (bf16*)p.out + (int64_t(t) * (n + 1) + qi) * p.d + h * HD;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      bf16x4 w = {bf16(oacc[hb][4 * r4] * inv), bf16(oacc[hb][4 * r4 + 1] * inv),
                  bf16(oacc[hb][4 * r4 + 2] * inv), bf16(oacc[hb][4 * r4 + 3] * inv)};
      *reinterpret_cast<bf16x4*>(out + hb * 32 + 8 * r4 + 4 * g) = w;
    }
}

}  // namespace

namespace tsk {

hipError_t attention(hipStream_t s, int act, const AttnArgs& a) {
  AttnP p{a.qkv, a.out, a.rows, a.n_union, a.d, a.H, a.n_tiles, a.n, a.local_pos, a.rope,
          a.maxl, a.pairs_t, a.pairs_h, 1.4426950408889634f / sqrtf(float(a.hd))};
  if (act == ACT_F32) {
    const dim3 grid((a.n + 1 + 63) / 64, a.H, a.n_tiles), block(64);
    if (a.hd == 32) hipLaunchKernelGGL(k_attn_f32<32>, grid, block, 0, s, p);
    else if (a.hd == 64) hipLaunchKernelGGL(k_attn_f32<64>, grid, block, 0, s, p);
    else hipLaunchKernelGGL(k_attn_f32<128>, grid, block, 0, s, p);
    return hipGetLastError();
  }
  const dim3 grid((a.n + 1 + QB - 1) / QB, a.H, a.n_tiles), block(256);
  if (a.hd == 64) hipLaunchKernelGGL(k_attn_bf16<64>, grid, block, 0, s, p);
  else if (a.hd == 128) hipLaunchKernelGGL(k_attn_bf16<128>, grid, block, 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tsk
