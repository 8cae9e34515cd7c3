// Projection GEMMs of the TileShare layer: QKV, out-projection, fc1, fc2
// (Table S6: "MLP GEMMs" and "QKV + out-projection GEMMs", which run once
// per token in shared layers).  C[M,N] = A[M,K] B[N,K]^T with fused epilogues
// (bias, exact GELU, fp32 residual add).
//
// bf16 / fp8: MFMA kernels for gfx950.  A workgroup computes a 256x256 output
// tile; its wavefronts form a 2 x WN grid (WN = 2: four wavefronts of 128x128,
// one per SIMD; WN = 4: eight of 128x64, two per SIMD so one can issue MFMAs
// while the other waits).  K is staged through LDS in two 64 KB buffers
// (128-byte rows: 64 bf16 or 128 fp8 per row) filled straight from global
// memory (global_load_lds, no staging registers) one K block ahead; 16-byte
// chunks are XOR-swizzled by row so both the loads and the MFMA fragment reads
// are free of bank conflicts; fragments of the next k-step are read while the
// current one's MFMAs run.  Tile ids are remapped so that the workgroups each
// XCD receives (the hardware deals workgroup b to XCD b % 8) form a compact
// group of output tiles that share A and B panels in that XCD's L2.  The
// epilogue goes through LDS so every lane writes 16 contiguous output bytes.
//
// fp32: a plain LDS-tiled FMA kernel, used by the fp32 configuration.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "ts_kernels.h"

namespace {

using tsk::EPI_BIAS;
using tsk::EPI_BIAS_GELU;
using tsk::EPI_F32;
using tsk::EPI_RESID;

struct GemmP {
  const void* A;
  const void* B;
  void* C;
  const float* bias;
  const float* sa;
  const float* sb;
  int M, N, K;
  // tile kernels: workgroups b < nlead take K-split parts: part b % ksplit
  // of tile tile0 + b / ksplit (K split ksplit ways), writing the raw
  // 256x256 fp32 partial product to part + b * 65536; workgroups b >= nlead
  // take tile b - nlead of the XCD-aware order over tile ids [0, ntiles)
  int ntiles, tile0, ksplit;
  float* part;
  // when set (bf16 output epilogues): atomic max of |output| as stored, in
  // float bits (all values are >= 0, so integer order is float order); the
  // fp8 quantisation of this output then needs no separate max pass
  unsigned* amax;
  // row pitches in elements of A (>= K) and C (>= N); B is [N, K] contiguous
  int lda, ldc;
  int nlead;
};

// Output stores of the tile epilogue, non-temporal: every output (qkv, the
// MLP hidden, the residual) is read by the next kernel from memory anyway, and
// streaming it past the L2 leaves the L2 to the A and B panels that the CUs'
// next tiles read (about -1 % per GEMM).
__device__ __forceinline__ void store4nt(float* p, f32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p)); }
__device__ __forceinline__ void store4nt(bf16* p, f32x4 v) {
  bf16x4 o = {bf16(v[0]), bf16(v[1]), bf16(v[2]), bf16(v[3])};
  __builtin_nontemporal_store(o, reinterpret_cast<bf16x4*>(p));
}

// |v| of a value as stored in bf16 (for the output max)
__device__ __forceinline__ float stored_abs(float v) { return fabsf(float(bf16(v))); }

// Maximum over a wavefront (all 64 lanes active), then one atomic max into
// one of the tsk::AMAX_SLOTS slots, chosen by workgroup and wavefront
// (atomics on one address serialise; the quantisation takes the max over the
// slots).
__device__ __forceinline__ void wave_amax(unsigned* amax, float m, int lane) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const int slot = int(blockIdx.x * 8u + (threadIdx.x >> 6)) & (tsk::AMAX_SLOTS - 1);
  if (lane == 0) atomicMax(amax + slot * tsk::AMAX_STRIDE, __float_as_uint(m));
}

// Epilogue code of a split part: the raw accumulator, no scale, no bias.
constexpr int EPI_RAW = 100;

// Store target of the epilogue lanes that fall outside a partial tile (16
// bytes per lane; the values written there are never read).
__device__ __attribute__((aligned(16))) float g_store_sink[64 * 4];

// GELU x Phi(x) = x (1 + erf(x / sqrt 2)) / 2 with erf from Abramowitz and
// Stegun, Handbook of Mathematical Functions, eq. 7.1.28: for z >= 0,
// erf(z) = 1 - (1 + a1 z + ... + a6 z^6)^-16, absolute error <= 3e-7 (about
// 2e-6 in fp32 arithmetic, i.e. <= 6e-7 on the GELU value, far below the
// bf16 rounding of the MFMA GEMMs' outputs).  One reciprocal and 11 FMA/MUL,
// no branches; large z overflows the power to +inf and gives erf = 1 exactly.
__device__ __forceinline__ float gelu_as(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  float q = fmaf(z, 0.0000430638f, 0.0002765672f);
  q = fmaf(q, z, 0.0001520143f);
  q = fmaf(q, z, 0.0092705272f);
  q = fmaf(q, z, 0.0422820123f);
  q = fmaf(q, z, 0.0705230784f);
  q = fmaf(q, z, 1.0f);
  q *= q;
  q *= q;
  q *= q;
  q *= q;
  const float e = 1.0f - __builtin_amdgcn_rcpf(q);  // erf(|x| / sqrt 2)
  const float hx = 0.5f * x;
  return fmaf(hx, copysignf(e, x), hx);
}

// FAST: GELU through gelu_as (MFMA kernels); otherwise the library erf
// (the fp32 kernel).
template <int EPI, bool FAST = false>
__device__ __forceinline__ float epi_value(float acc, float alpha, float bias) {
  if (EPI == EPI_RAW) return acc;
  float v = fmaf(acc, alpha, bias);
  if (EPI == EPI_BIAS_GELU) v = FAST ? gelu_as(v) : gelu_erf(v);
  return v;
}

// ---------------------------------------------------------------- fp32 --
constexpr int FT = 64, FK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmP p) {
  __shared__ float As[FK][FT + 4];
  __shared__ float Bs[FK][FT + 4];
  const float* A = (const float*)p.A;
  const float* B = (const float*)p.B;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * FT, n0 = blockIdx.x * FT;
  float acc[4][4] = {};
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  for (int k0 = 0; k0 < p.K; k0 += FK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = k0 + lk + e;
      const int am = m0 + lr, bn = n0 + lr;
      As[lk + e][lr] = (am < p.M && k < p.K) ? A[size_t(am) * p.lda + k] : 0.f;
      Bs[lk + e][lr] = (bn < p.N && k < p.K) ? B[size_t(bn) * p.K + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[k][ty * 4 + i];
        b[i] = Bs[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* C = (float*)p.C;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= p.N) continue;
      const float v = epi_value<EPI>(acc[i][j], 1.0f, p.bias ? p.bias[n] : 0.f);
      if (EPI == EPI_RESID) C[size_t(m) * p.ldc + n] += v;
      else C[size_t(m) * p.ldc + n] = v;
    }
  }
}

// ------------------------------------------------------------ MFMA ------
constexpr int BM = 256, BN = 256;

// s_setprio with a priority known after unrolling (the instruction takes an
// immediate)
__device__ __forceinline__ void set_prio(int v) {
  switch (v) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
}
constexpr int ROWB = 128;  // bytes per staged row: 64 bf16 or 128 fp8
constexpr int STAGE = (BM + BN) * ROWB;

// Tile id -> (tm, tn): groups of GROUP tile rows, column-major inside a group.
__device__ __forceinline__ void group_tile(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int grp = id / per_group;
  const int first_m = grp * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int in_grp = id - grp * per_group;
  tm = first_m + in_grp % gsize;
  tn = in_grp / gsize;
}

// Workgroup b of a launch of nblk tiles -> its tile: the hardware deals
// workgroup b to XCD b % 8, so each XCD gets a contiguous run of tile ids.
__device__ __forceinline__ void tile_coords(int bid, int nblk, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int xcd = bid & 7, loc = bid >> 3;
  const int q = nblk >> 3, r = nblk & 7;
  group_tile(xcd < r ? xcd * (q + 1) + loc : r * (q + 1) + (xcd - r) * q + loc, tiles_m, tiles_n, tm, tn);
}

// LDS swizzle: 16-byte chunk c of staged row r sits at chunk c ^ swz(r).  The
// LDS has 64 banks of 4 bytes and serves a 16-byte access 16 lanes at a time;
// with 128-byte rows a phase's 16 rows split by parity into the two 128-byte
// halves of the banks, and (r >> 1) & 7 gives the 8 rows of each parity 8
// different chunks (fragment reads of rows 0..15, writes of rows r, r+1).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Register fragments of one MFMA k-step for a wavefront's 128 x (32*NB)
// sub-tile: 4 A and NB B fragments (bf16: 8 values = 16 bytes; fp8: 32
// values = 32 bytes, two 16-byte chunks).  Any assignment of k to (lane
// group, element) works as long as A and B use the same one.
template <bool FP8, int NB> struct Frags;
template <int NB> struct Frags<false, NB> { bf16x8 a[4], b[NB]; };
template <int NB> struct Frags<true, NB> { i32x8 a[4], b[NB]; };

template <bool FP8, int NB>
__device__ __forceinline__ void load_frags(Frags<FP8, NB>& f, const char* sA, const char* sB, int s, int arow,
                                           int brow, int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  if constexpr (!FP8) {
    // k-step s covers bf16 columns 16s..16s+15: logical chunk 2s + g
    const int pc = ((2 * s + g) ^ swz(l32)) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.a[i] = *reinterpret_cast<const bf16x8*>(sA + (arow + i * 32 + l32) * ROWB + pc);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      f.b[j] = *reinterpret_cast<const bf16x8*>(sB + (brow + j * 32 + l32) * ROWB + pc);
  } else {
    // k-step s covers fp8 columns 64s..64s+63: logical chunks 4s+g and 4s+2+g
    const int pc0 = ((4 * s + g) ^ swz(l32)) * 16;
    const int pc1 = ((4 * s + 2 + g) ^ swz(l32)) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char* ra = sA + (arow + i * 32 + l32) * ROWB;
      const i32x4 a0 = *reinterpret_cast<const i32x4*>(ra + pc0);
      const i32x4 a1 = *reinterpret_cast<const i32x4*>(ra + pc1);
      f.a[i] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const char* rb = sB + (brow + j * 32 + l32) * ROWB;
      const i32x4 b0 = *reinterpret_cast<const i32x4*>(rb + pc0);
      const i32x4 b1 = *reinterpret_cast<const i32x4*>(rb + pc1);
      f.b[j] = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    }
  }
}

// FP8: e4m3 operands, 32x32x64 MFMA with unit block scales (E8M0 127 = 2^0).
template <bool FP8, int NB>
__device__ __forceinline__ void mfma_frags(const Frags<FP8, NB>& f, f32x16 (&acc)[4][NB]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if constexpr (!FP8)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 0, 0, 0,
                                                                    127, 0, 127);
    }
}

// Scheduling hint for one k-step: MFMAS MFMAs with READS LDS reads spread
// evenly between them (instruction groups in this order).
template <int MFMAS, int READS, int I = 0>
__device__ __forceinline__ void sched_interleave() {
  if constexpr (I < MFMAS) {
    constexpr int PER = (READS + MFMAS - 1) / MFMAS;
    constexpr int K = (I + 1) * PER <= READS ? PER : (I * PER < READS ? READS - I * PER : 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (K > 0) __builtin_amdgcn_sched_group_barrier(0x100, K, 0);
    sched_interleave<MFMAS, READS, I + 1>();
  }
}

// Epilogue of one wavefront's 128 x (32*NB) accumulator tile at (row0, col0):
// each 32-row block goes through the wavefront's own LDS staging area (32
// rows of 32*NB + 8 floats) so that every lane then writes 16 contiguous
// output bytes (4 columns) with the bias / GELU / residual applied.
// The destination is C with row pitch ldc, rows < mlim and columns < nlim
// stored (a split part: its own 256x256 block, raw sums).
template <int EPI, bool FP8, int NB>
__device__ __forceinline__ void store_tile(const GemmP& p, const f32x16 (&acc)[4][NB], float* stg, void* Cd,
                                           int64_t ldc, int mlim, int nlim, int row0, int col0, int lane) {
  constexpr int WCOLS = 32 * NB, EPI_LD = WCOLS + 8;
  float alpha = 1.0f;
  if (FP8 && EPI != EPI_RAW) alpha = (*p.sa) * (*p.sb);
  const int l32 = lane & 31, g = lane >> 5;
  // read-back mapping: LPR lanes cover one row (4 columns each), RPP rows per pass
  constexpr int LPR = WCOLS / 4, RPP = 64 / LPR;
  const int c4 = lane % LPR, rsub = lane / LPR;
  const int colb = col0 + c4 * 4;
  // No memory operation of the epilogue sits behind a branch: loads use
  // clamped indices and lanes past the tile's valid rows or columns store
  // into g_store_sink.  With branches around them the compiler loses count
  // of the outstanding loads and stores at every join and waits for all of
  // them (every earlier store included) before each store.
  const bool col_ok = colb < nlim;
  const int colc = col_ok ? colb : 0;
  f32x4 bias4 = {0.f, 0.f, 0.f, 0.f};
  if (EPI != EPI_RAW && p.bias) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float bv = p.bias[min(colb + e, nlim - 1)];
      bias4[e] = colb + e < nlim ? bv : 0.f;
    }
  }
  // residual: the old C values of 32-row block i+1 are loaded while block i
  // is written, so no pass waits on a load issued just before it
  constexpr int NP = 32 / RPP;
  f32x4 oldv[2][EPI == EPI_RESID ? NP : 1];
  auto load_old = [&](int i, f32x4 (&dst)[EPI == EPI_RESID ? NP : 1]) {
    if constexpr (EPI == EPI_RESID) {
#pragma unroll
      for (int it = 0; it < NP; ++it) {
        const int row = row0 + i * 32 + RPP * it + rsub;
        const f32x4 ov = load4((const float*)Cd + int64_t(min(row, mlim - 1)) * ldc + colc);
        dst[it] = (row < mlim && col_ok) ? ov : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  load_old(0, oldv[0]);
  float am = 0.f;  // max |output| of this lane (bf16 outputs)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i + 1 < 4) load_old(i + 1, oldv[(i + 1) & 1]);
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) stg[(8 * (r >> 2) + 4 * g + (r & 3)) * EPI_LD + j * 32 + l32] = acc[i][j][r];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < 32 / RPP; ++it) {
      const int rl = RPP * it + rsub;
      const int row = row0 + i * 32 + rl;
      const f32x4 v = *reinterpret_cast<const f32x4*>(stg + rl * EPI_LD + c4 * 4);
      const bool ok = row < mlim && col_ok;
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = epi_value<EPI, true>(v[e], alpha, bias4[e]);
      const int64_t off = int64_t(row) * ldc + colb;
      float* sink = g_store_sink + lane * 4;
      if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU) {
        if (ok)
#pragma unroll
          for (int e = 0; e < 4; ++e) am = fmaxf(am, stored_abs(o[e]));
      }
      if constexpr (EPI == EPI_RESID) {
        store4nt(ok ? (float*)Cd + off : sink, oldv[i & 1][it] + o);
      } else if (EPI == EPI_F32 || EPI == EPI_RAW) {
        store4nt(ok ? (float*)Cd + off : sink, o);
      } else {
        store4nt(ok ? (bf16*)Cd + off : reinterpret_cast<bf16*>(sink), o);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU)
    if (p.amax) wave_amax(p.amax, am, lane);
}

template <int EPI, bool FP8, int WN>
__global__ __launch_bounds__(128 * WN, 1) void k_gemm_mfma(GemmP p) {
  constexpr int NW = 2 * WN;                 // wavefronts: 2 (M) x WN (N)
  constexpr int NB = 8 / WN;                 // 32-column MFMA blocks per wavefront
  constexpr int WCOLS = 32 * NB;             // output columns per wavefront
  constexpr int LPO = 32 / NW;               // global_load_lds per operand per wavefront
  constexpr int STEPS = FP8 ? 2 : 4;         // MFMA k-steps per staged K block
  constexpr int READS = (4 + NB) * (FP8 ? 2 : 1);  // LDS reads per k-step
  constexpr int MFMAS = 4 * NB;              // MFMAs per k-step
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int arow = wm * 128, brow = wn * WCOLS;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int tm, tn;
  const int KTT = p.K * (FP8 ? 1 : 2) / ROWB;  // K blocks of the whole product
  int kb0 = 0, kb1 = KTT;                      // this workgroup's K blocks
  const bool is_part = int(blockIdx.x) < p.nlead;
  if (is_part) {
    const int part = blockIdx.x % p.ksplit;
    group_tile(p.tile0 + blockIdx.x / p.ksplit, tiles_m, tiles_n, tm, tn);
    kb0 = int(int64_t(KTT) * part / p.ksplit);
    kb1 = int(int64_t(KTT) * (part + 1) / p.ksplit);
  } else {
    tile_coords(blockIdx.x - p.nlead, p.ntiles, tiles_m, tiles_n, tm, tn);
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int ESZ = FP8 ? 1 : 2;               // element bytes
  const uint32_t lda8 = uint32_t(p.lda) * ESZ; // row pitches of A and B in bytes
  const uint32_t ldb8 = uint32_t(p.K) * ESZ;
  const char* A = (const char*)p.A;
  const char* B = (const char*)p.B;

  // Global -> LDS without registers (global_load_lds_dwordx4: lane l of a
  // wavefront instruction writes 16 bytes at LDS base + 16*l).  Instruction i
  // of wavefront w fills staged rows 8*(NW*i+w) .. +7 (1 KB); lane l covers row
  // 8*(NW*i+w) + (l>>3), LDS slot l&7, and so loads the logical chunk that the
  // swizzle puts in that slot, (l&7) ^ swz(row) (the same for every i).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lrow = 8 * wv + (lane >> 3);
  const int lchunk = (lane & 7) ^ swz(lrow);
  uint32_t offA[LPO], offB[LPO];  // byte offsets (the host checks they fit)
#pragma unroll
  for (int i = 0; i < LPO; ++i) {
    offA[i] = uint32_t(min(m0 + lrow + 8 * NW * i, p.M - 1)) * lda8 + lchunk * 16;
    offB[i] = uint32_t(min(n0 + lrow + 8 * NW * i, p.N - 1)) * ldb8 + lchunk * 16;
  }
  auto gload = [&](int kt, int st) {   // K block kb0 + kt into stage st
    const uint32_t kb = uint32_t(kb0 + kt) * ROWB;
    char* sA = smem + st * STAGE;
    char* sB = sA + BM * ROWB;
#pragma unroll
    for (int i = 0; i < LPO; ++i) {
      __builtin_amdgcn_global_load_lds((const void*)(A + offA[i] + kb),
                                       (TS_LDS void*)(sA + (NW * i + wv) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(B + offB[i] + kb),
                                       (TS_LDS void*)(sB + (NW * i + wv) * 1024), 16, 0, 0);
    }
  };

  // epilogue: the C tile, or this part's raw sums for a split launch
  auto store = [&](const f32x16 (&ac)[4][NB]) {
    float* stg = reinterpret_cast<float*>(smem) + wave * (32 * (WCOLS + 8));
    if (EPI == EPI_RAW || is_part)
      store_tile<EPI_RAW, FP8, NB>(p, ac, stg, p.part + int64_t(blockIdx.x) * (BM * BN), BN, BM, BN, arow, brow, lane);
    else
      store_tile<EPI, FP8, NB>(p, ac, stg, p.C, p.ldc, p.M, p.N, m0 + arow, n0 + brow, lane);
  };
  f32x16 acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Main loop, rotated so that no wavefront idles on LDS latency after the
  // per-block barrier: fragments are double buffered in registers (step s+1
  // is read while step s computes), and the last k-step of stage kt computes
  // after the barrier, from registers, while the first fragments of stage
  // kt+1 are read.  The barrier therefore only has to follow this wavefront's
  // reads of stage kt and its loads into stage kt+1; right after it, stage kt
  // is free for the loads of block kt+2.
  //
  // fp8 keeps the plain loop (next block's loads at the top, one barrier at
  // the end): its 32-byte fragments, double buffered across the barrier,
  // would not fit the register budget next to the accumulators.
  const int KT = kb1 - kb0;
  gload(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if constexpr (FP8) {
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      // the other stage was last read in the previous iteration, before its barrier
      if (kt + 1 < KT) gload(kt + 1, cur ^ 1);
      const char* sA = smem + cur * STAGE;
      const char* sB = sA + BM * ROWB;
      Frags<FP8, NB> fr[2];
      load_frags<FP8, NB>(fr[0], sA, sB, 0, arow, brow, lane);
      // k-step s at issue priority STEPS-s (the lagging wavefront of a SIMD
      // is preferred, as in the bf16 loop; fc2 -9.5 %, out -4 %)
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        set_prio(STEPS - s);
        if (s + 1 < STEPS) load_frags<FP8, NB>(fr[(s + 1) & 1], sA, sB, s + 1, arow, brow, lane);
        mfma_frags<FP8, NB>(fr[s & 1], acc);
        if (s == 0) __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
        if (s + 1 < STEPS) sched_interleave<MFMAS, READS>();
        else __builtin_amdgcn_sched_group_barrier(0x008, MFMAS, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      // this iteration's loads of the next stage must have landed before anyone reads it
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    store(acc);
    return;
  }
  if (KT > 1) gload(1, 1);
  Frags<FP8, NB> fr[2];
  load_frags<FP8, NB>(fr[0], smem, smem + BM * ROWB, 0, arow, brow, lane);
  static_assert(STEPS % 2 == 0, "the last step's fragments sit in fr[1]");
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const char* sA = smem + cur * STAGE;
    const char* sB = sA + BM * ROWB;
    // k-step s runs at issue priority STEPS-1-s, so that of the two
    // wavefronts of a SIMD the one that is behind is preferred (with equal
    // priorities the older one takes the MFMA slots first, reaches the
    // barrier early and the other finishes alone)
#pragma unroll
    for (int s = 0; s + 1 < STEPS; ++s) {
      set_prio(STEPS - 1 - s);
      load_frags<FP8, NB>(fr[(s + 1) & 1], sA, sB, s + 1, arow, brow, lane);
      mfma_frags<FP8, NB>(fr[s & 1], acc);
      sched_interleave<MFMAS, READS>();
    }
    __builtin_amdgcn_s_setprio(0);
    // this wavefront's loads of stage kt+1 have landed and its reads of stage
    // kt are done; after the barrier the same holds for every wavefront
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 2 < KT) gload(kt + 2, cur);
    if (kt + 1 < KT) {
      const char* nA = smem + (cur ^ 1) * STAGE;
      load_frags<FP8, NB>(fr[0], nA, nA + BM * ROWB, 0, arow, brow, lane);
    }
    mfma_frags<FP8, NB>(fr[1], acc);
    __builtin_amdgcn_sched_group_barrier(0x020, 2 * LPO, 0);  // global -> LDS loads
    __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);    // next stage's first fragments
    __builtin_amdgcn_sched_group_barrier(0x008, MFMAS, 0);    // this stage's last k-step
  }

  // ---- epilogue: per 32-row block, stage 32 x WCOLS fp32 through LDS ----
  store(acc);
}

// Rows of C past the last full 256-row tile when there are at most 32 of
// them (the TileShare row counts are multiples of 256 plus one global-token
// row per tile window): one 32 x 32 output block per workgroup, K split over
// its 8 wavefronts (128-byte k-groups dealt round robin, four in flight per
// wavefront), operands read straight from global memory (each row's 128 bytes
// of a k-group by the two lanes that own it), partial sums reduced through
// LDS, then the same epilogue as the tile kernels.
template <int EPI, bool FP8>
__global__ __launch_bounds__(512) void k_gemm_rows(GemmP p) {
  constexpr int NWR = 8, UNR = 4;
  __shared__ float red[NWR][32][33];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int n0 = blockIdx.x * 32;
  const int ESZ = FP8 ? 1 : 2;
  const char* ar = (const char*)p.A + int64_t(min(l32, p.M - 1)) * p.lda * ESZ;
  const char* br = (const char*)p.B + int64_t(min(n0 + l32, p.N - 1)) * p.K * ESZ;
  // byte offsets of this lane's four 16-byte chunks in a k-group: bf16 k-step
  // j takes chunk j (k 16j + 8g ..); fp8 k-step j2 takes chunks 2j2, 2j2+1
  // (k 64 j2 + 32 g ..); A and B use the same assignment
  int co[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) co[j] = FP8 ? 64 * (j >> 1) + 32 * g + 16 * (j & 1) : 32 * j + 16 * g;
  const int KT = p.K * ESZ / ROWB;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int kg0 = wave; kg0 < KT; kg0 += NWR * UNR) {
    i32x4 a[UNR][4], b[UNR][4];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int kg = kg0 + u * NWR;
      if (kg < KT) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a[u][j] = *reinterpret_cast<const i32x4*>(ar + int64_t(kg) * ROWB + co[j]);
          b[u][j] = *reinterpret_cast<const i32x4*>(br + int64_t(kg) * ROWB + co[j]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (kg0 + u * NWR >= KT) break;
      if constexpr (!FP8) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[u][j]),
                                                        __builtin_bit_cast(bf16x8, b[u][j]), acc, 0, 0, 0);
      } else {
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
          const i32x4 a0 = a[u][2 * j2], a1 = a[u][2 * j2 + 1], b0 = b[u][2 * j2], b1 = b[u][2 * j2 + 1];
          acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]},
              i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]}, acc, 0, 0, 0, 127, 0, 127);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][8 * (r >> 2) + 4 * g + (r & 3)][l32] = acc[r];
  __syncthreads();
  if (tid < 256) {
    const int row = tid >> 3, c = (tid & 7) * 4, col = n0 + c;
    float am = 0.f;
    if (row < p.M && col < p.N) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NWR; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += red[w][row][c + e];
      const float alpha = FP8 ? (*p.sa) * (*p.sb) : 1.0f;
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = epi_value<EPI, true>(v[e], alpha, p.bias ? p.bias[col + e] : 0.f);
      const int64_t off = int64_t(row) * p.ldc + col;
      if (EPI == EPI_RESID) {
        float* C = (float*)p.C;
        store4(C + off, load4(C + off) + o);
      } else if (EPI == EPI_F32) {
        store4((float*)p.C + off, o);
      } else {
        store4((bf16*)p.C + off, o);
#pragma unroll
        for (int e = 0; e < 4; ++e) am = fmaxf(am, stored_abs(o[e]));
      }
    }
    if (EPI != EPI_RESID && EPI != EPI_F32 && p.amax) wave_amax(p.amax, am, lane);  // waves 0-3, all lanes
  }
}

// Sum of the ksplit parts of each tile of a K-split launch, in part order
// (the same result on every run), then the epilogue.  One workgroup per 4 rows
// of a tile, 4 columns per thread.
template <int EPI, bool FP8>
__global__ __launch_bounds__(256) void k_gemm_reduce(GemmP p) {
  const int tl = blockIdx.x / (BM / 4), rb = blockIdx.x % (BM / 4);
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int tm, tn;
  group_tile(p.tile0 + tl, tiles_m, tiles_n, tm, tn);
  const int r = rb * 4 + int(threadIdx.x) / 64, c = (int(threadIdx.x) % 64) * 4;
  const int row = tm * BM + r, col = tn * BN + c;
  float am = 0.f;
  if (row < p.M && col < p.N) {
    const float* src = p.part + int64_t(tl) * p.ksplit * (BM * BN) + r * BN + c;
    f32x4 v = load4(src);
    for (int k = 1; k < p.ksplit; ++k) v += load4(src + int64_t(k) * (BM * BN));
    const float alpha = FP8 ? (*p.sa) * (*p.sb) : 1.0f;
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = epi_value<EPI, true>(v[e], alpha, p.bias ? p.bias[col + e] : 0.f);
    const int64_t off = int64_t(row) * p.ldc + col;
    if (EPI == EPI_RESID) {
      store4((float*)p.C + off, load4((const float*)p.C + off) + o);
    } else if (EPI == EPI_F32) {
      store4((float*)p.C + off, o);
    } else {
      store4((bf16*)p.C + off, o);
#pragma unroll
      for (int e = 0; e < 4; ++e) am = fmaxf(am, stored_abs(o[e]));
    }
  }
  if (EPI != EPI_RESID && EPI != EPI_F32 && p.amax) wave_amax(p.amax, am, int(threadIdx.x) & 63);
}

// Compute units of the current device (for the tile-round count).
int device_cus() {
  static int v = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
  }();
  return v;
}

// Wavefronts along N of the MFMA kernel: 2 (four wavefronts, 128x128 each) or
// 4 (eight wavefronts, 128x64 each, two per SIMD; the default).
// TS_GEMM_WAVES_N overrides it for measurements.
int gemm_waves_n() {
  static int v = [] {
    const char* e = getenv("TS_GEMM_WAVES_N");
    return (e && atoi(e) == 2) ? 2 : 4;
  }();
  return v;
}

// K-split lead parts for short-K residual GEMMs (the out-projection);
// TS_GEMM_LEAD_SPLIT=0 turns them off, for measurements.
bool lead_split() {
  static const bool v = [] {
    const char* e = getenv("TS_GEMM_LEAD_SPLIT");
    return !(e && atoi(e) == 0);
  }();
  return v;
}

}  // namespace

namespace tsk {

hipError_t gemm(hipStream_t s, int act, int epi, const void* A, const void* B, int M, int N, int K,
                const float* bias, void* C, const float* sa, const float* sb, float* ws, size_t ws_bytes,
                unsigned* amax, int lda, int ldc) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (lda == 0) lda = K;
  if (ldc == 0) ldc = N;
  if (lda < K || ldc < N) return hipErrorInvalidValue;
  // MFMA kernels: rows of A start on 16 bytes (staged and read in 16-byte
  // chunks), and the epilogue writes 4 elements per lane
  if (act != ACT_F32 && ((int64_t(lda) * (act == ACT_FP8 ? 1 : 2)) % 16 != 0 || ldc % 4 != 0))
    return hipErrorInvalidValue;
  if (act == ACT_F32) {
    GemmP p{A, B, C, bias, sa, sb, M, N, K, 0, 0, 1, nullptr, nullptr, lda, ldc, 0};
    const dim3 grid((N + FT - 1) / FT, (M + FT - 1) / FT), block(256);
    switch (epi) {
      case EPI_BIAS: hipLaunchKernelGGL(k_gemm_f32<EPI_BIAS>, grid, block, 0, s, p); break;
      case EPI_BIAS_GELU: hipLaunchKernelGGL(k_gemm_f32<EPI_BIAS_GELU>, grid, block, 0, s, p); break;
      case EPI_RESID: hipLaunchKernelGGL(k_gemm_f32<EPI_RESID>, grid, block, 0, s, p); break;
      default: hipLaunchKernelGGL(k_gemm_f32<EPI_F32>, grid, block, 0, s, p); break;
    }
    return hipGetLastError();
  }
  const bool f8 = act == ACT_FP8;
  const int esz = f8 ? 1 : 2, osz = (epi == EPI_RESID || epi == EPI_F32) ? 4 : 2;
  // Ragged rows (M % 256 <= 32) go to k_gemm_rows when that saves a round of
  // 256x256 tiles over the device's compute units (for tests, TS_GEMM_ROWS=
  // always: in every such case; never: not at all).
  const int tiles_n = (N + BN - 1) / BN, R = M % BM;
  int Mm = M;
  const char* rows_env = getenv("TS_GEMM_ROWS");
  if (R != 0 && R <= 32 && !(rows_env && strcmp(rows_env, "never") == 0)) {
    const int64_t ncu = device_cus();
    const int64_t all = int64_t((M + BM - 1) / BM) * tiles_n, full = int64_t(M / BM) * tiles_n;
    if ((rows_env && strcmp(rows_env, "always") == 0) || (full > 0 && (full + ncu - 1) / ncu < (all + ncu - 1) / ncu))
      Mm = M - R;
  }
  // The tiles of a partial last round over the CUs (when a workspace is
  // given) run K-split: ks parts per tile, as many workgroups as fit one
  // round, their raw sums reduced in part order by k_gemm_reduce.  At least 4
  // K blocks per part, at most 8 parts, and what the workspace holds.  Only
  // for long K (>= 64 K blocks, e.g. fc2): a short tile's last round runs at
  // a raised clock and gains less than the reduction costs (measured).
  const int64_t T = int64_t((Mm + BM - 1) / BM) * tiles_n;
  const int KTT = K * esz / ROWB;
  int64_t Tm = T;
  int ks = 1;
  bool lead = false;
  if (ws && T > 0 && KTT >= 64) {
    const int64_t ncu = device_cus(), rem = T % ncu;
    if (rem > 0) {
      int64_t k = std::min<int64_t>({ncu / rem, KTT / 4, 8, int64_t(ws_bytes / (size_t(rem) * BM * BN * 4))});
      if (k >= 2) {
        ks = int(k);
        Tm = T - rem;
      }
    }
  } else if (ws && T > 0 && epi == EPI_RESID && lead_split()) {
    // Short K, residual epilogue: the tiles of the partial last round run
    // first, as two K halves each, in the same launch as the full tiles.
    // The CUs that start with a half tile reach every later epilogue half a
    // tile after the others, so the HBM-bound fp32 residual epilogues of a
    // round no longer all run at once, and the rounds end together.
    const int64_t ncu = device_cus(), rem = T % ncu;
    if (rem > 0 && 2 * rem <= ncu && size_t(rem) * 2 * BM * BN * 4 <= ws_bytes && KTT >= 8) {
      ks = 2;
      Tm = T - rem;
      lead = true;
    }
  }
  const int nlead = lead ? int((T - Tm) * ks) : 0;
  GemmP pm{A, B, C, bias, sa, sb, Mm, N, K, int(Tm), int(Tm), ks, ws, amax, lda, ldc, nlead};
  GemmP ps{A, B, C, bias, sa, sb, Mm, N, K, 0, int(Tm), ks, ws, amax, lda, ldc, int((T - Tm) * ks)};
  GemmP pt{(const char*)A + int64_t(Mm) * lda * esz, B, (char*)C + int64_t(Mm) * ldc * osz, bias, sa, sb, M - Mm, N, K,
           0, 0, 1, nullptr, amax, lda, ldc, 0};
  const int wn = lead ? 4 : gemm_waves_n();
  const dim3 grid(static_cast<unsigned>(Tm + nlead)), block(128 * wn), tgrid((N + 31) / 32);
  const dim3 sgrid(static_cast<unsigned>((T - Tm) * ks)), rgrid(static_cast<unsigned>((T - Tm) * (BM / 4)));
#define TS_G(E, F8)                                                                          \
  do {                                                                                       \
    if (Tm + nlead == 0) {                                                                   \
    } else if (wn == 2) hipLaunchKernelGGL((k_gemm_mfma<E, F8, 2>), grid, block, 0, s, pm);   \
    else hipLaunchKernelGGL((k_gemm_mfma<E, F8, 4>), grid, block, 0, s, pm);                  \
    if (Tm < T) {                                                                            \
      if (!lead) hipLaunchKernelGGL((k_gemm_mfma<EPI_RAW, F8, 4>), sgrid, dim3(512), 0, s, ps); \
      hipLaunchKernelGGL((k_gemm_reduce<E, F8>), rgrid, dim3(256), 0, s, ps);                 \
    }                                                                                        \
    if (Mm < M) hipLaunchKernelGGL((k_gemm_rows<E, F8>), tgrid, dim3(512), 0, s, pt);         \
  } while (0)
  switch (epi) {
    case EPI_BIAS: if (f8) TS_G(EPI_BIAS, true); else TS_G(EPI_BIAS, false); break;
    case EPI_BIAS_GELU: if (f8) TS_G(EPI_BIAS_GELU, true); else TS_G(EPI_BIAS_GELU, false); break;
    case EPI_RESID: if (f8) TS_G(EPI_RESID, true); else TS_G(EPI_RESID, false); break;
    default: if (f8) TS_G(EPI_F32, true); else TS_G(EPI_F32, false); break;
  }
#undef TS_G
  return hipGetLastError();
}

}  // namespace tsk
