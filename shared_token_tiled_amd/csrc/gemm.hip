// Projection GEMMs of the TileShare layer: QKV, out-projection, fc1, fc2
// (Table S6: "MLP GEMMs" and "QKV + out-projection GEMMs", which run once
// per token in shared layers).  C[M,N] = A[M,K] B[N,K]^T with fused epilogues
// (bias, exact GELU, fp32 residual add).
//
// bf16 / fp8: MFMA kernels for gfx950.  256x256 output tile per workgroup of
// four wavefronts (2x2, 128x128 each, 4x4 MFMA 32x32 blocks), K staged through
// LDS in two buffers with 16-byte chunks XOR-swizzled by row so that both the
// row-wise global loads and the MFMA fragment reads are conflict free.  Tile
// ids are remapped so that the workgroups each XCD receives (the hardware
// deals workgroup b to XCD b % 8) form a compact group of output tiles that
// share A and B panels in that XCD's L2.  The epilogue goes through LDS so
// every lane writes 16 contiguous output bytes.
//
// fp32: a plain LDS-tiled FMA kernel, used by the fp32 configuration.
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
};

template <int EPI>
__device__ __forceinline__ float epi_value(float acc, float alpha, float bias) {
  float v = fmaf(acc, alpha, bias);
  if (EPI == EPI_BIAS_GELU) v = gelu_erf(v);
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
      As[lk + e][lr] = (am < p.M && k < p.K) ? A[size_t(am) * p.K + k] : 0.f;
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
      if (EPI == EPI_RESID) C[size_t(m) * p.N + n] += v;
      else C[size_t(m) * p.N + n] = v;
    }
  }
}

// ------------------------------------------------------------ MFMA ------
constexpr int BM = 256, BN = 256;
constexpr int ROWB = 128;  // bytes per staged row: 64 bf16 or 128 fp8
constexpr int STAGE = (BM + BN) * ROWB;
constexpr int EPI_LD = 136;  // fp32 row stride of the epilogue staging buffer

__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nblk = tiles_m * tiles_n;
  const int xcd = bid & 7, loc = bid >> 3;
  const int q = nblk >> 3, r = nblk & 7;
  const int id = xcd < r ? xcd * (q + 1) + loc : r * (q + 1) + (xcd - r) * q + loc;
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int grp = id / per_group;
  const int first_m = grp * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int in_grp = id - grp * per_group;
  tm = first_m + in_grp % gsize;
  tn = in_grp / gsize;
}

// FP8: e4m3 operands, 32x32x64 MFMA with unit block scales (E8M0 127 = 2^0).
template <bool FP8>
__device__ __forceinline__ void mfma_step(const char* sA, const char* sB, int s, int wm, int wn,
                                          int lane, f32x16 (&acc)[4][4]) {
  const int l32 = lane & 31, g = lane >> 5;
  if (!FP8) {
    // k-step s covers bf16 columns 16s..16s+15: logical chunk 2s + g
    bf16x8 af[4], bfr[4];
    const int pc = ((2 * s + g) ^ (lane & 7)) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = *reinterpret_cast<const bf16x8*>(sA + (wm * 128 + i * 32 + l32) * ROWB + pc);
      bfr[i] = *reinterpret_cast<const bf16x8*>(sB + (wn * 128 + i * 32 + l32) * ROWB + pc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  } else {
    // k-step s covers fp8 columns 64s..64s+63: logical chunks 4s+g and 4s+2+g
    i32x8 af[4], bfr[4];
    const int pc0 = ((4 * s + g) ^ (lane & 7)) * 16;
    const int pc1 = ((4 * s + 2 + g) ^ (lane & 7)) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char* ra = sA + (wm * 128 + i * 32 + l32) * ROWB;
      const char* rb = sB + (wn * 128 + i * 32 + l32) * ROWB;
      const i32x4 a0 = *reinterpret_cast<const i32x4*>(ra + pc0);
      const i32x4 a1 = *reinterpret_cast<const i32x4*>(ra + pc1);
      const i32x4 b0 = *reinterpret_cast<const i32x4*>(rb + pc0);
      const i32x4 b1 = *reinterpret_cast<const i32x4*>(rb + pc1);
      af[i] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      bfr[i] = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], acc[i][j], 0, 0,
                                                                    0, 127, 0, 127);
  }
}

template <int EPI, bool FP8>
__global__ __launch_bounds__(256, 1) void k_gemm_mfma(GemmP p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int ESZ = FP8 ? 1 : 2;                 // element bytes
  const int64_t ldab = int64_t(p.K) * ESZ;     // row pitch of A and B in bytes
  const char* A = (const char*)p.A;
  const char* B = (const char*)p.B;

  // Global -> LDS: chunk tid + 256*i is row (tid>>3) + 32*i, 16-byte chunk tid&7.
  const int lrow = tid >> 3, lkc = tid & 7;
  const int lds_off = lrow * ROWB + ((lkc ^ (lrow & 7)) * 16);
  int64_t offA[8], offB[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    offA[i] = int64_t(min(m0 + lrow + 32 * i, p.M - 1)) * ldab + lkc * 16;
    offB[i] = int64_t(min(n0 + lrow + 32 * i, p.N - 1)) * ldab + lkc * 16;
  }
  i32x4 ra[8], rb[8];
  auto gload = [&](int kt) {
    const int64_t kb = int64_t(kt) * ROWB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ra[i] = *reinterpret_cast<const i32x4*>(A + offA[i] + kb);
      rb[i] = *reinterpret_cast<const i32x4*>(B + offB[i] + kb);
    }
  };
  auto lstore = [&](int st) {
    char* sA = smem + st * STAGE;
    char* sB = sA + BM * ROWB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<i32x4*>(sA + lds_off + i * 32 * ROWB) = ra[i];
      *reinterpret_cast<i32x4*>(sB + lds_off + i * 32 * ROWB) = rb[i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = p.K * ESZ / ROWB;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const char* sA = smem + cur * STAGE;
    const char* sB = sA + BM * ROWB;
    constexpr int STEPS = FP8 ? 2 : 4;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) mfma_step<FP8>(sA, sB, s, wm, wn, lane, acc);
    if (kt + 1 < KT) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: per 32-row block, stage 32x128 fp32 through LDS ----
  float alpha = 1.0f;
  if (FP8) alpha = (*p.sa) * (*p.sb);
  float* stg = reinterpret_cast<float*>(smem) + wave * (32 * EPI_LD);
  const int l32 = lane & 31, g = lane >> 5;
  // read-back mapping: lane covers 4 columns c4*4.. of rows rr + 2*it
  const int c4 = lane & 31, rsub = lane >> 5;
  const int colb = n0 + wn * 128 + c4 * 4;
  f32x4 bias4 = {0.f, 0.f, 0.f, 0.f};
  if (p.bias) {
#pragma unroll
    for (int e = 0; e < 4; ++e) bias4[e] = colb + e < p.N ? p.bias[colb + e] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) stg[(8 * (r >> 2) + 4 * g + (r & 3)) * EPI_LD + j * 32 + l32] = acc[i][j][r];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): LDS writes of this wave done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int rl = 2 * it + rsub;
      const int row = m0 + wm * 128 + i * 32 + rl;
      const f32x4 v = *reinterpret_cast<const f32x4*>(stg + rl * EPI_LD + c4 * 4);
      if (row < p.M && colb < p.N) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = epi_value<EPI>(v[e], alpha, bias4[e]);
        const int64_t off = int64_t(row) * p.N + colb;
        if (EPI == EPI_RESID) {
          float* C = (float*)p.C;
          const f32x4 old = load4(C + off);
          store4(C + off, old + o);
        } else if (EPI == EPI_F32) {
          store4((float*)p.C + off, o);
        } else {
          store4((bf16*)p.C + off, o);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

namespace tsk {

hipError_t gemm(hipStream_t s, int act, int epi, const void* A, const void* B, int M, int N, int K,
                const float* bias, void* C, const float* sa, const float* sb) {
  if (M <= 0 || N <= 0) return hipSuccess;
  GemmP p{A, B, C, bias, sa, sb, M, N, K};
  if (act == ACT_F32) {
    const dim3 grid((N + FT - 1) / FT, (M + FT - 1) / FT), block(256);
    switch (epi) {
      case EPI_BIAS: hipLaunchKernelGGL(k_gemm_f32<EPI_BIAS>, grid, block, 0, s, p); break;
      case EPI_BIAS_GELU: hipLaunchKernelGGL(k_gemm_f32<EPI_BIAS_GELU>, grid, block, 0, s, p); break;
      case EPI_RESID: hipLaunchKernelGGL(k_gemm_f32<EPI_RESID>, grid, block, 0, s, p); break;
      default: hipLaunchKernelGGL(k_gemm_f32<EPI_F32>, grid, block, 0, s, p); break;
    }
    return hipGetLastError();
  }
  const dim3 grid(((M + BM - 1) / BM) * ((N + BN - 1) / BN)), block(256);
#define TS_G(E, F8) hipLaunchKernelGGL((k_gemm_mfma<E, F8>), grid, block, 0, s, p)
  if (act == ACT_BF16) {
    switch (epi) {
      case EPI_BIAS: TS_G(EPI_BIAS, false); break;
      case EPI_BIAS_GELU: TS_G(EPI_BIAS_GELU, false); break;
      case EPI_RESID: TS_G(EPI_RESID, false); break;
      default: TS_G(EPI_F32, false); break;
    }
  } else {
    switch (epi) {
      case EPI_BIAS: TS_G(EPI_BIAS, true); break;
      case EPI_BIAS_GELU: TS_G(EPI_BIAS_GELU, true); break;
      case EPI_RESID: TS_G(EPI_RESID, true); break;
      default: TS_G(EPI_F32, true); break;
    }
  }
#undef TS_G
  return hipGetLastError();
}

}  // namespace tsk
