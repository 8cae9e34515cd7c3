// Memory-bound kernels of the TileShare layer: norms, QK-norm, the w-bar
// blend (shared layers) and state merge (layer k), the per-tile gather, and
// e4m3 quantisation.  All are one pass over HBM; rows are handled by whole
// wavefronts with 16-byte (fp32) or 8-byte (bf16) vector accesses.
#include "device_common.h"
#include "ts_kernels.h"

namespace {

constexpr int kMaxChunks = 16;  // d <= 64 lanes * 4 elements * 16 = 4096

// ---- Norm1 / Norm2 (Table S1: once per token in shared layers) ---------
// One wavefront per row; the row stays in registers between the passes.
template <typename TOUT, bool RMS>
__global__ __launch_bounds__(256) void k_norm(const float* __restrict__ x, int M, int d,
                                              const float* __restrict__ g,
                                              const float* __restrict__ b, float eps,
                                              TOUT* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* xr = x + size_t(row) * d;
  const int nc = d >> 2;
  f32x4 v[kMaxChunks];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nc) {
      v[i] = load4(xr + 4 * c);
      s += RMS ? (v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3])
               : (v[i][0] + v[i][1] + v[i][2] + v[i][3]);
    }
  }
  s = wave_sum(s);
  const float inv_d = 1.0f / float(d);
  float mean = 0.f, inv;
  if (RMS) {
    inv = 1.0f / sqrtf(s * inv_d + eps);
  } else {
    mean = s * inv_d;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int c = lane + 64 * i;
      if (c < nc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float t = v[i][e] - mean;
          q += t * t;
        }
      }
    }
    q = wave_sum(q);
    inv = 1.0f / sqrtf(q * inv_d + eps);
  }
  TOUT* yr = y + size_t(row) * d;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nc) {
      const f32x4 gg = load4(g + 4 * c);
      f32x4 o;
      if (RMS) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = v[i][e] * inv * gg[e];
      } else {
        const f32x4 bb = load4(b + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (v[i][e] - mean) * inv * gg[e] + bb[e];
      }
      store4(yr + 4 * c, o);
    }
  }
}

// ---- per-head QK-RMSNorm (Table S1: once per token) and RoPE --------------
// HD/8 lanes per (row, head slice); slices 0..H-1 are q heads, H..2H-1 k heads,
// and slice s starts at column s*HD of the [q | k | v] row in both cases.
// NORM: RMS-normalise each head and scale by its gain first.  Then every q
// and k head is rotated by the row's grid coordinates (RopeRows): the angle
// of pair i of axis a is coord_a * base^(-i / pairs_a), so the score of two
// window tokens depends only on their coordinate difference, as with
// tile-local positions, and the attention kernels stage keys unchanged.
template <typename T, int HD, bool NORM>
__global__ __launch_bounds__(256) void k_qkprep(T* __restrict__ qkv, int M, int d, int H,
                                                const float* __restrict__ qg,
                                                const float* __restrict__ kg, float eps, tsk::RopeRows rr) {
  constexpr int LPS = HD / 8;
  // 32-bit index arithmetic (the host checks M * 2H * HD/8 < 2^31)
  const uint32_t gid = (blockIdx.x * 256u + threadIdx.x) / LPS;
  const int sub = threadIdx.x % LPS;
  const uint32_t total = uint32_t(M) * 2u * uint32_t(H);
  const bool ok = gid < total;
  const uint32_t row = ok ? gid / (2u * H) : 0u;
  const int sl = ok ? int(gid - row * (2u * H)) : 0;
  T* p = qkv + int64_t(row) * 3 * d + sl * HD + sub * 8;
  f32x4 a = {0, 0, 0, 0}, c = {0, 0, 0, 0};
  if (ok) load8(p, a, c);
  if constexpr (NORM) {
    float ss = a[0] * a[0] + a[1] * a[1] + a[2] * a[2] + a[3] * a[3] + c[0] * c[0] + c[1] * c[1] +
               c[2] * c[2] + c[3] * c[3];
    ss = group_sum(ss, LPS);
    const float inv = 1.0f / sqrtf(ss * (1.0f / HD) + eps);
    const float* gg = (sl < H ? qg : kg) + sub * 8;
    const f32x4 g0 = ok ? load4(gg) : f32x4{0, 0, 0, 0}, g1 = ok ? load4(gg + 4) : f32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = a[e] * inv * g0[e];
      c[e] = c[e] * inv * g1[e];
    }
  }
  if (!ok) return;
  // grid coordinates of the row
  int co[3];
  const int r = int(row);
  if (rr.shared && r < rr.n_union) {
    co[2] = r % rr.grid[2];
    co[1] = (r / rr.grid[2]) % rr.grid[1];
    co[0] = r / (rr.grid[2] * rr.grid[1]);
  } else {
    const int t = rr.shared ? r - rr.n_union : r / (rr.n + 1), i = rr.shared ? rr.n : r % (rr.n + 1);
    const int lp = i < rr.n ? rr.local_pos[i] : 0;
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) co[ax] = rr.tile_start[3 * t + ax] + ((lp >> (10 * ax)) & 1023);
  }
  float v[8] = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int k = 4 * sub + e;
    const int ax = k < rr.pairs[0] ? 0 : (k < rr.pairs[0] + rr.pairs[1] ? 1 : 2);
    const int i = ax == 0 ? k : (ax == 1 ? k - rr.pairs[0] : k - rr.pairs[0] - rr.pairs[1]);
    const int np = ax == 0 ? rr.pairs[0] : (ax == 1 ? rr.pairs[1] : rr.pairs[2]);
    const int off = ax == 0 ? rr.off[0] : (ax == 1 ? rr.off[1] : rr.off[2]);
    const int cc = ax == 0 ? co[0] : (ax == 1 ? co[1] : co[2]);
    const float2 cs = *reinterpret_cast<const float2*>(rr.tab + off + 2 * (cc * np + i));
    const float x = v[2 * e], y = v[2 * e + 1];
    v[2 * e] = x * cs.x - y * cs.y;
    v[2 * e + 1] = x * cs.y + y * cs.x;
  }
  store8(p, f32x4{v[0], v[1], v[2], v[3]}, f32x4{v[4], v[5], v[6], v[7]});
}

// ---- w-bar blend / state merge (Figure 2 caption: the only approximate step)
// One wavefront per output row; entries summed in ascending tile order.
template <typename TIN, typename TOUT>
__global__ __launch_bounds__(256) void k_blend(const TIN* __restrict__ in, int d, int n_union,
                                               int n_tiles, int n, const int* __restrict__ cover_ptr,
                                               const int* __restrict__ entry_row,
                                               const float* __restrict__ w,
                                               TOUT* __restrict__ out_union,
                                               TOUT* __restrict__ out_global) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nc = d >> 2;
  if (r < n_union) {
    const int e0 = cover_ptr[r], e1 = cover_ptr[r + 1];
    f32x4 acc[kMaxChunks];
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) acc[i] = f32x4{0, 0, 0, 0};
    for (int e = e0; e < e1; ++e) {
      const TIN* src = in + size_t(entry_row[e]) * d;
      const float we = w[e];
#pragma unroll
      for (int i = 0; i < kMaxChunks; ++i) {
        const int c = lane + 64 * i;
        if (c < nc) {
          const f32x4 v = load4(src + 4 * c);
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[i][k] = fmaf(we, v[k], acc[i][k]);
        }
      }
    }
    TOUT* dst = out_union + size_t(r) * d;
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int c = lane + 64 * i;
      if (c < nc) store4(dst + 4 * c, acc[i]);
    }
  } else if (r < n_union + n_tiles && out_global != nullptr) {
    const int t = r - n_union;
    const TIN* src = in + (size_t(t) * (n + 1) + n) * d;
    TOUT* dst = out_global + size_t(t) * d;
    for (int c = lane; c < nc; c += 64) store4(dst + 4 * c, load4(src + 4 * c));
  }
}

// ---- per-tile gather at stack entry (tile states = tile rows + global token)
__global__ __launch_bounds__(256) void k_gather(const float* __restrict__ x_in,
                                                const float* __restrict__ g, int64_t g_stride,
                                                const int* __restrict__ tile_rows, int n_tiles,
                                                int n, int d, float* __restrict__ X) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_tiles * (n + 1)) return;
  const int t = r / (n + 1), j = r % (n + 1);
  const float* src = j < n ? x_in + size_t(tile_rows[size_t(t) * n + j]) * d : g + t * g_stride;
  float* dst = X + size_t(r) * d;
  for (int c = lane; c < (d >> 2); c += 64) store4(dst + 4 * c, load4(src + 4 * c));
}

// X[t*(n+1)+j] += delta[tile_rows[t*n+j]], X[t*(n+1)+n] += delta[n_union+t]:
// one per-token result added to every tile's copy of the token.
__global__ __launch_bounds__(256) void k_add_to_tiles(float* __restrict__ X, const float* __restrict__ delta,
                                                      const int* __restrict__ tile_rows, int n_union,
                                                      int n_tiles, int n, int d) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_tiles * (n + 1)) return;
  const int t = r / (n + 1), j = r % (n + 1);
  const float* src = delta + size_t(j < n ? tile_rows[size_t(t) * n + j] : n_union + t) * d;
  float* dst = X + size_t(r) * d;
  for (int c = lane; c < (d >> 2); c += 64) store4(dst + 4 * c, load4(dst + 4 * c) + load4(src + 4 * c));
}

__global__ __launch_bounds__(256) void k_init_shared(const float* __restrict__ x_in,
                                                     const float* __restrict__ g, int n_union,
                                                     int n_tiles, int d, float* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_union + n_tiles) return;
  const float* src = r < n_union ? x_in + size_t(r) * d : g;
  float* dst = xs + size_t(r) * d;
  for (int c = lane; c < (d >> 2); c += 64) store4(dst + 4 * c, load4(src + 4 * c));
}

__global__ __launch_bounds__(256) void k_copy4(const float* __restrict__ src, float* __restrict__ dst,
                                               int64_t n4) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += int64_t(gridDim.x) * 256)
    store4(dst + 4 * i, load4(src + 4 * i));
}

// ---- e4m3 quantisation (Table S5 "V0 + FP8"; OCP e4m3, RNE, +-448) ------
__global__ void k_zero_u32(unsigned* p) { *p = 0u; }

template <typename T>
__global__ __launch_bounds__(256) void k_amax(const T* __restrict__ x, int64_t n,
                                              unsigned* __restrict__ amax_bits) {
  float m = 0.f;
  const int64_t n4 = n >> 2;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += int64_t(gridDim.x) * 256) {
    const f32x4 v = load4(x + 4 * i);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  }
  for (int64_t i = 4 * n4 + int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    m = fmaxf(m, fabsf(to_f32(x[i])));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(amax_bits, __float_as_uint(m));  // m >= 0: integer order = float order
  }
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

template <typename T>
__global__ __launch_bounds__(256) void k_quant(const T* __restrict__ x, int64_t n,
                                               const unsigned* __restrict__ amax_bits,
                                               uint8_t* __restrict__ q, float* __restrict__ scale_out) {
  const float amax = __uint_as_float(*amax_bits);
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0 && scale_out) *scale_out = s;
  const int64_t n4 = n >> 2;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += int64_t(gridDim.x) * 256) {
    const f32x4 v = load4(x + 4 * i);
    int pk = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(v[0] / s), clamp448(v[1] / s), 0, false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(v[2] / s), clamp448(v[3] / s), pk, true);
    reinterpret_cast<int*>(q)[i] = pk;
  }
  for (int64_t i = 4 * n4 + int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(to_f32(x[i]) / s), 0.f, 0, false);
    q[i] = uint8_t(pk & 0xff);
  }
}

inline int blocks_for_rows(int rows) { return (rows + 3) / 4; }
inline int grid_stride_blocks(int64_t items) {
  int64_t b = (items + 255) / 256;
  if (b > 4096) b = 4096;
  return int(b < 1 ? 1 : b);
}

}  // namespace

namespace tsk {

hipError_t norm(hipStream_t s, int act, bool rms, const float* x, int M, int d, const float* g,
                const float* b, float eps, void* y) {
  if (M <= 0) return hipSuccess;
  const dim3 grid(blocks_for_rows(M)), block(256);
  if (act == ACT_F32) {
    if (rms) hipLaunchKernelGGL((k_norm<float, true>), grid, block, 0, s, x, M, d, g, b, eps, (float*)y);
    else hipLaunchKernelGGL((k_norm<float, false>), grid, block, 0, s, x, M, d, g, b, eps, (float*)y);
  } else {
    if (rms) hipLaunchKernelGGL((k_norm<bf16, true>), grid, block, 0, s, x, M, d, g, b, eps, (bf16*)y);
    else hipLaunchKernelGGL((k_norm<bf16, false>), grid, block, 0, s, x, M, d, g, b, eps, (bf16*)y);
  }
  return hipGetLastError();
}

hipError_t qk_prep(hipStream_t s, int act, void* qkv, int M, int d, int H, int hd, const float* qg,
                   const float* kg, float eps, const RopeRows& rr) {
  if (M <= 0) return hipSuccess;
  const int64_t threads = int64_t(M) * 2 * H * (hd / 8);
  if (threads >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const dim3 grid(unsigned((threads + 255) / 256)), block(256);
  const bool norm = qg != nullptr;
#define TS_QK(T, HD)                                                                                         \
  do {                                                                                                       \
    if (norm) hipLaunchKernelGGL((k_qkprep<T, HD, true>), grid, block, 0, s, (T*)qkv, M, d, H, qg, kg, eps, rr); \
    else hipLaunchKernelGGL((k_qkprep<T, HD, false>), grid, block, 0, s, (T*)qkv, M, d, H, qg, kg, eps, rr);    \
  } while (0)
  if (act == ACT_F32) {
    if (hd == 32) TS_QK(float, 32); else if (hd == 64) TS_QK(float, 64); else TS_QK(float, 128);
  } else {
    if (hd == 32) TS_QK(bf16, 32); else if (hd == 64) TS_QK(bf16, 64); else TS_QK(bf16, 128);
  }
#undef TS_QK
  return hipGetLastError();
}

hipError_t blend(hipStream_t s, int tin, int tout, const void* in, int d, int n_union, int n_tiles,
                 int n, const int* cover_ptr, const int* entry_row, const float* w, void* out_union,
                 void* out_global) {
  const dim3 grid(blocks_for_rows(n_union + n_tiles)), block(256);
#define TS_BL(TI, TO)                                                                             \
  hipLaunchKernelGGL((k_blend<TI, TO>), grid, block, 0, s, (const TI*)in, d, n_union, n_tiles, n, \
                     cover_ptr, entry_row, w, (TO*)out_union, (TO*)out_global)
  if (tin == ACT_F32 && tout == ACT_F32) TS_BL(float, float);
  else if (tin == ACT_BF16 && tout == ACT_BF16) TS_BL(bf16, bf16);
  else if (tin == ACT_F32 && tout == ACT_BF16) TS_BL(float, bf16);
  else TS_BL(bf16, float);
#undef TS_BL
  return hipGetLastError();
}

hipError_t gather(hipStream_t s, const float* x_in, const float* g, int64_t g_stride, const int* tile_rows, int n_tiles,
                  int n, int d, float* X) {
  hipLaunchKernelGGL(k_gather, dim3(blocks_for_rows(n_tiles * (n + 1))), dim3(256), 0, s, x_in, g, g_stride,
                     tile_rows, n_tiles, n, d, X);
  return hipGetLastError();
}

hipError_t add_to_tiles(hipStream_t s, float* X, const float* delta, const int* tile_rows, int n_union,
                        int n_tiles, int n, int d) {
  hipLaunchKernelGGL(k_add_to_tiles, dim3(blocks_for_rows(n_tiles * (n + 1))), dim3(256), 0, s, X, delta,
                     tile_rows, n_union, n_tiles, n, d);
  return hipGetLastError();
}

hipError_t init_shared(hipStream_t s, const float* x_in, const float* g, int n_union, int n_tiles,
                       int d, float* xs) {
  hipLaunchKernelGGL(k_init_shared, dim3(blocks_for_rows(n_union + n_tiles)), dim3(256), 0, s, x_in,
                     g, n_union, n_tiles, d, xs);
  return hipGetLastError();
}

hipError_t copy_f32(hipStream_t s, const float* src, float* dst, int64_t n) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy4, dim3(grid_stride_blocks(n / 4)), dim3(256), 0, s, src, dst, n / 4);
  return hipGetLastError();
}

hipError_t fp8_quantize(hipStream_t s, int tin, const void* src, int64_t n, uint8_t* dst,
                        float* scale_out, unsigned* amax_slot) {
  hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, s, amax_slot);
  const int nb = grid_stride_blocks((n + 3) / 4);
  if (tin == ACT_F32) {
    hipLaunchKernelGGL(k_amax<float>, dim3(nb), dim3(256), 0, s, (const float*)src, n, amax_slot);
    hipLaunchKernelGGL(k_quant<float>, dim3(nb), dim3(256), 0, s, (const float*)src, n, amax_slot, dst,
                       scale_out);
  } else {
    hipLaunchKernelGGL(k_amax<bf16>, dim3(nb), dim3(256), 0, s, (const bf16*)src, n, amax_slot);
    hipLaunchKernelGGL(k_quant<bf16>, dim3(nb), dim3(256), 0, s, (const bf16*)src, n, amax_slot, dst,
                       scale_out);
  }
  return hipGetLastError();
}

}  // namespace tsk
