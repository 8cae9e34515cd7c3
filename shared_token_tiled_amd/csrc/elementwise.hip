// Memory-bound kernels of the TileShare layer: norms, QK-norm, the w-bar
// blend (shared layers) and state merge (layer k), the per-tile gather, and
// e4m3 quantisation.  All are one pass over HBM; rows are handled by whole
// wavefronts with 16-byte (fp32) or 8-byte (bf16) vector accesses.
#include <type_traits>

#include "device_common.h"
#include "ts_kernels.h"

namespace {

constexpr int kMaxChunks = 16;  // d <= 64 lanes * 4 elements * 16 = 4096

// Maximum of |v| over the four values of a chunk as stored in T.
template <typename T> __device__ __forceinline__ float stored_amax4(f32x4 v) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(to_f32(from_f32<T>(v[e]))));
  return m;
}
// Wavefront maximum (all 64 lanes active), then one atomic max in float bits
// (values >= 0, so integer order is float order) into one of the
// tsk::AMAX_SLOTS slots, chosen by workgroup and wavefront: atomics on one
// address serialise, so the producers spread them and the quantisation takes
// the max over the slots.
__device__ __forceinline__ void wave_amax(unsigned* amax, float m) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const int slot = int(blockIdx.x * 4u + (threadIdx.x >> 6)) & (tsk::AMAX_SLOTS - 1);
  if ((threadIdx.x & 63) == 0) atomicMax(amax + slot * tsk::AMAX_STRIDE, __float_as_uint(m));
}

// ---- Norm1 / Norm2 (Table S1: once per token in shared layers) ---------
// One wavefront per row; the row stays in registers between the passes.
// NCH: 4-element chunks per lane (d <= 256 NCH), so the register arrays are
// sized for the model width.  The gain (and LayerNorm bias) chunks are loaded
// together with the row, not after the reduction, so a row costs one memory
// round trip.
// amax (optional): max |y| as stored (for the fp8 quantisation of y).
template <typename TOUT, bool RMS, int NCH>
__global__ __launch_bounds__(256) void k_norm(const float* __restrict__ x, int M, int d,
                                              const float* __restrict__ g,
                                              const float* __restrict__ b, float eps,
                                              TOUT* __restrict__ y, unsigned* __restrict__ amax) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* xr = x + size_t(row) * d;
  const int nc = d >> 2;
  f32x4 v[NCH], gv[NCH], bv[RMS ? 1 : NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    if (c < nc) {
      v[i] = load4(xr + 4 * c);
      gv[i] = load4(g + 4 * c);
      if (!RMS) bv[i] = load4(b + 4 * c);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    if (c < nc)
      s += RMS ? (v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3])
               : (v[i][0] + v[i][1] + v[i][2] + v[i][3]);
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
    for (int i = 0; i < NCH; ++i) {
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
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    if (c < nc) {
      const f32x4 gg = gv[i];
      f32x4 o;
      if (RMS) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = v[i][e] * inv * gg[e];
      } else {
        const f32x4 bb = bv[RMS ? 0 : i];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (v[i][e] - mean) * inv * gg[e] + bb[e];
      }
      store4(yr + 4 * c, o);
      if (amax) am = fmaxf(am, stored_amax4<TOUT>(o));
    }
  }
  if (amax) wave_amax(amax, am);  // one row per wavefront: all lanes here
}

// ---- per-head QK-RMSNorm (Table S1: once per token) and RoPE --------------
// HD/8 lanes share a row, each owning 8 values (4 rotation pairs) of every
// head slice: slices 0..H-1 are the q heads, H..2H-1 the k heads, slice s
// starting at column s*HD of the [q | k | v] row.  A lane loads its gains
// and the (cos, sin) of its four pairs at the row's grid coordinates once and
// then streams the 2H slices of the row, U at a time.
// NORM: RMS-normalise each head and scale by its gain first.  Then every q
// and k head is rotated by the row's grid coordinates (RopeRows): the angle
// of pair i of axis a is coord_a * base^(-i / pairs_a), so the score of two
// window tokens depends only on their coordinate difference, as with
// tile-local positions, and the attention kernels stage keys unchanged.
// QKN: the largest q-head and k-head norms of the rows as stored into qkn[0],
// qkn[1], as float bits (atomic max per workgroup, skipped where the slot
// already holds more); a template flag, so the other versions carry none of it.
template <typename T, int HD, bool NORM, bool QKN>
__global__ __launch_bounds__(256) void k_qkprep(T* __restrict__ qkv, int M, int d, int H,
                                                const float* __restrict__ qg,
                                                const float* __restrict__ kg, float eps, tsk::RopeRows rr,
                                                unsigned* __restrict__ qkn) {
  constexpr int LPS = HD / 8;    // lanes per row
  constexpr int RPW = 64 / LPS;  // rows per wavefront
  constexpr int U = 4;           // head slices in flight per lane
  const int lane = threadIdx.x & 63, sub = lane % LPS;
  const int64_t row64 = (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * RPW + lane / LPS;
  const bool ok = row64 < M;
  const int r = ok ? int(row64) : 0;
  // grid coordinates of the row
  int co[3];
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
  float2 cs[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int k = 4 * sub + e;
    const int ax = k < rr.pairs[0] ? 0 : (k < rr.pairs[0] + rr.pairs[1] ? 1 : 2);
    const int i = ax == 0 ? k : (ax == 1 ? k - rr.pairs[0] : k - rr.pairs[0] - rr.pairs[1]);
    const int np = ax == 0 ? rr.pairs[0] : (ax == 1 ? rr.pairs[1] : rr.pairs[2]);
    const int off = ax == 0 ? rr.off[0] : (ax == 1 ? rr.off[1] : rr.off[2]);
    const int cc = ax == 0 ? co[0] : (ax == 1 ? co[1] : co[2]);
    cs[e] = *reinterpret_cast<const float2*>(rr.tab + off + 2 * (cc * np + i));
  }
  f32x4 gq0 = {1, 1, 1, 1}, gq1 = gq0, gk0 = gq0, gk1 = gq0;
  if constexpr (NORM) {
    gq0 = load4(qg + sub * 8);
    gq1 = load4(qg + sub * 8 + 4);
    gk0 = load4(kg + sub * 8);
    gk1 = load4(kg + sub * 8 + 4);
  }
  T* base = qkv + int64_t(r) * 3 * d + sub * 8;
  const int ns = 2 * H;
  float mq = 0.f, mk = 0.f;  // largest squared head norms as stored (qkn)
  for (int s0 = 0; s0 < ns; s0 += U) {
    f32x4 a[U], c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] = c[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (ok && s0 + u < ns) load8(base + (s0 + u) * HD, a[u], c[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sl = s0 + u;
      if constexpr (NORM) {
        float ss = a[u][0] * a[u][0] + a[u][1] * a[u][1] + a[u][2] * a[u][2] + a[u][3] * a[u][3] +
                   c[u][0] * c[u][0] + c[u][1] * c[u][1] + c[u][2] * c[u][2] + c[u][3] * c[u][3];
        ss = group_sum(ss, LPS);
        const float inv = 1.0f / sqrtf(ss * (1.0f / HD) + eps);
        const bool isq = sl < H;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[u][e] = a[u][e] * inv * (isq ? gq0[e] : gk0[e]);
          c[u][e] = c[u][e] * inv * (isq ? gq1[e] : gk1[e]);
        }
      }
      float v[8] = {a[u][0], a[u][1], a[u][2], a[u][3], c[u][0], c[u][1], c[u][2], c[u][3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = v[2 * e], y = v[2 * e + 1];
        v[2 * e] = x * cs[e].x - y * cs[e].y;
        v[2 * e + 1] = x * cs[e].y + y * cs[e].x;
      }
      // bf16: q takes the softmax scale log2(e)/sqrt(hd) before its one
      // rounding, so the attention's q.k is already in the log2 domain
      if (std::is_same<T, bf16>::value && sl < H) {
        constexpr float QSCALE = 1.4426950408889634f / (HD == 128 ? 11.313708498984761f : HD == 64 ? 8.0f : 5.656854249492381f);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= QSCALE;
      }
      if (ok && sl < ns) store8(base + sl * HD, f32x4{v[0], v[1], v[2], v[3]}, f32x4{v[4], v[5], v[6], v[7]});
      if constexpr (QKN) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = float(T(v[e]));
          ss += x * x;
        }
        ss = group_sum(ss, LPS);
        if (ok && sl < ns) {
          if (sl < H) mq = fmaxf(mq, ss);
          else mk = fmaxf(mk, ss);
        }
      }
    }
  }
  if constexpr (QKN) {
    __shared__ float red[2][4];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      mq = fmaxf(mq, __shfl_xor(mq, o, 64));
      mk = fmaxf(mk, __shfl_xor(mk, o, 64));
    }
    if (lane == 0) {
      red[0][threadIdx.x >> 6] = mq;
      red[1][threadIdx.x >> 6] = mk;
    }
    __syncthreads();
    if (threadIdx.x < 2) {
      const int t = threadIdx.x;
      const float m = fmaxf(fmaxf(red[t][0], red[t][1]), fmaxf(red[t][2], red[t][3]));
      const unsigned bits = __float_as_uint(sqrtf(m));
      if (bits > __hip_atomic_load(qkn + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(qkn + t, bits);
    }
  }
}

__global__ void k_zero_qkn(unsigned* qkn) {
  if (threadIdx.x < tsk::QKN_BYTES / 4) qkn[threadIdx.x] = 0u;
}

// ---- w-bar blend / state merge (Figure 2 caption: the only approximate step)
// One wavefront per output row; entries summed in ascending tile order.
// NCH: 8-element chunks per lane (d <= 512 NCH).  Entries are taken two at a
// time, both rows loaded before either is added, and added in entry order.
template <typename TIN, typename TOUT, int NCH>
__global__ __launch_bounds__(256) void k_blend(const TIN* __restrict__ in, int d, int n_union,
                                               int n_tiles, int n, const int* __restrict__ cover_ptr,
                                               const int* __restrict__ entry_row,
                                               const float* __restrict__ w,
                                               TOUT* __restrict__ out_union,
                                               TOUT* __restrict__ out_global, unsigned* __restrict__ amax) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nc = d >> 3;
  float am = 0.f;  // max |output| as stored (one row per wavefront)
  if (r < n_union) {
    const int e0 = cover_ptr[r], e1 = cover_ptr[r + 1];
    f32x4 acc[NCH][2];
#pragma unroll
    for (int i = 0; i < NCH; ++i) acc[i][0] = acc[i][1] = f32x4{0, 0, 0, 0};
    for (int e = e0; e < e1; e += 2) {
      const bool two = e + 1 < e1;
      const TIN* s0 = in + size_t(entry_row[e]) * d;
      const TIN* s1 = two ? in + size_t(entry_row[e + 1]) * d : s0;
      const float w0 = w[e], w1 = two ? w[e + 1] : 0.f;
      f32x4 v0[NCH][2], v1[NCH][2];
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c < nc) {
          load8(s0 + 8 * c, v0[i][0], v0[i][1]);
          if (two) load8(s1 + 8 * c, v1[i][0], v1[i][1]);
        }
      }
#pragma unroll
      for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[i][h][k] = fmaf(w0, v0[i][h][k], acc[i][h][k]);
      if (two) {
#pragma unroll
        for (int i = 0; i < NCH; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[i][h][k] = fmaf(w1, v1[i][h][k], acc[i][h][k]);
      }
    }
    TOUT* dst = out_union + size_t(r) * d;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + 64 * i;
      if (c < nc) {
        store8(dst + 8 * c, acc[i][0], acc[i][1]);
        if (amax) am = fmaxf(am, fmaxf(stored_amax4<TOUT>(acc[i][0]), stored_amax4<TOUT>(acc[i][1])));
      }
    }
  } else if (r < n_union + n_tiles && out_global != nullptr) {
    const int t = r - n_union;
    const TIN* src = in + (size_t(t) * (n + 1) + n) * d;
    TOUT* dst = out_global + size_t(t) * d;
    for (int c = lane; c < (d >> 2); c += 64) {
      const f32x4 v = load4(src + 4 * c);
      store4(dst + 4 * c, v);
      if (amax) am = fmaxf(am, stored_amax4<TOUT>(v));
    }
  }
  if (amax) wave_amax(amax, am);  // r is uniform over the wavefront
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
__global__ void k_zero_slots(unsigned* p, int nslots) {
  if (int(threadIdx.x) < nslots) p[threadIdx.x * tsk::AMAX_STRIDE] = 0u;
}

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
                                               const unsigned* __restrict__ amax_bits, int nslots,
                                               uint8_t* __restrict__ q, float* __restrict__ scale_out) {
  unsigned mb = 0u;  // max over the slots (float bits of values >= 0)
  for (int i = 0; i < nslots; ++i) mb = max(mb, amax_bits[i * tsk::AMAX_STRIDE]);
  const float amax = __uint_as_float(mb);
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0 && scale_out) *scale_out = s;
  // eight values per lane and step: one 16-byte (bf16) or two 16-byte (fp32)
  // loads, one 8-byte store of codes
  const int64_t n8 = n >> 3;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n8; i += int64_t(gridDim.x) * 256) {
    f32x4 a, b;
    load8(x + 8 * i, a, b);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a[0] / s), clamp448(a[1] / s), 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a[2] / s), clamp448(a[3] / s), lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(b[0] / s), clamp448(b[1] / s), 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(b[2] / s), clamp448(b[3] / s), hi, true);
    reinterpret_cast<int2*>(q)[i] = make_int2(lo, hi);
  }
  for (int64_t i = 8 * n8 + int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
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
                const float* b, float eps, void* y, unsigned* amax) {
  if (M <= 0) return hipSuccess;
  const dim3 grid(blocks_for_rows(M)), block(256);
#define TS_NORM(NCH)                                                                                       \
  do {                                                                                                     \
    if (act == ACT_F32) {                                                                                  \
      if (rms) hipLaunchKernelGGL((k_norm<float, true, NCH>), grid, block, 0, s, x, M, d, g, b, eps, (float*)y, amax);  \
      else hipLaunchKernelGGL((k_norm<float, false, NCH>), grid, block, 0, s, x, M, d, g, b, eps, (float*)y, amax);     \
    } else {                                                                                               \
      if (rms) hipLaunchKernelGGL((k_norm<bf16, true, NCH>), grid, block, 0, s, x, M, d, g, b, eps, (bf16*)y, amax);    \
      else hipLaunchKernelGGL((k_norm<bf16, false, NCH>), grid, block, 0, s, x, M, d, g, b, eps, (bf16*)y, amax);       \
    }                                                                                                      \
  } while (0)
  if (d <= 256 * 4) TS_NORM(4);
  else if (d <= 256 * 10) TS_NORM(10);
  else TS_NORM(kMaxChunks);
#undef TS_NORM
  return hipGetLastError();
}

hipError_t qk_prep(hipStream_t s, int act, void* qkv, int M, int d, int H, int hd, const float* qg,
                   const float* kg, float eps, const RopeRows& rr, unsigned* qkn) {
  if (qkn) hipLaunchKernelGGL(k_zero_qkn, dim3(1), dim3(64), 0, s, qkn);
  if (M <= 0) return hipGetLastError();
  // four wavefronts per block, 512 / hd rows per wavefront
  const int64_t rows_per_block = 4 * (512 / hd);
  const dim3 grid(unsigned((M + rows_per_block - 1) / rows_per_block)), block(256);
  const bool norm = qg != nullptr;
#define TS_QK(T, HD)                                                                                              \
  do {                                                                                                            \
    if (norm) hipLaunchKernelGGL((k_qkprep<T, HD, true, false>), grid, block, 0, s, (T*)qkv, M, d, H, qg, kg, eps, rr, qkn); \
    else if (qkn) hipLaunchKernelGGL((k_qkprep<T, HD, false, true>), grid, block, 0, s, (T*)qkv, M, d, H, qg, kg, eps, rr, qkn); \
    else hipLaunchKernelGGL((k_qkprep<T, HD, false, false>), grid, block, 0, s, (T*)qkv, M, d, H, qg, kg, eps, rr, qkn); \
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
                 void* out_global, unsigned* amax) {
  const dim3 grid(blocks_for_rows(n_union + n_tiles)), block(256);
#define TS_BLN(TI, TO, NCH)                                                                             \
  hipLaunchKernelGGL((k_blend<TI, TO, NCH>), grid, block, 0, s, (const TI*)in, d, n_union, n_tiles, n, \
                     cover_ptr, entry_row, w, (TO*)out_union, (TO*)out_global, amax)
#define TS_BL(TI, TO)                        \
  do {                                       \
    if (d <= 512 * 2) TS_BLN(TI, TO, 2);     \
    else if (d <= 512 * 5) TS_BLN(TI, TO, 5); \
    else TS_BLN(TI, TO, 8);                  \
  } while (0)
  if (tin == ACT_F32 && tout == ACT_F32) TS_BL(float, float);
  else if (tin == ACT_BF16 && tout == ACT_BF16) TS_BL(bf16, bf16);
  else if (tin == ACT_F32 && tout == ACT_BF16) TS_BL(float, bf16);
  else TS_BL(bf16, float);
#undef TS_BL
#undef TS_BLN
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
                        float* scale_out, unsigned* amax_slot, bool amax_ready, int nslots) {
  const int nb = grid_stride_blocks((n + 3) / 4);   // max pass: four values per lane and step
  const int nq = grid_stride_blocks((n + 7) / 8);   // codes: eight
  if (nslots < 1 || nslots > AMAX_SLOTS) return hipErrorInvalidValue;
  if (!amax_ready) hipLaunchKernelGGL(k_zero_slots, dim3(1), dim3(64), 0, s, amax_slot, nslots);
  if (tin == ACT_F32) {
    if (!amax_ready) hipLaunchKernelGGL(k_amax<float>, dim3(nb), dim3(256), 0, s, (const float*)src, n, amax_slot);
    hipLaunchKernelGGL(k_quant<float>, dim3(nq), dim3(256), 0, s, (const float*)src, n, amax_slot, nslots, dst,
                       scale_out);
  } else {
    if (!amax_ready) hipLaunchKernelGGL(k_amax<bf16>, dim3(nb), dim3(256), 0, s, (const bf16*)src, n, amax_slot);
    hipLaunchKernelGGL(k_quant<bf16>, dim3(nq), dim3(256), 0, s, (const bf16*)src, n, amax_slot, nslots, dst,
                       scale_out);
  }
  return hipGetLastError();
}

hipError_t zero_amax(hipStream_t s, unsigned* p) {
  hipLaunchKernelGGL(k_zero_slots, dim3(1), dim3(64), 0, s, p, AMAX_SLOTS);
  return hipGetLastError();
}

}  // namespace tsk
