// LayerNorm forward and backward, one wavefront per row.
//
// Forward: mu = mean(x), var = mean((x - mu)^2) (biased), rstd =
// (var + eps)^-1/2, y = g (x - mu) rstd + b. Backward (chain rule): with
// xhat = (x - mu) rstd and dxhat = dy g,
//   dx = rstd (dxhat - mean(dxhat) - xhat mean(dxhat xhat)),
// accumulated onto the incoming residual gradient, and per-block partial
// column sums of dy xhat (dg) and dy (db), reduced afterwards in a fixed order
// so the result is bit-reproducible.
// (LayerNorm layer: RustGPT page, file list; final LayerNorm before the
// vocabulary projection: Feste page, "Model Architecture".)
#include "kernels.h"

namespace lm {

// C = 128 * NV; a lane holds NV values in float4 chunks when NV is even
// (16-byte accesses), else in float2 chunks. Chunk j of a lane covers
// columns W (lane + 64 j) .. + W - 1, W the chunk width.
template <int NV, typename T>
__global__ void __launch_bounds__(256) ln_fwd_kernel(const float* __restrict__ x, const float* __restrict__ g,
                                                     const float* __restrict__ b, int M, float eps,
                                                     T* __restrict__ y, float* __restrict__ mu_out,
                                                     float* __restrict__ rstd_out) {
  constexpr int C = 128 * NV;
  constexpr int W = NV % 2 == 0 ? 4 : 2;  // floats per chunk
  constexpr int NC = C / (64 * W);        // chunks per lane
  const int lane = threadIdx.x & 63;
  const long m = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  float v[NC][W];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const long o = m * C + (long)W * (lane + 64 * j);
    if constexpr (W == 4) {
      const float4 t = *reinterpret_cast<const float4*>(x + o);
      v[j][0] = t.x; v[j][1] = t.y; v[j][2] = t.z; v[j][3] = t.w;
    } else {
      const float2 t = *reinterpret_cast<const float2*>(x + o);
      v[j][0] = t.x; v[j][1] = t.y;
    }
#pragma unroll
    for (int e = 0; e < W; ++e) s += v[j][e];
  }
  const float mu = wave_sum(s) * (1.0f / C);
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int e = 0; e < W; ++e) {
      const float a = v[j][e] - mu;
      q += a * a;
    }
  const float var = wave_sum(q) * (1.0f / C);
  const float r = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = W * (lane + 64 * j);
    float o[W];
#pragma unroll
    for (int e = 0; e < W; ++e) o[e] = (v[j][e] - mu) * r * g[c + e] + b[c + e];
    if constexpr (sizeof(T) == 2) {  // adjacent 16-bit values packed in pairs
      if constexpr (W == 4)
        *reinterpret_cast<uint2*>(y + m * C + c) = make_uint2(H16<T>::pack(o[0], o[1]), H16<T>::pack(o[2], o[3]));
      else
        *reinterpret_cast<uint32_t*>(y + m * C + c) = H16<T>::pack(o[0], o[1]);
    } else {
      if constexpr (W == 4)
        *reinterpret_cast<float4*>(y + m * C + c) = make_float4(o[0], o[1], o[2], o[3]);
      else
        *reinterpret_cast<float2*>(y + m * C + c) = make_float2(o[0], o[1]);
    }
  }
  if (lane == 0) {
    mu_out[m] = mu;
    rstd_out[m] = r;
  }
}

template <typename T>
void launch_ln_fwd(const float* x, const float* g, const float* b, int M, int C, float eps, T* y, float* mu,
                   float* rstd, hipStream_t s) {
  dim3 grid((M + 3) / 4), block(256);
  switch (C / 128) {
#define LN_CASE(NV) \
  case NV: hipLaunchKernelGGL((ln_fwd_kernel<NV, T>), grid, block, 0, s, x, g, b, M, eps, y, mu, rstd); break;
    LN_CASE(1) LN_CASE(2) LN_CASE(3) LN_CASE(4) LN_CASE(5) LN_CASE(6) LN_CASE(7) LN_CASE(8)
#undef LN_CASE
    default: break;
  }
}
template void launch_ln_fwd<float>(const float*, const float*, const float*, int, int, float, float*, float*,
                                   float*, hipStream_t);
template void launch_ln_fwd<bf16>(const float*, const float*, const float*, int, int, float, bf16*, float*,
                                  float*, hipStream_t);
template void launch_ln_fwd<f16>(const float*, const float*, const float*, int, int, float, f16*, float*,
                                 float*, hipStream_t);

// Backward. Each block owns kLnRowsPerBlock consecutive rows; wave w takes
// rows w, w+4, ... of them. g_out = g_in + dx (g_in may alias g_out or be
// null); g_act (nullable) receives g_out in the activation type. Per-block
// column partials: dgamma, dbeta and (part_dc non-null) the column sums of
// g_out itself, which are the gradient of the bias added to the residual
// stream just before this LayerNorm's input.
template <int NV, typename T>
__global__ void __launch_bounds__(256) ln_bwd_kernel(const float* __restrict__ dy, const float* __restrict__ x,
                                                     const float* __restrict__ mu_in,
                                                     const float* __restrict__ rstd_in,
                                                     const float* __restrict__ g, int M,
                                                     const float* g_in, float* g_out, T* __restrict__ g_act,
                                                     float* __restrict__ part_dg, float* __restrict__ part_db,
                                                     float* __restrict__ part_dc) {
  constexpr int C = 128 * NV;
  // a lane holds its values in float4 chunks when NV is even (16-byte
  // accesses), else in float2 chunks; chunk j covers columns
  // W (lane + 64 j) .. + W - 1
  constexpr int W = NV % 2 == 0 ? 4 : 2, NC = C / (64 * W);
  __shared__ float s_dg[4][C];
  __shared__ float s_db[4][C];
  __shared__ float s_dc[4][C];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  auto ld = [](const float* p, float* v) {
    if constexpr (W == 4) {
      const f32x4_t t = *reinterpret_cast<const f32x4_t*>(p);
      v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
    } else {
      const float2 t = *reinterpret_cast<const float2*>(p);
      v[0] = t.x; v[1] = t.y;
    }
  };
  float gg[NC][W], adg[NC][W], adb[NC][W], adc[NC][W];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    ld(g + W * (lane + 64 * j), gg[j]);
#pragma unroll
    for (int e = 0; e < W; ++e) adg[j][e] = adb[j][e] = adc[j][e] = 0.f;
  }
  const long r0 = (long)blockIdx.x * kLnRowsPerBlock;
  const long r1 = min((long)M, r0 + kLnRowsPerBlock);
  // the next row's inputs are loaded while the current row is computed
  float dn[NC][W], xn[NC][W], gn[NC][W];
  float mun = 0.f, rn = 0.f;
  auto load_row = [&](long m) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const long o = m * C + W * (lane + 64 * j);
      ld(dy + o, dn[j]);
      ld(x + o, xn[j]);
      if (g_in) ld(g_in + o, gn[j]);
      else
#pragma unroll
        for (int e = 0; e < W; ++e) gn[j][e] = 0.f;
    }
    mun = mu_in[m];
    rn = rstd_in[m];
  };
  if (r0 + w < r1) load_row(r0 + w);
  for (long m = r0 + w; m < r1; m += 4) {
    float dv[NC][W], xv[NC][W], gi[NC][W];
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int e = 0; e < W; ++e) {
        dv[j][e] = dn[j][e];
        xv[j][e] = xn[j][e];
        gi[j][e] = gn[j][e];
      }
    const float mu = mun, r = rn;
    if (m + 4 < r1) load_row(m + 4);
    float xh[NC][W], dxh[NC][W];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int e = 0; e < W; ++e) {
        const float d = dv[j][e];
        xh[j][e] = (xv[j][e] - mu) * r;
        dxh[j][e] = d * gg[j][e];
        s1 += dxh[j][e];
        s2 += dxh[j][e] * xh[j][e];
        adg[j][e] += d * xh[j][e];
        adb[j][e] += d;
      }
    const float m1 = wave_sum(s1) * (1.0f / C), m2 = wave_sum(s2) * (1.0f / C);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = W * (lane + 64 * j);
      float o[W];
#pragma unroll
      for (int e = 0; e < W; ++e) {
        o[e] = r * (dxh[j][e] - m1 - xh[j][e] * m2) + gi[j][e];
        adc[j][e] += o[e];
      }
      if constexpr (W == 4) {
        *reinterpret_cast<f32x4_t*>(g_out + m * C + c) = f32x4_t{o[0], o[1], o[2], o[3]};
        if (g_act) {
          if constexpr (sizeof(T) == 2)  // adjacent 16-bit values packed in pairs
            *reinterpret_cast<uint2*>(g_act + m * C + c) = make_uint2(H16<T>::pack(o[0], o[1]), H16<T>::pack(o[2], o[3]));
          else
            *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(g_act) + m * C + c) = f32x4_t{o[0], o[1], o[2], o[3]};
        }
      } else {
        *reinterpret_cast<float2*>(g_out + m * C + c) = make_float2(o[0], o[1]);
        if (g_act) {
          if constexpr (sizeof(T) == 2)
            *reinterpret_cast<uint32_t*>(g_act + m * C + c) = H16<T>::pack(o[0], o[1]);
          else
            *reinterpret_cast<float2*>(reinterpret_cast<float*>(g_act) + m * C + c) = make_float2(o[0], o[1]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = W * (lane + 64 * j);
#pragma unroll
    for (int e = 0; e < W; ++e) {
      s_dg[w][c + e] = adg[j][e];
      s_db[w][c + e] = adb[j][e];
      s_dc[w][c + e] = adc[j][e];
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += 256) {
    part_dg[(long)blockIdx.x * C + c] = ((s_dg[0][c] + s_dg[1][c]) + s_dg[2][c]) + s_dg[3][c];
    part_db[(long)blockIdx.x * C + c] = ((s_db[0][c] + s_db[1][c]) + s_db[2][c]) + s_db[3][c];
    if (part_dc) part_dc[(long)blockIdx.x * C + c] = ((s_dc[0][c] + s_dc[1][c]) + s_dc[2][c]) + s_dc[3][c];
  }
}

template <typename T>
void launch_ln_bwd(const float* dy, const float* x, const float* mu, const float* rstd, const float* g, int M,
                   int C, const float* g_in, float* g_out, T* g_act, float* part_dg, float* part_db,
                   float* part_dc, hipStream_t s) {
  dim3 grid((M + kLnRowsPerBlock - 1) / kLnRowsPerBlock), block(256);
  switch (C / 128) {
#define LN_CASE(NV)                                                                                    \
  case NV:                                                                                             \
    hipLaunchKernelGGL((ln_bwd_kernel<NV, T>), grid, block, 0, s, dy, x, mu, rstd, g, M, g_in, g_out, g_act, \
                       part_dg, part_db, part_dc);                                                     \
    break;
    LN_CASE(1) LN_CASE(2) LN_CASE(3) LN_CASE(4) LN_CASE(5) LN_CASE(6) LN_CASE(7) LN_CASE(8)
#undef LN_CASE
    default: break;
  }
}
template void launch_ln_bwd<float>(const float*, const float*, const float*, const float*, const float*, int, int,
                                   const float*, float*, float*, float*, float*, float*, hipStream_t);
template void launch_ln_bwd<bf16>(const float*, const float*, const float*, const float*, const float*, int, int,
                                  const float*, float*, bf16*, float*, float*, float*, hipStream_t);
template void launch_ln_bwd<f16>(const float*, const float*, const float*, const float*, const float*, int, int,
                                 const float*, float*, f16*, float*, float*, float*, hipStream_t);

// out[c] = sum over p < P of part[p][c] in a fixed order: a block covers 16
// columns with 64 row groups (a wavefront reads 4 rows x 64 bytes); thread
// (c, r) sums p = r, r + 64, ... for its column, then the group sums are
// added in r order (eight runs of eight, then the eight run sums). Up to
// three vectors at once (the dg, db and output-column partials of one
// LayerNorm); pb/pc and ob/oc may be null. The sums are latency-bound (a few
// MB, just written): many wavefronts, each with its loads in flight together.
constexpr int kPartCols = 16, kPartGroups = 64;
__device__ __forceinline__ void colsum_partials_block(const float* __restrict__ pa, const float* __restrict__ pb,
                                                      const float* __restrict__ pc, int P, int C,
                                                      float* __restrict__ oa, float* __restrict__ ob,
                                                      float* __restrict__ oc) {
  __shared__ float sm[3][kPartGroups][kPartCols];
  __shared__ float sr[3][8][kPartCols];
  const int cc = threadIdx.x % kPartCols, r = threadIdx.x / kPartCols;
  const int c = blockIdx.x * kPartCols + cc;
  float a = 0.f, b = 0.f, d = 0.f;
  if (c < C) {
    int p = r;
    for (; p + 7 * kPartGroups < P; p += 8 * kPartGroups) {
      float va[8], vb[8], vc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const long o = (long)(p + kPartGroups * u) * C + c;
        va[u] = pa[o];
        vb[u] = pb ? pb[o] : 0.f;
        vc[u] = pc ? pc[o] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a += va[u];
        b += vb[u];
        d += vc[u];
      }
    }
    for (; p < P; p += kPartGroups) {
      a += pa[(long)p * C + c];
      if (pb) b += pb[(long)p * C + c];
      if (pc) d += pc[(long)p * C + c];
    }
  }
  sm[0][r][cc] = a;
  sm[1][r][cc] = b;
  sm[2][r][cc] = d;
  __syncthreads();
  if (r < 8) {
    float ta = 0.f, tb = 0.f, td = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ta += sm[0][r * 8 + k][cc];
      tb += sm[1][r * 8 + k][cc];
      td += sm[2][r * 8 + k][cc];
    }
    sr[0][r][cc] = ta;
    sr[1][r][cc] = tb;
    sr[2][r][cc] = td;
  }
  __syncthreads();
  if (r == 0 && c < C) {
    float ta = 0.f, tb = 0.f, td = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ta += sr[0][k][cc];
      tb += sr[1][k][cc];
      td += sr[2][k][cc];
    }
    oa[c] = ta;
    if (ob) ob[c] = tb;
    if (oc) oc[c] = td;
  }
}

__global__ void __launch_bounds__(1024) colsum_partials_kernel(const float* __restrict__ pa, const float* __restrict__ pb,
                                                              const float* __restrict__ pc, int P, int C,
                                                              float* __restrict__ oa, float* __restrict__ ob,
                                                              float* __restrict__ oc) {
  colsum_partials_block(pa, pb, pc, P, C, oa, ob, oc);
}

// Several independent reductions of the same shape in one launch
// (blockIdx.y picks the set).
__global__ void __launch_bounds__(1024) colsum_partials_batch_kernel(ColsumBatch bt, int P, int C) {
  const int i = blockIdx.y;
  colsum_partials_block(bt.pa[i], bt.pb[i], bt.pc[i], P, C, bt.oa[i], bt.ob[i], bt.oc[i]);
}

void launch_colsum_partials(const float* pa, const float* pb, int P, int C, float* oa, float* ob,
                            hipStream_t s, const float* pc, float* oc) {
  static_assert(kPartCols * kPartGroups == 1024 && kPartGroups == 64, "block shape");
  hipLaunchKernelGGL(colsum_partials_kernel, dim3((C + kPartCols - 1) / kPartCols), dim3(1024), 0, s, pa, pb, pc, P,
                     C, oa, ob, oc);
}

void launch_colsum_partials_batch(const ColsumBatch& bt, int n, int P, int C, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(colsum_partials_batch_kernel, dim3((C + kPartCols - 1) / kPartCols, n), dim3(1024), 0, s, bt, P,
                     C);
}

// Column sums of an [M, N] matrix (bias gradients), N a multiple of 4. Stage
// 1: a block covers 256 columns (4 per thread) and kColRows rows, its four
// wavefronts taking every fourth row, combined in a fixed order into one
// partial row per block; stage 2 (colsum_partials) sums the partials.
template <typename T> struct Quad;
template <> struct Quad<float> {
  static __device__ __forceinline__ float4 ld(const float* p) { return *reinterpret_cast<const float4*>(p); }
};
template <typename T> struct Quad {  // 16-bit types
  static __device__ __forceinline__ float4 ld(const T* p) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(H16<T>::lo(u.x), H16<T>::hi(u.x), H16<T>::lo(u.y), H16<T>::hi(u.y));
  }
};

template <typename T>
__global__ void __launch_bounds__(256) colsum_stage1_kernel(const T* __restrict__ a, long lda, int M, int N,
                                                            float* __restrict__ part) {
  __shared__ float4 s[4][64];
  const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int c = (blockIdx.x * 64 + lane) * 4;
  const long r0 = (long)blockIdx.y * kColRows;
  const long r1 = min((long)M, r0 + kColRows);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < N) {
    long r = r0 + g;
    // batches of 8 rows: all loads in flight first, then added in row order
    for (; r + 28 < r1; r += 32) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = Quad<T>::ld(a + (r + 4 * u) * lda + c);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w;
      }
    }
    for (; r < r1; r += 4) {
      float4 v = Quad<T>::ld(a + r * lda + c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
  }
  s[g][lane] = acc;
  __syncthreads();
  if (g == 0 && c < N) {
    float4 t0 = s[0][lane], t1 = s[1][lane], t2 = s[2][lane], t3 = s[3][lane];
    float4 o = make_float4(((t0.x + t1.x) + t2.x) + t3.x, ((t0.y + t1.y) + t2.y) + t3.y,
                           ((t0.z + t1.z) + t2.z) + t3.z, ((t0.w + t1.w) + t2.w) + t3.w);
    *reinterpret_cast<float4*>(part + (long)blockIdx.y * N + c) = o;
  }
}

// 16-bit input with N and lda multiples of 8: 8 columns (one 16-byte load)
// per thread, 512 per block; the same row order per column as above.
template <typename T>
__device__ __forceinline__ void colsum8_h16_block(const T* __restrict__ a, long lda, int M, int N,
                                                  float* __restrict__ part) {
  __shared__ float s[4][8][64];
  const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int c = (blockIdx.x * 64 + lane) * 8;
  const long r0 = (long)blockIdx.y * kColRows;
  const long r1 = min((long)M, r0 + kColRows);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](uint4 u) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += H16<T>::lo(w[i]);
      acc[2 * i + 1] += H16<T>::hi(w[i]);
    }
  };
  if (c < N) {
    long r = r0 + g;
    for (; r + 28 < r1; r += 32) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const uint4*>(a + (r + 4 * u) * lda + c);
#pragma unroll
      for (int u = 0; u < 8; ++u) add(v[u]);
    }
    for (; r < r1; r += 4) add(*reinterpret_cast<const uint4*>(a + r * lda + c));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) s[g][i][lane] = acc[i];
  __syncthreads();
  if (g == 0 && c < N) {
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = ((s[0][i][lane] + s[1][i][lane]) + s[2][i][lane]) + s[3][i][lane];
    float* dst = part + (long)blockIdx.y * N + c;
    *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
  }
}

template <typename T>
__global__ void __launch_bounds__(256) colsum8_h16_kernel(const T* __restrict__ a, long lda, int M, int N,
                                                          float* __restrict__ part) {
  colsum8_h16_block<T>(a, lda, M, N, part);
}

// The same partial sums for several matrices of one shape in one launch
// (blockIdx.z: the matrix), each exactly as one colsum8_h16_kernel launch
// computes them.
template <typename T>
__global__ void __launch_bounds__(256) colsum8_h16_batch_kernel(Colsum16Batch b, long lda, int M, int N) {
  colsum8_h16_block<T>(reinterpret_cast<const T*>(b.a[blockIdx.z]), lda, M, N, b.part[blockIdx.z]);
}

template <typename T>
void launch_colsum_stage1_batch(const Colsum16Batch& b, int n, long lda, int M, int N, hipStream_t s) {
  if (n <= 0) return;
  const int P = (M + kColRows - 1) / kColRows;
  hipLaunchKernelGGL(colsum8_h16_batch_kernel<T>, dim3((N / 8 + 63) / 64, P, n), dim3(256), 0, s, b, lda, M, N);
}
template void launch_colsum_stage1_batch<bf16>(const Colsum16Batch&, int, long, int, int, hipStream_t);
template void launch_colsum_stage1_batch<f16>(const Colsum16Batch&, int, long, int, int, hipStream_t);

template <typename T>
void launch_colsum_stage1(const T* a, long lda, int M, int N, float* part, hipStream_t s) {
  const int P = (M + kColRows - 1) / kColRows;
  if constexpr (sizeof(T) == 2) {
    if (N % 8 == 0 && lda % 8 == 0) {
      hipLaunchKernelGGL(colsum8_h16_kernel<T>, dim3((N / 8 + 63) / 64, P), dim3(256), 0, s, a, lda, M, N, part);
      return;
    }
  }
  hipLaunchKernelGGL(colsum_stage1_kernel<T>, dim3((N / 4 + 63) / 64, P), dim3(256), 0, s, a, lda, M, N, part);
}

template <typename T>
void launch_colsum(const T* a, long lda, int M, int N, float* part, float* out, hipStream_t s) {
  launch_colsum_stage1<T>(a, lda, M, N, part, s);
  launch_colsum_partials(part, nullptr, (M + kColRows - 1) / kColRows, N, out, nullptr, s);
}
template void launch_colsum_stage1<float>(const float*, long, int, int, float*, hipStream_t);
template void launch_colsum_stage1<bf16>(const bf16*, long, int, int, float*, hipStream_t);
template void launch_colsum_stage1<f16>(const f16*, long, int, int, float*, hipStream_t);
template void launch_colsum<float>(const float*, long, int, int, float*, float*, hipStream_t);
template void launch_colsum<bf16>(const bf16*, long, int, int, float*, float*, hipStream_t);
template void launch_colsum<f16>(const f16*, long, int, int, float*, float*, hipStream_t);

}  // namespace lm
