// Fused softmax cross-entropy over the vocabulary, forward and backward.
//
// Over the valid rows (target >= 0, N of them): row loss = logsumexp(z) -
// z[target]; dz = (softmax(z) - onehot(target)) / N, written over z in place;
// rows with target -1 get dz = 0; padding columns V..ldz-1 are zeroed.
// (Cross-entropy loss: RustGPT page, technical-implementation list; the V
// outputs form a distribution summing to 1: Smallem page, "Ce qu'est un modele
// de langage".)
// One block per row: pass 1 keeps a per-thread running (max, sum of exp) over
// 16-byte vectors, combined across the block; pass 2 writes dz.
#include "kernels.h"

namespace lm {

template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const bf16* p, float* out) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(v[2 * i]) | ((uint32_t)f2bf(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const float* p, float* out) {
    float4 u = *reinterpret_cast<const float4*>(p);
    out[0] = u.x; out[1] = u.y; out[2] = u.z; out[3] = u.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  s = s * __expf(m - mm) + s2 * __expf(m2 - mm);
  m = mm;
}

template <typename T>
__global__ void __launch_bounds__(256) xent_kernel(T* __restrict__ z, long ldz, int V,
                                                   const int32_t* __restrict__ tgt,
                                                   const int32_t* __restrict__ n_valid,
                                                   float* __restrict__ row_loss) {
  constexpr int NV = Vec16<T>::N;
  __shared__ float s_m[256], s_s[256];
  const long row = blockIdx.x;
  T* zr = z + row * ldz;
  const int t = tgt[row];
  const bool valid = t >= 0 && t < V;
  const int nvec = (int)(ldz / NV);
  float m = -INFINITY, s = 0.f;
  if (valid) {
    for (int v = threadIdx.x; v < nvec; v += 256) {
      float x[NV];
      Vec16<T>::load(zr + (long)v * NV, x);
      float cm = -INFINITY;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (v * NV + i >= V) x[i] = -INFINITY;
        cm = fmaxf(cm, x[i]);
      }
      if (cm == -INFINITY) continue;
      if (cm > m) {
        s = s * __expf(m - cm);
        m = cm;
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) s += __expf(x[i] - m);
    }
  }
  s_m[threadIdx.x] = m;
  s_s[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      float mm = s_m[threadIdx.x], ss = s_s[threadIdx.x];
      merge_ms(mm, ss, s_m[threadIdx.x + o], s_s[threadIdx.x + o]);
      s_m[threadIdx.x] = mm;
      s_s[threadIdx.x] = ss;
    }
    __syncthreads();
  }
  const float lse = s_m[0] + __logf(s_s[0]);
  const int n = *n_valid;
  const float inv_n = n > 0 ? 1.0f / (float)n : 0.f;
  if (threadIdx.x == 0) row_loss[row] = valid ? lse - Act<T>::ld(zr, t) : 0.f;
  __syncthreads();  // every thread has read z[t] (via lse) before it is overwritten
  for (int v = threadIdx.x; v < nvec; v += 256) {
    float x[NV];
    Vec16<T>::load(zr + (long)v * NV, x);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int j = v * NV + i;
      float d = 0.f;
      if (valid && j < V) d = (__expf(x[i] - lse) - (j == t ? 1.f : 0.f)) * inv_n;
      x[i] = d;
    }
    Vec16<T>::store(zr + (long)v * NV, x);
  }
}

template <typename T>
void launch_xent(T* z, long ldz, int M, int V, const int32_t* tgt, const int32_t* n_valid, float* row_loss,
                 hipStream_t s) {
  hipLaunchKernelGGL(xent_kernel<T>, dim3(M), dim3(256), 0, s, z, ldz, V, tgt, n_valid, row_loss);
}
template void launch_xent<float>(float*, long, int, int, const int32_t*, const int32_t*, float*, hipStream_t);
template void launch_xent<bf16>(bf16*, long, int, int, const int32_t*, const int32_t*, float*, hipStream_t);

}  // namespace lm
