// Fused softmax cross-entropy over the vocabulary, forward and backward.
//
// Over the valid rows (target >= 0, N of them): row loss = logsumexp(z) -
// z[target]; dz = (softmax(z) - onehot(target)) / N, written over z in place;
// rows with target -1 get dz = 0; padding columns V..ldz-1 are zeroed. With
// a loss scale S (fp16 training), dz is multiplied by S: the gradient of S
// times the loss, so that small gradients stay above fp16's underflow; the
// reported loss is not scaled.
// (Cross-entropy loss: RustGPT page, technical-implementation list; the V
// outputs form a distribution summing to 1: Smallem page, "Ce qu'est un modele
// de langage".)
// One block per row: pass 1 keeps a per-thread running (max, sum of exp) over
// 16-byte vectors, combined across the block; pass 2 writes dz.
#include "kernels.h"

namespace lm {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte nontemporal load and store: the logits are streamed through once
// per pass (far more of them than the caches hold).
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_nt16(void* p, uint4 u) {
  __builtin_nontemporal_store(u32x4_t{u.x, u.y, u.z, u.w}, reinterpret_cast<u32x4_t*>(p));
}

template <typename T> struct Vec16 {  // 16-bit types (bf16, f16)
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const T* p, float* out) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = H16<T>::lo(w[i]);
      out[2 * i + 1] = H16<T>::hi(w[i]);
    }
  }
  static __device__ __forceinline__ void store(T* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = H16<T>::pack(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  static __device__ __forceinline__ void store_nt(T* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = H16<T>::pack(v[2 * i], v[2 * i + 1]);
    st_nt16(p, make_uint4(w[0], w[1], w[2], w[3]));
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
  static __device__ __forceinline__ void store_nt(float* p, const float* v) {
    st_nt16(p, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])));
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
                                                   const float* __restrict__ loss_scale,
                                                   float* __restrict__ row_loss) {
  constexpr int NV = Vec16<T>::N;
  constexpr int U = 4;  // vectors in flight per thread
  __shared__ float s_m[4], s_s[4];
  __shared__ float s_lse;
  const long row = blockIdx.x;
  T* zr = z + row * ldz;
  const int t = tgt[row];
  const bool valid = t >= 0 && t < V;
  const int nvec = (int)(ldz / NV);
  float m = -INFINITY, s = 0.f;
  if (valid) {
    for (int v0 = threadIdx.x; v0 < nvec; v0 += 256 * U) {
      float x[U][NV];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * 256;
        if (v < nvec) Vec16<T>::load(zr + (long)v * NV, x[u]);
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (v >= nvec || v * NV + i >= V) x[u][i] = -INFINITY;
      }
      float cm = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < NV; ++i) cm = fmaxf(cm, x[u][i]);
      if (cm == -INFINITY) continue;
      if (cm > m) {
        s = s * __expf(m - cm);
        m = cm;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < NV; ++i) s += __expf(x[u][i] - m);
    }
  }
  // combine (max, sum) pairs: within the wavefront, then the 4 wavefronts in order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) merge_ms(m, s, __shfl_xor(m, o, 64), __shfl_xor(s, o, 64));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_m[w] = m;
    s_s[w] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = s_m[0], ss = s_s[0];
    for (int q = 1; q < 4; ++q) merge_ms(mm, ss, s_m[q], s_s[q]);
    const float lse = mm + __logf(ss);
    s_lse = lse;
    row_loss[row] = valid ? lse - Act<T>::ld(zr, t) : 0.f;
  }
  __syncthreads();  // z[t] has been read before it is overwritten
  const float lse = s_lse;
  const int n = *n_valid;
  const float inv_n = (n > 0 ? 1.0f / (float)n : 0.f) * (loss_scale ? *loss_scale : 1.0f);
  for (int v0 = threadIdx.x; v0 < nvec; v0 += 256 * U) {
    float x[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * 256;
      if (v < nvec && valid) Vec16<T>::load(zr + (long)v * NV, x[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * 256;
      if (v >= nvec) continue;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int j = v * NV + i;
        float d = 0.f;
        if (valid && j < V) d = (__expf(x[u][i] - lse) - (j == t ? 1.f : 0.f)) * inv_n;
        x[u][i] = d;
      }
      Vec16<T>::store(zr + (long)v * NV, x[u]);
    }
  }
}

// The same computation with the row held in registers between the passes:
// BT threads, thread t owns the 16-byte vectors t, t + BT, ... (NCH of
// them), so the logits are read from memory once. Used when the row fits
// (ldz <= BT * NCH * vector width), with the narrowest block of 64, 256 or
// 1024 threads that holds it in at most 8 vectors a thread: a narrow row on
// 1024 threads (the 8000-wide vocabulary: one vector each) left a block of
// 16 wavefronts a short latency-bound pass, two blocks per CU. The vector work per logit is kept
// small: only the chunks that reach past column V - 1 are masked (a test
// uniform over the block), exponentials are exp2 of one fused multiply-add
// (the 1/N scale folded into the exponent of the gradient pass), and the
// one-hot term is subtracted by the one thread that holds the target.
template <typename T, int NCH, int BT>
__global__ void __launch_bounds__(BT) __attribute__((amdgpu_waves_per_eu(8))) xent_reg_kernel(T* __restrict__ z, long ldz, int V,
                                                        const int32_t* __restrict__ tgt,
                                                        const int32_t* __restrict__ n_valid,
                                                        const float* __restrict__ loss_scale,
                                                        float* __restrict__ row_loss) {
  constexpr int NV = Vec16<T>::N;
  constexpr float kL2e = 1.4426950408889634f;
  constexpr int NW = BT / 64;  // wavefronts of the block
  __shared__ float s_m[NW], s_s[NW];
  __shared__ float s_lse;
  const long row = blockIdx.x;
  T* zr = z + row * ldz;
  const int t = tgt[row];
  const bool valid = t >= 0 && t < V;
  const int nvec = (int)(ldz / NV);
  // the row stays in registers as loaded (16 bytes per vector), unpacked on
  // use; columns >= V (padding, and vectors past the row) are set to -inf
  // once, as loaded, so no pass tests them again
  uint4 raw[NCH];
  auto unpack = [&](int q, float* x) { Vec16<T>::load(reinterpret_cast<const T*>(&raw[q]), x); };
  float m = -INFINITY, s = 0.f;
  if (valid) {
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int v = threadIdx.x + q * BT;
      uint4 u = v < nvec ? ld_nt16(zr + (long)v * NV) : make_uint4(0, 0, 0, 0);
      const int lim = V - v * NV;  // elements of this vector below column V
      uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (NV == 8) {  // two 16-bit values per word, low first
          constexpr uint32_t ninf = sizeof(T) == 2 && std::is_same<T, bf16>::value ? 0xff80u : 0xfc00u;
          if (2 * k + 1 >= lim) wd[k] = (wd[k] & 0xffffu) | (ninf << 16);
          if (2 * k >= lim) wd[k] = (ninf << 16) | ninf;
        } else {
          if (k >= lim) wd[k] = 0xff800000u;
        }
      }
      raw[q] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      float x[NV];
      unpack(q, x);
#pragma unroll
      for (int i = 0; i < NV; ++i) m = fmaxf(m, x[i]);
    }
  }
  // the row maximum, then the sum of exp(z - max), each over the wavefront
  // (register reductions) and then over the 16 wavefronts in order
  const int w = threadIdx.x >> 6;
  const float mw = wave_max(m);
  // (the unpacked values are not kept from the first pass: that would hold
  // the whole row twice in registers)
#pragma unroll
  for (int q = 0; q < NCH; ++q) asm volatile("" : "+v"(raw[q].x), "+v"(raw[q].y), "+v"(raw[q].z), "+v"(raw[q].w));
  if (valid && mw != -INFINITY) {
    const float c = -mw * kL2e;
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      float x[NV];
      unpack(q, x);
#pragma unroll
      for (int i = 0; i < NV; ++i) s += __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], kL2e, c));
    }
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) {
    s_m[w] = mw;
    s_s[w] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = s_m[0], ss = s_s[0];
    for (int q = 1; q < NW; ++q) merge_ms(mm, ss, s_m[q], s_s[q]);
    const float lse = mm + __logf(ss);
    s_lse = lse;
    row_loss[row] = valid ? lse - Act<T>::ld(zr, t) : 0.f;
  }
  __syncthreads();  // z[t] has been read before it is overwritten
  const float lse = s_lse;
  const int n = *n_valid;
  const float inv_n = n > 0 ? 1.0f / (float)n : 0.f;
  const float scale = loss_scale ? *loss_scale : 1.0f;
  // dz = exp(z - lse) / N = exp2(z log2(e) - (lse log2(e) - log2(1/N))) (no
  // valid row: exp2(-inf) = 0), then times the loss scale as a separate
  // product, so a power-of-two scale changes the bits by exactly that power
  const float c = -(lse * kL2e - __log2f(inv_n));
  // the thread, chunk and element that hold the target column
  const int vt = valid ? t / NV : -1;
  const int t_thread = vt % BT, t_chunk = vt / BT, t_elem = valid ? t - vt * NV : 0;
#pragma unroll
  for (int q = 0; q < NCH; ++q) {
    const int v = threadIdx.x + q * BT;
    if (v >= nvec) continue;
    float x[NV];
    if (valid) {
      unpack(q, x);
#pragma unroll
      for (int i = 0; i < NV; ++i) x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], kL2e, c));
      if (q == t_chunk && (int)threadIdx.x == t_thread) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (i == t_elem) x[i] -= inv_n;
      }
      if (scale != 1.0f) {
#pragma unroll
        for (int i = 0; i < NV; ++i) x[i] *= scale;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i) x[i] = 0.f;
    }
    Vec16<T>::store_nt(zr + (long)v * NV, x);
  }
}

template <typename T>
void launch_xent(T* z, long ldz, int M, int V, const int32_t* tgt, const int32_t* n_valid, float* row_loss,
                 const float* loss_scale, hipStream_t s) {
  const long nvec = ldz / Vec16<T>::N;
#define XENT_REG(N, BT)                                                                                       \
  if ((nvec + BT - 1) / BT <= N) {                                                                            \
    hipLaunchKernelGGL((xent_reg_kernel<T, N, BT>), dim3(M), dim3(BT), 0, s, z, ldz, V, tgt, n_valid, loss_scale, \
                       row_loss);                                                                                   \
    return;                                                                                                   \
  }
  if (nvec <= 64 * 8) {
    XENT_REG(1, 64) XENT_REG(2, 64) XENT_REG(4, 64) XENT_REG(8, 64)
  }
  if (nvec <= 256 * 8) {
    XENT_REG(1, 256) XENT_REG(2, 256) XENT_REG(4, 256) XENT_REG(8, 256)
  }
  XENT_REG(1, 1024) XENT_REG(2, 1024) XENT_REG(4, 1024) XENT_REG(8, 1024)
#undef XENT_REG
  hipLaunchKernelGGL(xent_kernel<T>, dim3(M), dim3(256), 0, s, z, ldz, V, tgt, n_valid, loss_scale, row_loss);
}
template void launch_xent<float>(float*, long, int, int, const int32_t*, const int32_t*, float*, const float*,
                                 hipStream_t);
template void launch_xent<bf16>(bf16*, long, int, int, const int32_t*, const int32_t*, float*, const float*,
                                hipStream_t);
template void launch_xent<f16>(f16*, long, int, int, const int32_t*, const int32_t*, float*, const float*,
                               hipStream_t);

}  // namespace lm
