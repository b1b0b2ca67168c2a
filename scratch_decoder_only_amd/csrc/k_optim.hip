// Global gradient-norm clip and AdamW (Feste page, "Manual Backpropagation":
// AdamW with weight decay kept out of the gradient, and clipping against
// exploding gradients; RustGPT page: clip to an L2 norm of 5.0).
//
// n = ||g||_2 over the whole flat gradient buffer (fixed-order two-stage
// reduction in double), s = clip / n if n > clip else 1. Then per element,
// with gh = s g and a 1-based step t:
//   m = b1 m + (1 - b1) gh;  v = b2 v + (1 - b2) gh^2
//   p = p - lr (m / (1 - b1^t) / (sqrt(v / (1 - b2^t)) + eps) + wd p)
// and the 16-bit operand copy of p is refreshed in the same pass. A non-finite
// norm skips the update entirely (flags bit 0).
//
// fp16 training scales the loss by S (a power of two) before the backward
// (LucilleAI page: FP16 autocast with a GradScaler), so the buffer holds S g:
// the norm is taken of S g and divided by S, the clip factor comes from the
// true norm, and AdamW multiplies by (clip factor) / S. The scale then
// follows the usual dynamic rule: a non-finite norm (an overflow somewhere)
// skips the step and multiplies S by the backoff factor; after `interval`
// finite steps in a row S is multiplied by the growth factor.
#include "kernels.h"

namespace lm {

// Four 16-byte chunks per thread and iteration, nontemporal loads (one
// streaming read of the gradients), then the chunks added in index order.
__global__ void __launch_bounds__(256) sumsq_kernel(const float* __restrict__ g, long n, double* __restrict__ part) {
  __shared__ double s[256];
  double acc = 0.0;
  const long n4 = n / 4;
  const f32x4_t* g4 = reinterpret_cast<const f32x4_t*>(g);
  const long stride = (long)gridDim.x * 256;
  long i = (long)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    f32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(g4 + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc += (double)v[u][0] * v[u][0] + (double)v[u][1] * v[u][1] + (double)v[u][2] * v[u][2] +
             (double)v[u][3] * v[u][3];
  }
  for (; i < n4; i += stride) {
    const f32x4_t v = __builtin_nontemporal_load(g4 + i);
    acc += (double)v[0] * v[0] + (double)v[1] * v[1] + (double)v[2] * v[2] + (double)v[3] * v[3];
  }
  for (long i = n4 * 4 + (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256)
    acc += (double)g[i] * g[i];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = s[0];
}

void launch_sumsq_partials(const float* g, long n, double* part, hipStream_t s) {
  hipLaunchKernelGGL(sumsq_kernel, dim3(kNormBlocks), dim3(256), 0, s, g, n, part);
}

__global__ void __launch_bounds__(256) norm_finalize_kernel(const double* __restrict__ part, float clip,
                                                            float* __restrict__ norm_scale,
                                                            uint32_t* __restrict__ flags, float* __restrict__ stats,
                                                            LossScaler ls) {
  __shared__ double s[256];
  double acc = 0.0;
  for (int i = threadIdx.x; i < kNormBlocks; i += 256) acc += part[i];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double S = ls.state ? (double)ls.state[0] : 1.0;
    double n = sqrt(s[0]) / S;
    bool finite = isfinite(n);
    double sc = (finite && clip > 0.f && n > (double)clip) ? (double)clip / n : 1.0;
    norm_scale[0] = (float)n;
    norm_scale[1] = (float)(sc / S);
    if (!finite) atomicOr(flags, 1u);
    if (stats) stats[1] = (float)n;
    if (ls.state) {
      if (!finite) {
        ls.state[0] = (float)(S * (double)ls.backoff);
        ls.state[1] = 0.f;
      } else if (ls.state[1] + 1.f >= (float)ls.interval) {
        ls.state[0] = (float)(S * (double)ls.growth);
        ls.state[1] = 0.f;
      } else {
        ls.state[1] += 1.f;
      }
    }
  }
}

void launch_norm_finalize(const double* part, float clip, float* norm_scale, uint32_t* flags, float* stats,
                          LossScaler ls, hipStream_t s) {
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(1), dim3(256), 0, s, part, clip, norm_scale, flags, stats, ls);
}

// rb1, rb2: 1 / (1 - beta^t), computed once per thread; the per-element
// division by sqrt(v_hat) + eps uses the hardware reciprocal (about 1 ulp).
__device__ __forceinline__ void adam_one(float& p, float g, float& m, float& v, const AdamArgs& a, float sc,
                                         float rb1, float rb2) {
  const float gh = sc * g;
  m = a.beta1 * m + (1.0f - a.beta1) * gh;
  v = a.beta2 * v + (1.0f - a.beta2) * gh * gh;
  const float mh = m * rb1, vh = v * rb2;
  p = p - a.lr * (mh * __builtin_amdgcn_rcpf(sqrtf(vh) + a.eps) + a.wd * p);
}

// One 4-parameter chunk per thread and no grid-stride loop, with
// nontemporal loads and stores: the update streams 30 bytes per parameter
// through once, and measured on the device this shape keeps more loads in
// flight than a capped grid looping over the array (about 5.9 against 4.5
// TB/s for this 4-read, 3-write pattern).
__global__ void __launch_bounds__(256) adamw_kernel(AdamArgs a) {
  if (*a.flags & 1u) return;  // non-finite gradient norm: leave everything as it was
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.n / 4) return;
  const float sc = a.norm_scale[1];
  const float rb1 = 1.0f / a.bc1, rb2 = 1.0f / a.bc2;
  f32x4_t* pp = reinterpret_cast<f32x4_t*>(a.p) + i;
  f32x4_t* mp = reinterpret_cast<f32x4_t*>(a.m) + i;
  f32x4_t* vp = reinterpret_cast<f32x4_t*>(a.v) + i;
  f32x4_t p = __builtin_nontemporal_load(pp);
  const f32x4_t g = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(a.g) + i);
  f32x4_t m = __builtin_nontemporal_load(mp);
  f32x4_t v = __builtin_nontemporal_load(vp);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float pe = p[e], me = m[e], ve = v[e];
    adam_one(pe, g[e], me, ve, a, sc, rb1, rb2);
    p[e] = pe;
    m[e] = me;
    v[e] = ve;
  }
  __builtin_nontemporal_store(p, pp);
  __builtin_nontemporal_store(m, mp);
  __builtin_nontemporal_store(v, vp);
  if (a.shadow) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t w = a.shadow_f16 ? u32x2_t{H16<f16>::pack(p[0], p[1]), H16<f16>::pack(p[2], p[3])}
                                   : u32x2_t{H16<bf16>::pack(p[0], p[1]), H16<bf16>::pack(p[2], p[3])};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(a.shadow + i * 4));
  }
}

void launch_adamw(const AdamArgs& a, hipStream_t s) {
  const long n4 = a.n / 4;
  const long blocks = n4 > 0 ? (n4 + 255) / 256 : 1;
  hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
}

__global__ void make_shadow_kernel(const float* __restrict__ p, long n, uint16_t* __restrict__ shadow, int to_f16) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256)
    shadow[i] = (uint16_t)(to_f16 ? H16<f16>::bits(p[i]) : H16<bf16>::bits(p[i]));
}

void launch_make_shadow(const float* p, long n, uint16_t* shadow, bool to_f16, hipStream_t s) {
  long blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(make_shadow_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, shadow, to_f16 ? 1 : 0);
}

}  // namespace lm
