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

__global__ void __launch_bounds__(256) sumsq_kernel(const float* __restrict__ g, long n, double* __restrict__ part) {
  __shared__ double s[256];
  double acc = 0.0;
  const long n4 = n / 4;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
    float4 v = g4[i];
    acc += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
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

__global__ void __launch_bounds__(256) adamw_kernel(AdamArgs a) {
  if (*a.flags & 1u) return;  // non-finite gradient norm: leave everything as it was
  const float sc = a.norm_scale[1];
  const float rb1 = 1.0f / a.bc1, rb2 = 1.0f / a.bc2;
  const long n4 = a.n / 4;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
    float4 p = reinterpret_cast<float4*>(a.p)[i];
    float4 g = reinterpret_cast<const float4*>(a.g)[i];
    float4 m = reinterpret_cast<float4*>(a.m)[i];
    float4 v = reinterpret_cast<float4*>(a.v)[i];
    adam_one(p.x, g.x, m.x, v.x, a, sc, rb1, rb2);
    adam_one(p.y, g.y, m.y, v.y, a, sc, rb1, rb2);
    adam_one(p.z, g.z, m.z, v.z, a, sc, rb1, rb2);
    adam_one(p.w, g.w, m.w, v.w, a, sc, rb1, rb2);
    reinterpret_cast<float4*>(a.p)[i] = p;
    reinterpret_cast<float4*>(a.m)[i] = m;
    reinterpret_cast<float4*>(a.v)[i] = v;
    if (a.shadow) {
      const uint2 w = a.shadow_f16 ? make_uint2(H16<f16>::pack(p.x, p.y), H16<f16>::pack(p.z, p.w))
                                   : make_uint2(H16<bf16>::pack(p.x, p.y), H16<bf16>::pack(p.z, p.w));
      *reinterpret_cast<uint2*>(a.shadow + i * 4) = w;
    }
  }
}

void launch_adamw(const AdamArgs& a, hipStream_t s) {
  long n4 = a.n / 4;
  long blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
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
