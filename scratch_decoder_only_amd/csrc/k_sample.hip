// Next-token choice for generation (RustGPT page, technical list: greedy
// decoding for text generation; LucilleAI page: a sampler with temperature
// and top-k). One block of 1024 threads per row of logits.
//
// Greedy (temperature <= 0): the largest logit, ties to the smallest id.
// Sampling: the top_k largest logits (ties at the k-th value to the smaller
// ids), weights exp((z - z_max) / temperature), and the caller's uniform u
// picks the first id, in ascending id order, at which the running weight sum
// reaches u * total. Every reduction and scan has a fixed order, so the choice
// is a function of the inputs.
#include "kernels.h"

namespace lm {

namespace {

constexpr int kSampleThreads = 1024;

// Order-preserving map of an fp32 value to uint32 (larger value, larger key).
__device__ __forceinline__ uint32_t fkey(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive block scan of a float in thread order (fixed tree), returns the
// thread's inclusive prefix; *total receives the block total.
__device__ float block_scan_float(float v, float* red, float* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) red[w] = x;
  __syncthreads();
  float before = 0.f, t = 0.f;
  for (int i = 0; i < kSampleThreads / 64; ++i) {
    if (i < w) before += red[i];
    t += red[i];
  }
  *total = t;
  return before + x;
}

__global__ void __launch_bounds__(kSampleThreads) sample_kernel(const float* __restrict__ logits, int V, long ld,
                                                                float temperature, int top_k,
                                                                const float* __restrict__ uniforms,
                                                                int32_t* __restrict__ out) {
  __shared__ int s_hist[256];
  __shared__ int s_red[kSampleThreads / 64];
  __shared__ float s_fred[kSampleThreads / 64];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  __shared__ unsigned long long s_best;
  __shared__ int s_pick, s_last;
  const float* z = logits + (long)blockIdx.x * ld;
  const int tid = threadIdx.x;

  // ---- maximum (value, smallest id): key (fkey(z) << 32) | (0xffffffff - id)
  unsigned long long best = 0;
  for (int i = tid; i < V; i += kSampleThreads) {
    const unsigned long long k = ((unsigned long long)fkey(z[i]) << 32) | (0xffffffffu - (uint32_t)i);
    best = k > best ? k : best;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long y = __shfl_xor(best, o, 64);
    best = y > best ? y : best;
  }
  if (tid == 0) s_best = 0;
  __syncthreads();
  if ((tid & 63) == 0) atomicMax(&s_best, best);  // integer max: order-free
  __syncthreads();
  const int arg = (int)(0xffffffffu - (uint32_t)(s_best & 0xffffffffu));
  if (!(temperature > 0.f)) {
    if (tid == 0) out[blockIdx.x] = arg;
    return;
  }
  const float zmax = z[arg];
  const int k = (top_k <= 0 || top_k >= V) ? V : top_k;

  // ---- k-th largest value tau by radix selection over fkey (8 bits a pass);
  // afterwards s_need = how many of the ids with value tau are kept
  uint32_t prefix = 0;
  int need = k;
  if (k < V) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSampleThreads) s_hist[i] = 0;
      __syncthreads();
      const uint32_t hi_mask = shift == 24 ? 0u : (0xffffffffu << (shift + 8));
      for (int i = tid; i < V; i += kSampleThreads) {
        const uint32_t key = fkey(z[i]);
        if ((key & hi_mask) == (prefix & hi_mask)) atomicAdd(&s_hist[(key >> shift) & 255], 1);
      }
      __syncthreads();
      if (tid == 0) {
        // walk bins from the largest down until the running count reaches need
        int acc = 0, b = 255;
        for (; b > 0; --b) {
          if (acc + s_hist[b] >= need) break;
          acc += s_hist[b];
        }
        s_prefix = prefix | ((uint32_t)b << shift);
        s_need = need - acc;
      }
      __syncthreads();
      prefix = s_prefix;
      need = s_need;
    }
  }
  const uint32_t tau = prefix;

  // ---- weights and the pick: ids in ascending order, chunk by chunk; an id
  // is kept when fkey > tau, or fkey == tau and it is among the first `need`
  // such ids (k == V keeps every id)
  const float inv_t = 1.0f / temperature;
  auto weight = [&](int i, int eq_rank) -> float {
    if (i >= V) return 0.f;
    const uint32_t key = fkey(z[i]);
    const bool keep = k == V || key > tau || (key == tau && eq_rank < need);
    return keep ? __expf((z[i] - zmax) * inv_t) : 0.f;
  };
  // pass 1: total weight (same chunk order and tree as pass 2)
  float total = 0.f;
  int eq_base = 0;
  for (int c0 = 0; c0 < V; c0 += kSampleThreads) {
    const int i = c0 + tid;
    const int is_eq = (k < V && i < V && fkey(z[i]) == tau) ? 1 : 0;
    // rank of this id among the equal ones: exclusive prefix over the chunk
    int x = is_eq;
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == 63) s_red[w] = x;
    __syncthreads();
    int before = 0, ctot = 0;
    for (int q = 0; q < kSampleThreads / 64; ++q) {
      if (q < w) before += s_red[q];
      ctot += s_red[q];
    }
    const float wv = weight(i, eq_base + before + x - is_eq);
    float ct;
    block_scan_float(wv, s_fred, &ct);
    total += ct;
    eq_base += ctot;
  }
  const float target = uniforms[blockIdx.x] * total;
  // pass 2: the smallest kept id whose inclusive running sum reaches the
  // target (the running sums grow with the id, so that id is unique)
  if (tid == 0) {
    s_pick = 0x7fffffff;
    s_last = -1;
  }
  float run = 0.f;
  eq_base = 0;
  int last_kept = -1;
  for (int c0 = 0; c0 < V; c0 += kSampleThreads) {
    const int i = c0 + tid;
    const int is_eq = (k < V && i < V && fkey(z[i]) == tau) ? 1 : 0;
    int x = is_eq;
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == 63) s_red[w] = x;
    __syncthreads();
    int before = 0, ctot = 0;
    for (int q = 0; q < kSampleThreads / 64; ++q) {
      if (q < w) before += s_red[q];
      ctot += s_red[q];
    }
    const float wv = weight(i, eq_base + before + x - is_eq);
    float ct;
    const float incl = run + block_scan_float(wv, s_fred, &ct);
    if (wv > 0.f) {
      last_kept = i;
      if (incl >= target) atomicMin(&s_pick, i);  // integer min: order-free
    }
    __syncthreads();
    if (s_pick != 0x7fffffff) break;  // block-uniform
    run += ct;
    eq_base += ctot;
  }
  // rounding can leave the target above the final sum: then the last kept id
  if (last_kept >= 0) atomicMax(&s_last, last_kept);
  __syncthreads();
  if (tid == 0) out[blockIdx.x] = s_pick != 0x7fffffff ? s_pick : s_last;
}

}  // namespace

void launch_sample(const float* logits, int rows, int V, long ld, float temperature, int top_k, const float* u,
                   int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(sample_kernel, dim3(rows), dim3(kSampleThreads), 0, s, logits, V, ld, temperature, top_k, u,
                     out);
}

}  // namespace lm
