// Row-wise kernels of the step: fills, the packed-row index layout, the
// embedding gather, the valid-target count, and the loss reduction.
#include "kernels.h"

namespace lm {

// ---------------------------------------------------------------- fills
// A plain fill kernel (also used where a graph may capture the step).
__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, long n) {
  long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  long stride = (long)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

void launch_fill_u32(uint32_t* p, uint32_t v, long n, hipStream_t s) {
  if (n <= 0) return;
  long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, v, n);
}

// -------------------------------------------------------------- index layout
// Packed rows (several documents per row): a document is a maximal run of
// equal doc ids. start[t] = first index of t's run, end[t] = one past its last
// index, pos[t] = t - start[t]. Without doc ids: start = 0, end = T, pos = t.
// One block per row; block-wide max-scan (start) and min-scan (end) over the
// boundary indices. Sets flags bit 1 if doc ids decrease.
__global__ void __launch_bounds__(256) index_layout_kernel(const int32_t* __restrict__ doc, int T,
                                                           int32_t* __restrict__ start,
                                                           int32_t* __restrict__ end,
                                                           int32_t* __restrict__ pos,
                                                           uint32_t* __restrict__ flags) {
  __shared__ int s_max[256];
  __shared__ int s_min[256];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int per = (T + 255) / 256;
  const int t0 = tid * per, t1 = min(T, t0 + per);
  const int32_t* d = doc ? doc + (long)b * T : nullptr;
  // local reductions of boundary indices within this thread's chunk
  int lmax = 0, lmin = T;
  bool bad = false;
  for (int t = t0; t < t1; ++t) {
    if (d && t > 0 && d[t] != d[t - 1]) {
      lmax = t;
      lmin = min(lmin, t);
      if (d[t] < d[t - 1]) bad = true;
    }
  }
  s_max[tid] = lmax;
  s_min[tid] = lmin;
  __syncthreads();
  // prefix max over preceding chunks, suffix min over following chunks
  int pmax = 0, smin = T;
  for (int j = 0; j < tid; ++j) pmax = max(pmax, s_max[j]);
  for (int j = tid + 1; j < 256; ++j) smin = min(smin, s_min[j]);
  // end[t]: first boundary > t, scanning this chunk backwards
  int run_min = smin;
  for (int t = t1 - 1; t >= t0; --t) {
    long o = (long)b * T + t;
    end[o] = run_min;
    if (d && t > 0 && d[t] != d[t - 1]) run_min = t;
  }
  int run_max = pmax;
  for (int t = t0; t < t1; ++t) {
    if (d && t > 0 && d[t] != d[t - 1]) run_max = t;
    long o = (long)b * T + t;
    start[o] = run_max;
    pos[o] = t - run_max;
  }
  if (bad) atomicOr(flags, 2u);
}

void launch_index_layout(const int32_t* doc, int B, int T, int32_t* start, int32_t* end, int32_t* pos,
                         uint32_t* flags, hipStream_t s) {
  hipLaunchKernelGGL(index_layout_kernel, dim3(B), dim3(256), 0, s, doc, T, start, end, pos, flags);
}

// ------------------------------------------------------------ embedding fwd
// x[m, :] = wte[tok[m], :] + wpe[pos[m], :] (fp32 master rows). One wave per
// row, float2 per lane per step. Out-of-range tokens are clamped and flagged.
__global__ void __launch_bounds__(256) embed_fwd_kernel(const int32_t* __restrict__ tok,
                                                        const int32_t* __restrict__ pos,
                                                        const float* __restrict__ wte,
                                                        const float* __restrict__ wpe, int M, int C,
                                                        int V, float* __restrict__ x,
                                                        uint32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const long m = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  int t = tok[m];
  if (t < 0 || t >= V) {
    if (lane == 0) atomicOr(flags, 2u);
    t = t < 0 ? 0 : V - 1;
  }
  const float2* a = reinterpret_cast<const float2*>(wte + (long)t * C);
  const float2* p = reinterpret_cast<const float2*>(wpe + (long)pos[m] * C);
  float2* o = reinterpret_cast<float2*>(x + m * C);
  for (int j = lane; j < C / 2; j += 64) {
    float2 u = a[j], v = p[j];
    o[j] = make_float2(u.x + v.x, u.y + v.y);
  }
}

void launch_embed_fwd(const int32_t* tok, const int32_t* pos, const float* wte, const float* wpe, int M,
                      int C, int V, float* x, uint32_t* flags, hipStream_t s) {
  hipLaunchKernelGGL(embed_fwd_kernel, dim3((M + 3) / 4), dim3(256), 0, s, tok, pos, wte, wpe, M, C, V,
                     x, flags);
}

// ----------------------------------------------------- valid-target count
// n_valid = #{m : tgt[m] >= 0}; targets >= V are flagged and ignored.
// One block; writes an int (for the kernels) and its float (for the stats).
__global__ void __launch_bounds__(1024) count_valid_kernel(const int32_t* __restrict__ tgt, int M, int V,
                                                           int32_t* __restrict__ n_out,
                                                           float* __restrict__ stats,
                                                           uint32_t* __restrict__ flags) {
  __shared__ int s[1024];
  int c = 0;
  bool bad = false;
  for (int m = threadIdx.x; m < M; m += 1024) {
    int t = tgt[m];
    if (t >= V || t < -1) bad = true;
    if (t >= 0 && t < V) ++c;
  }
  s[threadIdx.x] = c;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
    __syncthreads();
  }
  if (bad) atomicOr(flags, 2u);
  if (threadIdx.x == 0) {
    *n_out = s[0];
    if (stats) stats[3] = (float)s[0];
  }
}

void launch_count_valid(const int32_t* tgt, int M, int V, int32_t* n_out, float* stats, uint32_t* flags,
                        hipStream_t s) {
  hipLaunchKernelGGL(count_valid_kernel, dim3(1), dim3(1024), 0, s, tgt, M, V, n_out, stats, flags);
}

// ------------------------------------------------------------ loss reduce
// loss = (sum over rows of row_loss) / n, summed in a fixed order (double).
__global__ void __launch_bounds__(1024) loss_reduce_kernel(const float* __restrict__ row_loss, int M,
                                                           const int32_t* __restrict__ n_valid,
                                                           float* __restrict__ out) {
  __shared__ double s[1024];
  double acc = 0.0;
  for (int m = threadIdx.x; m < M; m += 1024) acc += (double)row_loss[m];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int n = *n_valid;
    out[0] = n > 0 ? (float)(s[0] / (double)n) : 0.0f;
  }
}

void launch_loss_reduce(const float* row_loss, int M, const int32_t* n_valid, float* out, hipStream_t s) {
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(1024), 0, s, row_loss, M, n_valid, out);
}

// ---------------------------------------------------------- flags to stats
__global__ void write_flags_kernel(const uint32_t* flags, float* stats) { stats[2] = (float)(*flags); }

void launch_write_flags(const uint32_t* flags, float* stats, hipStream_t s) {
  hipLaunchKernelGGL(write_flags_kernel, dim3(1), dim3(1), 0, s, flags, stats);
}

// --------------------------------------------------- fp32 -> act conversion
template <typename T>
__global__ void convert_kernel(const float* __restrict__ src, T* __restrict__ dst, long n) {
  long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  long stride = (long)gridDim.x * blockDim.x;
  for (; i < n; i += stride) Act<T>::st(dst, i, src[i]);
}

template <typename T>
void launch_f32_to(const float* src, T* dst, long n, hipStream_t s) {
  if (n <= 0) return;
  long blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(convert_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
}
template void launch_f32_to<bf16>(const float*, bf16*, long, hipStream_t);
template void launch_f32_to<f16>(const float*, f16*, long, hipStream_t);

// Logits of the forward-only call: act [M, ldz] -> fp32 [M, V].
template <typename T>
__global__ void logits_out_kernel(const T* __restrict__ z, long ldz, int M, int V, float* __restrict__ out) {
  long m = blockIdx.y;
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < V; j += gridDim.x * blockDim.x)
    out[m * V + j] = Act<T>::ld(z, m * ldz + j);
}

template <typename T>
void launch_logits_out(const T* z, long ldz, int M, int V, float* out, hipStream_t s) {
  int bx = (V + 255) / 256;
  if (bx > 64) bx = 64;
  hipLaunchKernelGGL(logits_out_kernel<T>, dim3(bx, M), dim3(256), 0, s, z, ldz, M, V, out);
}
template void launch_logits_out<float>(const float*, long, int, int, float*, hipStream_t);
template void launch_logits_out<bf16>(const bf16*, long, int, int, float*, hipStream_t);
template void launch_logits_out<f16>(const f16*, long, int, int, float*, hipStream_t);

}  // namespace lm
