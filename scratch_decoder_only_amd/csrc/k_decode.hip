// Generation with a key/value cache: each new token's keys and values are
// appended to a per-layer cache, and its query attends to the cached keys of
// its row (causal: every cached position is at or before it). The attention
// of one query per (row, head) is the same operation as the training path's
// (Feste page, "Model Architecture": scores scaled by 1/sqrt(D), softmax,
// weighted sum of values), written here for one query at a time.
//
// Cache layout, per layer: K [B][S][C] then V [B][S][C] in the activation
// type (S = max_seq, C = d_model, head h at columns h*D .. h*D+D-1).
#include "kernels.h"

namespace lm {

namespace {

// cache rows (b, t0 .. t0+T-1) of layer l's K and V from qkv rows [B*T, 3C]
template <typename E>
__global__ void kv_store_kernel(const E* __restrict__ qkv, int B, int T, int C, int S, int t0,
                                E* __restrict__ kc, E* __restrict__ vc, const int32_t* __restrict__ d_pos) {
  if (d_pos) t0 = decode_pos(d_pos, S);
  const long r = blockIdx.x;  // b * T + t
  const int b = (int)(r / T), t = (int)(r % T);
  if (t0 + t >= S) return;
  const E* src = qkv + r * 3L * C;
  E* dk = kc + ((long)b * S + t0 + t) * C;
  E* dv = vc + ((long)b * S + t0 + t) * C;
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    dk[c] = src[C + c];
    dv[c] = src[2 * C + c];
  }
}

// One block per (row b, head h): query = qkv[b][h*D ..], keys/values 0 .. n-1
// of the cache. The block's scores, then their exponentials, sit in its own
// row of the global scratch sbuf (n <= S floats); fixed-order reductions;
// o[b][h*D + d] in the activation type.
template <typename T, int D>
__global__ void __launch_bounds__(256) attn_decode_kernel(const T* __restrict__ qkv, const T* __restrict__ kc,
                                                          const T* __restrict__ vc, int H, int S, int n,
                                                          T* __restrict__ o, float* __restrict__ sbuf,
                                                          const int32_t* __restrict__ d_pos) {
  if (d_pos) n = decode_pos(d_pos, S) + 1;
  constexpr int NT = 256;
  __shared__ float s_q[D];
  __shared__ float s_red[NT / 64];
  __shared__ float s_part[NT / D][D];
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int C = H * D, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float* sc = sbuf + (long)blockIdx.x * S;  // this block's scores
  if (tid < D) s_q[tid] = Act<T>::ld(qkv, (long)b * 3 * C + h * D + tid);
  __syncthreads();
  const float scale = 1.0f / sqrtf((float)D);
  const T* kb = kc + (long)b * S * C + h * D;
  const T* vb = vc + (long)b * S * C + h * D;
  // scores and their maximum
  float mx = -INFINITY;
  for (int j = tid; j < n; j += NT) {
    float acc = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) acc += s_q[d] * Act<T>::ld(kb, (long)j * C + d);
    acc *= scale;
    sc[j] = acc;
    mx = fmaxf(mx, acc);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) s_red[w] = mx;
  __syncthreads();
  mx = s_red[0];
  for (int q = 1; q < NT / 64; ++q) mx = fmaxf(mx, s_red[q]);
  __syncthreads();
  // exponentials and their sum (per thread in key order, then the block in order)
  float sum = 0.f;
  for (int j = tid; j < n; j += NT) {
    const float p = __expf(sc[j] - mx);
    sc[j] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  if (lane == 0) s_red[w] = sum;
  __syncthreads();
  sum = 0.f;
  for (int q = 0; q < NT / 64; ++q) sum += s_red[q];
  // o[d] = sum_j p_j v_j[d] / sum: thread (g, d) takes keys g, g + NT/D, ...
  const int d = tid % D, g = tid / D;
  float acc = 0.f;
  for (int j = g; j < n; j += NT / D) acc += sc[j] * Act<T>::ld(vb, (long)j * C + d);
  s_part[g][d] = acc;
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
    for (int q = 0; q < NT / D; ++q) t += s_part[q][tid];
    Act<T>::st(o, (long)b * C + h * D + tid, t / sum);
  }
}

}  // namespace

// 16-bit operands: the same operation with 16-byte accesses. A key's D
// values are split over LK = D/8 lanes (8 each), so a wavefront covers KPI =
// 64/LK keys per load; the dot products are finished with a shuffle tree over
// those LK lanes, and the weighted values are summed per lane over its keys,
// then over the lanes holding the same 8 columns (shuffles), then over the
// four wavefronts in order.
template <typename T, int D>
__global__ void __launch_bounds__(256) attn_decode16_kernel(const T* __restrict__ qkv, const T* __restrict__ kc,
                                                            const T* __restrict__ vc, int H, int S, int n,
                                                            T* __restrict__ o, float* __restrict__ sbuf,
                                                            const int32_t* __restrict__ d_pos) {
  if (d_pos) n = decode_pos(d_pos, S) + 1;
  constexpr int NT = 256, LK = D / 8, KPI = 64 / LK, KPB = KPI * (NT / 64);
  __shared__ float s_red[NT / 64];
  __shared__ float s_part[NT / 64][D];
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int C = H * D, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c8 = (lane % LK) * 8, kl = lane / LK;  // this lane's 8 columns and key slot
  float* sc = sbuf + (long)blockIdx.x * S;
  float q[8];
  {
    const uint4 u = *reinterpret_cast<const uint4*>(qkv + (long)b * 3 * C + h * D + c8);
    const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[2 * i] = H16<T>::lo(wv[i]);
      q[2 * i + 1] = H16<T>::hi(wv[i]);
    }
  }
  const float scale = 1.0f / sqrtf((float)D);
  const T* kb = kc + (long)b * S * C + h * D + c8;
  const T* vb = vc + (long)b * S * C + h * D + c8;
  // scores and their maximum
  float mx = -INFINITY;
  for (int j0 = w * KPI; j0 < n; j0 += KPB) {
    const int j = j0 + kl;
    float acc = 0.f;
    if (j < n) {
      const uint4 u = *reinterpret_cast<const uint4*>(kb + (long)j * C);
      const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = __builtin_fmaf(q[2 * i], H16<T>::lo(wv[i]), acc);
        acc = __builtin_fmaf(q[2 * i + 1], H16<T>::hi(wv[i]), acc);
      }
    }
#pragma unroll
    for (int off = 1; off < LK; off <<= 1) acc += __shfl_xor(acc, off, 64);
    acc *= scale;
    if (j < n) {
      if (lane % LK == 0) sc[j] = acc;
      mx = fmaxf(mx, acc);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) s_red[w] = mx;
  __syncthreads();  // (also orders the score stores before the reads below)
  mx = s_red[0];
  for (int qq = 1; qq < NT / 64; ++qq) mx = fmaxf(mx, s_red[qq]);
  __syncthreads();
  // exponentials and their sum (per thread in key order, then the block in order)
  float sum = 0.f;
  for (int j = tid; j < n; j += NT) {
    const float pv = __expf(sc[j] - mx);
    sc[j] = pv;
    sum += pv;
  }
  sum = wave_sum(sum);
  if (lane == 0) s_red[w] = sum;
  __syncthreads();
  sum = 0.f;
  for (int qq = 0; qq < NT / 64; ++qq) sum += s_red[qq];
  // o = sum_j p_j v_j / sum
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j0 = w * KPI; j0 < n; j0 += KPB) {
    const int j = j0 + kl;
    if (j < n) {
      const float pv = sc[j];
      const uint4 u = *reinterpret_cast<const uint4*>(vb + (long)j * C);
      const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(pv, H16<T>::lo(wv[i]), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(pv, H16<T>::hi(wv[i]), acc[2 * i + 1]);
      }
    }
  }
#pragma unroll
  for (int off = LK; off < 64; off <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], off, 64);
  if (kl == 0)
#pragma unroll
    for (int i = 0; i < 8; ++i) s_part[w][c8 + i] = acc[i];
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
    for (int qq = 0; qq < NT / 64; ++qq) t += s_part[qq][tid];
    Act<T>::st(o, (long)b * C + h * D + tid, t / sum);
  }
}

template <typename E>
void launch_kv_store(const E* qkv, int B, int T_, int C, int S, int t0, E* kc, E* vc, hipStream_t s,
                     const int32_t* d_pos) {
  hipLaunchKernelGGL(kv_store_kernel<E>, dim3(B * T_), dim3(256), 0, s, qkv, B, T_, C, S, t0, kc, vc, d_pos);
}
template void launch_kv_store<float>(const float*, int, int, int, int, int, float*, float*, hipStream_t,
                                     const int32_t*);
template void launch_kv_store<bf16>(const bf16*, int, int, int, int, int, bf16*, bf16*, hipStream_t, const int32_t*);
template void launch_kv_store<f16>(const f16*, int, int, int, int, int, f16*, f16*, hipStream_t, const int32_t*);

__global__ void fill_pos_kernel(int32_t* __restrict__ dst, const int32_t* __restrict__ d_pos, int S, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = decode_pos(d_pos, S);
}
void launch_fill_pos(int32_t* dst, const int32_t* d_pos, int S, long n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(fill_pos_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, d_pos, S, n);
}

template <typename T>
int launch_attn_decode(const T* qkv, const T* kc, const T* vc, int B, int H, int D, int S, int n, T* o, float* sbuf,
                       hipStream_t s, const int32_t* d_pos) {
  if (D != 64 && D != 32) return -1;
  if constexpr (sizeof(T) == 2) {
    if (D == 64)
      hipLaunchKernelGGL((attn_decode16_kernel<T, 64>), dim3(B * H), dim3(256), 0, s, qkv, kc, vc, H, S, n, o, sbuf,
                         d_pos);
    else
      hipLaunchKernelGGL((attn_decode16_kernel<T, 32>), dim3(B * H), dim3(256), 0, s, qkv, kc, vc, H, S, n, o, sbuf,
                         d_pos);
  } else {
    if (D == 64)
      hipLaunchKernelGGL((attn_decode_kernel<T, 64>), dim3(B * H), dim3(256), 0, s, qkv, kc, vc, H, S, n, o, sbuf,
                         d_pos);
    else
      hipLaunchKernelGGL((attn_decode_kernel<T, 32>), dim3(B * H), dim3(256), 0, s, qkv, kc, vc, H, S, n, o, sbuf,
                         d_pos);
  }
  return 0;
}
template int launch_attn_decode<float>(const float*, const float*, const float*, int, int, int, int, int, float*,
                                       float*, hipStream_t, const int32_t*);
template int launch_attn_decode<bf16>(const bf16*, const bf16*, const bf16*, int, int, int, int, int, bf16*, float*,
                                      hipStream_t, const int32_t*);
template int launch_attn_decode<f16>(const f16*, const f16*, const f16*, int, int, int, int, int, f16*, float*,
                                     hipStream_t, const int32_t*);

}  // namespace lm
