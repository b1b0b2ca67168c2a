// Causal multi-head self-attention, one wavefront per query (or key) row.
//
// Scores s_ij = q_i . k_j / sqrt(D) exist for start(i) <= j <= i (future
// positions and other packed documents are -inf before the softmax: Feste
// page, "Model Architecture"); P = softmax(s); o_i = sum_j P_ij v_j. The
// forward keeps a running max and sum (online softmax) and stores
// lse_i = log sum_j exp(s_ij). The backward (Feste page, "Manual
// Backpropagation") recomputes P_ij = exp(s_ij - lse_i):
//   delta_i = dO_i . O_i, dP_ij = dO_i . v_j, dS_ij = P_ij (dP_ij - delta_i),
//   dq_i = sum_j dS_ij k_j / sqrt(D), dk_j = sum_i dS_ij q_i / sqrt(D),
//   dv_j = sum_i P_ij dO_i.
// Lane d owns dimension d (D <= 64). This is the fp32 path, where the step is
// launch-bound; the bf16 path runs on the matrix cores (k_attn_mfma.hip).
#include "kernels.h"

namespace lm {

constexpr int kRowKeys = 4;  // keys (dK/dV: queries) whose loads go out together

template <typename E>
__global__ void __launch_bounds__(256) attn_fwd_rows_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // over B*H*T
  const int T = a.T, H = a.H, D = a.D, C = H * D;
  if (row >= (long)a.B * H * T) return;
  const int i = row % T, h = (row / T) % H, b = row / ((long)T * H);
  const E* qkv = reinterpret_cast<const E*>(a.qkv);
  const long ld = 3L * C;
  const long base = (long)b * T * ld;
  const bool act = lane < D;
  const float q = act ? Act<E>::ld(qkv, base + (long)i * ld + h * D + lane) : 0.f;
  const float scale = 1.0f / sqrtf((float)D);
  const int j0 = a.start[(long)b * T + i];
  float m = -INFINITY, l = 0.f, o = 0.f;
  auto key = [&](float kv, float vv) {
    float s = wave_sum(q * kv) * scale;
    float mn = fmaxf(m, s);
    float corr = __expf(m - mn);
    float p = __expf(s - mn);
    l = l * corr + p;
    o = o * corr + p * vv;
    m = mn;
  };
  auto kld = [&](int j) { return act ? Act<E>::ld(qkv, base + (long)j * ld + C + h * D + lane) : 0.f; };
  auto vld = [&](int j) { return act ? Act<E>::ld(qkv, base + (long)j * ld + 2 * C + h * D + lane) : 0.f; };
  // keys four at a time with their loads issued together (the row is a chain
  // of dependent updates; loading each key just before its update left a
  // memory latency per key), then the rest one by one, in key order
  int j = j0;
  for (; j + 3 <= i; j += kRowKeys) {
    float kv[kRowKeys], vv[kRowKeys];
#pragma unroll
    for (int u = 0; u < kRowKeys; ++u) {
      kv[u] = kld(j + u);
      vv[u] = vld(j + u);
    }
#pragma unroll
    for (int u = 0; u < kRowKeys; ++u) key(kv[u], vv[u]);
  }
  for (; j <= i; ++j) key(kld(j), vld(j));
  if (act) Act<E>::st(reinterpret_cast<E*>(a.o), ((long)b * T + i) * C + h * D + lane, o / l);
  if (lane == 0) a.lse[((long)b * H + h) * T + i] = m + __logf(l);
}

// delta_i = dO_i . O_i
template <typename E>
__global__ void __launch_bounds__(256) attn_delta_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int T = a.T, H = a.H, D = a.D, C = H * D;
  if (row >= (long)a.B * H * T) return;
  const int i = row % T, h = (row / T) % H, b = row / ((long)T * H);
  const long off = ((long)b * T + i) * C + h * D + lane;
  float v = 0.f;
  if (lane < D)
    v = Act<E>::ld(reinterpret_cast<const E*>(a.dout), off) * Act<E>::ld(reinterpret_cast<const E*>(a.o), off);
  v = wave_sum(v);
  if (lane == 0) a.delta[((long)b * H + h) * T + i] = v;
}

template <typename E>
__global__ void __launch_bounds__(256) attn_dq_rows_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int T = a.T, H = a.H, D = a.D, C = H * D;
  if (row >= (long)a.B * H * T) return;
  const int i = row % T, h = (row / T) % H, b = row / ((long)T * H);
  const E* qkv = reinterpret_cast<const E*>(a.qkv);
  const E* dout = reinterpret_cast<const E*>(a.dout);
  const long ld = 3L * C, base = (long)b * T * ld;
  const bool act = lane < D;
  const float scale = 1.0f / sqrtf((float)D);
  const float q = act ? Act<E>::ld(qkv, base + (long)i * ld + h * D + lane) : 0.f;
  const float g = act ? Act<E>::ld(dout, ((long)b * T + i) * C + h * D + lane) : 0.f;
  const float lse = a.lse[((long)b * H + h) * T + i];
  const float dl = a.delta[((long)b * H + h) * T + i];
  float dq = 0.f;
  auto key = [&](float kv, float vv) {
    float s = wave_sum(q * kv) * scale;
    float dp = wave_sum(g * vv);
    float p = __expf(s - lse);
    dq += p * (dp - dl) * kv;
  };
  auto kld = [&](int j) { return act ? Act<E>::ld(qkv, base + (long)j * ld + C + h * D + lane) : 0.f; };
  auto vld = [&](int j) { return act ? Act<E>::ld(qkv, base + (long)j * ld + 2 * C + h * D + lane) : 0.f; };
  int j = a.start[(long)b * T + i];
  for (; j + 3 <= i; j += kRowKeys) {
    float kv[kRowKeys], vv[kRowKeys];
#pragma unroll
    for (int u = 0; u < kRowKeys; ++u) {
      kv[u] = kld(j + u);
      vv[u] = vld(j + u);
    }
#pragma unroll
    for (int u = 0; u < kRowKeys; ++u) key(kv[u], vv[u]);
  }
  for (; j <= i; ++j) key(kld(j), vld(j));
  if (act) Act<E>::st(reinterpret_cast<E*>(a.dqkv), ((long)b * T + i) * ld + h * D + lane, dq * scale);
}

template <typename E>
__global__ void __launch_bounds__(256) attn_dkv_rows_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int T = a.T, H = a.H, D = a.D, C = H * D;
  if (row >= (long)a.B * H * T) return;
  const int j = row % T, h = (row / T) % H, b = row / ((long)T * H);
  const E* qkv = reinterpret_cast<const E*>(a.qkv);
  const E* dout = reinterpret_cast<const E*>(a.dout);
  const long ld = 3L * C, base = (long)b * T * ld;
  const bool act = lane < D;
  const float scale = 1.0f / sqrtf((float)D);
  const float kv = act ? Act<E>::ld(qkv, base + (long)j * ld + C + h * D + lane) : 0.f;
  const float vv = act ? Act<E>::ld(qkv, base + (long)j * ld + 2 * C + h * D + lane) : 0.f;
  float dk = 0.f, dv = 0.f;
  const int iend = a.end[(long)b * T + j];
  const float* lse = a.lse + ((long)b * H + h) * T;
  const float* dlt = a.delta + ((long)b * H + h) * T;
  auto query = [&](float q, float g, float ls, float de) {
    float s = wave_sum(q * kv) * scale;
    float dp = wave_sum(g * vv);
    float p = __expf(s - ls);
    float ds = p * (dp - de);
    dv += p * g;
    dk += ds * q;
  };
  auto qld = [&](int i) { return act ? Act<E>::ld(qkv, base + (long)i * ld + h * D + lane) : 0.f; };
  auto gld = [&](int i) { return act ? Act<E>::ld(dout, ((long)b * T + i) * C + h * D + lane) : 0.f; };
  int i = j;
  for (; i + 3 < iend; i += kRowKeys) {
    float q[kRowKeys], g[kRowKeys], ls[kRowKeys], de[kRowKeys];
#pragma unroll
    for (int u = 0; u < kRowKeys; ++u) {
      q[u] = qld(i + u);
      g[u] = gld(i + u);
      ls[u] = lse[i + u];
      de[u] = dlt[i + u];
    }
#pragma unroll
    for (int u = 0; u < kRowKeys; ++u) query(q[u], g[u], ls[u], de[u]);
  }
  for (; i < iend; ++i) query(qld(i), gld(i), lse[i], dlt[i]);
  if (act) {
    E* d = reinterpret_cast<E*>(a.dqkv);
    Act<E>::st(d, ((long)b * T + j) * ld + C + h * D + lane, dk * scale);
    Act<E>::st(d, ((long)b * T + j) * ld + 2 * C + h * D + lane, dv);
  }
}

template <typename E>
static int attn_fwd_rows(const AttnArgs& a, hipStream_t s) {
  if (a.D > 64) return -1;
  long rows = (long)a.B * a.H * a.T;
  hipLaunchKernelGGL(attn_fwd_rows_kernel<E>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
  return 0;
}

template <typename E>
static int attn_bwd_rows_part(const AttnArgs& a, int part, hipStream_t s) {
  if (a.D > 64) return -1;
  long rows = (long)a.B * a.H * a.T;
  dim3 g((unsigned)((rows + 3) / 4)), b(256);
  if (part == 0) hipLaunchKernelGGL(attn_delta_kernel<E>, g, b, 0, s, a);
  else if (part == 1) hipLaunchKernelGGL(attn_dq_rows_kernel<E>, g, b, 0, s, a);
  else hipLaunchKernelGGL(attn_dkv_rows_kernel<E>, g, b, 0, s, a);
  return 0;
}

int attn_fwd_f32(const AttnArgs& a, hipStream_t s) { return attn_fwd_rows<float>(a, s); }
int attn_bwd_part_f32(const AttnArgs& a, int part, hipStream_t s) { return attn_bwd_rows_part<float>(a, part, s); }
int attn_bwd_f32(const AttnArgs& a, hipStream_t s) {
  int rc = 0;
  for (int part = 0; part < 3; ++part) rc |= attn_bwd_part_f32(a, part, s);
  return rc;
}

}  // namespace lm
