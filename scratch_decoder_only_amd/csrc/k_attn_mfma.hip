// Causal (optionally block-diagonal) multi-head self-attention on the gfx950
// matrix cores, bf16 operands with fp32 accumulation.
//
// What is computed (Feste page, "Model Architecture": scores of future
// positions are -inf before the softmax; 768 = 12 heads x 64): for query i and
// key j of one head, s_ij = q_i . k_j / sqrt(D) if start(i) <= j <= i, else
// -inf; P = softmax over j; o_i = sum_j P_ij v_j; lse_i = log sum_j exp(s_ij).
// Backward (Feste page, "Manual Backpropagation"): P is recomputed from lse;
// dP = dO V^T, dS = P (dP - delta_i) with delta_i = dO_i . O_i,
// dQ = dS K / sqrt(D), dK = dS^T Q / sqrt(D), dV = P^T dO.
//
// gfx950 design. Every block has 4 wavefronts of 64 lanes; a wavefront owns
// 32 rows (queries in the forward and dQ passes, keys in the dK/dV pass) and
// walks 64-row tiles of the other side staged in LDS. The MFMA is
// v_mfma_f32_32x32x16_bf16 (lane l holds row l%32 of a 32x16 operand, k-slots
// 8(l/32)..8(l/32)+7; the 32x32 result gives lane l column l%32 and rows
// 8(e/4) + 4(l/32) + e%4, e = 0..15).
// Forward and dQ compute S^T = K Q^T, so lane l keeps one query (l%32): the
// running max and sum of the online softmax are per lane (two lanes, l and
// l^32, share a query and combine once per tile), and O^T += V^T P^T takes P
// straight from registers as the B operand. The key order inside an MFMA
// k-step is the order in which the lane holds its scores; V^T (and K^T) are
// read from LDS in that same order, so nothing is shuffled. dK/dV computes
// S = Q K^T so lane l keeps one key. There are no atomics: dQ and dK/dV are
// separate passes (P is recomputed in each), so results are bit-reproducible.
// Tiles of a block are skipped outside [start of its first query, its last
// query], so the block-diagonal mask of packed rows costs only the pairs it
// keeps (plus the partial tiles on its edges).
#include "kernels.h"

namespace lm {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Cfg {
  static constexpr int KS = D / 16;   // MFMA k-steps over the head dimension
  static constexpr int DT = D / 32;   // 32-wide tiles of the head dimension
  static constexpr int RP = D + 8;    // LDS pitch (bf16) of a row-major [rows][D] tile
  static constexpr int TP = 64 + 4;   // LDS pitch (bf16) of a transposed [D][64] tile
};

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

__device__ __forceinline__ bf16x8_t as_frag(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint4 pack_frag(const float* v) {
  return make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// Row-major tile: rows r0..r0+63 (zero beyond T) of a [*, ld] matrix,
// columns col0..col0+D-1 -> s[r][0..D) with pitch RP.
template <int D>
__device__ __forceinline__ void load_rows(bf16* __restrict__ s, const bf16* __restrict__ g, long ld, int r0, int T,
                                          int col0, int tid) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
  for (int c = tid; c < 64 * CH; c += 256) {
    int r = c / CH, k = c % CH;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + r < T) v = *reinterpret_cast<const uint4*>(g + (long)(r0 + r) * ld + col0 + k * 8);
    *reinterpret_cast<uint4*>(s + r * Cfg<D>::RP + k * 8) = v;
  }
}

// Transposed tile: s[d][r] = g[r0 + r][col0 + d] for r < 64 (zero beyond T),
// pitch TP. 8 x 8 blocks are transposed in registers.
template <int D>
__device__ __forceinline__ void load_cols(bf16* __restrict__ s, const bf16* __restrict__ g, long ld, int r0, int T,
                                          int col0, int tid) {
  constexpr int NB = 8 * (D / 8);
  for (int b = tid; b < NB; b += 256) {
    int rb = b % 8, db = b / 8;
    uint4 in[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int r = r0 + rb * 8 + j;
      in[j] = r < T ? *reinterpret_cast<const uint4*>(g + (long)r * ld + col0 + db * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t lo = word_of(in[2 * j], c >> 1), hi = word_of(in[2 * j + 1], c >> 1);
        o[j] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      bf16* dst = s + (db * 8 + c) * Cfg<D>::TP + rb * 8;
      *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
      *reinterpret_cast<uint2*>(dst + 4) = make_uint2(o[2], o[3]);
    }
  }
}

// A-operand fragment of a transposed tile: rows d (lane%32 of tile dt), the 8
// k-slots of k-step group `base` in the lanes' hold order: base + 4h + 0..3
// and base + 8 + 4h + 0..3 (h = lane / 32).
template <int D>
__device__ __forceinline__ bf16x8_t frag_t(const bf16* __restrict__ s, int dt, int base, int lane) {
  const bf16* p = s + (dt * 32 + (lane & 31)) * Cfg<D>::TP + base + (lane >> 5) * 4;
  uint2 a = *reinterpret_cast<const uint2*>(p);
  uint2 b = *reinterpret_cast<const uint2*>(p + 8);
  return as_frag(make_uint4(a.x, a.y, b.x, b.y));
}

// Operand fragment of a row-major tile: row r0 + lane%32, k-step ks.
template <int D>
__device__ __forceinline__ bf16x8_t frag_r(const bf16* __restrict__ s, int r0, int ks, int lane) {
  return *reinterpret_cast<const bf16x8_t*>(s + (r0 + (lane & 31)) * Cfg<D>::RP + ks * 16 + (lane >> 5) * 8);
}

// Register fragments of rows row0 + lane%32 straight from global memory.
template <int D>
__device__ __forceinline__ void frags_global(bf16x8_t* f, const bf16* __restrict__ g, long ld, int row, int T,
                                             int col0, int lane) {
#pragma unroll
  for (int ks = 0; ks < Cfg<D>::KS; ++ks) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < T) v = *reinterpret_cast<const uint4*>(g + (long)row * ld + col0 + ks * 16 + (lane >> 5) * 8);
    f[ks] = as_frag(v);
  }
}

__device__ __forceinline__ int acc_row(int e, int lane) { return (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3); }

// Store 16 accumulators of one 32-wide d tile for row `row`: d = dt*32 +
// acc_row(e) -> four 8-byte stores of 4 consecutive bf16.
__device__ __forceinline__ void store_acc_row(bf16* __restrict__ dst, const f32x16_t& acc, float scale, int lane) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    int d = g * 8 + (lane >> 5) * 4;
    uint2 w = make_uint2(pack2(acc[4 * g] * scale, acc[4 * g + 1] * scale),
                         pack2(acc[4 * g + 2] * scale, acc[4 * g + 3] * scale));
    *reinterpret_cast<uint2*>(dst + d) = w;
  }
}

// ----------------------------------------------------------------- forward
template <int D>
__global__ void __launch_bounds__(256) attn_fwd_kernel(AttnArgs a) {
  using C_ = Cfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 sK[64 * C_::RP];
  __shared__ __attribute__((aligned(16))) bf16 sVt[D * C_::TP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T = a.T, H = a.H, C = H * D;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int q0 = blockIdx.x * 128;
  const long ld = 3L * C;
  const bf16* base = reinterpret_cast<const bf16*>(a.qkv) + (long)b * T * ld;
  const int32_t* start = a.start + (long)b * T;

  const int q = q0 + w * 32 + (lane & 31);
  const bool qv = q < T;
  const int qs = qv ? start[q] : 0;
  bf16x8_t qf[C_::KS];
  frags_global<D>(qf, base, ld, q, T, h * D, lane);

  const float sc = kLog2e / sqrtf((float)D);
  float m = -INFINITY, l = 0.f;
  f32x16_t acc_o[C_::DT];
#pragma unroll
  for (int dt = 0; dt < C_::DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc_o[dt][e] = 0.f;

  const int k_lo = start[q0];
  const int k_hi = min(T, q0 + 128) - 1;
  for (int kt = k_lo / 64; kt <= k_hi / 64; ++kt) {
    const int k0 = kt * 64;
    __syncthreads();
    load_rows<D>(sK, base, ld, k0, T, C + h * D, tid);
    load_cols<D>(sVt, base, ld, k0, T, 2 * C + h * D, tid);
    __syncthreads();
    // S^T for 2 sub-tiles of 32 keys
    f32x16_t s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[sub][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C_::KS; ++ks)
        s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_r<D>(sK, sub * 32, ks, lane), qf[ks], s[sub], 0, 0, 0);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        int j = k0 + sub * 32 + acc_row(e, lane);
        float v = (qv && j >= qs && j <= q) ? s[sub][e] * sc : -INFINITY;
        s[sub][e] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(m, mt);
    const float corr = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
    float p[2][16];
    float ls = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = (mn == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[sub][e] - mn);
        p[sub][e] = v;
        ls += v;
      }
    l = l * corr + ls;
    m = mn;
#pragma unroll
    for (int dt = 0; dt < C_::DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_o[dt][e] *= corr;
    // O^T += V^T P^T over 4 k-steps of 16 keys
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x8_t pf = as_frag(pack_frag(&p[st >> 1][(st & 1) * 8]));
#pragma unroll
      for (int dt = 0; dt < C_::DT; ++dt)
        acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_t<D>(sVt, dt, st * 16, lane), pf, acc_o[dt], 0, 0, 0);
    }
  }
  l += __shfl_xor(l, 32, 64);
  if (qv) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16* orow = reinterpret_cast<bf16*>(a.o) + ((long)b * T + q) * C + h * D;
#pragma unroll
    for (int dt = 0; dt < C_::DT; ++dt) store_acc_row(orow + dt * 32, acc_o[dt], inv, lane);
    if (lane < 32) a.lse[((long)b * H + h) * T + q] = (m + __log2f(l)) * 0.6931471805599453f;
  }
}

// ---------------------------------------------------------------- delta
// delta_i = dO_i . O_i, one wavefront per (row, head), D/8 lanes x 8 values.
template <int D>
__global__ void __launch_bounds__(256) attn_delta_kernel_v(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  constexpr int LPR = D / 8;  // lanes per (row, head)
  const long idx = ((long)blockIdx.x * 256 + threadIdx.x) / LPR;  // (b, t, h) flat
  const int sub = threadIdx.x % LPR;
  const int H = a.H, T = a.T, C = H * D;
  const long total = (long)a.B * T * H;
  float v = 0.f;
  if (idx < total) {
    const int hh = idx % H;
    const long row = idx / H;
    const long off = row * C + hh * D + sub * 8;
    uint4 x = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16*>(a.dout) + off);
    uint4 y = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16*>(a.o) + off);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t xa = word_of(x, k), ya = word_of(y, k);
      v += __uint_as_float(xa << 16) * __uint_as_float(ya << 16);
      v += __uint_as_float(xa & 0xffff0000u) * __uint_as_float(ya & 0xffff0000u);
    }
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (idx < total && sub == 0) {
    const int hh = idx % H;
    const long row = idx / H;
    const long bb = row / T, t = row % T;
    a.delta[(bb * H + hh) * T + t] = v;
  }
  (void)lane;
}

// ------------------------------------------------------------ dQ pass
template <int D>
__global__ void __launch_bounds__(256) attn_dq_kernel(AttnArgs a) {
  using C_ = Cfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 sK[64 * C_::RP];
  __shared__ __attribute__((aligned(16))) bf16 sV[64 * C_::RP];
  __shared__ __attribute__((aligned(16))) bf16 sKt[D * C_::TP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T = a.T, H = a.H, C = H * D;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int q0 = blockIdx.x * 128;
  const long ld = 3L * C;
  const bf16* base = reinterpret_cast<const bf16*>(a.qkv) + (long)b * T * ld;
  const bf16* dob = reinterpret_cast<const bf16*>(a.dout) + (long)b * T * C;
  const int32_t* start = a.start + (long)b * T;

  const int q = q0 + w * 32 + (lane & 31);
  const bool qv = q < T;
  const int qs = qv ? start[q] : 0;
  const float lse2 = qv ? a.lse[((long)b * H + h) * T + q] * kLog2e : 0.f;
  const float dlt = qv ? a.delta[((long)b * H + h) * T + q] : 0.f;
  bf16x8_t qf[C_::KS], df[C_::KS];
  frags_global<D>(qf, base, ld, q, T, h * D, lane);
  frags_global<D>(df, dob, C, q, T, h * D, lane);
  const float sc = kLog2e / sqrtf((float)D);
  f32x16_t acc[C_::DT];
#pragma unroll
  for (int dt = 0; dt < C_::DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;

  const int k_lo = start[q0];
  const int k_hi = min(T, q0 + 128) - 1;
  for (int kt = k_lo / 64; kt <= k_hi / 64; ++kt) {
    const int k0 = kt * 64;
    __syncthreads();
    load_rows<D>(sK, base, ld, k0, T, C + h * D, tid);
    load_rows<D>(sV, base, ld, k0, T, 2 * C + h * D, tid);
    load_cols<D>(sKt, base, ld, k0, T, C + h * D, tid);
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16_t s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C_::KS; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_r<D>(sK, sub * 32, ks, lane), qf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_r<D>(sV, sub * 32, ks, lane), df[ks], dp, 0, 0, 0);
      }
      float ds[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        int j = k0 + sub * 32 + acc_row(e, lane);
        float p = (qv && j >= qs && j <= q) ? __builtin_amdgcn_exp2f(s[e] * sc - lse2) : 0.f;
        ds[e] = p * (dp[e] - dlt);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8_t f = as_frag(pack_frag(&ds[st * 8]));
#pragma unroll
        for (int dt = 0; dt < C_::DT; ++dt)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_t<D>(sKt, dt, sub * 32 + st * 16, lane), f, acc[dt],
                                                            0, 0, 0);
      }
    }
  }
  if (qv) {
    const float scale = 1.0f / sqrtf((float)D);
    bf16* row = reinterpret_cast<bf16*>(a.dqkv) + ((long)b * T + q) * ld + h * D;
#pragma unroll
    for (int dt = 0; dt < C_::DT; ++dt) store_acc_row(row + dt * 32, acc[dt], scale, lane);
  }
}

// ---------------------------------------------------------- dK / dV pass
template <int D>
__global__ void __launch_bounds__(256) attn_dkv_kernel(AttnArgs a) {
  using C_ = Cfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 sQ[64 * C_::RP];
  __shared__ __attribute__((aligned(16))) bf16 sdO[64 * C_::RP];
  __shared__ __attribute__((aligned(16))) bf16 sQt[D * C_::TP];
  __shared__ __attribute__((aligned(16))) bf16 sdOt[D * C_::TP];
  __shared__ float sL[64], sD[64];
  __shared__ int sS[64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T = a.T, H = a.H, C = H * D;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int kb0 = blockIdx.x * 128;
  const long ld = 3L * C;
  const bf16* base = reinterpret_cast<const bf16*>(a.qkv) + (long)b * T * ld;
  const bf16* dob = reinterpret_cast<const bf16*>(a.dout) + (long)b * T * C;
  const int32_t* start = a.start + (long)b * T;
  const float* lse = a.lse + ((long)b * H + h) * T;
  const float* dl = a.delta + ((long)b * H + h) * T;

  const int key = kb0 + w * 32 + (lane & 31);
  const bool kv = key < T;
  bf16x8_t kf[C_::KS], vf[C_::KS];
  frags_global<D>(kf, base, ld, key, T, C + h * D, lane);
  frags_global<D>(vf, base, ld, key, T, 2 * C + h * D, lane);
  const float sc = kLog2e / sqrtf((float)D);
  f32x16_t dk[C_::DT], dv[C_::DT];
#pragma unroll
  for (int dt = 0; dt < C_::DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[dt][e] = dv[dt][e] = 0.f;

  const int q_lo = kb0;
  const int q_hi = a.end[(long)b * T + min(T, kb0 + 128) - 1] - 1;
  for (int qt = q_lo / 64; qt <= q_hi / 64; ++qt) {
    const int qb = qt * 64;
    __syncthreads();
    load_rows<D>(sQ, base, ld, qb, T, h * D, tid);
    load_rows<D>(sdO, dob, C, qb, T, h * D, tid);
    load_cols<D>(sQt, base, ld, qb, T, h * D, tid);
    load_cols<D>(sdOt, dob, C, qb, T, h * D, tid);
    if (tid < 64) {
      int qq = qb + tid;
      bool ok = qq < T;
      sL[tid] = ok ? lse[qq] * kLog2e : 0.f;
      sD[tid] = ok ? dl[qq] : 0.f;
      sS[tid] = ok ? start[qq] : T;  // rows beyond T admit no key
    }
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16_t s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C_::KS; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_r<D>(sQ, sub * 32, ks, lane), kf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_r<D>(sdO, sub * 32, ks, lane), vf[ks], dp, 0, 0, 0);
      }
      float p[16], ds[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        int r = sub * 32 + acc_row(e, lane);
        int qq = qb + r;
        bool ok = kv && key >= sS[r] && key <= qq;
        float pv = ok ? __builtin_amdgcn_exp2f(s[e] * sc - sL[r]) : 0.f;
        p[e] = pv;
        ds[e] = pv * (dp[e] - sD[r]);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8_t pf = as_frag(pack_frag(&p[st * 8]));
        bf16x8_t sf = as_frag(pack_frag(&ds[st * 8]));
#pragma unroll
        for (int dt = 0; dt < C_::DT; ++dt) {
          dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_t<D>(sdOt, dt, sub * 32 + st * 16, lane), pf, dv[dt],
                                                           0, 0, 0);
          dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_t<D>(sQt, dt, sub * 32 + st * 16, lane), sf, dk[dt],
                                                           0, 0, 0);
        }
      }
    }
  }
  if (kv) {
    const float scale = 1.0f / sqrtf((float)D);
    bf16* row = reinterpret_cast<bf16*>(a.dqkv) + ((long)b * T + key) * ld;
#pragma unroll
    for (int dt = 0; dt < C_::DT; ++dt) {
      store_acc_row(row + C + h * D + dt * 32, dk[dt], scale, lane);
      store_acc_row(row + 2 * C + h * D + dt * 32, dv[dt], 1.0f, lane);
    }
  }
}

template <int D>
int fwd(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.T + 127) / 128, a.B * a.H);
  hipLaunchKernelGGL(attn_fwd_kernel<D>, grid, dim3(256), 0, s, a);
  return 0;
}

template <int D>
int bwd(const AttnArgs& a, hipStream_t s) {
  long rows = (long)a.B * a.T * a.H;
  long threads = rows * (D / 8);
  hipLaunchKernelGGL(attn_delta_kernel_v<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
  dim3 grid((a.T + 127) / 128, a.B * a.H);
  hipLaunchKernelGGL(attn_dq_kernel<D>, grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(attn_dkv_kernel<D>, grid, dim3(256), 0, s, a);
  return 0;
}

}  // namespace

int attn_fwd_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.D == 64) return fwd<64>(a, s);
  if (a.D == 32) return fwd<32>(a, s);
  return -1;
}

int attn_bwd_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.D == 64) return bwd<64>(a, s);
  if (a.D == 32) return bwd<32>(a, s);
  return -1;
}

}  // namespace lm
