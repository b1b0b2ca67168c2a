// Causal (optionally block-diagonal) multi-head self-attention on the gfx950
// matrix cores, 16-bit operands (bf16 or fp16, E) with fp32 accumulation.
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
// walks 64-row tiles of the other side, staged in LDS with a two-stage
// pipeline (the next tile's buffer loads are in flight during the MFMAs of the
// current one). The MFMA is v_mfma_f32_32x32x16_bf16 or _f16 (lane l holds row l%32 of
// a 32x16 operand, k-slots 8(l/32)..8(l/32)+7; the 32x32 result gives lane l
// column l%32 and rows 8(e/4) + 4(l/32) + e%4, e = 0..15).
// Forward and dQ compute S^T = K Q^T, so lane l keeps one query (l%32): the
// running max and sum of the online softmax are per lane (lanes l and l^32
// share a query and combine once per tile), and O^T += V^T P^T takes P
// straight from registers as the B operand. dK/dV computes S = Q K^T so lane l
// keeps one key. The k-slots of one MFMA step are taken in the order a lane
// holds its scores (slot j <-> row 8(j/4) + 4(l/32) + j%4 of the 16-row step);
// the transposed A operands (V^T, K^T, Q^T, dO^T) are read in that same order
// from the row-major LDS tiles with ds_read_b64_tr_b16, so no tile is ever
// transposed. There are no atomics: dQ and dK/dV are separate passes (P is
// recomputed in each), so results are bit-reproducible. Tiles outside
// [start of a block's first query, its last query] are skipped, so the
// block-diagonal mask of packed rows costs only the pairs it keeps (plus the
// partial tiles on its edges).
#include "kernels.h"

namespace lm {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;

// (an address-space cast, not a cast through an integer: the compiler keeps
// track of which LDS array the read addresses)
__device__ __forceinline__ bf16x4_t ds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(const __attribute__((address_space(3))) bf16*)p);
}

// Row-major [64 rows][D] LDS tile, 16-byte chunks XOR-swizzled per row so that
// both the 16-byte fragment reads of 16 consecutive rows and the transpose
// reads of 4 rows x 32 columns hit distinct banks.
template <int D>
struct RowTile {
  static constexpr int CH = D / 8;  // chunks per row
  static constexpr int ELEMS = 64 * D;
  static __device__ __forceinline__ int sw(int r) {
    if (D == 64) {
      const int x = (r >> 1) & 7;
      return ((x & 1) << 2) | (x >> 1);
    }
    return (r >> 2) & 3;
  }
  static __device__ __forceinline__ int off(int r, int c) { return r * D + ((c ^ sw(r)) << 3); }
};

// Fragments hold 8 raw 16-bit values; pairs of fp32 values become packed
// 16-bit pairs with one conversion instruction (round to nearest even).
__device__ __forceinline__ bf16x8_t as_frag(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
template <typename E>
__device__ __forceinline__ uint4 pack_frag(const float* v) {
  return make_uint4(H16<E>::pack(v[0], v[1]), H16<E>::pack(v[2], v[3]), H16<E>::pack(v[4], v[5]),
                    H16<E>::pack(v[6], v[7]));
}

// Loader of one 64-row tile (rows r0..r0+63 of a [T, ld] bf16 matrix, columns
// col0..col0+D-1) into a RowTile, through registers: buffer loads (rows past
// T read zeros), then LDS stores after the current tile's MFMAs.
template <int D>
struct TileLoad {
  static constexpr int N = 64 * D / 8 / 256;  // 16-byte chunks per thread (1 or 2)
  uint4 r[N];
  __amdgpu_buffer_rsrc_t rsrc;
  unsigned voff[N];
  int soff[N];
  long ld;
  __device__ __forceinline__ void init(const bf16* base, long ld_, int T, int col0, int tid) {
    ld = ld_;
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(base + col0), (short)0,
                                             (int)min(((long)(T - 1) * ld_ + D) * 2, (long)0x7fffffff), 0x00020000);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * 256;
      const int row = c / RowTile<D>::CH, ch = c % RowTile<D>::CH;
      voff[i] = (unsigned)(((long)row * ld_ + ch * 8) * 2);
      soff[i] = RowTile<D>::off(row, ch);
    }
  }
  // The whole byte offset is in the per-lane offset, which the range check
  // covers: rows at or past T read zeros.
  __device__ __forceinline__ void load(int r0) {
    const unsigned ro = (unsigned)r0 * (unsigned)(ld * 2);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(voff[i] + ro), 0, 0);
      r[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
  __device__ __forceinline__ void store(bf16* s) const {
#pragma unroll
    for (int i = 0; i < N; ++i) *reinterpret_cast<uint4*>(s + soff[i]) = r[i];
  }
};

// B/A operand fragment of rows r0 + lane%32 of a RowTile, k-step ks over D.
template <int D>
__device__ __forceinline__ bf16x8_t frag_r(const bf16* s, int r0, int ks, int lane) {
  const int r = r0 + (lane & 31), c = ks * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8_t*>(s + RowTile<D>::off(r, c));
}

// A operand "rows = d (tile dt), k-slots = 16 tile rows from base" of a
// RowTile, in the lanes' score order: slots 0..3 <-> rows base + 4h + 0..3,
// slots 4..7 <-> rows base + 8 + 4h + 0..3 (h = lane / 32). Two transpose
// reads: within each 16-lane group, source lane i reads row k0 + i/4, columns
// d0 + 4 (i % 4) .. + 3 and receives column d0 + i of rows k0 .. k0 + 3.
template <int D>
__device__ __forceinline__ bf16x8_t frag_t(const bf16* s, int dt, int base, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int d = dt * 32 + (g & 1) * 16 + 4 * (i & 3);
  const int k = base + (g >> 1) * 4 + (i >> 2);
  const int c = d >> 3, h = d & 7;
  bf16x4_t lo = ds_read_tr(s + RowTile<D>::off(k, c) + h);
  bf16x4_t hi = ds_read_tr(s + RowTile<D>::off(k + 8, c) + h);
  return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Register fragments of row `row` (zero past T) straight from global memory.
template <int D>
__device__ __forceinline__ void frags_global(bf16x8_t* f, const bf16* __restrict__ g, long ld, int row, int T,
                                             int col0, int lane) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < T) v = *reinterpret_cast<const uint4*>(g + (long)row * ld + col0 + ks * 16 + (lane >> 5) * 8);
    f[ks] = as_frag(v);
  }
}

__device__ __forceinline__ int acc_row(int e, int lane) { return (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3); }

// Store the 16 accumulators of one 32-wide d tile of row `dst`: d = acc_row(e).
template <typename E>
__device__ __forceinline__ void store_acc_row(bf16* __restrict__ dst, const f32x16_t& acc, float scale, int lane) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    int d = g * 8 + (lane >> 5) * 4;
    uint2 w = make_uint2(H16<E>::pack(acc[4 * g] * scale, acc[4 * g + 1] * scale),
                         H16<E>::pack(acc[4 * g + 2] * scale, acc[4 * g + 3] * scale));
    *reinterpret_cast<uint2*>(dst + d) = w;
  }
}

__device__ __forceinline__ void zero(f32x16_t& a) {
#pragma unroll
  for (int e = 0; e < 16; ++e) a[e] = 0.f;
}

// Work item of a block: (batch x head, first of its 128 rows). Under the
// causal mask a block's work grows with its query rows (forward, dQ) or
// shrinks with its key rows (dK/dV), so items are numbered longest first over
// the whole grid: item i takes size class i / (B H) and head row i % (B H).
// Consecutive blocks land on different XCDs, so every XCD gets the same mix
// of long and short items, and the long ones start first.
__device__ __forceinline__ void item_rows(const AttnArgs& a, bool queries, int& bh, int& r0) {
  const int BH = a.B * a.H, nt = (a.T + 127) / 128;
  const int k = blockIdx.x / BH;
  bh = blockIdx.x - k * BH;
  r0 = (queries ? nt - 1 - k : k) * 128;
}

// Occupancy: each kernel is compiled for as many wavefronts per SIMD as its
// registers allow without spilling (forward and dQ 3, dK/dV 2); left to
// itself the compiler took more registers (1-2 wavefronts per SIMD) and
// parked values in the accumulation registers, which measured 4-5% slower.

// ----------------------------------------------------------------- forward
template <int D, typename E>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) attn_fwd_kernel(AttnArgs a) {
  constexpr int KS = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 sK[2][RowTile<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][RowTile<D>::ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, H = a.H, C = H * D;
  int bh, q0;
  item_rows(a, true, bh, q0);
  const int b = bh / H, h = bh % H;
  const long ld = 3L * C;
  const bf16* base = reinterpret_cast<const bf16*>(a.qkv) + (long)b * T * ld;
  const int32_t* start = a.start + (long)b * T;

  const int qw0 = q0 + w * 32;
  const int q = qw0 + (lane & 31);
  const bool qv = q < T;
  const int qs = qv ? start[q] : 0;
  const bool wave_last_ok = qw0 + 31 < T;           // every query of the wave exists
  const int qs_last = __shfl(qs, 31, 64);           // start of the wave's last query
  // the smallest start of the wave's queries (starts never decrease along a
  // row); a wave with no query at all keeps every key masked
  const int qs_first = qw0 < T ? __builtin_amdgcn_readfirstlane(qs) : T;
  bf16x8_t qf[KS];
  frags_global<D>(qf, base, ld, q, T, h * D, lane);

  TileLoad<D> lk, lv;
  lk.init(base, ld, T, C + h * D, tid);
  lv.init(base, ld, T, 2 * C + h * D, tid);

  const float sc = kLog2e / sqrtf((float)D);
  float m = -INFINITY, l = 0.f;
  f32x16_t acc_o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) zero(acc_o[dt]);

  const int kt0 = start[q0] / 64, kt1 = (min(T, q0 + 128) - 1) / 64;
  lk.load(kt0 * 64);
  lv.load(kt0 * 64);
  lk.store(sK[0]);
  lv.store(sV[0]);
  __syncthreads();
  for (int kt = kt0; kt <= kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    const int k0 = kt * 64;
    if (kt < kt1) {
      lk.load(k0 + 64);
      lv.load(k0 + 64);
    }
    // 32-key halves of the tile that the mask removes for every query of the
    // wave (all keys after its last query, or before its first query's
    // start) add exact zeros: their matrix and softmax work is skipped
    // (wave-uniform tests)
    const bool live0 = k0 <= qw0 + 31 && k0 + 31 >= qs_first;
    const bool live1 = k0 + 32 <= qw0 + 31 && k0 + 63 >= qs_first;
    if (live0 || live1) {
    f32x16_t s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      zero(s[sub]);
      if (sub == 0 ? live0 : live1) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          s[sub] = mfma32<E>(frag_r<D>(sK[cur], sub * 32, ks, lane), qf[ks], s[sub]);
      }
    }
    // A tile every score of which is kept (all 64 keys at or before the
    // wave's first query and at or after its last query's start) needs no
    // mask: the max is taken on the raw scores and the scale folded into the
    // exponent.
    const bool full = wave_last_ok && k0 + 63 <= qw0 && qs_last <= k0;
    float mt = -INFINITY;
    float p[2][16];
    float ls = 0.f, mn;
    if (full) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, s[sub][e]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * sc;
      mn = fmaxf(m, mt);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float v = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][e], sc, -mn));
          p[sub][e] = v;
          ls += v;
        }
    } else {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = k0 + sub * 32 + acc_row(e, lane);
          const float v = (qv && j >= qs && j <= q) ? s[sub][e] * sc : -INFINITY;
          s[sub][e] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      mn = fmaxf(m, mt);
      // exp2(-inf) = 0 covers masked scores; a fully masked row so far keeps 0
      const float sub_mn = (mn == -INFINITY) ? 0.f : mn;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float v = __builtin_amdgcn_exp2f(s[sub][e] - sub_mn);
          p[sub][e] = v;
          ls += v;
        }
    }
    const float corr = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
    l = l * corr + ls;
    m = mn;
    // once the running maxima settle, no lane's changes: skip the rescale
    // (a wavefront-uniform test, so no divergence)
    if (__builtin_amdgcn_ballot_w64(corr != 1.f) != 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc_o[dt][e] *= corr;
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (!((st >> 1) == 0 ? live0 : live1)) continue;
      const bf16x8_t pf = as_frag(pack_frag<E>(&p[st >> 1][(st & 1) * 8]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        acc_o[dt] = mfma32<E>(frag_t<D>(sV[cur], dt, st * 16, lane), pf, acc_o[dt]);
    }
    }
    if (kt < kt1) {
      lk.store(sK[cur ^ 1]);
      lv.store(sV[cur ^ 1]);
    }
    __syncthreads();
  }
  l += __shfl_xor(l, 32, 64);
  if (qv) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16* orow = reinterpret_cast<bf16*>(a.o) + ((long)b * T + q) * C + h * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) store_acc_row<E>(orow + dt * 32, acc_o[dt], inv, lane);
    if (lane < 32) a.lse[((long)b * H + h) * T + q] = (m + __log2f(l)) * 0.6931471805599453f;
  }
}

// ------------------------------------------------------------ dQ pass
template <int D, typename E>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) attn_dq_kernel(AttnArgs a) {
  constexpr int KS = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 sK[2][RowTile<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][RowTile<D>::ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, H = a.H, C = H * D;
  int bh, q0;
  item_rows(a, true, bh, q0);
  const int b = bh / H, h = bh % H;
  const long ld = 3L * C;
  const bf16* base = reinterpret_cast<const bf16*>(a.qkv) + (long)b * T * ld;
  const bf16* dob = reinterpret_cast<const bf16*>(a.dout) + (long)b * T * C;
  const int32_t* start = a.start + (long)b * T;

  const int qw0 = q0 + w * 32;
  const int q = qw0 + (lane & 31);
  const bool qv = q < T;
  const int qs = qv ? start[q] : 0;
  const bool wave_last_ok = qw0 + 31 < T;
  const int qs_last = __shfl(qs, 31, 64);
  const int qs_first = qw0 < T ? __builtin_amdgcn_readfirstlane(qs) : T;
  const float lse2 = qv ? a.lse[((long)b * H + h) * T + q] * kLog2e : 0.f;
  bf16x8_t qf[KS], df[KS];
  frags_global<D>(qf, base, ld, q, T, h * D, lane);
  frags_global<D>(df, dob, C, q, T, h * D, lane);
  // delta_q = dO_q . O_q (lanes l and l ^ 32 hold the two halves of the row);
  // written out for the dK/dV pass, which runs after this one
  float dlt;
  {
    bf16x8_t of[KS];
    frags_global<D>(of, reinterpret_cast<const bf16*>(a.o) + (long)b * T * C, C, q, T, h * D, lane);
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 x = __builtin_bit_cast(uint4, df[ks]), y = __builtin_bit_cast(uint4, of[ks]);
      const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, yw[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        part += H16<E>::lo(xw[i]) * H16<E>::lo(yw[i]);
        part += H16<E>::hi(xw[i]) * H16<E>::hi(yw[i]);
      }
    }
    dlt = part + __shfl_xor(part, 32, 64);
    if (qv && lane < 32) a.delta[((long)b * H + h) * T + q] = dlt;
  }
  TileLoad<D> lk, lv;
  lk.init(base, ld, T, C + h * D, tid);
  lv.init(base, ld, T, 2 * C + h * D, tid);
  const float sc = kLog2e / sqrtf((float)D);
  f32x16_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) zero(acc[dt]);

  const int kt0 = start[q0] / 64, kt1 = (min(T, q0 + 128) - 1) / 64;
  lk.load(kt0 * 64);
  lv.load(kt0 * 64);
  lk.store(sK[0]);
  lv.store(sV[0]);
  __syncthreads();
  for (int kt = kt0; kt <= kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    const int k0 = kt * 64;
    if (kt < kt1) {
      lk.load(k0 + 64);
      lv.load(k0 + 64);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kb = k0 + sub * 32;
      // a 32-key block the mask removes for every query of the wave (after
      // its last query, or before its first query's start) adds exact zeros
      if (kb > qw0 + 31 || kb + 31 < qs_first) continue;
      f32x16_t s, dp;
      zero(s);
      zero(dp);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32<E>(frag_r<D>(sK[cur], sub * 32, ks, lane), qf[ks], s);
        dp = mfma32<E>(frag_r<D>(sV[cur], sub * 32, ks, lane), df[ks], dp);
      }
      float ds[16];
      if (wave_last_ok && kb + 31 <= qw0 && qs_last <= kb) {
        // every score of this 32 x 32 block is kept
#pragma unroll
        for (int e = 0; e < 16; ++e) ds[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], sc, -lse2)) * (dp[e] - dlt);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = kb + acc_row(e, lane);
          const bool ok = qv && j >= qs && j <= q;
          ds[e] = __builtin_amdgcn_exp2f(ok ? __builtin_fmaf(s[e], sc, -lse2) : -INFINITY) * (dp[e] - dlt);
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8_t f = as_frag(pack_frag<E>(&ds[st * 8]));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          acc[dt] = mfma32<E>(frag_t<D>(sK[cur], dt, sub * 32 + st * 16, lane), f,
                                                            acc[dt]);
      }
    }
    if (kt < kt1) {
      lk.store(sK[cur ^ 1]);
      lv.store(sV[cur ^ 1]);
    }
    __syncthreads();
  }
  if (qv) {
    const float scale = 1.0f / sqrtf((float)D);
    bf16* row = reinterpret_cast<bf16*>(a.dqkv) + ((long)b * T + q) * ld + h * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) store_acc_row<E>(row + dt * 32, acc[dt], scale, lane);
  }
}

// ---------------------------------------------------------- dK / dV pass
template <int D, typename E>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_dkv_kernel(AttnArgs a) {
  constexpr int KS = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 sQ[2][RowTile<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 sdO[2][RowTile<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) float sL[2][64];
  __shared__ __attribute__((aligned(16))) float sD[2][64];
  __shared__ __attribute__((aligned(16))) int sS[2][64];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, H = a.H, C = H * D;
  int bh, kb0;
  item_rows(a, false, bh, kb0);
  const int b = bh / H, h = bh % H;
  const long ld = 3L * C;
  const bf16* base = reinterpret_cast<const bf16*>(a.qkv) + (long)b * T * ld;
  const bf16* dob = reinterpret_cast<const bf16*>(a.dout) + (long)b * T * C;
  const int32_t* start = a.start + (long)b * T;
  const float* lse = a.lse + ((long)b * H + h) * T;
  const float* dl = a.delta + ((long)b * H + h) * T;

  const int kw0 = kb0 + w * 32;
  const int key = kw0 + (lane & 31);
  const bool kv = key < T;
  const bool wave_keys_ok = kw0 + 31 < T;  // every key of the wave exists
  bf16x8_t kf[KS], vf[KS];
  frags_global<D>(kf, base, ld, key, T, C + h * D, lane);
  frags_global<D>(vf, base, ld, key, T, 2 * C + h * D, lane);
  TileLoad<D> lq, ldo;
  lq.init(base, ld, T, h * D, tid);
  ldo.init(dob, C, T, h * D, tid);
  const float sc = kLog2e / sqrtf((float)D);
  f32x16_t dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    zero(dk[dt]);
    zero(dv[dt]);
  }
  auto load_vec = [&](int qb, int stage) {
    if (tid < 64) {
      const int qq = qb + tid;
      const bool ok = qq < T;
      sL[stage][tid] = ok ? lse[qq] * kLog2e : 0.f;
      sD[stage][tid] = ok ? -dl[qq] : 0.f;  // negated: the dP accumulators start from it
      sS[stage][tid] = ok ? start[qq] : T;  // rows past T admit no key
    }
  };

  const int qt0 = kb0 / 64;
  const int qt1 = (a.end[(long)b * T + min(T, kb0 + 128) - 1] - 1) / 64;
  lq.load(qt0 * 64);
  ldo.load(qt0 * 64);
  lq.store(sQ[0]);
  ldo.store(sdO[0]);
  load_vec(qt0 * 64, 0);
  __syncthreads();
  // one 64-query tile in stage CUR (compile-time: every LDS read is a per-lane
  // address plus an immediate offset)
  auto tile = [&](auto CUR_, int qt) {
    constexpr int cur = decltype(CUR_)::value;
    const int qb = qt * 64;
    if (qt < qt1) {
      lq.load(qb + 64);
      ldo.load(qb + 64);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      // a 32-query block the mask removes for every key of the wave (all its
      // queries before the wave's first key, or all their starts after its
      // last key; the block's first query has the smallest start, and rows
      // past T have start T) adds exact zeros
      if (qb + sub * 32 + 31 < kw0 || __builtin_amdgcn_readfirstlane(sS[cur][sub * 32]) > kw0 + 31) continue;
      // rows of element e: sub*32 + acc_row(e), four consecutive rows per
      // group of four elements, read as one vector. dP starts from -delta of
      // its row (read straight into the accumulators), so the MFMAs leave
      // dP - delta.
      f32x16_t s, dp;
      zero(s);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t D4 = *reinterpret_cast<const f32x4_t*>(&sD[cur][sub * 32 + g * 8 + (lane >> 5) * 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) dp[4 * g + i] = D4[i];
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32<E>(frag_r<D>(sQ[cur], sub * 32, ks, lane), kf[ks], s);
        dp = mfma32<E>(frag_r<D>(sdO[cur], sub * 32, ks, lane), vf[ks], dp);
      }
      float p[16], ds[16];
      const int rq = qb + sub * 32;  // first query of this 32-query block
      const bool full = wave_keys_ok && kw0 + 31 <= rq && rq + 31 < T && sS[cur][sub * 32 + 31] <= kw0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = sub * 32 + g * 8 + (lane >> 5) * 4;
        const f32x4_t L4 = *reinterpret_cast<const f32x4_t*>(&sL[cur][r0]);
        if (full) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + i], sc, -L4[i]));
            p[4 * g + i] = pv;
            ds[4 * g + i] = pv * dp[4 * g + i];
          }
        } else {
          const int4 S4 = *reinterpret_cast<const int4*>(&sS[cur][r0]);
          const int st4[4] = {S4.x, S4.y, S4.z, S4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // (non-short-circuit: the start read is not made conditional)
            const bool ok = kv & (key >= st4[i]) & (key <= qb + r0 + i);
            const float pv = __builtin_amdgcn_exp2f(ok ? __builtin_fmaf(s[4 * g + i], sc, -L4[i]) : -INFINITY);
            p[4 * g + i] = pv;
            ds[4 * g + i] = pv * dp[4 * g + i];
          }
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8_t pf = as_frag(pack_frag<E>(&p[st * 8]));
        const bf16x8_t sf = as_frag(pack_frag<E>(&ds[st * 8]));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          dv[dt] = mfma32<E>(frag_t<D>(sdO[cur], dt, sub * 32 + st * 16, lane), pf, dv[dt]);
          dk[dt] = mfma32<E>(frag_t<D>(sQ[cur], dt, sub * 32 + st * 16, lane), sf, dk[dt]);
        }
      }
    }
    if (qt < qt1) {
      lq.store(sQ[cur ^ 1]);
      ldo.store(sdO[cur ^ 1]);
      load_vec(qb + 64, cur ^ 1);
    }
    __syncthreads();
  };
  int qt = qt0;
  for (; qt + 1 <= qt1; qt += 2) {
    tile(std::integral_constant<int, 0>{}, qt);
    tile(std::integral_constant<int, 1>{}, qt + 1);
  }
  if (qt <= qt1) tile(std::integral_constant<int, 0>{}, qt);
  if (kv) {
    const float scale = 1.0f / sqrtf((float)D);
    bf16* row = reinterpret_cast<bf16*>(a.dqkv) + ((long)b * T + key) * ld;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      store_acc_row<E>(row + C + h * D + dt * 32, dk[dt], scale, lane);
      store_acc_row<E>(row + 2 * C + h * D + dt * 32, dv[dt], 1.0f, lane);
    }
  }
}

template <int D, typename E>
int fwd(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.T + 127) / 128 * a.B * a.H);
  hipLaunchKernelGGL((attn_fwd_kernel<D, E>), grid, dim3(256), 0, s, a);
  return 0;
}

// Backward in passes: part 0 (row dot products delta) has nothing left to do
// here, the dQ pass (part 1) computes and stores delta for its rows before
// the dK/dV pass (part 2) reads it.
template <int D, typename E>
int bwd_part(const AttnArgs& a, int part, hipStream_t s) {
  dim3 grid((a.T + 127) / 128 * a.B * a.H);
  if (part == 0) {
    return 0;
  } else if (part == 1) {
    hipLaunchKernelGGL((attn_dq_kernel<D, E>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_dkv_kernel<D, E>), grid, dim3(256), 0, s, a);
  }
  return 0;
}

}  // namespace

template <typename E>
int attn_fwd16(const AttnArgs& a, hipStream_t s) {
  if (a.D == 64) return fwd<64, E>(a, s);
  if (a.D == 32) return fwd<32, E>(a, s);
  return -1;
}

template <typename E>
int attn_bwd_part16(const AttnArgs& a, int part, hipStream_t s) {
  if (a.D == 64) return bwd_part<64, E>(a, part, s);
  if (a.D == 32) return bwd_part<32, E>(a, part, s);
  return -1;
}

template <typename E>
int attn_bwd16(const AttnArgs& a, hipStream_t s) {
  int rc = 0;
  for (int part = 0; part < 3; ++part) rc |= attn_bwd_part16<E>(a, part, s);
  return rc;
}

template int attn_fwd16<bf16>(const AttnArgs&, hipStream_t);
template int attn_fwd16<f16>(const AttnArgs&, hipStream_t);
template int attn_bwd_part16<bf16>(const AttnArgs&, int, hipStream_t);
template int attn_bwd_part16<f16>(const AttnArgs&, int, hipStream_t);
template int attn_bwd16<bf16>(const AttnArgs&, hipStream_t);
template int attn_bwd16<f16>(const AttnArgs&, hipStream_t);

}  // namespace lm
